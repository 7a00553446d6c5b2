"""CPU oracle for the FP16 x INT4 (group-128) linear layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The GPU library never loads it, and it loads nothing from the GPU library.

Two independent implementations live here:

* ``oracle.c`` (built into ``liboracle.so``): the plain C reference.  ``gemm(..., mode="f32")``
  accumulates in fp32 with k ascending and rounds to fp16 once, the precision the pages fix
  (Marlin deep-dive page "Marlin 完全拆解", section "让多个 warp 计算同一个输出 tile 的部分和":
  FP32 accumulators, FP16 only at write-out).  ``mode="f64"`` is the diagnostic truth.
* ``exact_gemm`` below: exact integer arithmetic on the dyadic values, correctly rounded to
  fp16 by its own routine.  It is slow and only for tiny shapes; it pins the C code.
* ``decode_along_k`` / ``decode_along_n``: checkpoint-style packed words (8 codes per word,
  along K or along N in a given nibble order) to codes, what the load-time repack must move.

2:4-sparse weights (MARLIN paper, sec. 1 "Contribution" and sec. 2.1.1: of every 4 consecutive
weights along K two are zero; Sparse-MARLIN section of the deep-dive page) need no routine of
their own: the product is the same definition with the pruned weights zero, i.e. code 8 in the
symmetric format, and ``gemm`` computes it from those dense codes.

A mixture-of-experts layer (deep-dive page, the section on where the format pays off, items 1
and 4: the layer regroups tokens by expert, so each expert's product has its own M) is
``moe_align`` (the regrouping) and ``moe_gemm`` (each assignment's row times its expert's
dequantised weights), in fp64 with one rounding to fp16 or bfloat16 (``bf16_round``).

The operation (MARLIN paper, arXiv 2408.11743, sec. 3.4 "Kernel Design"; deep-dive page,
section "Marlin 要解决的精确问题"):  C = A * Bhat,  Bhat[k, n] = s[k // group, n] * (q[k, n] - z),
z = 8 (symmetric) or a zero-point code z[k // group, n] in 0..15 (the page's general affine
form s_{g,n}(q_{k,n} - z_{g,n})).  group = 128, or group = K for one scale per column.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc.  -ffp-contract=off keeps multiply and add separate."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-pthread", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    p = ctypes.c_void_p
    i = ctypes.c_int
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_double_to_half.argtypes = [ctypes.c_double]
    lib.oracle_double_to_half.restype = ctypes.c_uint16
    lib.oracle_float_to_half.argtypes = [ctypes.c_float]
    lib.oracle_float_to_half.restype = ctypes.c_uint16
    lib.oracle_dequant.argtypes = [ctypes.c_uint8, ctypes.c_uint16]
    lib.oracle_dequant.restype = ctypes.c_double
    lib.oracle_dequant_zp.argtypes = [ctypes.c_uint8, ctypes.c_uint16, ctypes.c_uint8]
    lib.oracle_dequant_zp.restype = ctypes.c_double
    for name in ("oracle_gemm_zp_f32", "oracle_gemm_zp_f64"):
        fn = getattr(lib, name)
        fn.argtypes = [p, p, p, p, i, i, i, i, p, i]
        fn.restype = i
    for name in ("oracle_gemm_f32", "oracle_gemm_f64"):
        fn = getattr(lib, name)
        fn.argtypes = [p, p, p, i, i, i, i, p, i]
        fn.restype = i
    lib.oracle_gemv_f32.argtypes = [p, p, p, i, i, i, p]
    lib.oracle_gemv_f32.restype = i
    _lib = lib
    return lib


def lib():
    return _load()


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def default_threads() -> int:
    """Threads for the C oracle when the caller names none: the cores this process may use,
    capped by OMP_NUM_THREADS where the environment sets the process's CPU share.  (Any
    count gives the same bits: each output is summed by one thread in a fixed order.)"""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def gemm(A: np.ndarray, q: np.ndarray, s: np.ndarray, group: int = 128, mode: str = "f32",
         nthreads: int = 0, zeros: np.ndarray | None = None) -> np.ndarray:
    """C = A @ Bhat with A fp16 [M, K], q uint8 [K, N], s fp16 [K/group, N] and optional zero
    points uint8 [K/group, N] (default 8); returns fp16 [M, N]."""
    A = _c(np.asarray(A, dtype=np.float16))
    q = _c(np.asarray(q, dtype=np.uint8))
    s = _c(np.asarray(s, dtype=np.float16))
    M, K = A.shape
    K2, N = q.shape
    if K2 != K or s.shape != (K // group, N):
        raise ValueError(f"shape mismatch A{A.shape} q{q.shape} s{s.shape} group={group}")
    C = np.empty((M, N), dtype=np.float16)
    if nthreads <= 0:
        nthreads = default_threads()
    if zeros is None:
        fn = {"f32": _load().oracle_gemm_f32, "f64": _load().oracle_gemm_f64}[mode]
        rc = fn(A.ctypes.data, q.ctypes.data, s.ctypes.data, M, K, N, group, C.ctypes.data,
                int(nthreads))
    else:
        z = _c(np.asarray(zeros, dtype=np.uint8))
        if z.shape != s.shape:
            raise ValueError(f"zeros shape {z.shape} != scales shape {s.shape}")
        fn = {"f32": _load().oracle_gemm_zp_f32, "f64": _load().oracle_gemm_zp_f64}[mode]
        rc = fn(A.ctypes.data, q.ctypes.data, s.ctypes.data, z.ctypes.data, M, K, N, group,
                C.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_gemm_{mode} returned {rc}")
    return C


def gemv(a: np.ndarray, q: np.ndarray, s: np.ndarray, group: int = 128) -> np.ndarray:
    """The M = 1 product, coded separately from gemm; returns fp16 [N]."""
    a = _c(np.asarray(a, dtype=np.float16).reshape(-1))
    q = _c(np.asarray(q, dtype=np.uint8))
    s = _c(np.asarray(s, dtype=np.float16))
    K, N = q.shape
    if a.shape[0] != K:
        raise ValueError("length mismatch")
    c = np.empty((N,), dtype=np.float16)
    rc = _load().oracle_gemv_f32(a.ctypes.data, q.ctypes.data, s.ctypes.data, K, N, group,
                                 c.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_gemv_f32 returned {rc}")
    return c


def half_to_double(bits: int) -> float:
    return _load().oracle_half_to_double(int(bits))


def double_to_half(x: float) -> int:
    return int(_load().oracle_double_to_half(float(x)))


def float_to_half(x: float) -> int:
    return int(_load().oracle_float_to_half(float(x)))


def dequant(q: int, s_bits: int, z: int | None = None) -> float:
    if z is None:
        return _load().oracle_dequant(int(q), int(s_bits))
    return _load().oracle_dequant_zp(int(q), int(s_bits), int(z))


# --------------------------------------------------------------------------------------------
# Exact reference for tiny shapes: every finite fp16 value is an integer multiple of 2^-24, so
# a*w is an integer multiple of 2^-48 and the whole sum is one exact Python integer.

_SHIFT = 48


def _half_bits_to_scaled(h: int) -> int:
    """fp16 bits -> integer v with value = v * 2^-24 (finite inputs only)."""
    e = (h >> 10) & 0x1F
    m = h & 0x3FF
    if e == 31:
        raise ValueError("non-finite input")
    v = m if e == 0 else (m + 1024) << (e - 1)
    return -v if h & 0x8000 else v


def round_scaled_to_half(S: int, shift: int = _SHIFT) -> int:
    """Correctly round S * 2^-shift to fp16 bits (nearest, ties to even).  Exact zero -> +0."""
    if S == 0:
        return 0
    sign = 0x8000 if S < 0 else 0
    S = abs(S)
    e = S.bit_length() - 1 - shift          # 2^e <= value < 2^(e+1)
    ex = max(e, -14)
    sh = shift + ex - 10                    # value / ulp = S / 2^sh, ulp = 2^(ex-10)
    if sh > 0:
        qv, rem = divmod(S, 1 << sh)
        twice = rem << 1
        if twice > (1 << sh) or (twice == (1 << sh) and (qv & 1)):
            qv += 1
    else:
        qv = S << (-sh)
    if qv == 2048:                          # rounding carried into the next binade
        qv = 1024
        ex += 1
    if ex > 15 or (ex == 15 and qv > 2047):
        return sign | 0x7C00
    if qv < 1024:                           # only possible at ex == -14: subnormal
        return sign | qv
    return sign | ((ex + 15) << 10) | (qv - 1024)


def exact_gemm(A: np.ndarray, q: np.ndarray, s: np.ndarray, group: int = 128,
               zeros: np.ndarray | None = None):
    """Exact C per output: (correctly rounded fp16, exact value as float64, sum_k |a_k w_k|).

    Pure Python integer arithmetic; use only on tiny shapes.  zeros: uint8 [K/group, N] zero
    points (default 8).
    """
    A16 = np.asarray(A, dtype=np.float16).view(np.uint16)
    s16 = np.asarray(s, dtype=np.float16).view(np.uint16)
    q = np.asarray(q, dtype=np.uint8)
    M, K = A16.shape
    N = q.shape[1]
    z = None if zeros is None else np.asarray(zeros, dtype=np.uint8)

    def zp(k, n):
        return 8 if z is None else int(z[k // group, n])

    a_int = [[_half_bits_to_scaled(int(A16[m, k])) for k in range(K)] for m in range(M)]
    w_int = [[_half_bits_to_scaled(int(s16[k // group, n])) * (int(q[k, n]) - zp(k, n))
              for k in range(K)] for n in range(N)]
    out = np.empty((M, N), dtype=np.uint16)
    exact = np.empty((M, N), dtype=np.float64)
    absum = np.empty((M, N), dtype=np.float64)
    for m in range(M):
        am = a_int[m]
        for n in range(N):
            wn = w_int[n]
            tot = 0
            tabs = 0
            for k in range(K):
                p = am[k] * wn[k]
                tot += p
                tabs += abs(p)
            out[m, n] = round_scaled_to_half(tot)
            exact[m, n] = tot / float(1 << _SHIFT)
            absum[m, n] = tabs / float(1 << _SHIFT)
    return out.view(np.float16), exact, absum


# --------------------------------------------------------------------------------------------
# Checkpoint-style packed words -> codes.  Checkpoints labelled alike (INT4, group 128) differ
# in nibble order and arrangement, and converting one for the kernel moves codes without
# changing any (deep-dive page, section "直接生成 MMA 所需的寄存器 fragment" and the
# deployment section on checkpoint formats).  These are the plain definitions of the two
# arrangements the library's load-time repack takes: 8 codes per 32-bit word, nibble i in bits
# 4i..4i+3.

def _words(a, shape) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint32).reshape(shape)


def decode_along_k(qweight, K: int, N: int) -> np.ndarray:
    """Codes uint8 [K, N] from words [K/8, N]: word (r, n) holds rows 8r..8r+7 of column n,
    row 8r + i in nibble i."""
    w = _words(qweight, (K // 8, N))
    codes = np.empty((K, N), dtype=np.uint8)
    for i in range(8):
        codes[i::8, :] = (w >> np.uint32(4 * i)) & np.uint32(15)
    return codes


def check_order(order) -> list:
    order = list(range(8)) if order is None else [int(o) for o in order]
    if sorted(order) != list(range(8)):
        raise ValueError(f"order {order} is not a permutation of 0..7")
    return order


def decode_along_n(qweight, rows: int, N: int, order=None) -> np.ndarray:
    """Codes uint8 [rows, N] from words [rows, N/8]: word (k, c) holds columns 8c..8c+7 of row
    k, column 8c + order[i] in nibble i (order None: 0..7)."""
    order = check_order(order)
    w = _words(qweight, (rows, N // 8))
    codes = np.empty((rows, N), dtype=np.uint8)
    for i in range(8):
        codes[:, order[i]::8] = (w >> np.uint32(4 * i)) & np.uint32(15)
    return codes


# --------------------------------------------------------------------------------------------
# Mixture-of-experts layer: token t's j-th expert is topk_ids[t, j]; assignment a = t*topk + j
# is row a of the output, computed from row t of A with that expert's weights.  Deep-dive
# page, section on where the format pays off: item 1 (MoE regroups tokens by expert, so each
# expert's GEMM sees its own M) and item 4 (grouped GEMM).

def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value (8 significant bits, ties to even) of float64 x, as float64.
    bfloat16 is binary32 cut to 16 bits: same exponent range, 7 stored mantissa bits.  Values
    here stay far inside the normal range, where this is the whole definition."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2^e with 0.5 <= |m| < 1, or m = 0
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def bf16_bits(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of bf16_round(x): the upper half of the binary32 word."""
    r = bf16_round(x).astype(np.float32)   # exact: 8 significant bits
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """float64 values of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def moe_align(topk_ids, E: int):
    """The assignments grouped by expert: (sorted_ids int32, offsets int32 [E+1]) with expert
    e's assignments, in increasing order, at sorted_ids[offsets[e]:offsets[e+1]].  Entries
    outside 0..E-1 are left out."""
    flat = np.asarray(topk_ids).reshape(-1)
    lists = [np.flatnonzero(flat == e) for e in range(E)]
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum([len(x) for x in lists])
    ids = np.concatenate(lists) if lists else np.zeros(0, dtype=np.int64)
    return ids.astype(np.int32), offsets.astype(np.int32)


def moe_gemm(A, topk_ids, q, s, zeros=None, row_scale=None, act: str = "f16",
             group: int = 128):
    """Grouped product of an MoE layer.  A: float [T, K] (values of the activation type),
    topk_ids int [T, topk], q uint8 [E, K, N], s float [E, K/group, N] (values), zeros
    optional uint8 [E, K/group, N] (default 8), row_scale optional [T*topk].
    Returns (C float64 [T*topk, N], each listed row rounded once to fp16 or bfloat16, and a
    bool mask [T*topk] of the rows computed).  Per expert: Bhat = s (q - z) and
    C[a] = row_scale[a] * A[a // topk] @ Bhat in fp64."""
    A = np.asarray(A, dtype=np.float64)
    ids = np.asarray(topk_ids)
    T, topk = ids.shape
    E, K, N = q.shape
    R = T * topk
    C = np.zeros((R, N), dtype=np.float64)
    done = np.zeros(R, dtype=bool)
    order, offsets = moe_align(ids, E)
    for e in range(E):
        rows = order[offsets[e]:offsets[e + 1]].astype(np.int64)
        if rows.size == 0:
            continue
        z = 8.0 if zeros is None else np.repeat(np.asarray(zeros[e], np.float64), group, axis=0)
        W = np.repeat(np.asarray(s[e], np.float64), group, axis=0) * (q[e].astype(np.float64) - z)
        Y = A[rows // topk] @ W
        if row_scale is not None:
            Y = Y * np.asarray(row_scale, dtype=np.float64)[rows][:, None]
        C[rows] = Y
        done[rows] = True
    if act == "f16":
        C = C.astype(np.float16).astype(np.float64)
    elif act == "bf16":
        C = bf16_round(C)
    else:
        raise ValueError(act)
    return C, done

"""Thin Python binding of libw4a16 (the C ABI declared in include/w4a16.h).

Argument marshalling only: every step of the multiply runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  Importing this package fails loudly
when the compiled library is missing; there is no fallback path.

    packed, scales_p = pack(codes, scales)          # host, offline (numpy in, numpy out)
    packed_d, scales_d = to_device(packed, scales_p)
    C = gemm(A, packed_d, scales_d, N)              # A: fp16 [M, K] on the GPU

Other formats: pack(codes, scales, group=K) for one scale per column, and
pack(codes, scales, group, zeros=z) for zero points; pass the same group / zero_points to
gemm.  repack(...) converts checkpoint-style packed tensors already on the GPU into the same
layout on the GPU.  2:4-sparse weights: pack_24(codes, scales) and gemm_24(A, packed, scales, N).
"""
from __future__ import annotations

import ctypes
import functools
import os
import threading

import numpy as np

GROUP = 128
N_ALIGN = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
        "(or python mixed_precision_w4a16_amd/build.py) first")

# PyTorch ships its own HIP runtime (same SONAME as the system one, but its own libraries ask
# for it under another file name).  Loading torch first makes this library bind to that one
# runtime; loading this library first would leave two HIP runtimes in the process.
try:
    import torch as _torch  # noqa: F401
except ImportError:
    _torch = None

_lib = ctypes.CDLL(LIB_PATH)
_p, _i = ctypes.c_void_p, ctypes.c_int
_lib.w4a16_status_string.argtypes = [_i]
_lib.w4a16_status_string.restype = ctypes.c_char_p
_lib.w4a16_pack.argtypes = [_p, _p, _i, _i, _i, _p, _p]
_lib.w4a16_pack.restype = _i
_lib.w4a16_unpack.argtypes = [_p, _p, _i, _i, _i, _p, _p]
_lib.w4a16_unpack.restype = _i
_lib.w4a16_workspace_size.argtypes = [_i, _i, _i, ctypes.POINTER(ctypes.c_size_t)]
_lib.w4a16_workspace_size.restype = _i
_lib.w4a16_gemm.argtypes = [_p, _p, _p, _p, _i, _i, _i, _p, _p]
_lib.w4a16_gemm.restype = _i
_lib.w4a16_pack_zp.argtypes = [_p, _p, _p, _i, _i, _i, _p, _p]
_lib.w4a16_pack_zp.restype = _i
_lib.w4a16_unpack_zp.argtypes = [_p, _p, _i, _i, _i, _p, _p, _p]
_lib.w4a16_unpack_zp.restype = _i
_lib.w4a16_gemm_ex.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p]
_lib.w4a16_gemm_ex.restype = _i
_lib.w4a16_repack.argtypes = [_p, _i, _p, _p, _p, _i, _i, _i, _p, _p, _p]
_lib.w4a16_repack.restype = _i
_lib.w4a16_pack_24.argtypes = [_p, _p, _i, _i, _p, _p]
_lib.w4a16_pack_24.restype = _i
_lib.w4a16_unpack_24.argtypes = [_p, _p, _i, _i, _p, _p]
_lib.w4a16_unpack_24.restype = _i
_lib.w4a16_gemm_24.argtypes = [_p, _p, _p, _p, _i, _i, _i, _p, _p]
_lib.w4a16_gemm_24.restype = _i
_lib.w4a16_moe_align.argtypes = [_p, _i, _i, _i, _p, _p, _p]
_lib.w4a16_moe_align.restype = _i
_lib.w4a16_moe_gemm.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p]
_lib.w4a16_moe_gemm.restype = _i
_lib.w4a16_moe_gemm_topk.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p]
_lib.w4a16_moe_gemm_topk.restype = _i
_lib.w4a16_read_probe.argtypes = [_p, ctypes.c_size_t, _p, _p]
_lib.w4a16_read_probe.restype = _i
_lib.w4a16_mfma_probe.argtypes = [_p, ctypes.c_size_t, _i, _i, _i, _p, _p]
_lib.w4a16_mfma_probe.restype = _i
_lib.w4a16_gemm_noalloc.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p]
_lib.w4a16_gemm_noalloc.restype = _i

OK, EINVAL, ESHAPE, EUNSUPPORTED, EHIP = 0, -1, -2, -3, -4
PACKED_ALONG_K, PACKED_ALONG_N = 0, 1
ACT_F16, ACT_BF16 = 0, 1
EXPORTED = ("w4a16_status_string", "w4a16_pack", "w4a16_unpack", "w4a16_pack_zp",
            "w4a16_unpack_zp", "w4a16_workspace_size", "w4a16_gemm", "w4a16_gemm_ex",
            "w4a16_repack", "w4a16_pack_24", "w4a16_unpack_24", "w4a16_gemm_24",
            "w4a16_moe_align", "w4a16_moe_gemm", "w4a16_moe_gemm_topk", "w4a16_read_probe",
            "w4a16_mfma_probe", "w4a16_gemm_noalloc")
NOALLOC_SCRATCH_BYTES = (128 << 20) + 4096


class W4A16Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib.w4a16_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise W4A16Error(fn, status)


def library():
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib


# ------------------------------------------------------------------------------ host side

def pack(codes: np.ndarray, scales: np.ndarray, group: int = GROUP, zeros=None):
    """Offline reorder.  codes uint8 [K, N] (0..15), scales fp16 [K/group, N] (group 128, or
    K for one scale per column), zeros optional uint8 [K/group, N] (0..15) ->
    (packed uint32 [K*N/8], params fp16: the scales [(K/group)*N], or scales and zero terms
    [2*(K/group)*N] when zeros are given).  Scales given as uint16 are taken as raw 16-bit
    patterns (bf16 scales for w4a16_moe_gemm) and params come back as uint16."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    raw = np.asarray(scales).dtype == np.uint16
    scales = np.ascontiguousarray(scales, dtype=np.uint16 if raw else np.float16)
    K, N = codes.shape
    if not group or K % group or scales.shape != (K // group, N):
        raise ValueError(f"scales shape {scales.shape} does not match codes {codes.shape} "
                         f"with group {group}")
    packed = np.empty(K * N // 8, dtype=np.uint32)
    if zeros is None:
        params = np.empty(scales.size, dtype=scales.dtype)
        _check("w4a16_pack", _lib.w4a16_pack(codes.ctypes.data, scales.ctypes.data, K, N, group,
                                             packed.ctypes.data, params.ctypes.data))
    else:
        zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
        if zeros.shape != scales.shape:
            raise ValueError(f"zeros shape {zeros.shape} != scales shape {scales.shape}")
        params = np.empty(2 * scales.size, dtype=scales.dtype)
        _check("w4a16_pack_zp", _lib.w4a16_pack_zp(codes.ctypes.data, scales.ctypes.data,
                                                   zeros.ctypes.data, K, N, group,
                                                   packed.ctypes.data, params.ctypes.data))
    return packed, params


def unpack(packed: np.ndarray, params: np.ndarray, K: int, N: int, group: int = GROUP,
           zero_points: bool = False):
    """Inverse of pack: (codes uint8 [K, N], scales fp16 [K/group, N]), plus zeros uint8
    [K/group, N] when zero_points."""
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    params = np.ascontiguousarray(params, dtype=np.float16)
    per = 2 if zero_points else 1
    if not group or K % group or packed.size != K * N // 8 or params.size != per * (K // group) * N:
        raise ValueError("size mismatch")
    codes = np.empty((K, N), dtype=np.uint8)
    scales = np.empty((K // group, N), dtype=np.float16)
    if not zero_points:
        _check("w4a16_unpack", _lib.w4a16_unpack(packed.ctypes.data, params.ctypes.data, K, N,
                                                 group, codes.ctypes.data, scales.ctypes.data))
        return codes, scales
    zeros = np.empty((K // group, N), dtype=np.uint8)
    _check("w4a16_unpack_zp", _lib.w4a16_unpack_zp(packed.ctypes.data, params.ctypes.data, K, N,
                                                   group, codes.ctypes.data, scales.ctypes.data,
                                                   zeros.ctypes.data))
    return codes, scales, zeros


def pack_experts(codes: np.ndarray, scales: np.ndarray, zeros=None):
    """pack() for every expert of an MoE layer (group 128): codes uint8 [E, K, N], scales
    [E, K/128, N] (fp16 values, or uint16 bit patterns for bf16 scales), zeros optional uint8
    [E, K/128, N] -> (packed uint32 [E, K*N/8], params [E, P]) for moe_gemm."""
    E = codes.shape[0]
    outs = [pack(codes[e], scales[e], GROUP, None if zeros is None else zeros[e])
            for e in range(E)]
    return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])


# ------------------------------------------------------------------------------ device side

def to_device(packed: np.ndarray, scales_p: np.ndarray, device="cuda"):
    """Upload pack() output: (int32 tensor holding the uint32 words, fp16 tensor)."""
    import torch
    sp = np.ascontiguousarray(scales_p)
    if sp.dtype == np.uint16:
        sp = sp.view(np.int16)
    return (torch.from_numpy(np.ascontiguousarray(packed).view(np.int32)).to(device),
            torch.from_numpy(sp).to(device))


def workspace_bytes(M: int, K: int, N: int) -> int:
    """Exact workspace bytes for (M, K, N) on the current device (w4a16_workspace_size)."""
    n = ctypes.c_size_t(0)
    _check("w4a16_workspace_size", _lib.w4a16_workspace_size(M, K, N, ctypes.byref(n)))
    return n.value


@functools.lru_cache(maxsize=4096)
def _ws_need(M: int, K: int, N: int, device_index: int) -> int:
    # the answer depends only on the shape and the device (its compute-unit count); the
    # caller has made device_index current
    return workspace_bytes(M, K, N)


def workspace_bound(M: int, K: int, N: int) -> int:
    """The header's device-independent bound on workspace_bytes (w4a16_workspace_bound, a
    static inline function of include/w4a16.h), evaluated as the header writes it."""
    if M < 0 or K <= 0 or N < 0 or K % 128:
        return 0
    mt = 16 if M <= 16 else 32 if M <= 32 else 64 if M <= 64 else 128
    nt = min(N, 256)
    mcov = mt if M <= 64 else 128 * ((M + 127) // 128)
    stripes = min(2 * 1024 * mt * nt * 4, 8 * N * (K // 128) * mcov)
    pieces = min((N // 16 + 9) * 64 * 1024, 40 << 20) if M <= 128 else 0
    return 4096 + max(stripes, pieces)


_ws_lock = threading.Lock()
_ws = {}


def workspace(M: int, K: int, N: int, device=None, stream=None):
    """A zeroed workspace large enough for (M, K, N), cached per (device, stream) and grown on
    demand: calls queued on one stream never overlap, so they can share one; another stream
    gets its own."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    need = workspace_bytes(M, K, N)
    key = (dev, stream.cuda_stream)
    with _ws_lock:
        buf = _ws.get(key)
        if buf is None or buf.numel() < need:
            buf = torch.zeros(need, dtype=torch.uint8, device=dev)
            _ws[key] = buf
        return buf


def _check_ws(ws, A, M: int, K: int, N: int):
    """A caller's workspace must be a contiguous uint8 tensor on A's device holding at least
    workspace_bytes(M, K, N) bytes (the kernels size their partial tiles from the shape, not
    from the allocation)."""
    import torch
    if (not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or not ws.is_contiguous()
            or ws.device != A.device):
        raise ValueError("ws must be a contiguous uint8 tensor on A's device")
    need = _ws_need(M, K, N, A.device.index)
    if ws.numel() < need:
        raise ValueError(f"ws holds {ws.numel()} bytes; this shape needs {need}")


def new_workspace(M: int, K: int, N: int, device="cuda"):
    import torch
    return torch.zeros(workspace_bytes(M, K, N), dtype=torch.uint8, device=device)


def _gemm_args(A, packed, params, N, out, group, zero_points):
    """Checks of gemm()'s tensors; returns (M, K, out), out allocated if None."""
    import torch
    if A.dtype != torch.float16 or not A.is_cuda or A.dim() != 2 or not A.is_contiguous():
        raise ValueError("A must be a contiguous fp16 CUDA tensor of shape [M, K]")
    M, K = A.shape
    if packed.device != A.device or params.device != A.device:
        raise ValueError("packed and params must be on A's device")
    if packed.dtype != torch.int32 or packed.numel() * 8 != K * N or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous int32 tensor of K*N/8 words")
    per = 2 if zero_points else 1
    if (not group or K % group or params.dtype != torch.float16
            or params.numel() != per * (K // group) * N or not params.is_contiguous()):
        raise ValueError("params must be a contiguous fp16 tensor as pack() returned it")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=A.device)
    elif (out.dtype != torch.float16 or out.shape != (M, N) or not out.is_contiguous()
          or out.device != A.device):
        raise ValueError("out must be a contiguous fp16 tensor [M, N] on A's device")
    return M, K, out


def gemm(A, packed, params, N: int, out=None, ws=None, stream=None, group: int = GROUP,
         zero_points: bool = False):
    """C[M, N] = A[M, K] @ dequant(packed, params) on A's device and the current stream.

    A: fp16 [M, K] contiguous CUDA tensor.  packed: int32 [K*N/8], params: fp16, both from
    to_device(pack(...)) with the same group and zeros-or-not.  out: optional fp16 [M, N]
    contiguous tensor.
    """
    import torch
    M, K, out = _gemm_args(A, packed, params, N, out, group, zero_points)
    if M == 0:
        return out
    with torch.cuda.device(A.device):
        if stream is None:
            stream = torch.cuda.current_stream(A.device)
        if ws is None:
            ws = workspace(M, K, N, A.device, stream)
        else:
            _check_ws(ws, A, M, K, N)
        if group == GROUP and not zero_points:
            _check("w4a16_gemm", _lib.w4a16_gemm(A.data_ptr(), packed.data_ptr(),
                                                 params.data_ptr(), out.data_ptr(), M, K, N,
                                                 ws.data_ptr(), stream.cuda_stream))
        else:
            _check("w4a16_gemm_ex", _lib.w4a16_gemm_ex(A.data_ptr(), packed.data_ptr(),
                                                       params.data_ptr(), out.data_ptr(), M, K,
                                                       N, group, int(bool(zero_points)),
                                                       ws.data_ptr(), stream.cuda_stream))
    return out


def gemm_noalloc(A, packed, params, N: int, out=None, stream=None, group: int = GROUP,
                 zero_points: bool = False):
    """gemm() through w4a16_gemm_noalloc: the library's own per-GPU scratch instead of a
    workspace.  Calls that can overlap on one GPU (several streams or threads) race on that
    scratch: serialise them.  Same arguments and result as gemm() without ws."""
    import torch
    M, K, out = _gemm_args(A, packed, params, N, out, group, zero_points)
    if M == 0:
        return out
    with torch.cuda.device(A.device):
        if stream is None:
            stream = torch.cuda.current_stream(A.device)
        _check("w4a16_gemm_noalloc", _lib.w4a16_gemm_noalloc(
            A.data_ptr(), packed.data_ptr(), params.data_ptr(), out.data_ptr(), M, K, N, group,
            int(bool(zero_points)), stream.cuda_stream))
    return out


def repack(qweight, scales, K: int, N: int, layout: int, group: int = GROUP, qzeros=None,
           order=None, stream=None):
    """Device-side load-time conversion (w4a16_repack) -> (packed int32 [K*N/8], params fp16).

    qweight: int32 CUDA tensor holding the uint32 words, [K/8, N] for PACKED_ALONG_K or
    [K, N/8] for PACKED_ALONG_N.  scales: fp16 [K/group, N].  qzeros: optional int32
    [K/group, N/8] packed along N.  order: optional 8 column offsets, nibble i of a word packed
    along N holding offset order[i].  Pass the same group and zero_points=(qzeros is not None)
    to gemm.
    """
    import torch
    dev = qweight.device
    want = (K // 8, N) if layout == PACKED_ALONG_K else (K, N // 8)
    if (qweight.dtype != torch.int32 or not qweight.is_cuda or not qweight.is_contiguous()
            or tuple(qweight.shape) != want):
        raise ValueError(f"qweight must be a contiguous int32 CUDA tensor of shape {want}")
    if (not group or K % group or scales.dtype != torch.float16 or scales.device != dev
            or not scales.is_contiguous() or tuple(scales.shape) != (K // group, N)):
        raise ValueError("scales must be a contiguous fp16 tensor [K/group, N] on qweight's device")
    zp = 0
    if qzeros is not None:
        if (qzeros.dtype != torch.int32 or qzeros.device != dev or not qzeros.is_contiguous()
                or tuple(qzeros.shape) != (K // group, N // 8)):
            raise ValueError("qzeros must be a contiguous int32 tensor [K/group, N/8] on "
                             "qweight's device")
        zp = qzeros.data_ptr()
    order_buf = None
    if order is not None:
        order_buf = np.ascontiguousarray(order, dtype=np.uint8)
        if order_buf.shape != (8,):
            raise ValueError("order must hold 8 entries")
    packed = torch.empty(K * N // 8, dtype=torch.int32, device=dev)
    params = torch.empty((2 if qzeros is not None else 1) * (K // group) * N,
                         dtype=torch.float16, device=dev)
    with torch.cuda.device(dev):
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        _check("w4a16_repack", _lib.w4a16_repack(
            qweight.data_ptr(), int(layout),
            None if order_buf is None else order_buf.ctypes.data, scales.data_ptr(), zp or None,
            K, N, group, packed.data_ptr(), params.data_ptr(), stream.cuda_stream))
    return packed, params


# ------------------------------------------------------------------------------ 2:4 sparse

def pack_24(codes: np.ndarray, scales: np.ndarray):
    """Offline reorder of 2:4-sparse weights (group 128, zero point 8).  codes uint8 [K, N]
    with at most 2 codes other than 8 in every aligned group of 4 rows of a column ->
    (packed uint32 [K*N*3/32], scales fp16 [(K/128)*N])."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float16)
    K, N = codes.shape
    if K % GROUP or scales.shape != (K // GROUP, N):
        raise ValueError(f"scales shape {scales.shape} does not match codes {codes.shape}")
    packed = np.empty(K * N * 3 // 32, dtype=np.uint32)
    sp = np.empty(scales.size, dtype=np.float16)
    _check("w4a16_pack_24", _lib.w4a16_pack_24(codes.ctypes.data, scales.ctypes.data, K, N,
                                               packed.ctypes.data, sp.ctypes.data))
    return packed, sp


def unpack_24(packed: np.ndarray, scales_p: np.ndarray, K: int, N: int):
    """Inverse of pack_24: (codes uint8 [K, N] with 8 at pruned positions, scales fp16)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    scales_p = np.ascontiguousarray(scales_p, dtype=np.float16)
    if K % GROUP or packed.size != K * N * 3 // 32 or scales_p.size != (K // GROUP) * N:
        raise ValueError("size mismatch")
    codes = np.empty((K, N), dtype=np.uint8)
    scales = np.empty((K // GROUP, N), dtype=np.float16)
    _check("w4a16_unpack_24", _lib.w4a16_unpack_24(packed.ctypes.data, scales_p.ctypes.data, K,
                                                   N, codes.ctypes.data, scales.ctypes.data))
    return codes, scales


def gemm_24(A, packed, scales, N: int, out=None, ws=None, stream=None):
    """C[M, N] = A @ Bhat for 2:4-sparse Bhat from to_device(pack_24(...)); ws as for gemm."""
    import torch
    if A.dtype != torch.float16 or not A.is_cuda or A.dim() != 2 or not A.is_contiguous():
        raise ValueError("A must be a contiguous fp16 CUDA tensor of shape [M, K]")
    M, K = A.shape
    if packed.device != A.device or scales.device != A.device:
        raise ValueError("packed and scales must be on A's device")
    if packed.dtype != torch.int32 or packed.numel() * 32 != K * N * 3 or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous int32 tensor of K*N*3/32 words")
    if (K % GROUP or scales.dtype != torch.float16 or scales.numel() != (K // GROUP) * N
            or not scales.is_contiguous()):
        raise ValueError("scales must be a contiguous fp16 tensor as pack_24() returned it")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=A.device)
    elif (out.dtype != torch.float16 or out.shape != (M, N) or not out.is_contiguous()
          or out.device != A.device):
        raise ValueError("out must be a contiguous fp16 tensor [M, N] on A's device")
    if M == 0:
        return out
    with torch.cuda.device(A.device):
        if stream is None:
            stream = torch.cuda.current_stream(A.device)
        if ws is None:
            ws = workspace(M, K, N, A.device, stream)
        else:
            _check_ws(ws, A, M, K, N)
        _check("w4a16_gemm_24", _lib.w4a16_gemm_24(A.data_ptr(), packed.data_ptr(),
                                                   scales.data_ptr(), out.data_ptr(), M, K, N,
                                                   ws.data_ptr(), stream.cuda_stream))
    return out


def moe_align(topk_ids, E: int, stream=None):
    """Regroup the assignments of topk_ids (int32 [T, topk] on the GPU) by expert
    (w4a16_moe_align) -> (sorted_ids int32 [T*topk], expert_offsets int32 [E+1])."""
    import torch
    if (topk_ids.dtype != torch.int32 or not topk_ids.is_cuda or topk_ids.dim() != 2
            or not topk_ids.is_contiguous()):
        raise ValueError("topk_ids must be a contiguous int32 CUDA tensor [T, topk]")
    T, topk = topk_ids.shape
    sorted_ids = torch.empty(T * topk, dtype=torch.int32, device=topk_ids.device)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=topk_ids.device)
    with torch.cuda.device(topk_ids.device):
        if stream is None:
            stream = torch.cuda.current_stream(topk_ids.device)
        _check("w4a16_moe_align", _lib.w4a16_moe_align(topk_ids.data_ptr(), T, topk, E,
                                                       sorted_ids.data_ptr(), offsets.data_ptr(),
                                                       stream.cuda_stream))
    return sorted_ids, offsets


MOE_ROUTE_MAX = 2048


def _moe_args(A, packed, params, topk, E, N, row_scale, zero_points, out):
    import torch
    if A.dtype not in (torch.float16, torch.bfloat16) or not A.is_cuda or A.dim() != 2 \
            or not A.is_contiguous():
        raise ValueError("A must be a contiguous fp16 or bf16 CUDA tensor [T, K]")
    T, K = A.shape
    dev = A.device
    per = 2 if zero_points else 1
    if (packed.dtype != torch.int32 or packed.numel() * 8 != E * K * N or not packed.is_contiguous()
            or packed.device != dev):
        raise ValueError("packed must be a contiguous int32 tensor of E*K*N/8 words on A's device")
    if (K % GROUP or params.element_size() != 2 or params.numel() != E * per * (K // GROUP) * N
            or not params.is_contiguous() or params.device != dev):
        raise ValueError("params must be the 16-bit tensor pack_experts() returned, on A's device")
    if row_scale is not None and (row_scale.dtype != torch.float32 or row_scale.numel() != T * topk
                                  or not row_scale.is_contiguous() or row_scale.device != dev):
        raise ValueError("row_scale must be a contiguous float32 tensor [T*topk]")
    if out is None:
        out = torch.empty((T * topk, N), dtype=A.dtype, device=dev)
    elif (out.dtype != A.dtype or tuple(out.shape) != (T * topk, N) or not out.is_contiguous()
          or out.device != dev):
        raise ValueError("out must be a contiguous [T*topk, N] tensor of A's dtype on A's device")
    act = ACT_BF16 if A.dtype == torch.bfloat16 else ACT_F16
    return T, K, out, act


def moe_gemm_topk(A, packed, params, topk_ids, E: int, N: int, row_scale=None,
                  zero_points: bool = False, out=None, stream=None):
    """moe_gemm with the regrouping inside the product (w4a16_moe_gemm_topk): topk_ids int32
    [T, topk] on the GPU, T*topk <= MOE_ROUTE_MAX.  Same result as moe_align + moe_gemm."""
    import torch
    if (topk_ids.dtype != torch.int32 or not topk_ids.is_cuda or topk_ids.dim() != 2
            or not topk_ids.is_contiguous() or topk_ids.device != A.device
            or topk_ids.shape[0] != A.shape[0]):
        raise ValueError("topk_ids must be a contiguous int32 [T, topk] tensor on A's device")
    topk = topk_ids.shape[1]
    T, K, out, act = _moe_args(A, packed, params, topk, E, N, row_scale, zero_points, out)
    with torch.cuda.device(A.device):
        if stream is None:
            stream = torch.cuda.current_stream(A.device)
        _check("w4a16_moe_gemm_topk", _lib.w4a16_moe_gemm_topk(
            A.data_ptr(), packed.data_ptr(), params.data_ptr(), topk_ids.data_ptr(),
            None if row_scale is None else row_scale.data_ptr(), out.data_ptr(), T, topk, E, K,
            N, int(bool(zero_points)), act, stream.cuda_stream))
    return out


def moe_gemm(A, packed, params, sorted_ids, offsets, topk: int, E: int, N: int, row_scale=None,
             zero_points: bool = False, out=None, stream=None):
    """Grouped MoE product (w4a16_moe_gemm): out[a] = row_scale[a] * A[a // topk] @ Bhat_e for
    each assignment a listed in sorted_ids.  A: fp16 or bf16 [T, K]; packed int32 [E, K*N/8]
    and params [E, P] from to_device(pack_experts(...)); out: optional [T*topk, N] of A's
    dtype (rows not listed keep their contents)."""
    import torch
    T, K, out, act = _moe_args(A, packed, params, topk, E, N, row_scale, zero_points, out)
    dev = A.device
    for t, n in ((sorted_ids, T * topk), (offsets, E + 1)):
        if t.dtype != torch.int32 or t.numel() < n or not t.is_contiguous() or t.device != dev:
            raise ValueError("sorted_ids / offsets must be moe_align()'s int32 tensors")
    with torch.cuda.device(dev):
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        _check("w4a16_moe_gemm", _lib.w4a16_moe_gemm(
            A.data_ptr(), packed.data_ptr(), params.data_ptr(), sorted_ids.data_ptr(),
            offsets.data_ptr(), None if row_scale is None else row_scale.data_ptr(),
            out.data_ptr(), T, topk, E, K, N, int(bool(zero_points)), act, stream.cuda_stream))
    return out


def mfma_probe(src, shape: int = 0, workgroups: int = 1024, iters: int = 2000, out=None,
               stream=None):
    """Measurement support (w4a16_mfma_probe): fp16 matrix instructions on operand fragments
    from CUDA tensor src (random fp16 values), shape 0 = 16x16x32, 1 = 32x32x16.  Returns
    (out float32 [workgroups*256], flops of the launch)."""
    import torch
    if not src.is_cuda or not src.is_contiguous() or (src.numel() * src.element_size()) % 16:
        raise ValueError("src must be a contiguous CUDA tensor of a multiple of 16 bytes")
    if out is None:
        out = torch.empty(workgroups * 256, dtype=torch.float32, device=src.device)
    with torch.cuda.device(src.device):
        if stream is None:
            stream = torch.cuda.current_stream(src.device)
        _check("w4a16_mfma_probe", _lib.w4a16_mfma_probe(
            src.data_ptr(), src.numel() * src.element_size(), int(shape), int(workgroups),
            int(iters), out.data_ptr(), stream.cuda_stream))
    return out, workgroups * 4 * iters * 64 * (16384 if shape == 0 else 32768)


def read_probe(x, out=None, stream=None):
    """Measurement support (w4a16_read_probe): stream the bytes of CUDA tensor x (each
    workgroup one contiguous chunk) and discard them.  out: optional int32 [2048] tensor."""
    import torch
    if not x.is_cuda or not x.is_contiguous() or (x.numel() * x.element_size()) % 16:
        raise ValueError("x must be a contiguous CUDA tensor of a multiple of 16 bytes")
    if out is None:
        out = torch.zeros(2048, dtype=torch.int32, device=x.device)
    with torch.cuda.device(x.device):
        if stream is None:
            stream = torch.cuda.current_stream(x.device)
        _check("w4a16_read_probe", _lib.w4a16_read_probe(x.data_ptr(), x.numel() * x.element_size(),
                                                         out.data_ptr(), stream.cuda_stream))
    return out

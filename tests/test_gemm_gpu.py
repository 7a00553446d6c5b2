"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Bar: relative Frobenius error <= 1e-3 and max |C - C_ref| <= 1e-2 * max |C_ref|, C_ref the
fp32-accumulating oracle rounded to fp16.  Cases with an exactly representable answer
(one-hot activations, integer sums, the zero point, power-of-two scaling) must match bit for
bit.  Full-size workloads run in the same launch configuration the benchmark times and are
checked on every column at every M.
"""
import gc

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mixed_precision_w4a16_amd as w4
import oracle
from workloads import (ALL, COMPUTE_SWEEP, LARGE, LLAMA2_70B, LLAMA2_70B_TP8, LLAMA2_7B, SMALL,
                       draw)

pytestmark = pytest.mark.gpu

REL_FRO = 1e-3
MAX_ABS = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def bits(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def same(a, b):
    x, y = bits(a).copy(), bits(b).copy()
    x[x == 0x8000] = 0
    y[y == 0x8000] = 0
    return np.array_equal(x, y)


class Weights:
    """Packed weights resident on the GPU."""

    def __init__(self, q, s):
        self.K, self.N = q.shape
        packed, sp = w4.pack(q, s)
        self.packed, self.scales = w4.to_device(packed, sp)

    def run(self, A, out=None, ws=None):
        Ad = torch.from_numpy(np.ascontiguousarray(A)).cuda()
        C = w4.gemm(Ad, self.packed, self.scales, self.N, out=out, ws=ws)
        torch.cuda.synchronize()
        return C.cpu().numpy()


def gpu_gemm(A, q, s):
    return Weights(q, s).run(A)


def check(C, ref, what=""):
    d = C.astype(np.float64) - ref.astype(np.float64)
    nref = np.linalg.norm(ref.astype(np.float64))
    rel = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    mref = np.abs(ref.astype(np.float64)).max()
    mx = np.abs(d).max() / mref if mref > 0 else np.abs(d).max()
    print(f"  {what} rel_fro={rel:.2e} max_abs/max|C|={mx:.2e}", flush=True)
    assert np.isfinite(C).all(), what
    assert rel <= REL_FRO, (what, rel)
    assert mx <= MAX_ABS, (what, mx)
    return rel, mx


def test_one_hip_runtime_in_process_and_device_supported():
    maps = open("/proc/self/maps").read().splitlines()
    hip = {l.split()[-1] for l in maps if "libamdhip64" in l}
    assert len(hip) == 1, hip
    assert w4.workspace_bytes(16, 1024, 1024) >= 4096


# ------------------------------------------------------------------ small and ragged shapes

def test_small_workload_1024x1024_m16():
    sh = SMALL.shapes[0]
    A, q, s = draw(sh.K, sh.N, 16, seed=0)
    check(gpu_gemm(A, q, s), oracle.gemm(A, q, s), "1024x1024 M=16")


@pytest.mark.parametrize("M", list(range(1, 18)) + [31, 32, 33, 47, 48, 49, 63, 64, 65, 100,
                                                     128, 129, 200])
def test_m_sweep_ragged_rows(M):
    A, q, s = draw(1024, 512, M, seed=M)
    check(gpu_gemm(A, q, s), oracle.gemm(A, q, s), f"K=1024 N=512 M={M}")


@pytest.mark.parametrize("K,N", [(128, 64), (128, 256), (256, 192), (384, 320), (1152, 64),
                                 (18432, 64), (4096, 4096), (2048, 1344)])
@pytest.mark.parametrize("M", [1, 16, 40])
def test_shapes_tiles_and_reduction(K, N, M):
    # N = 64 / 192 / 320: one 16-column slab per wave; K = 128: one tile per slice;
    # K = 18432, N = 64: one slice split over up to 144 workgroups.
    A, q, s = draw(K, N, M, seed=K + N + M)
    check(gpu_gemm(A, q, s), oracle.gemm(A, q, s), f"K={K} N={N} M={M}")


@pytest.mark.parametrize("M,K,N", [(64, 18432, 4096), (128, 4096, 8192), (64, 18432, 1024),
                                   (100, 8192, 4096), (16, 18432, 2048), (32, 18432, 4096)])
def test_long_stripes_many_contributors_fresh_workspaces(M, K, N):
    # Slices shared by many stripes, more workgroups than fit on the chip at once (so some
    # start late, on whichever XCD has room), and a freshly zero-filled workspace whose lines
    # other caches may still hold: the device-scope release/acquire must make every
    # partial visible to the stripe that sums it.
    A, q, s = draw(K, N, M, seed=M + K + N)
    W = Weights(q, s)
    ref = oracle.gemm(A, q, s)
    for rep in range(2):
        ws = w4.new_workspace(M, K, N)
        check(W.run(A, ws=ws), ref, f"M={M} K={K} N={N} rep={rep}")
        assert int(ws[:4096].count_nonzero()) == 0


@pytest.mark.parametrize("M,K,N", [(128, 4096, 768), (300, 2048, 1280), (129, 1024, 256),
                                   (256, 4096, 1536), (513, 1024, 2048)])
def test_wide_tiles_both_shapes_ragged_rows(M, K, N):
    # M > 64 takes the 128-row tiles: 512-column slices where N allows (N = 1536, 2048),
    # else 256-column slices (N = 768, 1280, 256); M = 129, 300, 513 leave ragged row blocks.
    A, q, s = draw(K, N, M, seed=M * 7 + N)
    check(gpu_gemm(A, q, s), oracle.gemm(A, q, s), f"M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(128, 18432, 512), (200, 18432, 768), (96, 9216, 256)])
def test_one_slice_split_over_many_stripes(M, K, N):
    # Very few output tiles over a long K: slices are shared by dozens of one- or two-tile
    # stripes that all finish together, so the slice's owner is sometimes the last to arrive
    # (and sums from its registers) and sometimes not (and stores its piece like the others).
    # Whoever sums, the order is fixed: repeated runs must agree bit for bit.
    A, q, s = draw(K, N, M, seed=M + N)
    W = Weights(q, s)
    ref = oracle.gemm(A, q, s)
    first = W.run(A)
    check(first, ref, f"M={M} K={K} N={N}")
    for rep in range(4):
        ws = w4.new_workspace(M, K, N)
        assert np.array_equal(bits(W.run(A, ws=ws)), bits(first)), rep
        assert int(ws[:4096].count_nonzero()) == 0


def test_m1_equals_gemv():
    A, q, s = draw(4096, 1024, 1, seed=21)
    check(gpu_gemm(A, q, s)[0], oracle.gemv(A[0], q, s), "M=1 vs gemv")


# ------------------------------------------------------------------ exact cases

def test_one_hot_rows_are_bit_exact():
    # Row m of A is 1 at k_m: C[m, :] = fp16(s[k_m // 128, :] * (q[k_m, :] - 8)) exactly.
    # Positions cover every nibble slot of a packed word, every MFMA k-step and group edges.
    K, N = 384, 256
    hot = [0, 1, 2, 3, 4, 5, 6, 7, 8, 15, 31, 32, 63, 64, 96, 127, 128, 129, 200, 255, 256, 383]
    A, q, s = draw(K, N, len(hot), seed=22)
    A[:] = 0
    for m, k in enumerate(hot):
        A[m, k] = -2.0 if m % 3 == 0 else 1.0
    C = gpu_gemm(A, q, s)
    for m, k in enumerate(hot):
        w = s[k // 128].astype(np.float64) * (q[k].astype(np.float64) - 8.0) * float(A[m, k])
        assert same(C[m], w.astype(np.float16)), (m, k)


def test_integer_sums_are_bit_exact():
    # A in {-1, 0, 1} and power-of-two scales: every partial sum is exact in fp32, so the
    # result equals the oracle's bit for bit under any summation order or split.
    rng = np.random.default_rng(23)
    K, N, M = 4096, 1024, 33
    A = rng.integers(-1, 2, (M, K)).astype(np.float16)
    q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    s = rng.choice(np.array([0.25, 0.5, 1.0, 2.0], dtype=np.float16), (K // 128, N))
    assert same(gpu_gemm(A, q, s), oracle.gemm(A, q, s))


def test_zero_point_gives_zero():
    A, q, s = draw(2048, 512, 16, seed=24)
    q[:] = 8
    assert (bits(gpu_gemm(A, q, s)) & 0x7FFF == 0).all()


def test_power_of_two_scaling_is_exact():
    A, q, s = draw(4096, 1024, 16, seed=25)
    W = Weights(q, s)
    C = W.run(A).astype(np.float32)
    C2 = W.run((A.astype(np.float32) * 2).astype(np.float16)).astype(np.float32)
    big = np.abs(C) >= 2.0 ** -13
    assert np.array_equal(C2[big], 2 * C[big])


def test_repeated_runs_are_bitwise_identical():
    # many slices split between workgroups: the cross-workgroup sum order is fixed
    A, q, s = draw(18432, 512, 16, seed=26)
    W = Weights(q, s)
    first = W.run(A)
    for _ in range(3):
        assert np.array_equal(bits(W.run(A)), bits(first))
    check(first, oracle.gemm(A, q, s), "K=18432 N=512 M=16")


def test_nested_m_agrees():
    A, q, s = draw(2048, 1024, 128, seed=27)
    W = Weights(q, s)
    c128 = W.run(A)
    c16 = W.run(A[:16])
    check(c16, c128[:16].astype(np.float16), "M=16 vs M=128 rows")


# ------------------------------------------------------------------ boundary behaviour

def test_m_zero_is_a_no_op():
    _, q, s = draw(256, 64, 1, seed=28)
    W = Weights(q, s)
    out = torch.full((0, 64), 7.0, dtype=torch.float16, device="cuda")
    Ad = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    r = w4.gemm(Ad, W.packed, W.scales, 64, out=out)
    assert r.shape == (0, 64)
    lib = w4.library()
    ws = w4.new_workspace(1, 256, 64)
    st = lib.w4a16_gemm(Ad.data_ptr() or 16, W.packed.data_ptr(), W.scales.data_ptr(),
                        out.data_ptr() or 16, 0, 256, 64, ws.data_ptr(), None)
    assert st == w4.OK


def test_bad_shapes_rejected_on_device():
    _, q, s = draw(256, 64, 1, seed=29)
    W = Weights(q, s)
    A = torch.zeros((4, 256), dtype=torch.float16, device="cuda")
    lib = w4.library()
    ws = w4.new_workspace(4, 256, 64)
    out = torch.empty((4, 64), dtype=torch.float16, device="cuda")
    args = (A.data_ptr(), W.packed.data_ptr(), W.scales.data_ptr(), out.data_ptr())
    assert lib.w4a16_gemm(*args, 4, 200, 64, ws.data_ptr(), None) == w4.ESHAPE
    assert lib.w4a16_gemm(*args, 4, 256, 100, ws.data_ptr(), None) == w4.ESHAPE
    assert lib.w4a16_gemm(*args, 4, 256, 64, None, None) == w4.EINVAL


def test_workspace_shared_across_shapes_stays_clean():
    shapes = [(18432, 256, 16), (1024, 512, 3), (4096, 1024, 64), (18432, 64, 1), (1024, 512, 3)]
    need = max(w4.workspace_bytes(M, K, N) for K, N, M in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, (K, N, M) in enumerate(shapes):
        A, q, s = draw(K, N, M, seed=30 + i)
        check(Weights(q, s).run(A, ws=ws), oracle.gemm(A, q, s), f"shared ws K={K} N={N} M={M}")
        assert int(ws[:4096].count_nonzero()) == 0      # counters back to zero


# The 128-row kernel on the 72k x 18k weight at M = 128 splits column slices between stripes.
# Its pieces once went out with element 0 of row block 7 zeroed now and then (a 128-bit store's
# data register reset right behind the store): the same call must give the same bits on every
# run, and rows 112..127 must match the oracle on columns at every lane position of a slab.
def test_128_row_tiles_repeat_bit_for_bit_and_last_row_block_on_the_full_weight():
    K, N, M = 18432, 73728, 128
    A, q, s = draw(K, N, M, seed=5)
    W = Weights(q, s)
    first = W.run(A)
    for _ in range(4):
        assert np.array_equal(bits(W.run(A)), bits(first))
    cols = np.concatenate([np.arange(16 * j, 16 * j + 16) for j in (0, 1011, 2303, 4607)])
    ref = oracle.gemm(A[112:128], np.ascontiguousarray(q[:, cols]), np.ascontiguousarray(s[:, cols]))
    check(first[112:128, cols], ref, "M=128 rows 112..127")
    del W, q
    gc.collect()
    torch.cuda.empty_cache()


# Every kernel that splits slices between stripes, on a weight whose 16-tile slices split
# unevenly: the same call repeats bit for bit (a race in the piece stores shows as differing
# elements from run to run, whatever the oracle's tolerance).
@pytest.mark.parametrize("M", [24, 48, 64, 96, 113, 128])
def test_split_slices_repeat_bit_for_bit(M):
    K, N = 2048, 73728
    A, q, s = draw(K, N, M, seed=6)
    W = Weights(q, s)
    first = W.run(A)
    for _ in range(3):
        assert np.array_equal(bits(W.run(A)), bits(first)), M


# ------------------------------------------------------------------ full-size workloads

def _full_check(shape, seed=0):
    # every column at every M of the workload, in the launch configuration the benchmark
    # times; the oracle runs once at the largest M (its rows do not depend on M: pinned)
    A, q, s = draw(shape.K, shape.N, max(shape.Ms), seed=seed, sigma=shape.sigma)
    W = Weights(q, s)
    ref_all = oracle.gemm(A, q, s)
    del q, s
    gc.collect()
    for M in shape.Ms:
        C = W.run(A[:M])
        assert np.isfinite(C).all()
        check(C, ref_all[:M], f"{shape.name} M={M} (all {shape.N} columns)")
    del W
    torch.cuda.empty_cache()


@pytest.mark.slow
@pytest.mark.parametrize("shape", [sh for wl in (SMALL, LARGE, LLAMA2_7B, LLAMA2_70B,
                                                 COMPUTE_SWEEP) for sh in wl.shapes],
                         ids=lambda sh: sh.name)
def test_full_size_workloads_all_columns(shape):
    _full_check(shape)


# One tensor-parallel rank's shapes of the 70B block, every column against the oracle.
@pytest.mark.parametrize("shape", LLAMA2_70B_TP8.shapes, ids=lambda sh: sh.name)
def test_tensor_parallel_rank_shapes(shape):
    A, q, s = draw(shape.K, shape.N, max(shape.Ms), seed=3)
    W = Weights(q, s)
    ref = oracle.gemm(A, q, s)
    for M in shape.Ms:
        check(W.run(A[:M]), ref[:M], f"{shape.name} M={M}")


# ------------------------------------------------------------------ other packed formats
# One scale per column (group = K) and zero points per group and column (w4a16_pack_zp,
# w4a16_gemm_ex), against the oracle with the same group and zero points.

from workloads import draw_zeros  # noqa: E402

FORMATS = {"column": (True, False), "zeros": (False, True), "column_zeros": (True, True)}


class FmtWeights:
    def __init__(self, q, s, group, zeros=None):
        self.K, self.N = q.shape
        self.group, self.zp = group, zeros is not None
        packed, params = w4.pack(q, s, group=group, zeros=zeros)
        self.packed, self.params = w4.to_device(packed, params)

    def run(self, A, ws=None):
        Ad = torch.from_numpy(np.ascontiguousarray(A)).cuda()
        C = w4.gemm(Ad, self.packed, self.params, self.N, ws=ws, group=self.group,
                    zero_points=self.zp)
        torch.cuda.synchronize()
        return C.cpu().numpy()


def fmt_case(fmt, K, N, M, seed):
    col, zp = FORMATS[fmt]
    g = K if col else 128
    A, q, s = draw(K, N, M, seed=seed, group=g)
    z = draw_zeros(K, N, seed=seed, group=g) if zp else None
    return A, q, s, g, z


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("M,K,N", [(1, 1024, 512), (16, 2048, 1024), (33, 1024, 320),
                                   (64, 4096, 192), (130, 2048, 1024), (300, 1024, 768),
                                   (16, 18432, 512), (128, 9216, 256), (5, 384, 64)])
def test_formats_against_oracle(fmt, M, K, N):
    A, q, s, g, z = fmt_case(fmt, K, N, M, seed=M + K + N)
    C = FmtWeights(q, s, g, z).run(A)
    check(C, oracle.gemm(A, q, s, group=g, zeros=z), f"{fmt} M={M} K={K} N={N}")


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("M", [3, 40, 129])
def test_formats_one_hot_rows_are_bit_exact(fmt, M):
    # row m is 1 at k_m: C[m, :] = fp16(s * (q[k_m] - z)) exactly (one rounding)
    K, N = 384, 256
    A, q, s, g, z = fmt_case(fmt, K, N, M, seed=60 + M)
    A[:] = 0
    ks = [(7 * m + 3) % K for m in range(M)]
    for m, k in enumerate(ks):
        A[m, k] = 1.0
    C = FmtWeights(q, s, g, z).run(A)
    for m, k in enumerate(ks):
        zz = 8 if z is None else z[k // g].astype(np.float64)
        w = s[k // g].astype(np.float64) * (q[k].astype(np.float64) - zz)
        assert same(C[m], w.astype(np.float16)), (fmt, m, k)


@pytest.mark.parametrize("col", [False, True])
@pytest.mark.parametrize("M", [16, 64, 128])
def test_code_equal_to_zero_point_gives_zero_on_gpu(col, M):
    K, N = 1024, 512
    g = K if col else 128
    A, _, s = draw(K, N, M, seed=70, group=g)
    z = draw_zeros(K, N, seed=70, group=g)
    q = np.repeat(z, g, axis=0)
    assert (bits(FmtWeights(q, s, g, z).run(A)) & 0x7FFF == 0).all()


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_formats_repeat_bit_for_bit_with_split_slices(fmt):
    K, N, M = 18432, 512, 128
    A, q, s, g, z = fmt_case(fmt, K, N, M, seed=71)
    W = FmtWeights(q, s, g, z)
    first = W.run(A)
    check(first, oracle.gemm(A, q, s, group=g, zeros=z), f"{fmt} K={K} N={N} M={M}")
    for _ in range(2):
        assert np.array_equal(bits(W.run(A, ws=w4.new_workspace(M, K, N))), bits(first))


@pytest.mark.slow
@pytest.mark.parametrize("fmt", list(FORMATS))
def test_formats_full_size_72kx18k_all_columns(fmt):
    K, N = LARGE.shapes[0].K, LARGE.shapes[0].N
    Ms = [1, 16, 32, 64, 128]
    A, q, s, g, z = fmt_case(fmt, K, N, max(Ms), seed=0)
    W = FmtWeights(q, s, g, z)
    ref = oracle.gemm(A, q, s, group=g, zeros=z)
    del q
    gc.collect()
    for M in Ms:
        C = W.run(A[:M])
        assert np.isfinite(C).all()
        check(C, ref[:M], f"{fmt} 72k x 18k M={M} (all columns)")
    del W
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ nothing written past C

@pytest.mark.parametrize("fmt", ["group128", "zeros"])
@pytest.mark.parametrize("M,K,N", [(1, 1024, 512), (3, 2048, 256), (15, 1024, 1024),
                                   (17, 1024, 512), (33, 1024, 512), (63, 2048, 256),
                                   (65, 1024, 1024), (100, 1024, 512), (129, 2048, 1024),
                                   (200, 1024, 768), (1, 18432, 512)])
def test_no_write_past_the_rows_of_c(M, K, N, fmt):
    # C is the head of a larger buffer whose tail covers every row a padded tile could
    # address (up to 128 rows past M); the tail must keep its fill pattern.
    zp = fmt == "zeros"
    A, q, s = draw(K, N, M, seed=M + N)
    z = draw_zeros(K, N, seed=M) if zp else None
    packed, params = w4.to_device(*w4.pack(q, s, zeros=z))
    Ad = torch.from_numpy(A).cuda()
    pad = 128 * ((M + 127) // 128) + 128
    buf = torch.full((pad * N + M * N,), -7.0, dtype=torch.float16, device="cuda")
    C = buf[:M * N].view(M, N)
    w4.gemm(Ad, packed, params, N, out=C, zero_points=zp)
    torch.cuda.synchronize()
    tail = buf[M * N:]
    bad = int((tail != -7.0).sum())
    assert bad == 0, f"{bad} fp16 values written past C (M={M}, N={N})"
    check(C.cpu().numpy(), oracle.gemm(A, q, s, zeros=z), f"{fmt} M={M} K={K} N={N}")


# ------------------------------------------------------------------ M <= 16: whole-K workgroups

# M = 20 and 32 run the kernel's two-row-block form (one workgroup per CU only), M = 40 and
# 64 its four-row-block form where N takes at most four slabs per CU, M = 100 and 128 two
# 64-row sub-problems of it side by side where that still fits (1024 x 8192 here).
# N chosen for 2 to 9 slabs per workgroup: one workgroup per CU up to 7 slabs (8192 -> 2,
# 9216 -> 3, 12544 -> 4, 16640 -> 5, 26880 -> 7 on 256 CUs), 73728 -> 6 or 9 with two or three
# per CU; 8960 (560 slabs in workgroups of three), 17152 (1072 in fives) and 27904 (1744 in
# sevens) leave a last workgroup short, and odd slab counts put first slabs at every offset
# mod 4.  K = 128..384 so that some waves of a workgroup get no K tile at all.
SKINNY_SHAPES = [(128, 9216), (256, 16640), (384, 26880), (1024, 16640), (4096, 8448),
                 (2048, 73728), (640, 12544), (1024, 8192), (4096, 8960), (256, 17152),
                 (384, 27904)]


@pytest.mark.parametrize("fmt", ["group128"] + list(FORMATS))
@pytest.mark.parametrize("K,N", SKINNY_SHAPES)
@pytest.mark.parametrize("M", [1, 5, 16, 20, 32, 40, 64, 100, 128])
def test_whole_k_workgroups_against_oracle(M, K, N, fmt):
    if fmt == "group128":
        A, q, s = draw(K, N, M, seed=M + K + N)
        W, g, z = FmtWeights(q, s, 128), 128, None
    else:
        A, q, s, g, z = fmt_case(fmt, K, N, M, seed=M + K + N)
        W = FmtWeights(q, s, g, z)
    C = W.run(A)
    check(C, oracle.gemm(A, q, s, group=g, zeros=z), f"{fmt} M={M} K={K} N={N}")
    # bitwise repeatable: the four waves' sums meet in a fixed order
    assert np.array_equal(bits(W.run(A)), bits(C))


@pytest.mark.parametrize("fmt", ["group128", "zeros", "column_zeros"])
def test_whole_k_workgroups_one_hot_rows_are_bit_exact(fmt):
    K, N, M = 512, 16640, 16
    if fmt == "group128":
        A, q, s = draw(K, N, M, seed=90)
        g, z = 128, None
    else:
        A, q, s, g, z = fmt_case(fmt, K, N, M, seed=90)
    A[:] = 0
    ks = [0, 7, 127, 128, 200, 255, 256, 300, 383, 384, 385, 450, 500, 510, 511, 64]
    for m, k in enumerate(ks):
        A[m, k] = 1.0
    C = FmtWeights(q, s, g, z).run(A)
    for m, k in enumerate(ks):
        zz = 8 if z is None else z[k // g].astype(np.float64)
        w = s[k // g].astype(np.float64) * (q[k].astype(np.float64) - zz)
        assert same(C[m], w.astype(np.float16)), (fmt, m, k)


# Whole-K workgroups with K split between several workgroups (few slab groups over a long K;
# M = 17..32 and 33..64 run the kernel's two- and four-row-block forms, M = 65..128 two 64-row
# sub-problems side by side, each with its own counters and pieces).  The selection takes,
# as (slabs per workgroup, splits): 8192 x 1280 (2, 6) or (4, 8); 14336 x 2048 (4, 8);
# 28672 x 1024 (2, 8); 6144 x 256 (1, 6); 11008 x 4096 (4, 4), whose 86 K tiles make splits of
# 21 and 22.  The last workgroup to finish a slab group sums the pieces: two calls on one
# workspace check that the counters come back to zero and that results repeat bit for bit.
SPLIT_K_SHAPES = [(8192, 1280), (14336, 2048), (28672, 1024), (6144, 256), (11008, 4096)]


@pytest.mark.parametrize("fmt", ["group128"] + list(FORMATS))
@pytest.mark.parametrize("K,N", SPLIT_K_SHAPES)
@pytest.mark.parametrize("M", [1, 5, 16, 17, 32, 33, 64, 65, 128])
def test_whole_k_split_k_against_oracle(M, K, N, fmt):
    if fmt == "group128":
        A, q, s = draw(K, N, M, seed=M + K + N + 1)
        W, g, z = FmtWeights(q, s, 128), 128, None
    else:
        A, q, s, g, z = fmt_case(fmt, K, N, M, seed=M + K + N + 1)
        W = FmtWeights(q, s, g, z)
    ws = w4.workspace(M, K, N, torch.device("cuda"))
    C = W.run(A, ws=ws)
    check(C, oracle.gemm(A, q, s, group=g, zeros=z), f"split-K {fmt} M={M} K={K} N={N}")
    assert np.array_equal(bits(W.run(A, ws=ws)), bits(C))
    assert int(ws[:4096].count_nonzero()) == 0        # the counters are back at zero


# More than four slabs per workgroup where A has real rows: 8192 x 10240 at M = 9..32 takes
# 5 slabs and 2 splits, 28672 x 8192 at M = 9..16 8 slabs and 4 splits; longer walks of the
# whole-K kernel: 28672 x 8192 at M = 32 (two row blocks, 28 tiles a wave), 8192 x 10240 at
# M = 40 and 64 (four row blocks by DMA, 16 tiles a wave); four row blocks over 5, 6 and 7
# slabs: 4096 x 20480, 4096 x 22016, 8192 x 28672; two 64-row sub-problems of 6 and 5 slabs:
# 4096 x 12288 at M = 96, 8192 x 10240 at M = 128.
@pytest.mark.parametrize("fmt", ["group128"] + list(FORMATS))
@pytest.mark.parametrize("K,N,M", [(8192, 10240, 12), (8192, 10240, 24), (8192, 10240, 32),
                                   (28672, 8192, 16), (28672, 8192, 32), (8192, 10240, 40),
                                   (8192, 10240, 64), (4096, 20480, 64), (4096, 22016, 40),
                                   (8192, 28672, 64), (4096, 12288, 96), (8192, 10240, 128)])
def test_whole_k_wide_slab_groups_against_oracle(K, N, M, fmt):
    if fmt == "group128":
        A, q, s = draw(K, N, M, seed=M + K + N + 2)
        W, g, z = FmtWeights(q, s, 128), 128, None
    else:
        A, q, s, g, z = fmt_case(fmt, K, N, M, seed=M + K + N + 2)
        W = FmtWeights(q, s, g, z)
    ws = w4.workspace(M, K, N, torch.device("cuda"))
    C = W.run(A, ws=ws)
    check(C, oracle.gemm(A, q, s, group=g, zeros=z), f"wide slab groups {fmt} M={M} K={K} N={N}")
    assert np.array_equal(bits(W.run(A, ws=ws)), bits(C))
    assert int(ws[:4096].count_nonzero()) == 0


# At M <= 8 with up to three slabs per workgroup and at least six K tiles a wave the whole-K
# kernel keeps one more tile of registers in flight (three buffers): 8192 x 8192 (2 slabs),
# 4096 x 12288 (3), 8192 x 1280 (slabs and K splits from the split search), 6144 x 256
# (1 slab, K split).
@pytest.mark.parametrize("fmt", ["group128"] + list(FORMATS))
@pytest.mark.parametrize("K,N", [(8192, 8192), (4096, 12288), (8192, 1280), (6144, 256)])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_whole_k_three_buffers_against_oracle(M, K, N, fmt):
    if fmt == "group128":
        A, q, s = draw(K, N, M, seed=M + K + N + 3)
        W, g, z = FmtWeights(q, s, 128), 128, None
    else:
        A, q, s, g, z = fmt_case(fmt, K, N, M, seed=M + K + N + 3)
        W = FmtWeights(q, s, g, z)
    ws = w4.workspace(M, K, N, torch.device("cuda"))
    C = W.run(A, ws=ws)
    check(C, oracle.gemm(A, q, s, group=g, zeros=z), f"three buffers {fmt} M={M} K={K} N={N}")
    assert np.array_equal(bits(W.run(A, ws=ws)), bits(C))
    assert int(ws[:4096].count_nonzero()) == 0


@pytest.mark.parametrize("fmt", ["group128", "column_zeros"])
def test_whole_k_split_k_one_hot_rows_are_bit_exact(fmt):
    # the other splits' pieces of a one-hot row are zeros: the sum is the one product
    K, N, M = 14336, 2048, 16
    if fmt == "group128":
        A, q, s = draw(K, N, M, seed=91)
        g, z = 128, None
    else:
        A, q, s, g, z = fmt_case(fmt, K, N, M, seed=91)
    A[:] = 0
    ks = [0, 127, 128, 3583, 3584, 7167, 7168, 7200, 10751, 10752, 14335, 5000, 9000, 12000,
          1, 14000]
    for m, k in enumerate(ks):
        A[m, k] = 1.0
    C = FmtWeights(q, s, g, z).run(A)
    for m, k in enumerate(ks):
        zz = 8 if z is None else z[k // g].astype(np.float64)
        w = s[k // g].astype(np.float64) * (q[k].astype(np.float64) - zz)
        assert same(C[m], w.astype(np.float16)), (fmt, m, k)


# Seeded random shapes across every kernel choice (whole-K at M <= 16 with two or three
# workgroups per CU, 16/32/64-row stripes, 128-row tiles, several row sub-problems), the
# stripe-count model's range of split pieces and N from one to many slices, for all four
# formats.  The oracle runs them in seconds.
def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([1, 2, 3, 5, 8, 11, 16, 17, 24, 31, 32, 40, 64, 65, 100, 128, 129, 200]))
        K = 128 * int(rng.integers(1, 17))
        N = 64 * int(rng.integers(1, 49))
        if rng.random() < 0.4:
            N = 256 * int(rng.integers(1, 13))
        out.append((M, K, N))
    return out


@pytest.mark.parametrize("zp", [False, True])
@pytest.mark.parametrize("col", [False, True])
@pytest.mark.parametrize("M,K,N", _random_shapes(12, 2026))
def test_random_shapes_every_format(M, K, N, col, zp):
    A, q, s = draw(K, N, M, seed=M * 7 + K + N)
    group = K if col else 128
    if col:
        s = s[:1].copy()
    z = None
    if zp:
        from workloads import draw_zeros
        z = draw_zeros(K, N, seed=M + K, group=group)
    packed, params = w4.pack(q, s, group=group, zeros=z)
    pd, prm = w4.to_device(packed, params)
    Ad = torch.from_numpy(A).cuda()
    C = w4.gemm(Ad, pd, prm, N, group=group, zero_points=zp)
    torch.cuda.synchronize()
    ref = oracle.gemm(A, q, s, group=group, zeros=z)
    check(C.cpu().numpy(), ref, f"M={M} K={K} N={N} col={col} zp={zp}")


def test_read_probe_streams_without_writing():
    # all-ones fp16 words XOR to zero, never the checksum that would store
    x = torch.ones(1 << 22, dtype=torch.float16, device="cuda")
    out = w4.read_probe(x)
    torch.cuda.synchronize()
    assert int(out.count_nonzero()) == 0


# ------------------------------------------------------------------ workspace sizing and checks

def test_header_workspace_bound_covers_what_the_device_asks_for():
    shapes = [(M, K, N) for M in (1, 2, 8, 16, 17, 24, 32, 48, 64, 65, 100, 128, 129, 256, 1024)
              for K, N in ((128, 64), (1024, 1024), (18432, 73728), (8192, 28672), (8192, 1280),
                           (28672, 8192), (4096, 4096), (11008, 4096), (1024, 192), (2048, 73728))]
    for M, K, N in shapes:
        assert w4.workspace_bytes(M, K, N) <= w4.workspace_bound(M, K, N), (M, K, N)


def test_caller_workspace_is_checked_before_the_call():
    A, q, s = draw(4096, 73728, 64, seed=33)
    W = Weights(q, s)
    Ad = torch.from_numpy(A).cuda()
    need = w4.workspace_bytes(64, 4096, 73728)
    assert need > 4096
    with pytest.raises(ValueError):
        w4.gemm(Ad, W.packed, W.scales, W.N, ws=torch.zeros(need - 1, dtype=torch.uint8,
                                                               device="cuda"))
    with pytest.raises(ValueError):
        w4.gemm(Ad, W.packed, W.scales, W.N, ws=torch.zeros(need // 4 + 1, dtype=torch.int32,
                                                               device="cuda"))
    with pytest.raises(ValueError):
        w4.gemm(Ad, W.packed, W.scales, W.N, ws=torch.zeros(need, dtype=torch.uint8))
    C = w4.gemm(Ad, W.packed, W.scales, W.N, ws=torch.zeros(need, dtype=torch.uint8,
                                                           device="cuda"))
    torch.cuda.synchronize()
    check(C.cpu().numpy(), oracle.gemm(A, q, s), "exact-size caller workspace")


def test_cached_workspaces_are_per_stream():
    side = torch.cuda.Stream()
    a = w4.workspace(16, 1024, 1024, torch.device("cuda", 0))
    b = w4.workspace(16, 1024, 1024, torch.device("cuda", 0), stream=side)
    assert a.data_ptr() != b.data_ptr()
    assert w4.workspace(16, 1024, 1024, torch.device("cuda", 0)).data_ptr() == a.data_ptr()


def test_mfma_probe_runs_on_random_operands():
    src = (torch.randn(1 << 16, device="cuda") * 0.5).half()
    for shape in (0, 1):
        out, fl = w4.mfma_probe(src, shape=shape, workgroups=8, iters=4)
        torch.cuda.synchronize()
        assert fl == 8 * 4 * 4 * 64 * (16384 if shape == 0 else 32768)
        assert torch.isfinite(out).all()
        assert out.abs().sum() > 0


# ------------------------------------------------------------------ 32 rows, two per CU
# M = 17..32 on weights of more than seven slabs per CU (symmetric formats): whole-K
# workgroups of seven to nine slabs, two per CU, the raw-decode sums formed slab by slab.
# N = 73472, 65536 and 57344 give 4592, 4096 and 3584 slabs (nine, eight and seven per
# workgroup; the last workgroup of the first is two slabs short); K = 128 leaves three of four
# waves without tiles.  N = 32768 (four slabs) takes the stripe kernel; the zero-point formats
# take it everywhere; both are run too.
@pytest.mark.parametrize("fmt", ["group128"] + list(FORMATS))
@pytest.mark.parametrize("K,N", [(1024, 32768), (256, 73472), (384, 65536), (128, 57344)])
@pytest.mark.parametrize("M", [17, 24, 32])
def test_32_row_two_per_cu_form_against_oracle(M, K, N, fmt):
    if fmt == "group128":
        A, q, s = draw(K, N, M, seed=M * 7 + K + N)
        W, g, z = FmtWeights(q, s, 128), 128, None
    else:
        A, q, s, g, z = fmt_case(fmt, K, N, M, seed=M * 7 + K + N)
        W = FmtWeights(q, s, g, z)
    C = W.run(A)
    check(C, oracle.gemm(A, q, s, group=g, zeros=z), f"two-per-CU {fmt} M={M} K={K} N={N}")
    assert np.array_equal(bits(W.run(A)), bits(C))


def test_32_row_two_per_cu_form_bit_exact_cases():
    # one-hot rows, q = 8 everywhere and power-of-two scaling on the 9-slab form
    K, N, M = 256, 73472, 32
    _, q, s = draw(K, N, M, seed=91)
    W = Weights(q, s)
    A = np.zeros((M, K), dtype=np.float16)
    ks = np.arange(M) * 7 % K
    A[np.arange(M), ks] = 1.0
    C = W.run(A)
    want = (s[ks // 128].astype(np.float32) * (q[ks].astype(np.float32) - 8)).astype(np.float16)
    assert same(C, want)
    q8 = np.full_like(q, 8)
    A2, _, _ = draw(K, N, M, seed=92)
    assert (bits(Weights(q8, s).run(A2)) & 0x7FFF == 0).all()
    C1 = W.run(A2).astype(np.float32)
    C2 = W.run((A2.astype(np.float32) * 2).astype(np.float16)).astype(np.float32)
    big = np.abs(C1) >= 2.0 ** -13
    assert np.array_equal(C2[big], 2 * C1[big])

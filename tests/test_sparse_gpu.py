"""GPU parity of the 2:4-sparse path (w4a16_pack_24 + w4a16_gemm_24) against the oracle.

The oracle needs nothing new: a 2:4-sparse weight is the dense weight with code 8 (zero) at
the pruned positions, and oracle.gemm computes the product from those codes.  Same bar as the
dense path: relative Frobenius <= 1e-3, max abs <= 1e-2 * max |C_ref|; bit-exact where the
answer is exactly representable.
"""
import gc

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mixed_precision_w4a16_amd as w4
import oracle
from workloads import LARGE, draw, sparsify_24

pytestmark = pytest.mark.gpu


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


def check(C, ref, what=""):
    d = C.astype(np.float64) - ref.astype(np.float64)
    nref = np.linalg.norm(ref.astype(np.float64))
    rel = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    mref = np.abs(ref.astype(np.float64)).max()
    mx = np.abs(d).max() / mref if mref > 0 else np.abs(d).max()
    print(f"  {what} rel_fro={rel:.2e} max_abs/max|C|={mx:.2e}", flush=True)
    assert np.isfinite(C).all(), what
    assert rel <= 1e-3, (what, rel)
    assert mx <= 1e-2, (what, mx)


class Sparse:
    def __init__(self, q, s):
        self.K, self.N = q.shape
        self.packed, self.scales = w4.to_device(*w4.pack_24(q, s))

    def run(self, A, out=None):
        Ad = torch.from_numpy(np.ascontiguousarray(A)).cuda()
        C = w4.gemm_24(Ad, self.packed, self.scales, self.N, out=out)
        torch.cuda.synchronize()
        return C.cpu().numpy()


def case(K, N, M, seed):
    A, q, s = draw(K, N, M, seed=seed)
    return A, sparsify_24(q, seed), s


# M <= 16 (whole-K workgroups): N = 256 .. 16640 gives 1 to 3 slabs per workgroup (16640: the
# last workgroup holds two); K = 128 / 384: waves without a K tile.  M > 16 (stripes of
# 32- and 64-row tiles): one to three row sub-problems (65, 130), slices split between
# several workgroups (K = 18432 with N = 256: up to one tile per workgroup) or whole.
@pytest.mark.parametrize("K,N", [(128, 256), (384, 512), (1024, 1024), (2048, 16640),
                                 (4096, 9216), (18432, 256)])
@pytest.mark.parametrize("M", [1, 3, 16, 17, 32, 33, 64, 65, 130])
def test_sparse_against_oracle(M, K, N):
    A, q, s = case(K, N, M, seed=M + K + N)
    W = Sparse(q, s)
    C = W.run(A)
    check(C, oracle.gemm(A, q, s), f"2:4 M={M} K={K} N={N}")
    assert np.array_equal(bits(W.run(A)), bits(C))       # fixed summation order


@pytest.mark.parametrize("M", [5, 16, 40])
def test_sparse_one_hot_rows_are_bit_exact(M):
    # row m is 1 at k_m: C[m] = fp16(s * (q[k_m] - 8)) exactly -- zero where k_m was pruned
    K, N = 512, 512
    A, q, s = case(K, N, M, seed=40 + M)
    A[:] = 0
    ks = [(37 * m + 5) % K for m in range(M)]
    for m, k in enumerate(ks):
        A[m, k] = 1.0
    C = Sparse(q, s).run(A)
    for m, k in enumerate(ks):
        w = s[k // 128].astype(np.float64) * (q[k].astype(np.float64) - 8.0)
        assert same(C[m], w.astype(np.float16)), (m, k)


def test_sparse_all_pruned_gives_zero_and_integer_sums_are_exact():
    K, N, M = 1024, 512, 24
    A, q, s = case(K, N, M, seed=9)
    assert (bits(Sparse(np.full_like(q, 8), s).run(A)) & 0x7FFF == 0).all()
    rng = np.random.default_rng(10)
    Ai = rng.integers(-1, 2, (M, K)).astype(np.float16)
    sp2 = rng.choice(np.array([0.25, 0.5, 1.0, 2.0], dtype=np.float16), (K // 128, N))
    assert same(Sparse(q, sp2).run(Ai), oracle.gemm(Ai, q, sp2))


@pytest.mark.parametrize("M,N", [(1, 512), (17, 1024), (65, 256)])
def test_sparse_no_write_past_the_rows_of_c(M, N):
    K = 1024
    A, q, s = case(K, N, M, seed=M)
    W = Sparse(q, s)
    Ad = torch.from_numpy(A).cuda()
    buf = torch.full((M * N + 128 * N,), -7.0, dtype=torch.float16, device="cuda")
    w4.gemm_24(Ad, W.packed, W.scales, N, out=buf[:M * N].view(M, N))
    torch.cuda.synchronize()
    assert int((buf[M * N:] != -7.0).sum()) == 0
    check(buf[:M * N].view(M, N).cpu().numpy(), oracle.gemm(A, q, s), f"M={M} N={N}")


def test_sparse_leaves_the_counters_zero_and_repeats_across_workspaces():
    # split slices count arrivals in the workspace's first 4 KiB; every call leaves them 0
    K, N, M = 4096, 1024, 50
    A, q, s = case(K, N, M, seed=77)
    W = Sparse(q, s)
    Ad = torch.from_numpy(A).cuda()
    ws = w4.new_workspace(M, K, N, "cuda")
    C0 = w4.gemm_24(Ad, W.packed, W.scales, N, ws=ws).cpu().numpy()
    torch.cuda.synchronize()
    assert int(ws[:4096].count_nonzero()) == 0
    ws2 = w4.new_workspace(M, K, N, "cuda")
    C1 = w4.gemm_24(Ad, W.packed, W.scales, N, ws=ws2).cpu().numpy()
    assert np.array_equal(bits(C0), bits(C1))
    check(C0, oracle.gemm(A, q, s), "counters")


@pytest.mark.slow
def test_sparse_full_size_72kx18k_all_columns():
    sh = LARGE.shapes[0]
    K, N = sh.K, sh.N
    A, q, s = case(K, N, max(sh.Ms), seed=0)
    W = Sparse(q, s)
    ref = oracle.gemm(A, q, s)
    del q
    gc.collect()
    for M in sh.Ms:
        C = W.run(A[:M])
        assert np.isfinite(C).all()
        check(C, ref[:M], f"2:4 72k x 18k M={M} (all columns)")
    del W
    torch.cuda.empty_cache()

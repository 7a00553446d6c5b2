"""w4a16_gemm_noalloc, the entry point that allocates nothing (its scratch is the library's
own per-GPU device array), called through the C ABI and compared with w4a16_gemm_ex on the
same inputs: the same kernels run, so the outputs must agree bit for bit (and with the oracle
within the parity bar).  Two calls in a row, the second on a smaller input, so the second
call runs on the scratch the first one left (counters back at zero, stale partial tiles)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mixed_precision_w4a16_amd as w4
import oracle
from workloads import draw

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def bits(t):
    return t.cpu().numpy().view(np.uint16)


def run_both(M, K, N, group, zp, seed):
    A, q, s = draw(K, N, M, seed=seed)
    z = None
    if group != 128:
        s = np.ascontiguousarray(s[:1])
    if zp:
        z = np.random.default_rng(seed + 1).integers(0, 16, s.shape, dtype=np.uint8)
    packed, params = w4.pack(q, s, group=group, zeros=z)
    pd, sd = w4.to_device(packed, params)
    Ad = torch.from_numpy(A).cuda()
    lib = w4.library()
    c_ex = torch.empty((M, N), dtype=torch.float16, device="cuda")
    c_na = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    ws = w4.new_workspace(M, K, N)
    st = torch.cuda.current_stream().cuda_stream
    print(f"  noalloc M={M} K={K} N={N} group={group} zp={zp}", flush=True)
    assert lib.w4a16_gemm_ex(Ad.data_ptr(), pd.data_ptr(), sd.data_ptr(), c_ex.data_ptr(), M, K,
                             N, group, int(zp), ws.data_ptr(), st) == w4.OK
    assert lib.w4a16_gemm_noalloc(Ad.data_ptr(), pd.data_ptr(), sd.data_ptr(), c_na.data_ptr(),
                                  M, K, N, group, int(zp), st) == w4.OK
    torch.cuda.synchronize()
    assert np.array_equal(bits(c_na), bits(c_ex)), (M, K, N)
    ref = oracle.gemm(A, q, s, group=group, zeros=z).astype(np.float64)
    d = c_na.cpu().numpy().astype(np.float64) - ref
    assert np.linalg.norm(d) / np.linalg.norm(ref) <= 1e-3
    assert np.abs(d).max() <= 1e-2 * np.abs(ref).max()


# first call: split slices with fp32 partial tiles (128-row tiles over 288 slices); second,
# smaller: whole-K workgroups with K splits (1 KiB pieces and counters)
@pytest.mark.parametrize("fmt", [(128, False), (None, True)])
def test_noalloc_equals_gemm_ex_two_calls_second_smaller(fmt):
    group, zp = fmt
    run_both(128, 2048, 73728, group or 2048, zp, seed=81)
    run_both(16, 8192, 1280, group or 8192, zp, seed=82)


def test_noalloc_rejects_bad_arguments():
    lib = w4.library()
    d = torch.zeros(4096, dtype=torch.uint8, device="cuda").data_ptr()
    assert lib.w4a16_gemm_noalloc(None, d, d, d, 16, 1024, 1024, 128, 0, None) == w4.EINVAL
    assert lib.w4a16_gemm_noalloc(d, d, d, d, -1, 1024, 1024, 128, 0, None) == w4.EINVAL
    assert lib.w4a16_gemm_noalloc(d, d, d, d, 16, 1000, 1024, 128, 0, None) == w4.ESHAPE
    assert lib.w4a16_gemm_noalloc(d, d, d, d, 16, 1024, 1024, 64, 0, None) == w4.ESHAPE
    assert lib.w4a16_gemm_noalloc(d, d, d, d, 16, 1024, 1024, 128, 2, None) == w4.EINVAL
    assert lib.w4a16_gemm_noalloc(d, d, d, d, 0, 1024, 1024, 128, 0, None) == w4.OK


def test_every_workload_shape_fits_the_scratch():
    for M, K, N in [(128, 18432, 73728), (1024, 8192, 28672), (64, 18432, 73728),
                    (128, 8192, 57344), (16, 28672, 8192), (200, 1024, 768)]:
        assert w4.workspace_bytes(M, K, N) <= w4.NOALLOC_SCRATCH_BYTES, (M, K, N)

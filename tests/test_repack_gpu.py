"""GPU parity of the load-time repack (w4a16_repack): checkpoint-style packed words on the
device -> the multiply's layout on the device.

Expected values: the oracle's decoders give the codes (and zero points) the source words
hold; the documented layout of those codes (tests/layouts.py) is what the repack must write,
bit for bit.  The repacked weights then go through the multiply and are checked against the
oracle's product of the decoded codes.
"""
import gc

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mixed_precision_w4a16_amd as w4
import oracle
from layouts import encode_along_k, encode_along_n, layout_reference, params_layout_reference
from workloads import LARGE, draw, draw_zeros

pytestmark = pytest.mark.gpu

AWQ_LIKE = (0, 2, 4, 6, 1, 3, 5, 7)
ORDERS = {"k": None, "n": None, "n_interleaved": AWQ_LIKE, "n_shuffled": (5, 0, 7, 2, 6, 1, 3, 4)}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def dev_words(w):
    return torch.from_numpy(np.ascontiguousarray(w).view(np.int32)).cuda()


def source(q, z, src, order):
    """Device source tensors and what the oracle reads back from them."""
    K, N = q.shape
    if src == "k":
        qw = encode_along_k(q)
        codes = oracle.decode_along_k(qw, K, N)
        layout = w4.PACKED_ALONG_K
    else:
        qw = encode_along_n(q, order)
        codes = oracle.decode_along_n(qw, K, N, order)
        layout = w4.PACKED_ALONG_N
    zw = zeros = None
    if z is not None:
        zw = encode_along_n(z, order)
        zeros = oracle.decode_along_n(zw, z.shape[0], N, order)
    return layout, dev_words(qw), (None if zw is None else dev_words(zw)), codes, zeros


def run_repack(q, s, z, src, group):
    order = ORDERS[src]
    K, N = q.shape
    layout, qw, zw, codes, zeros = source(q, z, src, order)
    sd = torch.from_numpy(np.ascontiguousarray(s)).cuda()
    packed, params = w4.repack(qw, sd, K, N, layout, group=group, qzeros=zw,
                               order=None if order is None else list(order))
    torch.cuda.synchronize()
    return packed, params, codes, zeros


@pytest.mark.parametrize("src", list(ORDERS))
@pytest.mark.parametrize("zp", [False, True])
@pytest.mark.parametrize("col", [False, True])
@pytest.mark.parametrize("K,N", [(128, 16), (256, 48), (384, 320), (1024, 1024), (256, 272),
                                 (2048, 4096), (640, 1552), (256, 384), (128, 1280)])
def test_repack_writes_the_documented_layout(K, N, src, zp, col):
    # N = 16 / 48 / 272 / 320 / 384 / 1552: tiles of 64 and 256 columns cut short at the right
    # edge; N = 384 and 1280 put 2 and 4 slabs' parameters side by side
    g = K if col else 128
    _, q, s = draw(K, N, 1, seed=K + 3 * N, group=g)
    z = draw_zeros(K, N, seed=K + N, group=g) if zp else None
    packed, params, codes, zeros = run_repack(q, s, z, src, g)
    ref_p, ref_s = layout_reference(codes, s.view(np.uint16))
    assert np.array_equal(packed.cpu().numpy().view(np.uint32), ref_p)
    want = ref_s if zeros is None else params_layout_reference(s, zeros)
    assert np.array_equal(params.cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("src", ["k", "n_interleaved"])
@pytest.mark.parametrize("zp,col", [(False, False), (True, False), (True, True), (False, True)])
@pytest.mark.parametrize("M,K,N", [(16, 1024, 512), (70, 2048, 768), (1, 4096, 256)])
def test_repacked_weights_multiply_like_the_oracle(M, K, N, src, zp, col):
    g = K if col else 128
    A, q, s = draw(K, N, M, seed=M + K, group=g)
    z = draw_zeros(K, N, seed=M, group=g) if zp else None
    packed, params, codes, zeros = run_repack(q, s, z, src, g)
    Ad = torch.from_numpy(A).cuda()
    C = w4.gemm(Ad, packed, params, N, group=g, zero_points=zp)
    torch.cuda.synchronize()
    ref = oracle.gemm(A, codes, s, group=g, zeros=zeros)
    d = C.cpu().numpy().astype(np.float64) - ref.astype(np.float64)
    rel = np.linalg.norm(d) / np.linalg.norm(ref.astype(np.float64))
    mx = np.abs(d).max() / np.abs(ref.astype(np.float64)).max()
    print(f"  {src} zp={zp} col={col} M={M} K={K} N={N} rel_fro={rel:.2e} max={mx:.2e}", flush=True)
    assert rel <= 1e-3 and mx <= 1e-2


@pytest.mark.slow
@pytest.mark.parametrize("src", ["k", "n_interleaved"])
def test_full_size_72kx18k_repack_sampled_blocks(src):
    # the 18432 x 73728 weight with zero points: 64 sampled 1 KiB output blocks and their
    # parameters against the documented layout of the decoded codes
    sh = LARGE.shapes[0]
    K, N = sh.K, sh.N
    _, q, s = draw(K, N, 1, seed=0)
    z = draw_zeros(K, N, seed=0)
    packed, params, codes, zeros = run_repack(q, s, z, src, 128)
    del q
    gc.collect()
    pk = packed.cpu().numpy().view(np.uint32)
    pr = params.cpu().numpy().view(np.uint16)
    del packed, params
    torch.cuda.empty_cache()
    G, Q = K // 128, 4
    rng = np.random.default_rng(5)
    blocks = [(0, 0), (N // 16 - 1, G - 1)] + [tuple(x) for x in zip(rng.integers(0, N // 16, 62),
                                                                    rng.integers(0, G, 62))]
    for j, g in blocks:
        sub = codes[128 * g:128 * g + 128, 16 * j:16 * j + 16]
        ref_p, _ = layout_reference(sub, np.zeros((1, 16), np.uint16))
        got = pk[(j * G + g) * 256:(j * G + g + 1) * 256]
        assert np.array_equal(got, ref_p), (j, g)
        for c in range(16):
            i = (((j // Q) * G + g) * 16 + c) * 2 * Q + j % Q
            assert pr[i] == s[g, 16 * j + c].view(np.uint16), (j, g, c)
            assert pr[i + Q] == 0x6400 | int(zeros[g, 16 * j + c]), (j, g, c)

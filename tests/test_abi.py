"""Host-side tests of the C ABI: exported symbols, the offline pack, argument checking.

No GPU needed: w4a16_pack / w4a16_unpack are host code, and w4a16_gemm rejects bad
arguments before touching the HIP runtime.
"""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import mixed_precision_w4a16_amd as w4
from layouts import NIBBLE, layout_reference, params_layout_reference
from workloads import ALL, draw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "paper_constants.json")


def _header_code():
    return re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)


def header_inline_functions():
    """Functions the header defines itself (static inline): evaluated by the caller, not
    exported by the library."""
    return sorted(set(re.findall(r"static\s+inline\s+[a-z_0-9 ]+?\b(w4a16_[a-z0-9_]+)\s*\(",
                                 _header_code())))


def declared_functions():
    names = set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", _header_code()))
    return sorted(names - set(header_inline_functions()))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(w4.EXPORTED)
    lib = ctypes.CDLL(w4.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_header_inline_workspace_bound_matches_the_binding(tmp_path):
    # the header's w4a16_workspace_bound, compiled as C, against the binding's statement of
    # the same formula, over shapes on both sides of every branch
    assert header_inline_functions() == ["w4a16_workspace_bound"]
    shapes = [(M, K, N) for M in (0, 1, 16, 17, 32, 33, 64, 65, 128, 129, 1024, -1)
              for K, N in ((128, 64), (1024, 1024), (18432, 73728), (8192, 28672), (4096, 192),
                           (100, 256), (0, 256))]
    src = tmp_path / "bound.c"
    src.write_text('#include <stdio.h>\n#include "w4a16.h"\nint main(void){\n' + "".join(
        f'printf("%zu\\n", w4a16_workspace_bound({M}, {K}, {N}));\n' for M, K, N in shapes)
        + "return 0;}\n")
    exe = tmp_path / "bound"
    import subprocess
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                    str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got == [w4.workspace_bound(M, K, N) for M, K, N in shapes]
    # values written out by hand: M = 1 on 1024 x 1024 is bounded by its 64 tiles of 16 x 256;
    # M = 128 on the 72k x 18k weight by 1024 stripes of two 128 x 256 tiles
    assert w4.workspace_bound(1, 1024, 1024) == 4096 + max(8 * 1024 * 8 * 16, (64 + 9) * 65536)
    assert w4.workspace_bound(128, 18432, 73728) == 4096 + 2 * 1024 * 128 * 256 * 4
    assert w4.workspace_bound(5, 1000, 256) == 0


def test_noalloc_gemm_rejects_bad_arguments_before_any_device_call():
    lib = w4.library()
    d = ctypes.c_void_p(16)
    assert lib.w4a16_gemm_noalloc(None, d, d, d, 16, 1024, 1024, 128, 0, None) == w4.EINVAL
    assert lib.w4a16_gemm_noalloc(d, None, d, d, 16, 1024, 1024, 128, 0, None) == w4.EINVAL
    assert lib.w4a16_gemm_noalloc(d, d, d, d, -1, 1024, 1024, 128, 0, None) == w4.EINVAL
    assert lib.w4a16_gemm_noalloc(d, d, d, d, 16, 1024, 1024, 128, 3, None) == w4.EINVAL
    assert lib.w4a16_gemm_noalloc(d, d, d, d, 16, 1000, 1024, 128, 0, None) == w4.ESHAPE
    assert lib.w4a16_gemm_noalloc(d, d, d, d, 16, 1024, 1000, 128, 0, None) == w4.ESHAPE
    assert lib.w4a16_gemm_noalloc(d, d, d, d, 16, 1024, 1024, 256, 0, None) == w4.ESHAPE
    assert w4.NOALLOC_SCRATCH_BYTES == (128 << 20) + 4096


def test_mfma_probe_rejects_bad_arguments_before_any_device_call():
    lib = w4.library()
    d = ctypes.c_void_p(256)
    assert lib.w4a16_mfma_probe(None, 4096, 0, 1, 1, d, None) == w4.EINVAL
    assert lib.w4a16_mfma_probe(d, 4096, 0, 1, 1, None, None) == w4.EINVAL
    assert lib.w4a16_mfma_probe(d, 0, 0, 1, 1, d, None) == w4.EINVAL
    assert lib.w4a16_mfma_probe(d, 4100, 0, 1, 1, d, None) == w4.EINVAL
    assert lib.w4a16_mfma_probe(ctypes.c_void_p(264), 4096, 0, 1, 1, d, None) == w4.EINVAL
    assert lib.w4a16_mfma_probe(d, 4096, 2, 1, 1, d, None) == w4.EINVAL
    assert lib.w4a16_mfma_probe(d, 4096, 0, 0, 1, d, None) == w4.EINVAL
    assert lib.w4a16_mfma_probe(d, 4096, 1, 1, 0, d, None) == w4.EINVAL


def test_status_strings():
    for st in (w4.OK, w4.EINVAL, w4.ESHAPE, w4.EUNSUPPORTED, w4.EHIP, 12345):
        assert w4.library().w4a16_status_string(st)


@pytest.mark.parametrize("K,N", [(128, 16), (256, 64), (384, 48), (1024, 1024), (256, 384),
                                 (128, 128), (256, 320)])
def test_pack_matches_documented_layout(K, N):
    _, q, s = draw(K, N, 1, seed=K + N)
    packed, sp = w4.pack(q, s)
    ref_p, ref_s = layout_reference(q, s)
    assert np.array_equal(packed, ref_p)
    assert np.array_equal(sp.view(np.uint16), ref_s.view(np.uint16))


def _patterns(K, N, rng):
    yield rng.integers(0, 16, (K, N), dtype=np.uint8)
    yield np.zeros((K, N), dtype=np.uint8)
    yield np.full((K, N), 15, dtype=np.uint8)
    yield ((np.arange(K)[:, None] + np.arange(N)[None, :]) % 2 * 15).astype(np.uint8)
    yield ((np.arange(K)[:, None] * 7 + np.arange(N)[None, :] * 3) % 16).astype(np.uint8)


@pytest.mark.parametrize("K,N", [(128, 16), (256, 64), (640, 208), (4096, 512)])
def test_pack_unpack_round_trip_is_bit_exact(K, N):
    rng = np.random.default_rng(K * N)
    s = rng.uniform(0.005, 0.02, (K // 128, N)).astype(np.float16)
    s[0, 0] = np.float16(-0.0)
    s[-1, -1] = np.float16(65504.0)
    for q in _patterns(K, N, rng):
        packed, sp = w4.pack(q, s)
        q2, s2 = w4.unpack(packed, sp, K, N)
        assert np.array_equal(q2, q)
        assert np.array_equal(s2.view(np.uint16), s.view(np.uint16))


def test_round_trip_at_every_workload_shape_sampled():
    # Full-size shapes, pack/unpack on a 1024-row band (the layout is per 128-row group, so
    # any multiple of 128 exercises the same code for every column slab of the real N).
    for wl in ALL:
        for sh in wl.shapes:
            K = min(sh.K, 1024)
            _, q, s = draw(K, sh.N, 1, seed=1)
            packed, sp = w4.pack(q, s)
            q2, s2 = w4.unpack(packed, sp, K, sh.N)
            assert np.array_equal(q2, q), sh.name
            assert np.array_equal(s2.view(np.uint16), s.view(np.uint16)), sh.name


def test_footprint_is_4_125_bits_per_weight():
    g = json.load(open(GOLDEN))
    K, N = 18432, 256
    _, q, s = draw(K, N, 1, seed=2)
    packed, sp = w4.pack(q, s)
    bits = (packed.nbytes + sp.nbytes) * 8 / (K * N)
    assert bits == g["bits_per_weight_group128"]["value"]
    # large-shape byte count at the 72k x 18k workload (codes + scales)
    Kl, Nl = 18432, 73728
    assert Kl * Nl // 2 + Kl // 128 * Nl * 2 == 700_710_912


def test_pack_rejects_bad_arguments():
    lib = w4.library()
    q = np.zeros((256, 32), dtype=np.uint8)
    s = np.ones((2, 32), dtype=np.float16)
    out = np.zeros(256 * 32 // 8, dtype=np.uint32)
    so = np.zeros(64, dtype=np.float16)
    P = lambda a: a.ctypes.data
    assert lib.w4a16_pack(None, P(s), 256, 32, 128, P(out), P(so)) == w4.EINVAL
    assert lib.w4a16_pack(P(q), P(s), -1, 32, 128, P(out), P(so)) == w4.EINVAL
    assert lib.w4a16_pack(P(q), P(s), 256, 32, 64, P(out), P(so)) == w4.ESHAPE
    assert lib.w4a16_pack(P(q), P(s), 200, 32, 128, P(out), P(so)) == w4.ESHAPE
    assert lib.w4a16_pack(P(q), P(s), 256, 24, 128, P(out), P(so)) == w4.ESHAPE
    assert lib.w4a16_pack(P(q), P(s), 0, 32, 128, P(out), P(so)) == w4.ESHAPE
    q[5, 7] = 16
    assert lib.w4a16_pack(P(q), P(s), 256, 32, 128, P(out), P(so)) == w4.EINVAL
    with pytest.raises(w4.W4A16Error):
        w4.pack(q, s)


def test_gemm_rejects_bad_arguments_before_any_device_call():
    lib = w4.library()
    d = ctypes.c_void_p(16)   # never dereferenced: every case fails validation first
    assert lib.w4a16_gemm(None, d, d, d, 16, 1024, 1024, d, None) == w4.EINVAL
    assert lib.w4a16_gemm(d, d, d, d, 16, 1024, 1024, None, None) == w4.EINVAL
    assert lib.w4a16_gemm(d, d, d, d, -1, 1024, 1024, d, None) == w4.EINVAL
    assert lib.w4a16_gemm(d, d, d, d, 16, 1000, 1024, d, None) == w4.ESHAPE
    assert lib.w4a16_gemm(d, d, d, d, 16, 0, 1024, d, None) == w4.ESHAPE
    assert lib.w4a16_gemm(d, d, d, d, 16, 1024, 1000, d, None) == w4.ESHAPE
    assert lib.w4a16_gemm(d, d, d, d, 16, 1024, 32, d, None) == w4.ESHAPE
    # size limits of the 32-bit buffer ranges
    assert lib.w4a16_gemm(d, d, d, d, 2 ** 20, 4096, 1024, d, None) == w4.ESHAPE
    assert lib.w4a16_gemm(d, d, d, d, 16, 2 ** 20, 2 ** 14, d, None) == w4.ESHAPE
    assert lib.w4a16_gemm(d, d, d, d, 2 ** 15, 128, 2 ** 16, d, None) == w4.ESHAPE   # C >= 4 GiB
    n = ctypes.c_size_t(7)
    assert lib.w4a16_workspace_size(16, 1000, 1024, ctypes.byref(n)) == w4.ESHAPE
    assert lib.w4a16_workspace_size(16, 1024, 1024, None) == w4.EINVAL
    assert n.value == 7


# ------------------------------------------------------------------ one scale per column, zero points

@pytest.mark.parametrize("K,N,col", [(256, 64, False), (384, 256, False), (256, 128, True),
                                     (512, 48, True), (128, 16, False)])
def test_pack_zp_matches_documented_layout(K, N, col):
    from workloads import draw_zeros
    g = K if col else 128
    _, q, s = draw(K, N, 1, seed=K + N, group=g)
    z = draw_zeros(K, N, seed=K, group=g)
    packed, params = w4.pack(q, s, group=g, zeros=z)
    ref_p, _ = layout_reference(q, np.zeros((K // 128, N), np.float16))
    assert np.array_equal(packed, ref_p)
    assert np.array_equal(params.view(np.uint16), params_layout_reference(s, z))


@pytest.mark.parametrize("K,N", [(256, 64), (640, 208), (1024, 512)])
def test_column_scale_pack_round_trip_and_layout(K, N):
    _, q, s = draw(K, N, 1, seed=K * 3 + N, group=K)
    packed, sp = w4.pack(q, s, group=K)
    Q = 4 if N % 256 == 0 else (2 if N % 128 == 0 else 1)
    ref = s.view(np.uint16).reshape(1, N // (16 * Q), Q, 16).transpose(1, 0, 3, 2).reshape(-1)
    assert np.array_equal(sp.view(np.uint16), ref)
    q2, s2 = w4.unpack(packed, sp, K, N, group=K)
    assert np.array_equal(q2, q) and np.array_equal(s2.view(np.uint16), s.view(np.uint16))


@pytest.mark.parametrize("K,N,col", [(256, 64, False), (640, 208, True), (1024, 512, False)])
def test_zero_point_pack_round_trip_is_bit_exact(K, N, col):
    rng = np.random.default_rng(K + N)
    g = K if col else 128
    s = rng.uniform(0.005, 0.02, (K // g, N)).astype(np.float16)
    for q in _patterns(K, N, rng):
        for z in (rng.integers(0, 16, (K // g, N), dtype=np.uint8),
                  np.zeros((K // g, N), np.uint8), np.full((K // g, N), 15, np.uint8)):
            packed, params = w4.pack(q, s, group=g, zeros=z)
            q2, s2, z2 = w4.unpack(packed, params, K, N, group=g, zero_points=True)
            assert np.array_equal(q2, q) and np.array_equal(z2, z)
            assert np.array_equal(s2.view(np.uint16), s.view(np.uint16))


def test_new_pack_calls_reject_bad_arguments():
    lib = w4.library()
    K, N = 256, 32
    q = np.zeros((K, N), dtype=np.uint8)
    s = np.ones((2, N), dtype=np.float16)
    z = np.full((2, N), 8, dtype=np.uint8)
    out = np.zeros(K * N // 8, dtype=np.uint32)
    po = np.zeros(4 * N, dtype=np.float16)
    P = lambda a: a.ctypes.data
    assert lib.w4a16_pack_zp(P(q), P(s), None, K, N, 128, P(out), P(po)) == w4.EINVAL
    assert lib.w4a16_pack_zp(P(q), P(s), P(z), K, N, 64, P(out), P(po)) == w4.ESHAPE
    assert lib.w4a16_pack(P(q), P(s), K, N, 512, P(out), P(po)) == w4.ESHAPE      # not 128 or K
    assert lib.w4a16_pack(P(q), P(s), K, N, K, P(out), P(po)) == w4.OK            # group = K
    z[1, 3] = 16
    assert lib.w4a16_pack_zp(P(q), P(s), P(z), K, N, 128, P(out), P(po)) == w4.EINVAL
    # unpack_zp refuses parameters that were not written as zero terms
    z[1, 3] = 2
    assert lib.w4a16_pack_zp(P(q), P(s), P(z), K, N, 128, P(out), P(po)) == w4.OK
    bad = po.copy()
    bad.view(np.uint16)[1] = 0x3C00
    qo = np.zeros((K, N), np.uint8)
    so = np.zeros((2, N), np.float16)
    zo = np.zeros((2, N), np.uint8)
    assert lib.w4a16_unpack_zp(P(out), P(bad), K, N, 128, P(qo), P(so), P(zo)) == w4.EINVAL
    assert lib.w4a16_unpack_zp(P(out), P(po), K, N, 128, P(qo), P(so), None) == w4.EINVAL


def test_gemm_ex_rejects_bad_arguments_before_any_device_call():
    lib = w4.library()
    d = ctypes.c_void_p(16)
    assert lib.w4a16_gemm_ex(d, d, d, d, 16, 1024, 1024, 128, 2, d, None) == w4.EINVAL
    assert lib.w4a16_gemm_ex(d, d, d, d, 16, 1024, 1024, 128, -1, d, None) == w4.EINVAL
    assert lib.w4a16_gemm_ex(None, d, d, d, 16, 1024, 1024, 128, 0, d, None) == w4.EINVAL
    assert lib.w4a16_gemm_ex(d, d, d, d, 16, 1024, 1024, 256, 0, d, None) == w4.ESHAPE
    assert lib.w4a16_gemm_ex(d, d, d, d, 16, 1024, 1024, 0, 1, d, None) == w4.ESHAPE
    assert lib.w4a16_gemm_ex(d, d, d, d, 16, 1000, 1024, 1000, 0, d, None) == w4.ESHAPE


def test_repack_rejects_bad_arguments_before_any_device_call():
    lib = w4.library()
    d = ctypes.c_void_p(256)
    K, N = 1024, 512
    ok_order = (ctypes.c_uint8 * 8)(0, 2, 4, 6, 1, 3, 5, 7)
    dup = (ctypes.c_uint8 * 8)(0, 1, 2, 3, 4, 5, 6, 6)
    big = (ctypes.c_uint8 * 8)(0, 1, 2, 3, 4, 5, 6, 8)
    R = lib.w4a16_repack
    assert R(None, 0, None, d, None, K, N, 128, d, d, None) == w4.EINVAL
    assert R(d, 0, None, None, None, K, N, 128, d, d, None) == w4.EINVAL
    assert R(d, 0, None, d, None, K, N, 128, None, d, None) == w4.EINVAL
    assert R(d, 0, None, d, None, K, N, 128, d, None, None) == w4.EINVAL
    assert R(d, 2, None, d, None, K, N, 128, d, d, None) == w4.EINVAL
    assert R(d, -1, None, d, None, K, N, 128, d, d, None) == w4.EINVAL
    assert R(d, 1, dup, d, None, K, N, 128, d, d, None) == w4.EINVAL
    assert R(d, 1, big, d, None, K, N, 128, d, d, None) == w4.EINVAL
    assert R(d, 0, None, d, None, -128, N, 128, d, d, None) == w4.EINVAL
    assert R(d, 0, None, d, None, K, N, 128, ctypes.c_void_p(264), d, None) == w4.EINVAL  # 8-aligned out
    assert R(d, 0, None, d, ctypes.c_void_p(258), K, N, 128, d, d, None) == w4.EINVAL      # 2-aligned zeros
    assert R(d, 1, ok_order, d, None, 1000, N, 128, d, d, None) == w4.ESHAPE
    assert R(d, 1, ok_order, d, None, K, 520, 128, d, d, None) == w4.ESHAPE
    assert R(d, 0, None, d, None, K, N, 256, d, d, None) == w4.ESHAPE
    assert R(d, 0, None, d, None, 0, N, 128, d, d, None) == w4.ESHAPE


# ------------------------------------------------------------------ 2:4-sparse weights

def _sparse_cases(K, N, seed):
    from workloads import sparsify_24
    _, q, s = draw(K, N, 1, seed=seed)
    q = sparsify_24(q, seed)
    # some groups with fewer non-zeros: one, and none at all
    q[0:4, 0] = [8, 8, 3, 8]
    q[4:8, 1] = [8, 8, 8, 8]
    q[8:12, 2] = [15, 8, 8, 0]
    return q, s


@pytest.mark.parametrize("K,N", [(128, 16), (256, 64), (384, 48), (1024, 256)])
def test_pack_24_matches_documented_layout(K, N):
    q, s = _sparse_cases(K, N, K + N)
    packed, sp = w4.pack_24(q, s)
    from layouts import layout_reference_24
    assert np.array_equal(packed, layout_reference_24(q))
    assert np.array_equal(sp.view(np.uint16), layout_reference(q, s)[1].view(np.uint16))


@pytest.mark.parametrize("K,N", [(128, 16), (512, 272), (2048, 1024)])
def test_pack_24_round_trip_is_bit_exact(K, N):
    q, s = _sparse_cases(K, N, 7 * K + N)
    q2, s2 = w4.unpack_24(*w4.pack_24(q, s), K, N)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2.view(np.uint16), s.view(np.uint16))


def test_pack_24_rejects_groups_with_three_nonzero_weights_and_bad_shapes():
    q, s = _sparse_cases(256, 64, 3)
    bad = q.copy()
    bad[4:8, 5] = [1, 8, 2, 3]
    with pytest.raises(w4.W4A16Error) as e:
        w4.pack_24(bad, s)
    assert e.value.status == w4.EINVAL
    bad = q.copy()
    bad[9, 9] = 16
    with pytest.raises(w4.W4A16Error) as e:
        w4.pack_24(bad, s)
    assert e.value.status == w4.EINVAL
    lib = w4.library()
    d = ctypes.c_void_p(64)
    assert lib.w4a16_pack_24(d, d, 200, 64, d, d) == w4.ESHAPE
    assert lib.w4a16_pack_24(d, d, 256, 40, d, d) == w4.ESHAPE
    assert lib.w4a16_pack_24(None, d, 256, 64, d, d) == w4.EINVAL
    # unpack refuses positions that pack never writes (two equal positions in a group)
    packed, sp = w4.pack_24(q, s)
    packed[2] = 0
    with pytest.raises(w4.W4A16Error):
        w4.unpack_24(packed, sp, 256, 64)


def test_gemm_24_rejects_bad_arguments_before_any_device_call():
    lib = w4.library()
    d = ctypes.c_void_p(256)
    assert lib.w4a16_gemm_24(None, d, d, d, 16, 1024, 1024, d, None) == w4.EINVAL
    assert lib.w4a16_gemm_24(d, d, d, d, 16, 1024, 1024, None, None) == w4.EINVAL  # workspace
    assert lib.w4a16_gemm_24(d, d, d, d, -1, 1024, 1024, d, None) == w4.EINVAL
    assert lib.w4a16_gemm_24(d, d, d, d, 16, 1024, 320, d, None) == w4.ESHAPE     # N % 256
    assert lib.w4a16_gemm_24(d, d, d, d, 16, 1000, 1024, d, None) == w4.ESHAPE
    assert lib.w4a16_gemm_24(d, d, d, d, 16, 98304, 65536, d, None) == w4.ESHAPE  # 2.4 GB


def test_sparsify_24_keeps_two_of_every_four():
    from workloads import sparsify_24
    _, q, _ = draw(512, 96, 1, seed=5)
    z = sparsify_24(q, 5)
    g = z.reshape(128, 4, 96)
    assert ((g == 8).sum(axis=1) >= 2).all()
    assert np.array_equal(z[z != 8], q[z != 8])
    # every one of the six pairs occurs
    kept = (np.arange(512) % 4)[:, None] * np.ones((1, 96), int)
    pairs = set()
    for a in range(0, 512, 4):
        for n in range(96):
            pairs.add(tuple(np.flatnonzero(z[a:a + 4, n] != 8)))
    assert {(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)} <= pairs


def test_moe_entry_points_reject_bad_arguments_before_any_device_call():
    lib = w4.library()
    d = ctypes.c_void_p(256)
    # w4a16_moe_align(topk_ids, T, topk, E, sorted_ids, expert_offsets, stream)
    assert lib.w4a16_moe_align(None, 4, 2, 8, d, d, None) == w4.EINVAL
    assert lib.w4a16_moe_align(d, -1, 2, 8, d, d, None) == w4.EINVAL
    assert lib.w4a16_moe_align(d, 4, 0, 8, d, d, None) == w4.EINVAL
    assert lib.w4a16_moe_align(d, 4, 2, 0, d, d, None) == w4.EINVAL
    assert lib.w4a16_moe_align(d, 4, 2, 1025, d, d, None) == w4.ESHAPE
    assert lib.w4a16_moe_align(d, 1 << 30, 4, 8, d, d, None) == w4.ESHAPE
    # w4a16_moe_gemm(A, packed, params, sorted, offsets, row_scale, C, T, topk, E, K, N,
    #                zero_points, act_dtype, stream)
    ok = [d, d, d, d, d, None, d, 4, 2, 8, 1024, 1024, 0, w4.ACT_F16, None]

    def call(**kw):
        a = list(ok)
        names = ["A", "packed", "params", "sorted", "offsets", "row_scale", "C", "T", "topk",
                 "E", "K", "N", "zp", "act", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return lib.w4a16_moe_gemm(*a)
    assert call(A=None) == w4.EINVAL
    assert call(sorted=None) == w4.EINVAL
    assert call(C=None) == w4.EINVAL
    assert call(T=-1) == w4.EINVAL
    assert call(topk=0) == w4.EINVAL
    assert call(E=0) == w4.EINVAL
    assert call(zp=2) == w4.EINVAL
    assert call(act=2) == w4.EINVAL
    assert call(K=1000) == w4.ESHAPE
    assert call(N=320) == w4.ESHAPE                    # N a multiple of 256
    assert call(K=65536, N=65536) == w4.ESHAPE         # 2 GiB of codes per expert
    assert call(T=600000, K=4096) == w4.ESHAPE         # A past 2^31 bytes


def test_moe_routing_entry_rejects_bad_arguments_before_any_device_call():
    lib = w4.library()
    d = ctypes.c_void_p(256)
    # w4a16_moe_gemm_topk(A, packed, params, topk_ids, row_scale, C, T, topk, E, K, N,
    #                     zero_points, act_dtype, stream)
    assert lib.w4a16_moe_gemm_topk(d, d, d, None, None, d, 4, 2, 8, 1024, 1024, 0, 0,
                                   None) == w4.EINVAL
    assert lib.w4a16_moe_gemm_topk(None, d, d, d, None, d, 4, 2, 8, 1024, 1024, 0, 0,
                                   None) == w4.EINVAL
    assert lib.w4a16_moe_gemm_topk(d, d, d, d, None, d, 1025, 2, 8, 1024, 1024, 0, 0,
                                   None) == w4.ESHAPE        # more than 2048 assignments
    assert lib.w4a16_moe_gemm_topk(d, d, d, d, None, d, 4, 2, 8, 1024, 1000, 0, 0,
                                   None) == w4.ESHAPE
    assert lib.w4a16_moe_gemm_topk(d, d, d, d, None, d, 4, 2, 1025, 1024, 1024, 0, 0,
                                   None) == w4.ESHAPE        # more than 1024 experts
    # w4a16_moe_gemm(A, packed, params, sorted_ids, offsets, row_scale, C, T, topk, E, K, N,
    #                zero_points, act_dtype, stream)
    assert lib.w4a16_moe_gemm(d, d, d, d, d, None, d, 4, 2, 1025, 1024, 1024, 0, 0,
                              None) == w4.ESHAPE
    assert w4.MOE_ROUTE_MAX == 2048


def test_read_probe_rejects_bad_arguments_before_any_device_call():
    lib = w4.library()
    d = ctypes.c_void_p(256)
    assert lib.w4a16_read_probe(None, 4096, d, None) == w4.EINVAL
    assert lib.w4a16_read_probe(d, 0, d, None) == w4.EINVAL
    assert lib.w4a16_read_probe(d, 4100, d, None) == w4.EINVAL
    assert lib.w4a16_read_probe(ctypes.c_void_p(264), 4096, d, None) == w4.EINVAL
    assert lib.w4a16_read_probe(d, 4096, None, None) == w4.EINVAL

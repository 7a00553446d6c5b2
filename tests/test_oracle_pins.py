"""Pins for the CPU oracle: each test ties it to something other than itself.

The oracle computes C = A * Bhat, Bhat[k, n] = s[k // 128, n] * (q[k, n] - 8), fp32 accumulation
and one fp16 rounding (MARLIN paper sec. 3.4 "Kernel Design"; Marlin deep-dive page
"Marlin 完全拆解", sections "Marlin 要解决的精确问题" and on warp partial sums).  The pins:

* the fp16 conversions against numpy's IEEE binary16 conversions (a library routine), and
  against this package's exact integer rounder;
* tiny shapes against exact integer arithmetic (``oracle.exact_gemm``), bitwise for the fp64
  variant and within the textbook inner-product error bound for the fp32 one;
* special cases with a closed form (zero point, one-hot activations, integer-exact sums);
* invariants (power-of-two scaling, nested M, the M = 1 product, thread count, per-group
  locality of the scales) and the output's second moment.

A plausible slip anywhere in the oracle -- a dropped "- 8", a wrong group index, a transposed
operand, a wrong rounding -- fails at least one of these.
"""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import draw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paper_constants.json")


def bits(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def same(a, b):
    """Bitwise equality of fp16 arrays with -0 and +0 identified (a sum that starts at +0
    returns +0 for an all-zero input, where the closed form may give -0)."""
    x, y = bits(a).copy(), bits(b).copy()
    x[x == 0x8000] = 0
    y[y == 0x8000] = 0
    return np.array_equal(x, y)


# ------------------------------------------------------------------ fp16 conversions

def test_half_to_double_every_bit_pattern():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = allbits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(b) for b in allbits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    assert np.isnan(got[np.isnan(ref)]).all()
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def _rounding_probe_values():
    vals = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    nxt = np.append(vals[1:], 65536.0)
    mids = (vals + nxt) / 2.0                     # exact ties between neighbours
    probe = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                            [65504.0, 65519.999, 65520.0, 65536.0, 1e9, 2.0 ** -25,
                             np.nextafter(2.0 ** -25, 1.0), 2.0 ** -26, 1e-30]])
    return np.concatenate([probe, -probe])


def test_double_to_half_against_numpy_and_exact_rounder():
    x = _rounding_probe_values()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.double_to_half(v) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)
    # the exact integer rounder used by the brute force agrees on the same values
    for v, r in zip(x[:: 97], ref[:: 97]):
        if v == 0:
            continue
        num, den = float(v).as_integer_ratio()
        shift = den.bit_length() - 1              # den is a power of two
        assert oracle.round_scaled_to_half(num, shift) == r, v


def test_float_to_half_against_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(100),
        (rng.standard_normal(20000) * 1e-6).astype(np.float32),
        np.array([65519.996, 65520.0, 6.0e-8, 3.0e-8, 2.9802322e-08], dtype=np.float32)])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half(v) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ dequantisation

def test_dequant_is_affine_in_code_with_slope_scale_and_zero_at_8():
    # every positive finite fp16 scale (normal and subnormal), all 16 codes
    for sb in list(range(1, 0x7C00, 7)) + [1, 0x3C00, 0x7BFF]:
        s = oracle.half_to_double(sb)
        w = [oracle.dequant(q, sb) for q in range(16)]
        assert w[8] == 0.0
        assert all(w[q + 1] - w[q] == s for q in range(15))   # uniform grid, step s
        assert w[0] == -8 * s and w[15] == 7 * s


# ------------------------------------------------------------------ brute force, tiny shapes

TINY = [(1, 128, 16), (2, 256, 16), (3, 384, 8), (5, 128, 48), (16, 256, 4), (17, 128, 3)]


@pytest.mark.parametrize("M,K,N", TINY)
def test_tiny_shapes_against_exact_integer_sum(M, K, N):
    A, q, s = draw(K, N, M, seed=100 + M * K + N)
    C64 = oracle.gemm(A, q, s, mode="f64")
    C32 = oracle.gemm(A, q, s, mode="f32")
    E, exact, absum = oracle.exact_gemm(A, q, s)
    # fp64 accumulation is far more accurate than fp16 spacing: same correctly rounded result
    assert np.array_equal(bits(C64), bits(E))
    # fp32 accumulation: |acc - exact| <= gamma_K * sum|a_k w_k| (Higham, Accuracy and
    # Stability of Numerical Algorithms, 2nd ed., eq. (3.5)), then one fp16 rounding.
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    c = C32.astype(np.float64)
    x = np.abs(exact) + gamma * absum
    ulp16 = 2.0 ** (np.maximum(np.floor(np.log2(np.maximum(x, 2.0 ** -30))), -14) - 10)
    # half an fp16 ulp at the larger of the two binades the rounded value can fall in
    assert (np.abs(c - exact) <= gamma * absum + ulp16).all()


def test_tiny_shapes_extreme_values():
    rng = np.random.default_rng(7)
    M, K, N = 3, 256, 8
    A = np.zeros((M, K), dtype=np.float16)
    A[0] = rng.choice(np.array([6.0e-8, -6.0e-8, 1.0e-5, 2048.0, -1024.0], dtype=np.float16), K)
    A[1] = np.float16(65504.0) * rng.choice(np.array([1, -1], dtype=np.float16), K) / np.float16(64)
    A[2, ::3] = np.float16(1.0)
    q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    s = rng.choice(np.array([6.0e-8, 0.5, 0.019989, 2.0], dtype=np.float16), (K // 128, N))
    E, _, _ = oracle.exact_gemm(A, q, s)
    assert np.array_equal(bits(oracle.gemm(A, q, s, mode="f64")), bits(E))


# ------------------------------------------------------------------ closed forms

def test_zero_point_code_8_gives_positive_zero():
    A, q, s = draw(256, 64, 4, seed=3)
    q[:] = 8
    assert (bits(oracle.gemm(A, q, s)) == 0).all()


def test_code_9_unit_scale_gives_row_sums():
    rng = np.random.default_rng(4)
    M, K, N = 5, 384, 32
    A = rng.integers(-4, 5, (M, K)).astype(np.float16)
    q = np.full((K, N), 9, dtype=np.uint8)
    s = np.ones((K // 128, N), dtype=np.float16)
    rows = A.astype(np.int64).sum(axis=1)
    assert np.array_equal(oracle.gemm(A, q, s).astype(np.int64), np.repeat(rows[:, None], N, 1))


@pytest.mark.parametrize("k_hot", [0, 1, 7, 8, 31, 32, 33, 127, 128, 200, 255, 256, 383])
def test_one_hot_activation_selects_one_dequantised_row(k_hot):
    K, N = 384, 40
    A, q, s = draw(K, N, 2, seed=5)
    A[:] = 0
    A[0, k_hot] = 1.0
    A[1, k_hot] = -2.0
    C = oracle.gemm(A, q, s)
    w = s[k_hot // 128].astype(np.float64) * (q[k_hot].astype(np.float64) - 8.0)   # exact
    assert same(C[0], w.astype(np.float16))
    assert same(C[1], (-2.0 * w).astype(np.float16))


def test_scales_act_only_inside_their_group():
    K, N = 512, 24
    A, q, s = draw(K, N, 3, seed=6)
    for g in range(K // 128):
        s2 = s.copy()
        s2[g] = (s2[g].astype(np.float32) * 2).astype(np.float16)    # exact doubling
        inside = np.zeros_like(A)
        inside[:, g * 128:(g + 1) * 128] = A[:, g * 128:(g + 1) * 128]
        outside = A - inside
        assert np.array_equal(bits(oracle.gemm(outside, q, s2)), bits(oracle.gemm(outside, q, s)))
        c1 = oracle.gemm(inside, q, s).astype(np.float32)
        c2 = oracle.gemm(inside, q, s2).astype(np.float32)
        big = np.abs(c1) >= 2.0 ** -13
        assert np.array_equal(c2[big], 2 * c1[big])


# ------------------------------------------------------------------ invariants

def test_power_of_two_scaling_of_activations_and_scales():
    A, q, s = draw(1024, 256, 8, seed=8)
    C = oracle.gemm(A, q, s).astype(np.float32)
    big = np.abs(C) >= 2.0 ** -13
    C2a = oracle.gemm((A.astype(np.float32) * 2).astype(np.float16), q, s).astype(np.float32)
    C2s = oracle.gemm(A, q, (s.astype(np.float32) * 2).astype(np.float16)).astype(np.float32)
    assert np.array_equal(C2a[big], 2 * C[big])
    assert np.array_equal(C2s[big], 2 * C[big])


def test_gemv_equals_gemm_row_and_nested_m():
    A, q, s = draw(1024, 512, 32, seed=9)
    C32 = oracle.gemm(A, q, s)
    C16 = oracle.gemm(A[:16], q, s)
    assert np.array_equal(bits(C16), bits(C32[:16]))
    assert np.array_equal(bits(oracle.gemv(A[0], q, s)), bits(C32[0]))
    assert np.array_equal(bits(oracle.gemm(A[:1], q, s)), bits(C32[:1]))


def test_thread_count_does_not_change_result():
    A, q, s = draw(512, 300, 6, seed=10)
    ref = bits(oracle.gemm(A, q, s, nthreads=1))
    for t in (2, 3, 8, 300):
        assert np.array_equal(bits(oracle.gemm(A, q, s, nthreads=t)), ref)


def test_fp64_library_matmul_agrees():
    # numpy's fp64 matmul (a library routine) on the exactly dequantised matrix
    A, q, s = draw(1024, 512, 16, seed=11)
    Bhat = np.repeat(s.astype(np.float64), 128, axis=0) * (q.astype(np.float64) - 8.0)
    ref = (A.astype(np.float64) @ Bhat).astype(np.float16)
    C64 = oracle.gemm(A, q, s, mode="f64")
    assert (bits(C64) != bits(ref)).sum() <= 2     # only where fp64 rounding straddles a tie
    C32 = oracle.gemm(A, q, s).astype(np.float64)
    rel = np.linalg.norm(C32 - ref.astype(np.float64)) / np.linalg.norm(ref.astype(np.float64))
    assert rel < 1e-4


def test_output_second_moment_matches_closed_form():
    # std(C) = sqrt(K * sigma^2 * E[s^2] * E[(q-8)^2]), E[s^2] = (b^3-a^3)/(3(b-a)) for
    # s ~ U[a, b], E[(q-8)^2] = 344/16 for q uniform on 0..15.
    K, N, M = 1024, 1024, 16
    A, q, s = draw(K, N, M, seed=0)
    a, b = 0.005, 0.02
    es2 = (b ** 3 - a ** 3) / (3 * (b - a))
    pred = np.sqrt(K * 1.0 * es2 * 344 / 16)
    C = oracle.gemm(A, q, s).astype(np.float64)
    assert abs(C.std() / pred - 1) < 0.03


def test_bad_arguments_rejected():
    A, q, s = draw(256, 16, 2, seed=12)
    q2 = q.copy()
    q2[3, 4] = 16
    with pytest.raises(ValueError):
        oracle.gemm(A, q2, s)
    with pytest.raises(ValueError):
        oracle.gemm(A[:, :200], q[:200], s[:1])


# ------------------------------------------------------------------ printed figures

def test_printed_footprint_and_bound():
    g = json.load(open(GOLDEN))
    G = g["group_size"]["value"]
    bpw = 4 + 16 / G
    assert bpw == g["bits_per_weight_group128"]["value"]
    assert abs(16 / bpw - g["ideal_speedup_vs_fp16"]["value"]) < 0.01


def test_printed_dequant_constants_reproduce_code_minus_8():
    # The page's masks and OR constant, applied to fp16 bit patterns: the low nibble of each
    # half gives 1024 + q, the next nibble 1024 + 16 q; the fix-ups recover q - 8 exactly.
    g = json.load(open(GOLDEN))["dequant_masks"]["value"]
    lo, hi, magic = (int(g[k], 16) for k in ("lo_mask", "hi_mask", "or_magic"))
    z = json.load(open(GOLDEN))["symmetric_zero_point"]["value"]
    for qa in range(16):
        for qb in range(16):
            word = np.uint32(qa | (qb << 4) | (qb << 16) | (qa << 20))
            x = np.array([(word & lo) | magic], dtype=np.uint32).view(np.float16).astype(np.float64)
            y = np.array([(word & hi) | magic], dtype=np.uint32).view(np.float16).astype(np.float64)
            assert list(x - (1024 + z)) == [qa - z, qb - z]
            assert list(y / 16 - (64 + z)) == [qb - z, qa - z]


# ------------------------------------------------------------------ zero points, one scale per column
# The general affine dequantisation s_{g,n} (q_{k,n} - z_{g,n}) of the deep-dive page (section
# "Marlin 要解决的精确问题") and one scale per column (group = K; section "scale 为什么有时在内环乘，
# 有时在末尾乘": AB = (AQ) diag(s)).

from workloads import draw_zeros  # noqa: E402


def test_dequant_with_zero_point_is_affine_and_vanishes_at_z():
    for z in range(16):
        for sb in (0x2000, 0x1E1F, 0x3C00):
            s = float(np.uint16(sb).view(np.float16))
            w = [oracle.dequant(q, sb, z) for q in range(16)]
            assert w[z] == 0.0
            assert all(w[q] == s * (q - z) for q in range(16))
    assert all(oracle.dequant(q, 0x2000, 8) == oracle.dequant(q, 0x2000) for q in range(16))


@pytest.mark.parametrize("group_is_k", [False, True])
def test_zero_point_8_equals_the_symmetric_path(group_is_k):
    K, N, M = 384, 24, 5
    g = K if group_is_k else 128
    A, q, s = draw(K, N, M, seed=41, group=g)
    z = np.full((K // g, N), 8, dtype=np.uint8)
    for mode in ("f32", "f64"):
        assert np.array_equal(bits(oracle.gemm(A, q, s, group=g, mode=mode, zeros=z)),
                              bits(oracle.gemm(A, q, s, group=g, mode=mode)))


@pytest.mark.parametrize("M,K,N,group_is_k", [(1, 128, 16, False), (3, 256, 8, False),
                                              (5, 384, 6, False), (2, 256, 8, True),
                                              (4, 384, 5, True)])
def test_zero_points_and_column_scales_against_exact_integer_sum(M, K, N, group_is_k):
    g = K if group_is_k else 128
    A, q, s = draw(K, N, M, seed=200 + M * K + N, group=g)
    z = draw_zeros(K, N, seed=200 + M, group=g)
    E, exact, absum = oracle.exact_gemm(A, q, s, group=g, zeros=z)
    assert np.array_equal(bits(oracle.gemm(A, q, s, group=g, mode="f64", zeros=z)), bits(E))
    C32 = oracle.gemm(A, q, s, group=g, zeros=z).astype(np.float64)
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    x = np.abs(exact) + gamma * absum
    ulp16 = 2.0 ** (np.maximum(np.floor(np.log2(np.maximum(x, 2.0 ** -30))), -14) - 10)
    assert (np.abs(C32 - exact) <= gamma * absum + ulp16).all()


def test_code_equal_to_zero_point_gives_zero():
    K, N, M = 256, 32, 4
    A, _, s = draw(K, N, M, seed=43)
    z = draw_zeros(K, N, seed=43)
    q = np.repeat(z, 128, axis=0)                 # q[k, n] = z[k // 128, n]
    assert (bits(oracle.gemm(A, q, s, zeros=z)) & 0x7FFF == 0).all()


@pytest.mark.parametrize("k_hot", [0, 5, 127, 128, 255])
def test_one_hot_activation_with_zero_points(k_hot):
    K, N = 256, 40
    _, q, s = draw(K, N, 1, seed=44)
    z = draw_zeros(K, N, seed=44)
    A = np.zeros((1, K), dtype=np.float16)
    A[0, k_hot] = 1.0
    g = k_hot // 128
    want = (s[g].astype(np.float64) * (q[k_hot].astype(np.float64) - z[g])).astype(np.float16)
    assert same(oracle.gemm(A, q, s, zeros=z)[0], want)


def test_shifting_codes_and_zero_points_together_changes_nothing():
    # q - z is what matters: q + d, z + d (codes still 0..15) give the same C bit for bit
    K, N, M = 256, 16, 3
    rng = np.random.default_rng(45)
    A, _, s = draw(K, N, M, seed=45)
    q = rng.integers(0, 8, (K, N), dtype=np.uint8)
    z = rng.integers(0, 8, (K // 128, N), dtype=np.uint8)
    C0 = oracle.gemm(A, q, s, zeros=z)
    for d in (1, 5, 8):
        assert np.array_equal(bits(oracle.gemm(A, q + d, s, zeros=z + d)), bits(C0))


def test_zero_points_act_only_inside_their_group():
    K, N, M = 384, 8, 2
    A, q, s = draw(K, N, M, seed=46)
    z = draw_zeros(K, N, seed=46)
    for g in range(K // 128):
        A1 = np.zeros_like(A)
        A1[:, 128 * g:128 * (g + 1)] = A[:, 128 * g:128 * (g + 1)]
        z2 = z.copy()
        z2[(g + 1) % 3] = (z2[(g + 1) % 3] + 3) % 16      # another group's zero points
        assert np.array_equal(bits(oracle.gemm(A1, q, s, zeros=z)), bits(oracle.gemm(A1, q, s, zeros=z2)))


def test_column_scale_equals_group_scales_all_equal():
    # one scale per column (group = K) is the grouped form with the same scale in every group
    K, N, M = 512, 24, 6
    A, q, s1 = draw(K, N, M, seed=47, group=K)
    z1 = draw_zeros(K, N, seed=47, group=K)
    s128 = np.repeat(s1, K // 128, axis=0)
    z128 = np.repeat(z1, K // 128, axis=0)
    for mode in ("f32", "f64"):
        assert np.array_equal(bits(oracle.gemm(A, q, s1, group=K, mode=mode)),
                              bits(oracle.gemm(A, q, s128, group=128, mode=mode)))
        assert np.array_equal(bits(oracle.gemm(A, q, s1, group=K, mode=mode, zeros=z1)),
                              bits(oracle.gemm(A, q, s128, group=128, mode=mode, zeros=z128)))


def test_column_scale_factors_out_of_the_sum():
    # AB = (AQ) diag(s): with power-of-two column scales the scaling is exact, so scaling the
    # unit-scale product by s gives the same bits
    K, N, M = 512, 16, 4
    A, q, _ = draw(K, N, M, seed=48, group=K)
    z = draw_zeros(K, N, seed=48, group=K)
    rng = np.random.default_rng(48)
    s = rng.choice(np.array([0.25, 0.5, 2.0, 0.0078125], dtype=np.float16), (1, N))
    one = np.ones((1, N), dtype=np.float16)
    C1 = oracle.gemm(A, q, one, group=K, zeros=z).astype(np.float32)
    Cs = oracle.gemm(A, q, s, group=K, zeros=z).astype(np.float32)
    big = np.abs(C1) >= 2.0 ** -6                 # away from fp16 subnormals after scaling
    assert np.array_equal((C1 * s.astype(np.float32))[big], Cs[big])


def test_bad_zero_points_rejected():
    K, N, M = 128, 16, 1
    A, q, s = draw(K, N, M, seed=49)
    z = np.full((1, N), 16, dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.gemm(A, q, s, zeros=z)


# ------------------------------------------------------------------ checkpoint-style words

def test_decode_along_k_literal_words():
    # word (0, 0) = 0x76543210: rows 0..7 of column 0 hold 0..7; word (0, 1) rows 8..15 -> 8..15
    w = np.array([[0x76543210, 0xFEDCBA98]], dtype=np.uint32)
    codes = oracle.decode_along_k(w, 8, 2)
    assert codes[:, 0].tolist() == list(range(8))
    assert codes[:, 1].tolist() == list(range(8, 16))


def test_decode_along_n_literal_words():
    w = np.array([[0x76543210], [0x01234567]], dtype=np.uint32)
    assert oracle.decode_along_n(w, 2, 8).tolist() == [list(range(8)), list(range(7, -1, -1))]
    # nibble i holds column order[i]: with (0, 2, 4, 6, 1, 3, 5, 7) the nibbles 0..7 of
    # 0x76543210 land in columns 0, 2, 4, 6, 1, 3, 5, 7
    got = oracle.decode_along_n(w[:1], 1, 8, order=(0, 2, 4, 6, 1, 3, 5, 7))
    assert got.tolist() == [[0, 4, 1, 5, 2, 6, 3, 7]]


@pytest.mark.parametrize("along", ["k", "n"])
def test_decode_single_nibble_probes(along):
    # one nibble set to 15 at a time: exactly one code is 15, at the position the definition
    # names; every other code is 0.
    K, N = 16, 16
    order = (3, 1, 7, 5, 0, 2, 6, 4)
    shape = (K // 8, N) if along == "k" else (K, N // 8)
    for a in range(shape[0]):
        for b in range(shape[1]):
            for i in range(8):
                w = np.zeros(shape, dtype=np.uint32)
                w[a, b] = np.uint32(15) << np.uint32(4 * i)
                if along == "k":
                    codes = oracle.decode_along_k(w, K, N)
                    where = (8 * a + i, b)
                else:
                    codes = oracle.decode_along_n(w, K, N, order=order)
                    where = (a, 8 * b + order[i])
                assert codes[where] == 15 and int(codes.sum()) == 15, (a, b, i)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_inverts_nibble_by_nibble_encoders(seed):
    from layouts import encode_along_k, encode_along_n
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 16, (64, 48), dtype=np.uint8)
    order = rng.permutation(8)
    assert np.array_equal(oracle.decode_along_k(encode_along_k(codes), 64, 48), codes)
    assert np.array_equal(oracle.decode_along_n(encode_along_n(codes, order), 64, 48, order), codes)
    assert np.array_equal(oracle.decode_along_n(encode_along_n(codes), 64, 48), codes)


def test_decode_rejects_orders_that_are_not_permutations():
    w = np.zeros((1, 1), dtype=np.uint32)
    for bad in [(0, 1, 2, 3, 4, 5, 6, 6), (0, 1, 2, 3, 4, 5, 6, 8), (0, 1, 2)]:
        with pytest.raises(ValueError):
            oracle.decode_along_n(w, 1, 8, order=bad)

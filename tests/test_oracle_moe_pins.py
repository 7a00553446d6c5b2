"""Pins for the oracle's mixture-of-experts routines and its bfloat16 rounding.

The MoE layer (deep-dive page, section on where the format pays off, items 1 and 4) is the
dense product applied per assignment: row a = t*topk + j of the output is row t of A times the
dequantised weights of expert topk_ids[t, j].  The pins:

* ``bf16_round`` / ``bf16_bits`` against values worked out by hand from the binary format
  (ties to even included) and against torch's float32 -> bfloat16 cast (a library routine);
* ``moe_align`` against a worked example and against its definition on random routings;
* ``moe_gemm`` against the exact integer reference ``exact_gemm`` row by row (each row with
  its own expert's codes, scales and zero points), bitwise;
* properties: power-of-two router weights scale rows exactly; rows with no valid expert are
  not computed; bf16 results are the exact sums rounded once.
"""
import numpy as np
import pytest

import oracle


def f16(x):
    return np.asarray(x, dtype=np.float16)


# ------------------------------------------------------------------------- bf16 rounding

@pytest.mark.parametrize("x,want", [
    (1.0, 1.0),
    (1 + 2**-8, 1.0),                  # halfway between 1 and 1 + 2^-7: even mantissa wins
    (1 + 3 * 2**-8, 1 + 2**-6),        # halfway between 1 + 2^-7 and 1 + 2^-6: even wins
    (1 + 2**-7 + 2**-9, 1 + 2**-7),    # below halfway
    (1 + 2**-7 + 2**-8 + 2**-12, 1 + 2**-6),   # above halfway
    (255.5, 256.0),                    # spacing 1 in [128, 256): tie, 256 is even
    (-3.0, -3.0),
    (0.0, 0.0),
    (2**-20 * (1 + 2**-9), 2**-20),
])
def test_bf16_round_worked_values(x, want):
    assert float(oracle.bf16_round(x)) == want


@pytest.mark.parametrize("x,bits", [(1.0, 0x3F80), (-2.0, 0xC000), (0.5, 0x3F00), (3.0, 0x4040),
                                    (-0.0078125, 0xBC00)])
def test_bf16_bits_worked_values(x, bits):
    assert int(oracle.bf16_bits(x)) == bits
    assert float(oracle.bf16_value(bits)) == x


def test_bf16_matches_torch_cast_on_float32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-6, 6, 200000)).astype(np.float32)
    # ties: float32 values whose low 16 bits are exactly 0x8000 (finite, both signs)
    hi = rng.integers(0x3000, 0x4F00, 1000, dtype=np.uint32) | (rng.integers(0, 2, 1000,
                                                                             dtype=np.uint32) << 15)
    ties = (hi << 16) | 0x8000
    x = np.concatenate([x, ties.view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits(x.astype(np.float64)), want)
    assert np.array_equal(oracle.bf16_value(want), oracle.bf16_round(x.astype(np.float64)))


# ------------------------------------------------------------------------------ regrouping

def test_moe_align_worked_example():
    # tokens 0..2 pick (1, 0), (1, 2), (0, 1): expert 0 has assignments 1 and 4, expert 1 has
    # 0, 2 and 5, expert 2 has 3
    ids, off = oracle.moe_align(np.array([[1, 0], [1, 2], [0, 1]]), 3)
    assert ids.tolist() == [1, 4, 0, 2, 5, 3]
    assert off.tolist() == [0, 2, 5, 6]


def test_moe_align_leaves_out_invalid_experts_and_empty_experts_have_empty_ranges():
    ids, off = oracle.moe_align(np.array([[3, -1], [0, 4], [3, 0]]), 4)
    assert ids.tolist() == [2, 5, 0, 4]
    assert off.tolist() == [0, 2, 2, 2, 4]


@pytest.mark.parametrize("seed", [0, 1])
def test_moe_align_against_its_definition(seed):
    rng = np.random.default_rng(seed)
    E = 9
    topk = rng.integers(-1, E + 1, size=(50, 3))
    ids, off = oracle.moe_align(topk, E)
    flat = topk.reshape(-1)
    for e in range(E):
        got = ids[off[e]:off[e + 1]]
        assert np.all(np.diff(got) > 0)
        assert set(got.tolist()) == {a for a in range(flat.size) if flat[a] == e}
    assert off[-1] == np.sum((flat >= 0) & (flat < E))


# ----------------------------------------------------------------------------- the product

def tiny(E, T, topk, K, N, seed, zeros=False):
    rng = np.random.default_rng(seed)
    A = f16(rng.standard_normal((T, K)))
    q = rng.integers(0, 16, (E, K, N), dtype=np.uint8)
    s = f16(rng.uniform(0.005, 0.02, (E, K // 128, N)))
    z = rng.integers(0, 16, (E, K // 128, N), dtype=np.uint8) if zeros else None
    ids = np.stack([rng.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    return A, q, s, z, ids


@pytest.mark.parametrize("zeros", [False, True])
def test_moe_gemm_rows_equal_the_exact_product_with_their_expert(zeros):
    E, T, topk, K, N = 3, 4, 2, 256, 8
    A, q, s, z, ids = tiny(E, T, topk, K, N, seed=7, zeros=zeros)
    C, done = oracle.moe_gemm(A.astype(np.float64), ids, q, s.astype(np.float64), zeros=z)
    assert done.all()
    for a in range(T * topk):
        t, e = a // topk, ids[a // topk, a % topk]
        want, _, _ = oracle.exact_gemm(A[t:t + 1], q[e], s[e], zeros=None if z is None else z[e])
        assert np.array_equal(f16(C[a]).view(np.uint16), want[0].view(np.uint16)), a


def test_moe_gemm_one_expert_one_slot_is_the_dense_product():
    A, q, s, _, _ = tiny(1, 5, 1, 384, 16, seed=8)
    C, _ = oracle.moe_gemm(A.astype(np.float64), np.zeros((5, 1), np.int32), q,
                           s.astype(np.float64))
    want, _, _ = oracle.exact_gemm(A, q[0], s[0])
    assert np.array_equal(f16(C).view(np.uint16), want.view(np.uint16))


def test_moe_gemm_router_weights_of_a_power_of_two_scale_rows_exactly():
    A, q, s, _, ids = tiny(4, 6, 2, 256, 8, seed=9)
    base, _ = oracle.moe_gemm(A.astype(np.float64), ids, q, s.astype(np.float64))
    rs = np.array([0.5, 2.0, 0.25, 1.0] * 3, dtype=np.float32)
    C, _ = oracle.moe_gemm(A.astype(np.float64), ids, q, s.astype(np.float64), row_scale=rs)
    assert np.array_equal(C, base * rs[:, None])


def test_moe_gemm_skips_rows_without_a_valid_expert():
    A, q, s, _, ids = tiny(3, 4, 2, 128, 8, seed=10)
    ids[1, 0] = -1
    ids[2, 1] = 3
    C, done = oracle.moe_gemm(A.astype(np.float64), ids, q, s.astype(np.float64))
    assert done.tolist() == [True, True, False, True, True, False, True, True]
    assert not C[~done].any()


def test_moe_gemm_bf16_is_the_exact_sum_rounded_once():
    # inputs exact in both formats: the exact sums come from the integer reference
    rng = np.random.default_rng(11)
    E, T, topk, K, N = 2, 3, 2, 256, 8
    A = f16(rng.integers(-2, 3, (T, K)))
    q = rng.integers(0, 16, (E, K, N), dtype=np.uint8)
    s = f16(2.0 ** rng.integers(-7, -3, (E, K // 128, N)))
    ids = np.array([[0, 1], [1, 0], [1, 0]], dtype=np.int32)
    C, _ = oracle.moe_gemm(A.astype(np.float64), ids, q, s.astype(np.float64), act="bf16")
    for a in range(T * topk):
        t, e = a // topk, ids[a // topk, a % topk]
        _, exact, _ = oracle.exact_gemm(A[t:t + 1], q[e], s[e])
        assert np.array_equal(C[a], oracle.bf16_round(exact[0])), a
    assert np.array_equal(oracle.bf16_round(C), C)

"""GPU parity of the mixture-of-experts path (w4a16_moe_align + w4a16_moe_gemm) against the
oracle (oracle.moe_align / oracle.moe_gemm).

Regrouping is integer work: bit-exact.  The product: relative Frobenius error <= 1e-3 and max
abs error <= 1e-2 * max|C_ref| for fp16 outputs (the dense path's bar).  For bf16 outputs both
sides round the same fp32-or-better sum once to bfloat16, so an element differs by at most one
bf16 ulp (2^-8 relative) where the two sums straddle a rounding boundary: relative Frobenius
<= 4e-3 (below 2^-8 even if every element differed) and max abs <= 1e-2 * max|C_ref|.
With fp16 activations a row is also bit-identical to the dense w4a16_gemm of the same token
and expert when the dense call takes its whole-K kernel (same decode, same K split, same
summation order).  The routing entry (w4a16_moe_gemm_topk) lists the same rows in the same
order as w4a16_moe_align, so its results equal the presorted entry's bit for bit.
"""
import gc

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mixed_precision_w4a16_amd as w4
import oracle
from workloads import MOE_64E, MOE_8E, draw_moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


TOL = {"f16": 1e-3, "bf16": 4e-3}


def check(C, ref, act, what=""):
    d = C - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    mref = np.abs(ref).max()
    mx = np.abs(d).max() / mref if mref > 0 else np.abs(d).max()
    print(f"  {what} rel_fro={rel:.2e} max_abs/max|C|={mx:.2e}", flush=True)
    assert np.isfinite(C).all(), what
    assert rel <= TOL[act], (what, rel)
    assert mx <= 1e-2, (what, mx)


def to_torch(bits, act):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.bfloat16 if act == "bf16" else torch.float16)


def values(t):
    """float64 values of a fp16 / bf16 CUDA tensor."""
    return t.float().cpu().numpy().astype(np.float64)


class Moe:
    def __init__(self, d):
        self.act = d["act"]
        self.E, self.K, self.N = d["q"].shape
        self.zp = d["zeros"] is not None
        scales = d["s_bits"] if self.act == "bf16" else d["s"].astype(np.float16)
        self.packed, self.params = w4.to_device(*w4.pack_experts(d["q"], scales, d["zeros"]))

    def run(self, d, row_scale=True, out=None, topk_ids=None, routed=False):
        ids = d["topk_ids"] if topk_ids is None else topk_ids
        A = to_torch(d["A_bits"], self.act)
        ids_d = torch.from_numpy(np.ascontiguousarray(ids)).cuda()
        rs = torch.from_numpy(d["row_scale"]).cuda() if row_scale else None
        if routed:
            C = w4.moe_gemm_topk(A, self.packed, self.params, ids_d, self.E, self.N,
                                 row_scale=rs, zero_points=self.zp, out=out)
        else:
            sorted_ids, offsets = w4.moe_align(ids_d, self.E)
            C = w4.moe_gemm(A, self.packed, self.params, sorted_ids, offsets, ids.shape[1],
                            self.E, self.N, row_scale=rs, zero_points=self.zp, out=out)
        torch.cuda.synchronize()
        return C


def ref(d, row_scale=True, topk_ids=None, cols=None):
    q, s, z = d["q"], d["s"], d["zeros"]
    if cols is not None:
        q, s = q[:, :, cols], s[:, :, cols]
        z = None if z is None else z[:, :, cols]
    return oracle.moe_gemm(d["A"], d["topk_ids"] if topk_ids is None else topk_ids, q, s, z,
                           d["row_scale"] if row_scale else None, d["act"])


# ------------------------------------------------------------------------------ regrouping

@pytest.mark.parametrize("T,topk,E", [(1, 1, 1), (5, 2, 8), (64, 6, 64), (700, 8, 16),
                                      (3, 2, 1024), (257, 4, 3)])
def test_align_against_oracle(T, topk, E):
    rng = np.random.default_rng(T * 31 + E)
    ids = rng.integers(0, E, (T, topk)).astype(np.int32)
    if T > 100:
        ids[rng.random((T, topk)) < 0.05] = -1          # assignments of no expert here
        ids[rng.random((T, topk)) < 0.05] = E
    want_ids, want_off = oracle.moe_align(ids, E)
    got_ids, got_off = w4.moe_align(torch.from_numpy(ids).cuda(), E)
    got_off = got_off.cpu().numpy()
    assert np.array_equal(got_off, want_off)
    assert np.array_equal(got_ids.cpu().numpy()[:want_off[-1]], want_ids)


def test_align_is_repeatable_across_calls():
    ids = np.random.default_rng(3).integers(0, 10, (2000, 4)).astype(np.int32)
    t = torch.from_numpy(ids).cuda()
    a = [w4.moe_align(t, 10) for _ in range(3)]
    for x in a[1:]:
        assert torch.equal(x[0], a[0][0]) and torch.equal(x[1], a[0][1])


# ----------------------------------------------------------------------------- the product

# (E, topk, K, N, T): one expert; a few experts with 1..16 rows each (16-row blocks); 32 and
# 64 mean rows (32- and 64-row blocks, several blocks per expert); 64 experts over few tokens
# (most workgroups find no rows); K = 128 (three of four waves without a K tile); N = 2816
# (eleven 256-column parameter groups, slab groups crossing them).
SHAPES = [(1, 1, 128, 256, 1), (8, 2, 384, 512, 5), (8, 2, 1024, 1024, 40),
          (4, 2, 1024, 512, 64), (4, 1, 512, 768, 300), (64, 6, 256, 2816, 16),
          (16, 4, 128, 256, 2)]


@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("zp", [False, True])
@pytest.mark.parametrize("E,topk,K,N,T", SHAPES)
def test_moe_against_oracle(E, topk, K, N, T, zp, act):
    d = draw_moe(E, topk, K, N, T, seed=E + K + N + T, act=act, zero_points=zp)
    W = Moe(d)
    C = W.run(d)
    want, done = ref(d)
    assert done.all()
    check(values(C), want, act, f"{act} zp={zp} E={E} topk={topk} K={K} N={N} T={T}")
    assert torch.equal(W.run(d), C)                      # fixed summation order
    assert torch.equal(W.run(d, routed=True), C)         # the routing entry: same bits


# Experts with row counts on every side of the pass sizes: 8 experts at 16 mean rows take
# passes of up to two 16-row blocks (0, 3, 16, 17, 32, 33 rows ...), 4 experts at 32 mean rows
# passes of up to four (31, 33, 64 rows; 110 rows: a pass of four, then one more of four), 16
# experts at 3.6 mean rows passes of one (9, 12, 16 rows).  K = 4096 (8 K tiles a wave and
# more) takes the whole-line A loads in passes of more than 8 rows, K = 512 the fragment-order
# loads throughout.
@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("zp", [False, True])
@pytest.mark.parametrize("K", [512, 4096])
@pytest.mark.parametrize("E,counts", [(8, [0, 3, 16, 17, 32, 33, 20, 7]),
                                      (4, [0, 33, 64, 31]), (4, [1, 17, 110, 0]),
                                      (16, [12, 16, 9, 8, 1, 0, 2, 0, 0, 3, 0, 5, 0, 0, 0, 2])])
def test_expert_row_counts_around_the_pass_sizes(E, counts, K, zp, act):
    topk, N = 2, 512
    R = sum(counts)
    T = R // topk
    d = draw_moe(E, topk, K, N, T, seed=R + E + K + len(counts), act=act, zero_points=zp)
    experts = np.repeat(np.arange(E, dtype=np.int32), counts)
    np.random.default_rng(E).shuffle(experts)
    d["topk_ids"] = experts.reshape(T, topk)
    W = Moe(d)
    C = W.run(d)
    want, done = ref(d)
    assert done.all()
    check(values(C), want, act, f"{act} zp={zp} E={E} K={K} rows per expert {counts}")
    assert torch.equal(W.run(d, routed=True), C)


# Few rows over a long K with at most a workgroup per CU: three register buffers (K = 8192, 64
# K tiles: 16 a wave).
@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("zp", [False, True])
@pytest.mark.parametrize("T", [1, 3])
def test_three_buffer_passes_against_oracle(T, zp, act):
    E, topk, K, N = 8, 2, 8192, 1024
    d = draw_moe(E, topk, K, N, T, seed=78 + T, act=act, zero_points=zp)
    W = Moe(d)
    C = W.run(d)
    want, done = ref(d)
    assert done.all()
    check(values(C), want, act, f"three buffers {act} zp={zp} T={T}")
    assert torch.equal(W.run(d, routed=True), C)


# Passes of two row blocks over at least two rounds of workgroups take six slabs per
# workgroup: 8 experts x 28672 columns (299 slab groups each), 64 tokens, top 2.
@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("zp", [False, True])
def test_six_slab_passes_against_oracle(zp, act):
    E, topk, K, N, T = 8, 2, 512, 28672, 64
    d = draw_moe(E, topk, K, N, T, seed=77, act=act, zero_points=zp)
    W = Moe(d)
    C = W.run(d)
    want, done = ref(d)
    assert done.all()
    check(values(C), want, act, f"six slabs {act} zp={zp}")
    assert torch.equal(W.run(d, routed=True), C)


@pytest.mark.parametrize("routed", [False, True])
@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_rows_of_no_expert_are_not_written(act, routed):
    E, topk, K, N, T = 6, 3, 512, 512, 20
    d = draw_moe(E, topk, K, N, T, seed=5, act=act)
    ids = d["topk_ids"].copy()
    ids[::3, 0] = -1
    ids[1::4, 2] = E
    W = Moe(d)
    dt = torch.bfloat16 if act == "bf16" else torch.float16
    out = torch.full((T * topk, N), -7.0, dtype=dt, device="cuda")
    W.run(d, out=out, topk_ids=ids, routed=routed)
    want, done = ref(d, topk_ids=ids)
    got = values(out)
    assert (got[~done] == -7.0).all()
    check(got[done], want[done], act, "partial routing")


def test_f16_rows_equal_the_dense_product_of_their_token_and_expert():
    E, topk, K, N, T = 4, 2, 2048, 1024, 8
    d = draw_moe(E, topk, K, N, T, seed=6, act="f16")
    W = Moe(d)
    C = W.run(d, row_scale=False).cpu()
    A = to_torch(d["A_bits"], "f16")
    ids = d["topk_ids"].reshape(-1)
    per = K * N // 8
    for e in range(E):
        rows = np.flatnonzero(ids == e)
        if rows.size == 0:
            continue
        assert rows.size <= 16                           # the dense whole-K kernel's range
        Ae = A[torch.from_numpy(rows // topk).cuda()].contiguous()
        De = w4.gemm(Ae, W.packed[e].reshape(per), W.params[e].view(torch.float16).reshape(-1), N)
        torch.cuda.synchronize()
        assert torch.equal(De.cpu(), C[torch.from_numpy(rows)]), e


# The workgroups of the experts in use come first whatever their numbers: a few scattered
# experts of 64 (the last one among them), and two of 1024 (the most experts the entries take).
@pytest.mark.parametrize("routed", [False, True])
@pytest.mark.parametrize("E,ids", [(64, [[63, 5], [17, 63], [5, 40]]),
                                   (1024, [[1023, 0], [0, 1023], [511, 1023]])])
def test_scattered_experts_in_use(E, ids, routed):
    ids = np.array(ids, dtype=np.int32)
    T, topk = ids.shape
    d = draw_moe(E, topk, 128, 256, T, seed=E + 1, act="f16")
    d["topk_ids"] = ids
    W = Moe(d)
    C = W.run(d, routed=routed)
    want, done = ref(d)
    assert done.all()
    check(values(C), want, "f16", f"E={E} experts {sorted(set(ids.ravel().tolist()))}")


def test_routing_entry_at_its_limit():
    # T * topk = 2048, the most the routing entry takes
    E, topk, K, N, T = 16, 8, 256, 512, 256
    d = draw_moe(E, topk, K, N, T, seed=12, act="f16")
    ids = d["topk_ids"].copy()
    W = Moe(d)
    with pytest.raises(ValueError):
        w4.moe_gemm_topk(to_torch(d["A_bits"][:T - 1], "f16"), W.packed, W.params,
                         torch.from_numpy(ids).cuda(), E, N)
    C = W.run(d, routed=True)
    assert torch.equal(C, W.run(d))
    want, _ = ref(d)
    check(values(C), want, "f16", "routing at 2048 assignments")


def test_row_scale_none_is_one():
    d = draw_moe(8, 2, 512, 256, 9, seed=8, act="bf16")
    W = Moe(d)
    d1 = dict(d, row_scale=np.ones_like(d["row_scale"]))
    assert torch.equal(W.run(d, row_scale=False), W.run(d1, row_scale=True))


def test_moe_rejects_bad_arguments():
    d = draw_moe(2, 1, 256, 256, 2, seed=1)
    W = Moe(d)
    A = to_torch(d["A_bits"], "f16")
    s_ids, off = w4.moe_align(torch.from_numpy(d["topk_ids"]).cuda(), 2)
    lib = w4.library()
    args = [A.data_ptr(), W.packed.data_ptr(), W.params.data_ptr(), s_ids.data_ptr(),
            off.data_ptr(), None]
    out = torch.empty(2, 256, dtype=torch.float16, device="cuda")
    assert lib.w4a16_moe_gemm(*args, out.data_ptr(), 2, 1, 2, 256, 320, 0, 0, None) == w4.ESHAPE
    assert lib.w4a16_moe_gemm(*args, out.data_ptr(), 2, 1, 2, 200, 256, 0, 0, None) == w4.ESHAPE
    assert lib.w4a16_moe_gemm(*args, out.data_ptr(), 2, 1, 2, 256, 256, 0, 2, None) == w4.EINVAL
    assert lib.w4a16_moe_gemm(*args, out.data_ptr(), 2, 0, 2, 256, 256, 0, 0, None) == w4.EINVAL
    assert lib.w4a16_moe_gemm(*args, out.data_ptr(), 0, 1, 2, 256, 256, 0, 0, None) == w4.OK
    assert lib.w4a16_moe_align(None, 2, 1, 2, s_ids.data_ptr(), off.data_ptr(), None) == w4.EINVAL
    assert lib.w4a16_moe_align(s_ids.data_ptr(), 2, 1, 1025, s_ids.data_ptr(), off.data_ptr(),
                               None) == w4.ESHAPE


# The layer shapes at their full sizes, every token count of the workload, every column.
@pytest.mark.slow
@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("sh", [sh for wl in (MOE_8E, MOE_64E) for sh in wl.shapes],
                         ids=lambda sh: sh.name)
def test_moe_full_size_all_columns(sh, act):
    d = draw_moe(sh.E, sh.topk, sh.K, sh.N, max(sh.Ts), seed=0, act=act)
    W = Moe(d)
    for T in sh.Ts:
        dT = dict(d, A=d["A"][:T], A_bits=d["A_bits"][:T], topk_ids=d["topk_ids"][:T],
                  row_scale=d["row_scale"][:T * sh.topk])
        Ct = W.run(dT)
        C = values(Ct)
        want, done = ref(dT)
        assert done.all()
        check(C, want, act, f"{sh.name} {act} T={T} (all columns)")
        if T * sh.topk <= w4.MOE_ROUTE_MAX:
            assert torch.equal(W.run(dT, routed=True), Ct)
    del W, d
    gc.collect()
    torch.cuda.empty_cache()

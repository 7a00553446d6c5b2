"""Benchmark: W4A16 GEMM effective GB/s on the 72k x 18k weight (K = 18432, N = 73728,
group 128) over the batch sweep M = 1, 2, 4, ..., 128.

One step = one call per M in the sweep (the whole multiply path for that batch).  `value` is
the sweep's algorithmic bytes divided by its wall time, inputs resident in HBM.  Algorithmic
bytes per call: D = 2MK (A) + KN/2 (codes) + KN/64 (scales) + 2MN (C); flops F = 2MKN.
Roofline per call: T_bound = max(D / 8 TB/s, F / 2.5 PFLOP/s); fp16-weight byte bound
D16 = 2MK + 2KN + 2MN (the MARLIN paper's uncompressed reference point).

`roofline` covers the dominant kernel: the whole-K-workgroup kernel as it serves M = 1..8,
four of the eight calls; HBM-bound, so achieved = its algorithmic bytes per launch / its mean
launch time (HIP events on the launch stream around every call).  `roofline_by_kernel` gives
the same for every kernel of the sweep, the compute-bound ones against the fp16 MFMA peak;
`traffic` is the measured HBM bytes per launch from the committed counter runs, while the
kernel source is the one they were taken on.

The stdout line (kept to a few KB) also holds the per-M `sweep` (with each row's speed-up
over torch.matmul on fp16 weights, hipBLASLt, the pages' comparison point: `x_fp16_gemm`),
the compute-bound 8192 x 28672 sweep at M = 256, 512, 1024 (`compute_sweep`), the measured
stream-read and random-operand MFMA rates (`references`), the CPU baseline (the oracle on a
column sample) and the run state (clocks, power cap and ECC state from sysfs, CPU model, core
counts).
The rest goes to stderr and to the `--details` JSON file: the other packed formats, the
load-time repack, the 2:4-sparse path, the MoE layers, the tensor-parallel rank and
model-layer shapes, each with its fraction of the roofline bound.

Single GPU only.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMM effective GB/s (% HBM peak) + TFLOP/s at M=1..128, vs 3.87x bound"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix
GROUP = 128
CALIB_BYTES = 512 << 20
SETTLE_S = 1.0                  # untimed sweep before the warm-up steps (clock ramp)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_72kx18k.json")

# The kernel each M of the sweep runs (the library picks it from M: workgroups that own nine
# 16-column slabs over all of K up to M = 16, 32-row tiles up to 32, 64-row up to 64, then
# 128-row tiles on this shape), and the roof that bounds it.
KERNELS = [
    ("w4a16_gemm_skinny_kernel<1,6> (whole-K workgroups, 6 slabs, 3 per CU)", (1, 2, 4, 8), "hbm"),
    ("w4a16_gemm_skinny_kernel<1,9,fl> (whole-K workgroups, 9 slabs, 2 per CU, whole-line A)",
     (16,), "hbm"),
    ("w4a16_gemm_skinny_kernel<2,9,two,dma> (whole-K workgroups, 9 slabs, 32 rows, 2 per CU, "
     "A lines by DMA)", (32,), "hbm"),
    ("w4a16_gemm_kernel<4,4> (64-row tiles)", (64,), "hbm"),
    ("w4a16_gemm_wide_kernel<4,2> (128-row tiles)", (128,), "mfma"),
]
KERNEL_SOURCE = os.path.join(ROOT, "mixed_precision_w4a16_amd", "csrc", "gemm.hip")


def measured_traffic():
    """HBM bytes per launch from the committed counter runs, if they were taken on the
    kernel source as it is now (else None)."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
        sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec


def algorithmic_bytes(M, K, N):
    return 2 * M * K + K * N // 2 + K * N // 64 + 2 * M * N


def format_bytes(M, K, N, group, zero_points):
    """Algorithmic bytes of one call in a given packed format: A, codes, the stored per-group
    parameters (fp16 scale, plus the fp16 zero term with zero points) and C."""
    per_col = (K // group) * 2 * (2 if zero_points else 1)
    return 2 * M * K + K * N // 2 + per_col * N + 2 * M * N


def fp16_weight_bytes(M, K, N):
    return 2 * M * K + 2 * K * N + 2 * M * N


def flops(M, K, N):
    return 2 * M * K * N


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_SPIN_CYCLES_PER_US = None


def hold_gpu(torch, stream, us):
    """Keep `stream` busy for about `us` microseconds with torch's spin kernel, so that calls
    enqueued right after are all queued before the GPU reaches them: back-to-back timing of
    kernels shorter than the host's per-call cost (the Python binding takes ~15-25 us a call)
    then sees kernel time, not the host's launch rate.  The spin's clock is calibrated once."""
    global _SPIN_CYCLES_PER_US
    if _SPIN_CYCLES_PER_US is None:
        torch.cuda._sleep(1000)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        torch.cuda._sleep(2_000_000)
        e1.record(stream)
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_US = 2_000_000 / max(e0.elapsed_time(e1) * 1e3, 1.0)
    torch.cuda._sleep(int(us * _SPIN_CYCLES_PER_US))


def queued_batch(torch, stream, calls, warmup=5):
    """GPU time per call of `calls(i)` for i in range(n) run back to back: `warmup` untimed
    calls (which also measure the host's cost per call), a spin that outlasts enqueuing the
    batch, then the batch between one event pair.  Returns (us per call, queued) where
    queued says the first event was still waiting behind the spin when the last call had
    been enqueued, i.e. the GPU never waited for the host."""
    n = calls.n
    t0 = time.perf_counter()
    for i in range(warmup):
        calls(i)
    host_us = (time.perf_counter() - t0) * 1e6 / max(warmup, 1)
    torch.cuda.synchronize()
    hold_gpu(torch, stream, 1.5 * host_us * n + 500.0)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        calls(warmup + i)
    e1.record(stream)
    queued = not e0.query()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n, queued


def cpu_baseline(A, q, s, Ms, ncols, nthreads):
    """The oracle as it stands, on a column sample of the same workload and every M."""
    import oracle
    K = q.shape[0]
    qc = np.ascontiguousarray(q[:, :ncols])
    sc = np.ascontiguousarray(s[:, :ncols])
    t = time.perf_counter()
    for M in Ms:
        oracle.gemm(A[:M], qc, sc, nthreads=nthreads)
    dt = time.perf_counter() - t
    byts = sum(algorithmic_bytes(M, K, ncols) for M in Ms)
    return {"value": byts / dt / 1e9, "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": f"all M in {list(Ms)}, K={K}, first {ncols} of the N columns "
                      f"(the same draws as the GPU run); {dt:.1f} s of CPU time"}


FORMATS = (("column", True, False), ("zeros", False, True), ("column_zeros", True, True))
FORMAT_MS = (1, 16, 64, 128)


def time_formats(w4, torch, dev, Ad, q, s, K, N, steps, warmup, copies, stream, sym):
    """Per-call time of the other packed formats on the same codes: one scale per column
    (group = K; the first row of scale groups serves as that column's scale), zero points per
    group and column, and both.  The calls of all four formats (the group-128 symmetric one
    included, `sym` = its rotated weight copies) alternate call by call, so every format is
    timed in the same clock and power state."""
    from workloads import draw_zeros
    fmts = [("group128_symmetric", GROUP, False, sym)]
    for name, col, zp in FORMATS:
        group = K if col else GROUP
        sf = np.ascontiguousarray(s[:1]) if col else s
        z = draw_zeros(K, N, seed=0, group=group) if zp else None
        packed, params = w4.pack(q, sf, group=group, zeros=z)
        pd, sd = w4.to_device(packed, params, dev)
        del packed, params
        fmts.append((name, group, zp, [(pd, sd)] + [(pd.clone(), sd.clone())
                                                     for _ in range(copies - 1)]))
    rows = []
    for M in FORMAT_MS:
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
        ws = w4.new_workspace(M, K, N, dev)
        evs = {name: [] for name, *_ in fmts}
        for i in range(warmup + steps):
            for name, group, zp, cps in fmts:
                p_, s_ = cps[i % len(cps)]
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                w4.gemm(Ad[:M], p_, s_, N, out=out, ws=ws, stream=stream, group=group,
                        zero_points=zp)
                e1.record(stream)
                if i >= warmup:
                    evs[name].append((e0, e1))
        torch.cuda.synchronize()
        us = {name: float(np.mean([a.elapsed_time(b) for a, b in e])) * 1e3
              for name, e in evs.items()}
        for name, group, zp, _ in fmts:
            D = format_bytes(M, K, N, group, zp)
            rows.append({"format": name, "group": group, "zero_points": zp, "M": M,
                         "us": round(us[name], 2), "GBps": round(D / us[name] / 1e3, 1),
                         "hbm_frac": round(D / us[name] / 1e3 / HBM_PEAK_GBPS, 4),
                         "TFLOPs": round(flops(M, K, N) / us[name] / 1e6, 2),
                         "time_vs_group128_symmetric":
                             round(us[name] / us["group128_symmetric"], 3)})
            log(f"{name:19s} M={M:4d} {us[name]:8.1f} us  {D / us[name] / 1e3:7.0f} GB/s  "
                f"x{us[name] / us['group128_symmetric']:.3f}")
    del fmts
    torch.cuda.empty_cache()
    return rows


def sparse_bytes(M, K, N):
    """Algorithmic bytes of one 2:4-sparse call: A, kept codes and their positions (3 bits
    per weight), scales, C."""
    return 2 * M * K + K * N * 3 // 8 + K * N // 64 + 2 * M * N


def time_sparse(w4, torch, dev, Ad, q, s, K, N, Ms, steps, warmup, copies, stream, dense):
    """The 2:4-sparse path (w4a16_pack_24 / w4a16_gemm_24) on the same codes with two of
    every four along K pruned, every M of the sweep; each call alternated with a dense call
    on the original codes, so both are timed in the same clock and power state.  TFLOP/s
    counts the dense product's 2MKN."""
    from workloads import sparsify_24
    t = time.perf_counter()
    qs = sparsify_24(q, seed=0)
    packed, sp = w4.pack_24(qs, s)
    del qs
    log(f"2:4 weights drawn and packed in {time.perf_counter() - t:.1f} s")
    pd, sd = w4.to_device(packed, sp, dev)
    del packed, sp
    cps = [(pd, sd)] + [(pd.clone(), sd.clone()) for _ in range(copies - 1)]
    rows = []
    for M in Ms:
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
        ws = w4.new_workspace(M, K, N, dev)
        ev_s, ev_d = [], []
        for i in range(warmup + steps):
            for kind in ("sparse", "dense"):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                if kind == "sparse":
                    p_, s_ = cps[i % len(cps)]
                    w4.gemm_24(Ad[:M], p_, s_, N, out=out, stream=stream)
                else:
                    p_, s_ = dense[i % len(dense)]
                    w4.gemm(Ad[:M], p_, s_, N, out=out, ws=ws, stream=stream)
                e1.record(stream)
                if i >= warmup:
                    (ev_s if kind == "sparse" else ev_d).append((e0, e1))
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in ev_s])) * 1e3
        usd = float(np.mean([a.elapsed_time(b) for a, b in ev_d])) * 1e3
        D = sparse_bytes(M, K, N)
        rows.append({"M": M, "us": round(us, 2), "GBps": round(D / us / 1e3, 1),
                     "hbm_frac": round(D / us / 1e3 / HBM_PEAK_GBPS, 4),
                     "TFLOPs_dense_equivalent": round(flops(M, K, N) / us / 1e6, 2),
                     "dense_us": round(usd, 2), "speedup_vs_dense": round(usd / us, 3)})
        log(f"2:4 sparse M={M:4d} {us:8.1f} us  {D / us / 1e3:7.0f} GB/s "
            f"({D / us / 1e3 / HBM_PEAK_GBPS:5.1%} HBM)  dense {usd:8.1f} us  x{usd / us:.3f}")
    del cps, pd, sd
    torch.cuda.empty_cache()
    return rows


def time_repack(w4, torch, dev, K, N, steps, stream):
    """Load-time repack (w4a16_repack) of the same-sized weight with zero points, from words
    packed along K and along N: random words (every 32-bit word is 8 valid codes).  Bytes:
    codes read and written (K*N/2 each), scales and packed zero points read, scales and zero
    terms written."""
    G = K // GROUP
    g = torch.Generator(device=dev).manual_seed(0)
    rows = []
    for name, layout, shape in (("along_k", w4.PACKED_ALONG_K, (K // 8, N)),
                                ("along_n", w4.PACKED_ALONG_N, (K, N // 8))):
        qw = torch.randint(-2**31, 2**31 - 1, shape, dtype=torch.int32, device=dev, generator=g)
        qz = torch.randint(-2**31, 2**31 - 1, (G, N // 8), dtype=torch.int32, device=dev,
                           generator=g)
        sc = (torch.rand((G, N), device=dev, generator=g) * 0.015 + 0.005).half()
        order = None if layout == w4.PACKED_ALONG_K else [0, 2, 4, 6, 1, 3, 5, 7]
        evs = []
        for i in range(2 + steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            out = w4.repack(qw, sc, K, N, layout, qzeros=qz, order=order, stream=stream)
            e1.record(stream)
            if i >= 2:
                evs.append((e0, e1))
            del out
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
        D = K * N // 2 * 2 + G * N * 2 + G * N // 2 + G * N * 4
        rows.append({"source": name, "zero_points": True, "us": round(us, 1),
                     "GBps": round(D / us / 1e3, 1), "hbm_frac": round(D / us / 1e3 / HBM_PEAK_GBPS, 4)})
        log(f"repack {name}: {us:8.1f} us  {D / us / 1e3:7.0f} GB/s")
        del qw, qz, sc
        torch.cuda.empty_cache()
    return rows


def time_moe(w4, torch, dev, steps, stream):
    """Mixture-of-experts layers on the Mixtral-shaped and 64-expert shapes, fp16 and bf16
    activations, every token count of the workload: w4a16_moe_align + w4a16_moe_gemm (two
    launches) and w4a16_moe_gemm_topk (routing inside the product, one launch), alternated
    call by call.  Bytes per call: the weights and scales of the experts the call's tokens
    use, A, and C (T * topk rows).  Enough weight copies rotate between calls that a copy's
    experts are not still in the memory-side cache when they come round again."""
    from workloads import MOE_64E, MOE_8E, draw_moe
    rows = []
    for wl in (MOE_8E, MOE_64E):
        for sh in wl.shapes:
            G = sh.K // GROUP
            per_expert = sh.K * sh.N // 2 + G * sh.N * 2
            for act in ("f16", "bf16"):
                t = time.perf_counter()
                d = draw_moe(sh.E, sh.topk, sh.K, sh.N, max(sh.Ts), seed=0, act=act)
                scales = d["s_bits"] if act == "bf16" else d["s"].astype(np.float16)
                pk, pr = w4.to_device(*w4.pack_experts(d["q"], scales), dev)
                log(f"moe {sh.name} {act}: drawn and packed in {time.perf_counter() - t:.1f} s")
                dt = torch.bfloat16 if act == "bf16" else torch.float16
                A_all = torch.from_numpy(d["A_bits"].view(np.int16)).to(dev).view(dt)
                used = {T: len(np.unique(d["topk_ids"][:T])) for T in sh.Ts}
                touched = min(used.values()) * per_expert
                ncp = int(min(max(2, -(-600e6 // touched)), max(2, 8e9 // (sh.E * per_expert))))
                cps = [(pk, pr)] + [(pk.clone(), pr.clone()) for _ in range(ncp - 1)]
                for T in sh.Ts:
                    A = A_all[:T].contiguous()
                    ids = torch.from_numpy(np.ascontiguousarray(d["topk_ids"][:T])).to(dev)
                    rs = torch.from_numpy(d["row_scale"][:T * sh.topk]).to(dev)
                    out = torch.empty((T * sh.topk, sh.N), dtype=dt, device=dev)
                    ev, evt = [], []

                    def iteration(i):
                        p_, r_ = cps[i % len(cps)]
                        e0, e1, e2, e3 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
                        e0.record(stream)
                        sid, off = w4.moe_align(ids, sh.E, stream=stream)
                        e1.record(stream)
                        w4.moe_gemm(A, p_, r_, sid, off, sh.topk, sh.E, sh.N, row_scale=rs,
                                    out=out, stream=stream)
                        e2.record(stream)
                        p_, r_ = cps[(i + len(cps) // 2) % len(cps)]
                        w4.moe_gemm_topk(A, p_, r_, ids, sh.E, sh.N, row_scale=rs, out=out,
                                         stream=stream)
                        e3.record(stream)
                        return e0, e1, e2, e3
                    # warm-up iterations measure the host's cost of one; the timed ones are
                    # queued behind a spin that outlasts enqueuing them all, so the decode-size
                    # calls (a few us each) are timed on the GPU, not at the host's launch rate
                    t0 = time.perf_counter()
                    for i in range(4):
                        iteration(i)
                    host_us = (time.perf_counter() - t0) * 1e6 / 4
                    torch.cuda.synchronize()
                    hold_gpu(torch, stream, 1.5 * host_us * steps + 500.0)
                    for i in range(4, 4 + steps):
                        e0, e1, e2, e3 = iteration(i)
                        ev.append((e0, e1, e2))
                        evt.append((e2, e3))
                    queued = not ev[0][0].query()
                    torch.cuda.synchronize()
                    ua = float(np.mean([a.elapsed_time(b) for a, b, _ in ev])) * 1e3
                    ug = float(np.mean([b.elapsed_time(c) for _, b, c in ev])) * 1e3
                    ut = float(np.mean([a.elapsed_time(b) for a, b in evt])) * 1e3
                    D = used[T] * per_expert + T * sh.K * 2 + T * sh.topk * sh.N * 2
                    rows.append({"workload": wl.name, "shape": sh.name, "act": act, "T": T,
                                 "E": sh.E, "topk": sh.topk, "K": sh.K, "N": sh.N,
                                 "experts_used": used[T], "align_us": round(ua, 2),
                                 "gemm_us": round(ug, 2), "us": round(ua + ug, 2),
                                 "gemm_GBps": round(D / ug / 1e3, 1),
                                 "gemm_hbm_frac": round(D / ug / 1e3 / HBM_PEAK_GBPS, 4),
                                 "routed_us": round(ut, 2),
                                 "routed_GBps": round(D / ut / 1e3, 1),
                                 "weight_copies_rotated": ncp,
                                 "queued_ahead_of_gpu": queued})
                    log(f"moe {sh.name:12s} {act:4s} T={T:3d} experts={used[T]:2d}  align "
                        f"{ua:6.1f} us  gemm {ug:7.1f} us  {D / ug / 1e3:6.0f} GB/s "
                        f"({D / ug / 1e3 / HBM_PEAK_GBPS:5.1%} HBM)  routed {ut:7.1f} us "
                        f"{D / ut / 1e3:6.0f} GB/s")
                del cps, pk, pr, d
                torch.cuda.empty_cache()
    return rows


def time_compute_sweep(w4, torch, dev, steps, stream):
    """The compute-bound transition sweep (K = 8192, N = 28672, M = 256, 512, 1024, A ~ N(0,
    0.5^2)): us per call, TFLOP/s and its fraction of the 2.5 PFLOP/s dense fp16 matrix peak
    (MFMA utilisation), GB/s of the algorithmic bytes and the speed-up over the fp16-weight
    byte bound.  Five weight copies (585 MB) rotate, more than the memory-side cache holds."""
    from workloads import COMPUTE_SWEEP, draw_shape
    sh = COMPUTE_SWEEP.shapes[0]
    K, N = sh.K, sh.N
    A, q, s = draw_shape(sh, seed=0)
    pd, sd = w4.to_device(*w4.pack(q, s), dev)
    cps = [(pd, sd)] + [(pd.clone(), sd.clone()) for _ in range(4)]
    Ad = torch.from_numpy(A).to(dev)
    rows = []
    for M in sh.Ms:
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
        ws = w4.new_workspace(M, K, N, dev)
        evs = []
        for i in range(5 + steps):
            p_, s_ = cps[i % len(cps)]
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            w4.gemm(Ad[:M], p_, s_, N, out=out, ws=ws, stream=stream)
            e1.record(stream)
            if i >= 5:
                evs.append((e0, e1))
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
        F, D, D16 = flops(M, K, N), algorithmic_bytes(M, K, N), fp16_weight_bytes(M, K, N)
        rows.append({"M": M, "K": K, "N": N, "us": round(us, 2),
                     "TFLOPs": round(F / us / 1e6, 1),
                     "mfma_frac": round(F / us / 1e6 / MFMA_F16_PEAK_TFLOPS, 4),
                     "GBps": round(D / us / 1e3, 1),
                     "speedup_vs_fp16_bound": round(max(D16 / (HBM_PEAK_GBPS * 1e3),
                                                        F / (MFMA_F16_PEAK_TFLOPS * 1e6)) / us, 3)})
        log(f"compute sweep M={M:5d} {us:8.1f} us  {F / us / 1e6:7.1f} TFLOP/s "
            f"({F / us / 1e6 / MFMA_F16_PEAK_TFLOPS:5.1%} of fp16 MFMA peak)")
    del cps, pd, sd
    torch.cuda.empty_cache()
    return rows


def time_fp16_gemm(torch, dev, Ad, q, s, Ms, steps, stream, w4_us):
    """The pages' comparison point (MARLIN paper, Figure 1; deep-dive page, "性能结果应该怎样读"):
    the same product with uncompressed fp16 weights, torch.matmul (hipBLASLt) on a fp16 copy
    of the dequantised weight, per M of the sweep, against the W4A16 call's time in this run.
    The fp16 weight (K x N x 2 bytes, 2.7 GB on 72k x 18k) exceeds the memory-side cache."""
    K, N = q.shape
    g = torch.from_numpy(np.ascontiguousarray(s)).to(dev).float()
    W = torch.empty((K, N), dtype=torch.float16, device=dev)
    step = 2048
    for k0 in range(0, K, step):            # dequantise on the GPU in K blocks
        qk = torch.from_numpy(np.ascontiguousarray(q[k0:k0 + step])).to(dev).float()
        W[k0:k0 + step] = (qk - 8.0).mul_(g[k0 // GROUP:(k0 + step) // GROUP].repeat_interleave(GROUP, 0)).half()
        del qk
    rows = []
    for M in Ms:
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
        for _ in range(3):
            torch.matmul(Ad[:M], W, out=out)
        evs = []
        for _ in range(steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            torch.matmul(Ad[:M], W, out=out)
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
        rows.append({"M": M, "fp16_us": round(us, 2), "w4a16_us": w4_us[M],
                     "speedup": round(us / w4_us[M], 3)})
        log(f"fp16 torch.matmul M={M:4d} {us:8.1f} us   W4A16 {w4_us[M]:8.1f} us   "
            f"speedup {us / w4_us[M]:.2f}x")
    del W, g
    torch.cuda.empty_cache()
    return rows


def time_shapes(w4, torch, dev, steps, stream, workload, tag):
    """Per-call time of every shape and M of a workload: back-to-back calls between one event
    pair, queued behind a spin so the host's launch rate does not set the time (these kernels
    run for a few to a few hundred us); enough weight copies rotate (600 MB or more) that each
    call's weights come from HBM."""
    from workloads import draw_shape
    rows = []
    for sh in workload.shapes:
        A, q, s = draw_shape(sh, seed=0)
        pd, sd = w4.to_device(*w4.pack(q, s), dev)
        del q, s
        wbytes = sh.K * sh.N // 2 + sh.K // GROUP * sh.N * 2
        ncp = max(2, -(-600_000_000 // wbytes))
        cps = [(pd, sd)] + [(pd.clone(), sd.clone()) for _ in range(ncp - 1)]
        Ad = torch.from_numpy(A).to(dev)
        for M in sh.Ms:
            out = torch.empty((M, sh.N), dtype=torch.float16, device=dev)
            ws = w4.new_workspace(M, sh.K, sh.N, dev)
            Am = Ad[:M]

            def calls(i, Am=Am, out=out, ws=ws):
                p_, s_ = cps[i % len(cps)]
                w4.gemm(Am, p_, s_, sh.N, out=out, ws=ws, stream=stream)
            calls.n = steps
            us, queued = queued_batch(torch, stream, calls)
            D, F = algorithmic_bytes(M, sh.K, sh.N), flops(M, sh.K, sh.N)
            t_bound = max(D / (HBM_PEAK_GBPS * 1e3), F / (MFMA_F16_PEAK_TFLOPS * 1e6))
            rows.append({"shape": sh.name, "M": M, "K": sh.K, "N": sh.N, "us": round(us, 2),
                         "GBps": round(D / us / 1e3, 1),
                         "hbm_frac": round(D / us / 1e3 / HBM_PEAK_GBPS, 4),
                         "TFLOPs": round(F / us / 1e6, 1),
                         "roofline_frac": round(t_bound / us, 4),
                         "weight_copies_rotated": ncp, "queued_ahead_of_gpu": queued})
            log(f"{tag} {sh.name:16s} M={M:4d} {us:7.1f} us  {D / us / 1e3:6.0f} GB/s  "
                f"roofline {t_bound / us:5.1%}")
        del cps, pd, sd, Ad
        torch.cuda.empty_cache()
    return rows


def time_tp8_rank(w4, torch, dev, steps, stream):
    """One 8-way tensor-parallel rank's share of the Llama-2-70B block (the kernel at the
    local shapes a sharded layer runs), M = 16, 32, 128."""
    from workloads import LLAMA2_70B_TP8
    return time_shapes(w4, torch, dev, steps, stream, LLAMA2_70B_TP8, "tp8")


def time_layers(w4, torch, dev, steps, stream):
    """The Llama-2-7B block's layers at M = 1, 16, 64 and the Llama-2-70B block's at M = 16,
    32, 128 (the model-layer configurations of the benchmark's workload list)."""
    from workloads import LLAMA2_70B, LLAMA2_7B
    return {wl.name: time_shapes(w4, torch, dev, steps, stream, wl, "layer")
            for wl in (LLAMA2_7B, LLAMA2_70B)}


def stream_read_rate(w4, torch, dev, stream):
    """Context for the HBM fraction: the read rate of a plain streaming read (w4a16_read_probe:
    each workgroup one contiguous chunk, the fastest pattern measured) over 4 GiB, best of 5
    calls."""
    x = torch.empty(1 << 31, dtype=torch.float16, device=dev)
    x.fill_(1.0)
    out = torch.zeros(2048, dtype=torch.int32, device=dev)
    best = 0.0
    for _ in range(6):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        w4.read_probe(x, out=out, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        best = max(best, x.numel() * 2 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del x
    torch.cuda.empty_cache()
    return {"kernel": "w4a16_read_probe over 4 GiB (contiguous chunk per workgroup, 128-bit "
                      "non-temporal loads)",
            "GBps": round(best, 1), "frac_of_spec": round(best / HBM_PEAK_GBPS, 4)}


def _read(path, limit=400):
    try:
        with open(path) as f:
            return f.read(limit).strip()
    except OSError:
        return None


def gpu_sysfs_state(pci_bus_id=None):
    """Clocks, power cap and ECC state of the GPU from sysfs (amdgpu's files; reading them
    starts no process and does not touch the GPU).  The card is the one at `pci_bus_id`
    when known, else the only amdgpu card with clock tables."""
    import glob
    cards = []
    for dev in sorted(glob.glob("/sys/class/drm/card[0-9]*/device")):
        if os.path.exists(os.path.join(dev, "pp_dpm_sclk")):
            cards.append(dev)
    pick = None
    if pci_bus_id is not None:
        for dev in cards:
            if os.path.realpath(dev).lower().endswith(f":{pci_bus_id:02x}:00.0"):
                pick = dev
    if pick is None and len(cards) == 1:
        pick = cards[0]
    if pick is None:
        return {"sysfs": f"{len(cards)} amdgpu cards with clock tables, none matched"}

    def levels(table):
        # the DPM levels ("0: 500Mhz", ...); which one is current at the moment of reading
        # says nothing about the timed region, so it is not reported
        if not table:
            return None
        return [ln.strip().rstrip("*").strip() for ln in table.splitlines() if ln.strip()]

    state = {"card": os.path.realpath(pick).rsplit("/", 1)[-1],
             "sclk_levels": levels(_read(os.path.join(pick, "pp_dpm_sclk"))),
             "mclk_levels": levels(_read(os.path.join(pick, "pp_dpm_mclk")))}
    caps = sorted(glob.glob(os.path.join(pick, "hwmon", "hwmon*", "power1_cap")))
    if caps:
        cap = _read(caps[0])
        state["power_cap_w"] = int(cap) / 1e6 if cap and cap.isdigit() else cap
    feats = _read(os.path.join(pick, "ras", "features"))
    umc = _read(os.path.join(pick, "ras", "umc_err_count"))
    if feats is None and umc is None:
        # no per-device RAS files: the driver's module parameters (ras_enable -1 = auto,
        # 0 = off, 1 = on; ras_mask: the RAS blocks asked for, bit 0 = memory/UMC)
        par = "/sys/module/amdgpu/parameters"
        state["ecc"] = {"ras_files": "absent",
                        "amdgpu_ras_enable": _read(os.path.join(par, "ras_enable")),
                        "amdgpu_ras_mask": _read(os.path.join(par, "ras_mask"))}
    else:
        # RAS feature mask: bit 0 is the memory controller block (UMC), i.e. HBM ECC on
        mask = None
        if feats:
            for tok in feats.replace(":", " ").split():
                if tok.lower().startswith("0x"):
                    mask = int(tok, 16)
                    break
        state["ecc"] = {"ras_features": feats,
                        "hbm_ecc_enabled": None if mask is None else bool(mask & 1),
                        "umc_err_count": umc}
    return state


def host_state():
    """The host the CPU baseline runs on: CPU model and core counts."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count()
    return {"cpu_model": model, "host_cores": os.cpu_count(), "cores_allowed": allowed,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def oracle_threads(host):
    """Threads for the CPU baseline: every core this process may use, capped by
    OMP_NUM_THREADS where the environment sets the process's CPU share (the GPU machines give a
    one-GPU job 16 threads, whatever the host's core count)."""
    n = host["cores_allowed"] or 1
    omp = host["omp_num_threads"]
    if omp and omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return n


def device_state(torch, props, sysfs, host):
    """Software, device, clock, ECC and host state of the run."""
    return {"hip": getattr(torch.version, "hip", None), "torch": torch.__version__,
            "gpu": props.name, "arch": getattr(props, "gcnArchName", ""),
            "cus": props.multi_processor_count, "gpu_sysfs": sysfs, **host}


def mfma_rate(w4, torch, dev, stream):
    """Context for the compute-bound fraction: the sustained fp16 matrix rate on random
    operands (w4a16_mfma_probe: 1024 workgroups of 4 waves, 64 independent instructions per
    round), both instruction shapes, best of 3 launches each."""
    g = torch.Generator(device=dev).manual_seed(0)
    src = (torch.randn(1 << 20, device=dev, generator=g) * 0.5).half()
    res = {}
    for shape, name in ((0, "16x16x32"), (1, "32x32x16")):
        best = 0.0
        for _ in range(4):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            _, fl = w4.mfma_probe(src, shape=shape, workgroups=1024, iters=400, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            best = max(best, fl / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        res[name] = round(best, 1)
    del src
    return {"kernel": "w4a16_mfma_probe, random fp16 operands", "TFLOPs": res,
            "frac_of_spec": {k: round(v / MFMA_F16_PEAK_TFLOPS, 4) for k, v in res.items()}}


SHORT_NAMES = {
    "w4a16_gemm_skinny_kernel": "skinny",
    "w4a16_gemm_kernel": "stripe",
    "w4a16_gemm_wide_kernel": "wide",
}


def compose_line(args, value, ms_per_step, config, kernels, sweep, cpu, refs, state,
                 compute_sweep, details_path):
    """The one JSON line bench.py prints: headline, roofline of the dominant kernel and of
    each kernel of the sweep, the per-M sweep, the CPU baseline, reference rates and the run
    state.  Everything else goes to the details file (kept to a few KB so that a driver
    reading the tail of stdout gets the whole line)."""
    by_kernel = [{k: v for k, v in r.items() if k in ("kernel", "M", "bound", "achieved", "unit",
                                                      "frac", "traffic", "mean_launch_us")}
                 for r in kernels]
    line = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": config,
        "roofline": kernels[0],
        "roofline_by_kernel": by_kernel,
        "sweep": sweep,
        "compute_sweep": compute_sweep,
        "references": refs,
        "cpu_baseline": cpu,
        "run_state": state,
        "details": details_path,
    }
    return json.dumps(line, separators=(",", ":"))


ABLATION_MS = (1, 16, 32, 64, 128)


def run_ablation(args):
    """The pages' Figure 12 on this chip: the shipped library against measurement-only builds
    with one design choice undone each (build.py --ablation all), on the 72k x 18k weight,
    every call of every build alternated so all see the same clock and cache state.  Prints
    one JSON line of mean us per call and the ratio to the shipped build; checks that every
    build's output equals the shipped one bit for bit (the switches change speed, not
    results)."""
    import ctypes
    import torch
    import mixed_precision_w4a16_amd as w4
    from mixed_precision_w4a16_amd import build as B
    from workloads import LARGE, draw
    libs = {"shipped": w4.library()}
    for name in B.ABLATIONS:
        path = B.ablation_lib(name)
        if not os.path.exists(path):
            sys.exit(f"{path} is not built: python mixed_precision_w4a16_amd/build.py "
                     "--ablation all")
        lib = ctypes.CDLL(path)
        lib.w4a16_gemm.argtypes = w4.library().w4a16_gemm.argtypes
        lib.w4a16_gemm.restype = ctypes.c_int
        libs[name] = lib
    sh = LARGE.shapes[0]
    K, N = sh.K, sh.N
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    A, q, s = draw(K, N, max(ABLATION_MS), seed=0)
    pd, sd = w4.to_device(*w4.pack(q, s), dev)
    del q, s
    copies = [(pd, sd)] + [(pd.clone(), sd.clone()) for _ in range(args.copies - 1)]
    Ad = torch.from_numpy(A).to(dev)
    ws = w4.new_workspace(max(ABLATION_MS), K, N, dev)
    outs = {(v, M): torch.empty((M, N), dtype=torch.float16, device=dev)
            for v in libs for M in ABLATION_MS}
    stream = torch.cuda.current_stream(dev)
    n = [0]

    def call(v, M):
        p_, s_ = copies[n[0] % len(copies)]
        n[0] += 1
        rc = libs[v].w4a16_gemm(Ad.data_ptr(), p_.data_ptr(), s_.data_ptr(),
                                outs[(v, M)].data_ptr(), M, K, N, ws.data_ptr(),
                                stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"{v}: w4a16_gemm returned {rc}")

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.settle_s:
        for M in ABLATION_MS:
            for v in libs:
                call(v, M)
        torch.cuda.synchronize()
    for M in ABLATION_MS:
        ref = outs[("shipped", M)].cpu()
        for v in libs:
            if not torch.equal(outs[(v, M)].cpu().view(torch.int16), ref.view(torch.int16)):
                raise RuntimeError(f"ablation build {v} differs from the shipped one at M={M}")
    ev = {(v, M): [] for v in libs for M in ABLATION_MS}
    for _ in range(args.steps):
        for M in ABLATION_MS:
            for v in libs:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                call(v, M)
                e1.record(stream)
                ev[(v, M)].append((e0, e1))
    torch.cuda.synchronize()
    res = {}
    for M in ABLATION_MS:
        base = float(np.mean([a.elapsed_time(b) for a, b in ev[("shipped", M)]])) * 1e3
        kern = next(k for k, ms, _ in KERNELS if M in ms)
        row = {"kernel": kern, "shipped_us": round(base, 2),
               "shipped_hbm_frac": round(algorithmic_bytes(M, K, N) / base / 1e3 / HBM_PEAK_GBPS, 4)}
        for v in libs:
            if v == "shipped":
                continue
            us = float(np.mean([a.elapsed_time(b) for a, b in ev[(v, M)]])) * 1e3
            row[v] = {"us": round(us, 2), "time_vs_shipped": round(us / base, 3)}
        res[M] = row
        log(f"M={M:4d} shipped {base:7.1f} us  " + "  ".join(
            f"{v} x{row[v]['time_vs_shipped']:.3f}" for v in libs if v != "shipped"))
    print(json.dumps({"ablation": res, "workload": LARGE.name, "steps": args.steps,
                      "weight_copies_rotated": args.copies,
                      "builds": {v: os.path.basename(B.ablation_lib(v)) for v in B.ABLATIONS}}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-cols", type=int, default=65536,
                    help="columns of the CPU-baseline sample (0 skips it)")
    ap.add_argument("--copies", type=int, default=9,
                    help="weight copies rotated between calls: more copies than calls per step, "
                         "so no call finds its weights still in the 256 MB memory-side cache")
    ap.add_argument("--format-steps", type=int, default=20,
                    help="timed calls per M for each other packed format (0 skips them)")
    ap.add_argument("--moe-steps", type=int, default=20,
                    help="timed calls per token count of each MoE layer shape (0 skips them)")
    ap.add_argument("--extra-steps", type=int, default=20,
                    help="timed calls per M of the compute sweep, the tensor-parallel rank and the "
                         "model-layer shapes, plus the reference rates (0 skips them)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain fp16 copy kernel of known size (for counter scaling)")
    ap.add_argument("--details", default=os.path.join(ROOT, "gpurun_out", "bench_details.json"),
                    help="file for the sections not in the stdout line ('' skips it)")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="seconds of untimed sweep before the warm-up steps (0 under a counter "
                         "profiler, where every dispatch is slow)")
    ap.add_argument("--ablation", action="store_true",
                    help="instead of the benchmark: the shipped library against the "
                         "measurement-only builds (build.py --ablation all), M = 1..128")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.ablation:
        run_ablation(args)
        return

    host = host_state()
    import torch
    import mixed_precision_w4a16_amd as w4
    from workloads import LARGE, draw

    shape = LARGE.shapes[0]
    K, N, Ms = shape.K, shape.N, shape.Ms
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")
    state = device_state(torch, props, gpu_sysfs_state(getattr(props, "pci_bus_id", None)), host)
    log(f"run state: {json.dumps(state)}")

    t = time.perf_counter()
    A, q, s = draw(K, N, max(Ms), seed=0, sigma=shape.sigma)
    packed, sp = w4.pack(q, s)
    log(f"inputs drawn and packed in {time.perf_counter() - t:.1f} s")
    pd, sd = w4.to_device(packed, sp, dev)
    del packed, sp
    copies = [(pd, sd)] + [(pd.clone(), sd.clone()) for _ in range(args.copies - 1)]
    Ad = torch.from_numpy(A).to(dev)
    outs = {M: torch.empty((M, N), dtype=torch.float16, device=dev) for M in Ms}
    ws = w4.new_workspace(max(Ms), K, N, dev)
    stream = torch.cuda.current_stream(dev)

    ncall = [0]

    def call(M):
        p_, s_ = copies[ncall[0] % len(copies)]
        ncall[0] += 1
        w4.gemm(Ad[:M], p_, s_, N, out=outs[M], ws=ws, stream=stream)

    # Settle: untimed sweep steps for SETTLE_S seconds before the W warm-up steps.  Under a
    # sustained load the GPU's clocks take about a tenth of a second to reach their steady
    # state; without this the first timed steps of a short run (5 warm-up steps are ~7 ms)
    # run at the ramping clock.
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for M in Ms:
            call(M)
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        for M in Ms:
            call(M)
    torch.cuda.synchronize()

    # Timed region: K steps, each one call per M, with a HIP event pair around every call
    # on the stream the kernels run on.
    ev = {M: [] for M in Ms}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for M in Ms:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call(M)
            e1.record(stream)
            ev[M].append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    if args.calib_copy:
        # a plain elementwise kernel that reads CALIB_BYTES and writes CALIB_BYTES
        x = torch.ones(CALIB_BYTES // 2, dtype=torch.float16, device=dev)
        y = torch.empty_like(x)
        for _ in range(2):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        del x, y

    sweep = []
    tot_bytes = 0.0
    for M in Ms:
        us = float(np.mean([a.elapsed_time(b) for a, b in ev[M]])) * 1e3
        D, D16, F = algorithmic_bytes(M, K, N), fp16_weight_bytes(M, K, N), flops(M, K, N)
        t_bound = max(D / (HBM_PEAK_GBPS * 1e3), F / (MFMA_F16_PEAK_TFLOPS * 1e6))   # us
        gbps = D / us / 1e3
        sweep.append({
            "M": M, "us": round(us, 2), "GBps": round(gbps, 1),
            "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "TFLOPs": round(F / us / 1e6, 1),
            "mfma_frac": round(F / us / 1e6 / MFMA_F16_PEAK_TFLOPS, 4),
            "roofline_frac": round(t_bound / us, 4),
            "x_fp16_bound": round(D16 / (HBM_PEAK_GBPS * 1e3) / us, 3),
        })
        tot_bytes += D
        log(f"M={M:4d}  {us:8.1f} us  {gbps:7.0f} GB/s ({gbps / HBM_PEAK_GBPS:5.1%} HBM)  "
            f"{F / us / 1e6:7.1f} TFLOP/s  roofline {t_bound / us:5.1%}  "
            f"vs fp16 bound {D16 / (HBM_PEAK_GBPS * 1e3) / us:4.2f}x")

    ms_per_step = wall / args.steps * 1e3
    value = tot_bytes * args.steps / wall / 1e9
    traffic = measured_traffic()
    by_M = {row["M"]: row for row in sweep}

    def roof(name, ms, bound):
        ms = [m for m in ms if m in by_M]
        us = float(np.mean([by_M[m]["us"] for m in ms]))
        if bound == "hbm":
            a = float(np.mean([algorithmic_bytes(m, K, N) for m in ms])) / us / 1e3
            peak, unit = HBM_PEAK_GBPS, "GB/s"
        else:
            a = float(np.mean([flops(m, K, N) for m in ms])) / us / 1e6
            peak, unit = MFMA_F16_PEAK_TFLOPS, "TFLOP/s"
        tb = None
        if traffic is not None:
            tb = float(np.mean([traffic["per_M"][str(m)]["hbm_bytes"] for m in ms]))
        return {"bound": bound, "achieved": round(a, 1), "peak": peak, "unit": unit,
                "frac": round(a / peak, 4), "traffic": tb, "kernel": name, "M": ms,
                "mean_launch_us": round(us, 2)}

    kernels = [roof(*k) for k in KERNELS]
    details = {"sweep_traffic_source": None if traffic is None else os.path.relpath(TRAFFIC_FILE, ROOT)}
    if traffic is not None:
        details["hbm_bytes_measured_by_M"] = {m: traffic["per_M"][str(m)]["hbm_bytes"] for m in Ms}

    if args.format_steps > 0:
        details["repack"] = time_repack(w4, torch, dev, K, N, 10, stream)
        details["sparse_24"] = time_sparse(w4, torch, dev, Ad, q, s, K, N, Ms, args.format_steps,
                                           max(2, args.warmup // 4), args.copies, stream, copies)
    if args.moe_steps > 0:
        details["moe"] = time_moe(w4, torch, dev, args.moe_steps, stream)
    refs = None
    compute_sweep = None
    if args.extra_steps > 0:
        compute_sweep = time_compute_sweep(w4, torch, dev, args.extra_steps, stream)
        details["compute_sweep"] = compute_sweep
        details["tp8_rank_shapes"] = time_tp8_rank(w4, torch, dev, args.extra_steps, stream)
        details["layer_shapes"] = time_layers(w4, torch, dev, args.extra_steps, stream)
        sref = stream_read_rate(w4, torch, dev, stream)
        mref = mfma_rate(w4, torch, dev, stream)
        log(f"stream read reference: {sref}")
        log(f"MFMA reference: {mref}")
        refs = {"stream_read_GBps": sref["GBps"], "stream_read_frac_of_spec": sref["frac_of_spec"],
                "mfma_f16_TFLOPs": mref["TFLOPs"], "mfma_f16_frac_of_spec": mref["frac_of_spec"]}
        details["stream_read_reference"] = sref
        details["mfma_reference"] = mref
        compute_sweep = [{k: r[k] for k in ("M", "us", "TFLOPs", "mfma_frac")} for r in compute_sweep]
    fp16 = None
    if args.extra_steps > 0:
        del copies
        torch.cuda.empty_cache()
        fp16 = time_fp16_gemm(torch, dev, Ad, q, s, Ms, args.extra_steps, stream,
                              {r["M"]: r["us"] for r in sweep})
        details["fp16_gemm_baseline"] = fp16
        copies = [(pd, sd)] + [(pd.clone(), sd.clone()) for _ in range(args.copies - 1)]
    if args.format_steps > 0:
        details["formats"] = time_formats(w4, torch, dev, Ad, q, s, K, N, args.format_steps,
                                          max(2, args.warmup // 4), args.copies, stream, copies)
    del copies, pd, sd, Ad, outs, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    cpu = None
    if args.cpu_cols > 0:
        cpu = cpu_baseline(A, q, s, Ms, args.cpu_cols, oracle_threads(host))
        cpu.update(cpu_model=host["cpu_model"], host_cores=host["host_cores"])
        log(f"cpu baseline: {cpu}")
    config = {"workload": LARGE.name, "K": K, "N": N, "M": list(Ms), "group": GROUP,
              "weights": "int4 codes + fp16 scales (4.125 bits/weight)",
              "weight_copies_rotated": args.copies, "untimed_settle_s": round(settle_s, 2)}
    details_path = None
    if args.details:
        os.makedirs(os.path.dirname(os.path.abspath(args.details)), exist_ok=True)
        with open(args.details, "w") as f:
            json.dump({"config": config, "sweep": sweep, "roofline_by_kernel": kernels,
                       **details}, f, indent=1)
        details_path = os.path.relpath(os.path.abspath(args.details), ROOT)
        log(f"details written to {details_path}")
    if fp16 is not None:
        for row, f in zip(sweep, fp16):
            row["x_fp16_gemm"] = f["speedup"]
    print(compose_line(args, round(value, 1), round(ms_per_step, 4), config, kernels, sweep, cpu,
                       refs, state, compute_sweep, details_path), flush=True)


if __name__ == "__main__":
    main()

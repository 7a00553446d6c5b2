"""Seeded synthetic inputs and the layer shapes they are drawn for.

Shared by the tests, the smoke check and the benchmark.  This module holds no part of the
layer's arithmetic: it only draws codes, scales and activations and names shapes.

Distributions (the same for every shape):
  codes  q  ~ uniform integers 0..15 (uint8, one code per byte, [K, N] row-major)
  scales s  ~ uniform [0.005, 0.02], rounded to fp16 ([K/group, N] row-major)
  A         ~ N(0, sigma^2) drawn in fp32, rounded to fp16 ([M, K] row-major)
Draw order per weight shape: q, then s, then A (largest M; smaller M use the leading rows),
all from one ``numpy.random.default_rng(seed)`` stream.

The shapes stand in for the pages' workloads: one 72k x 18k weight at group 128 (the MARLIN
paper's Figure 1 layer, read as K = 18432 reduction rows by N = 73728 output columns) and
Llama-2-7B / Llama-2-70B decoder-block linears (the per-layer benchmarks at batch 16).
No model weights or datasets are used: only the shapes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GROUP = 128


@dataclass(frozen=True)
class Shape:
    name: str
    K: int
    N: int
    Ms: tuple
    sigma: float = 1.0


@dataclass(frozen=True)
class Workload:
    name: str
    shapes: tuple = field(default_factory=tuple)


SMALL = Workload("single_1024x1024_m16", (Shape("1024x1024", 1024, 1024, (16,)),))

LARGE = Workload("single_72kx18k_m1_128", (
    Shape("18432x73728", 18432, 73728, (1, 2, 4, 8, 16, 32, 64, 128)),))

LLAMA2_7B = Workload("llama2_7b_block_m1_16_64", (
    Shape("7b_qkv", 4096, 12288, (1, 16, 64)),
    Shape("7b_o", 4096, 4096, (1, 16, 64)),
    Shape("7b_gate_up", 4096, 22016, (1, 16, 64)),
    Shape("7b_down", 11008, 4096, (1, 16, 64)),
))

LLAMA2_70B = Workload("llama2_70b_block_m16_32_128", (
    Shape("70b_qkv", 8192, 10240, (16, 32, 128)),
    Shape("70b_o", 8192, 8192, (16, 32, 128)),
    Shape("70b_gate_up", 8192, 57344, (16, 32, 128)),
    Shape("70b_down", 28672, 8192, (16, 32, 128)),
))

# One rank's share of the Llama-2-70B block under 8-way tensor parallelism (column-parallel
# qkv and gate+up split N, row-parallel o and down split K): the kernel at the local shapes.
LLAMA2_70B_TP8 = Workload("llama2_70b_tp8_rank_m16_32_128", (
    Shape("70b_tp8_qkv", 8192, 1280, (16, 32, 128)),
    Shape("70b_tp8_o", 1024, 8192, (16, 32, 128)),
    Shape("70b_tp8_gate_up", 8192, 7168, (16, 32, 128)),
    Shape("70b_tp8_down", 3584, 8192, (16, 32, 128)),
))

COMPUTE_SWEEP = Workload("compute_8192x28672_m256_1024", (
    Shape("8192x28672", 8192, 28672, (256, 512, 1024), sigma=0.5),))

ALL = (SMALL, LARGE, LLAMA2_7B, LLAMA2_70B, COMPUTE_SWEEP)


@dataclass(frozen=True)
class MoeShape:
    name: str
    E: int          # experts
    topk: int       # experts per token
    K: int
    N: int
    Ts: tuple       # tokens per call


# Mixture-of-experts layers (the pages name the case, not a model): experts shaped like a
# Mixtral-8x7B block (8 experts, top-2, hidden 4096, expert width 14336; gate and up fused)
# and like a 64-expert, top-6 block with hidden 2048 and expert width 1408.
MOE_8E = Workload("moe_8e_top2_4096", (
    MoeShape("8e_gate_up", 8, 2, 4096, 28672, (1, 4, 16, 64)),
    MoeShape("8e_down", 8, 2, 14336, 4096, (1, 4, 16, 64)),
))
MOE_64E = Workload("moe_64e_top6_2048", (
    MoeShape("64e_gate_up", 64, 6, 2048, 2816, (1, 4, 16, 64)),
    MoeShape("64e_down", 64, 6, 1408, 2048, (1, 4, 16, 64)),
))


def draw(K: int, N: int, M: int, seed: int = 0, sigma: float = 1.0, group: int = GROUP):
    """Return (A fp16 [M,K], q uint8 [K,N], s fp16 [K/group,N]) from one seeded stream."""
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    s = rng.uniform(0.005, 0.02, size=(K // group, N)).astype(np.float16)
    A = (rng.standard_normal((M, K), dtype=np.float32) * np.float32(sigma)).astype(np.float16)
    return A, q, s


def draw_zeros(K: int, N: int, seed: int = 0, group: int = GROUP) -> np.ndarray:
    """Zero points z ~ U{0..15} per (group, column), uint8 [K/group, N], from a stream of their
    own (numpy.random.default_rng([seed, 1])), so the draws of ``draw`` are unchanged."""
    rng = np.random.default_rng([seed, 1])
    return rng.integers(0, 16, size=(K // group, N), dtype=np.uint8)


def draw_shape(shape: Shape, seed: int = 0, group: int = GROUP):
    """Inputs for every M of a shape: A has max(Ms) rows; M uses A[:M]."""
    return draw(shape.K, shape.N, max(shape.Ms), seed=seed, sigma=shape.sigma, group=group)


# The six ways to keep 2 of 4 positions.
_PAIRS_24 = np.array([[1, 1, 0, 0], [1, 0, 1, 0], [1, 0, 0, 1], [0, 1, 1, 0], [0, 1, 0, 1],
                      [0, 0, 1, 1]], dtype=bool)


def sparsify_24(q: np.ndarray, seed: int = 0) -> np.ndarray:
    """2:4 structure along K: in every aligned group of 4 rows of each column two positions,
    drawn uniformly from the six pairs (numpy.random.default_rng([seed, 2])), keep their code
    and the other two become 8 (weight 0).  Returns a new uint8 [K, N]."""
    K, N = q.shape
    if K % 4:
        raise ValueError("K must be a multiple of 4")
    rng = np.random.default_rng([seed, 2])
    out = np.array(q, dtype=np.uint8, copy=True)
    step = 4096                                    # rows per chunk, to bound the mask's memory
    for k0 in range(0, K, step):
        rows = min(step, K - k0)
        pick = rng.integers(0, 6, size=(rows // 4, N), dtype=np.uint8)
        keep = _PAIRS_24[pick].transpose(0, 2, 1).reshape(rows, N)     # [rows, N]
        blk = out[k0:k0 + rows]
        blk[~keep] = 8
    return out


def to_act(x: np.ndarray, act: str):
    """Round float32 draws to the activation type: (16-bit patterns uint16, values float64).
    fp16 by numpy's cast, bf16 by torch's (both round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if act == "f16":
        h = x.astype(np.float16)
        return h.view(np.uint16), h.astype(np.float64)
    if act == "bf16":
        import torch
        b = torch.from_numpy(x).to(torch.bfloat16)
        bits = b.view(torch.int16).numpy().view(np.uint16).copy()
        return bits, b.to(torch.float64).numpy()
    raise ValueError(act)


def draw_moe(E: int, topk: int, K: int, N: int, T: int, seed: int = 0, act: str = "f16",
             zero_points: bool = False, group: int = GROUP) -> dict:
    """Inputs of one MoE layer call, from numpy.random.default_rng([seed, 3]):
      q [E, K, N] ~ U{0..15}; scales [E, K/group, N] ~ U[0.005, 0.02]; A [T, K] ~ N(0, 1);
      router: logits [T, E] ~ N(0, 1) plus a per-expert N(0, 1/4) offset (some experts are
      picked more often than others, as with a trained router); each token takes its topk
      largest; row_scale [T*topk] ~ U[0.1, 1] (router weights); zero points ~ U{0..15}.
    A and the scales are rounded to the activation type ("f16" or "bf16")."""
    rng = np.random.default_rng([seed, 3])
    q = rng.integers(0, 16, size=(E, K, N), dtype=np.uint8)
    s32 = rng.uniform(0.005, 0.02, size=(E, K // group, N)).astype(np.float32)
    A32 = rng.standard_normal((T, K), dtype=np.float32)
    logits = rng.standard_normal((T, E)) + 0.5 * rng.standard_normal(E)
    topk_ids = np.argsort(-logits, axis=1, kind="stable")[:, :topk].astype(np.int32)
    row_scale = rng.uniform(0.1, 1.0, size=T * topk).astype(np.float32)
    z = rng.integers(0, 16, size=(E, K // group, N), dtype=np.uint8) if zero_points else None
    A_bits, A = to_act(A32, act)
    s_bits, s = to_act(s32, act)
    return {"A": A, "A_bits": A_bits, "q": q, "s": s, "s_bits": s_bits, "zeros": z,
            "topk_ids": topk_ids, "row_scale": row_scale, "act": act}

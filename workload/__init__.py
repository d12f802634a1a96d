"""Seeded synthetic inputs for the SwiGLU MLP training step.

This module is shared by the fp64 oracle (``oracle/``) and by the HIP path's
tests and benchmark.  It holds shapes, value distributions and a seeded
bf16 generator, and none of the MLP's arithmetic: no products, no
activations, no gradients.

Shapes are (M tokens, D model dim, I intermediate dim, Dout output dim).
The weight layouts follow the note "SwiGLU MLP forward principle, backward
chain and optimisation" (section 1, forward): ``W1`` is ``[D, 2I]`` with
columns ``[0, I)`` the un-gated ("left", up) branch and ``[I, 2I)`` the gate
branch, and ``W_down`` is ``[I, Dout]``.

Distributions: ``N(0, s)`` means mean 0 and *standard deviation* s.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 1234
# one seed offset per tensor, so every tensor is reproducible on its own
SEED_X, SEED_W1, SEED_WD, SEED_DY = 0, 1, 2, 3
# expert routing of the MoE workloads; expert e's weights use seed offsets
# SEED_W1 + 16 * (e + 1) and SEED_WD + 16 * (e + 1)
SEED_ROUTE = 4


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    D: int
    I: int
    Dout: int
    x_std: float
    w1_std: float
    wd_std: float
    dy_std: float
    gate_scale: float = 1.0   # multiplies W1's gate half [I, 2I) after rounding
    fwd_only: bool = False
    note: str = field(default="", compare=False)


def _fan_in(n: int) -> float:
    return 1.0 / float(np.sqrt(n))


# The five workloads the pages' method is exercised on.  The target shape
# [M, D, H, Dout] = [11136, 3584, 14336, 3584] is the one the drop-h report
# times its MLP block on (performance table); the others are a tiny
# correctness case, a small 8/3-sized MLP, a Llama-like MLP with an
# intermediate size of 11008 whose gate half is stretched so that sigmoid
# saturates, and a decode-shaped forward of 16 tokens.
WORKLOADS = {
    "tiny": Workload("tiny", 128, 256, 512, 256,
                     1.0, _fan_in(256), _fan_in(512), 1.0,
                     note="correctness case; full oracle in seconds"),
    "small": Workload("small", 2048, 1024, 2816, 1024,
                      1.0, _fan_in(1024), _fan_in(2816), 1.0,
                      note="I = 8/3 * D rounded up to a multiple of 128"),
    "target": Workload("target", 11136, 3584, 14336, 3584,
                       1.0, 0.02, 0.02, 0.01,
                       note="the drop-h report's target shape"),
    "llama": Workload("llama", 8192, 4096, 11008, 4096,
                      1.0, _fan_in(4096), _fan_in(11008), 1.0,
                      gate_scale=8.0,
                      note="gate half of W1 x8: |gate| reaches ~30, sigmoid saturates"),
    "decode": Workload("decode", 16, 4096, 14336, 4096,
                       1.0, 0.02, 0.02, 0.0, fwd_only=True,
                       note="decode-shaped forward, weight-streaming bound"),
}


def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, round to nearest, ties to even.

    Non-finite values never arise from the generator (finite normals)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> exact fp32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> exact fp64 values."""
    return bf16_bits_to_f32(b).astype(np.float64)


def normal_bf16(shape, std: float, seed: int) -> np.ndarray:
    """Seeded N(0, std) samples drawn in fp32 (PCG64), rounded RNE to bf16.

    Returns the uint16 bit patterns, C-contiguous (row-major)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return round_to_bf16_bits(v)


def scale_pow2_bf16(bits: np.ndarray, factor: float) -> np.ndarray:
    """Multiply bf16 values by a power of two (exact unless it overflows)."""
    m, e = np.frexp(factor)
    assert m == 0.5, "only powers of two keep bf16 values exact"
    return round_to_bf16_bits(bf16_bits_to_f32(bits) * np.float32(factor))


def make_inputs(w: Workload, seed: int = BASE_SEED, M: int | None = None):
    """bf16 bit patterns for x [M,D], W1 [D,2I], W_down [I,Dout], dy [M,Dout].

    ``M`` may override the workload's token count (same distributions); the
    weights do not depend on it.  ``dy`` is None for forward-only workloads.
    """
    M = w.M if M is None else M
    x = normal_bf16((M, w.D), w.x_std, seed + SEED_X)
    W1 = normal_bf16((w.D, 2 * w.I), w.w1_std, seed + SEED_W1)
    if w.gate_scale != 1.0:
        W1 = W1.copy()
        W1[:, w.I:] = scale_pow2_bf16(W1[:, w.I:], w.gate_scale)
    Wd = normal_bf16((w.I, w.Dout), w.wd_std, seed + SEED_WD)
    dy = None if w.fwd_only else normal_bf16((M, w.Dout), w.dy_std, seed + SEED_DY)
    return x, W1, Wd, dy


def make_custom(M: int, D: int, I: int, Dout: int, seed: int = BASE_SEED,
                x_std: float = 1.0, dy_std: float = 1.0, gate_scale: float = 1.0):
    """Inputs for an arbitrary shape with the fan-in rule used by the tiny
    and small workloads."""
    w = Workload("custom", M, D, I, Dout, x_std, _fan_in(D), _fan_in(I), dy_std,
                 gate_scale=gate_scale)
    return make_inputs(w, seed)


# ---------------------------------------------------------------------------
# Mixture-of-experts workloads ("Lesson 24", sections 41-43): every expert is
# its own SwiGLU MLP block, tokens are routed to top_k experts each, and the
# routed rows arrive sorted and packed by expert, so that expert e owns rows
# [offsets[e], offsets[e+1]).  Routing itself is not modelled: the expert of
# each routed row is drawn from a skewed (Zipf-like) popularity, which gives
# the uneven per-expert token counts the grouped GEMM is for.  The routed
# rows of x and dy are independent draws (the GEMMs do not care whether two
# rows are copies of one token).
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class MoEWorkload:
    name: str
    tokens: int       # tokens before routing
    top_k: int        # experts per token
    experts: int
    D: int
    I: int            # each expert's intermediate size
    Dout: int
    x_std: float
    w1_std: float
    wd_std: float
    dy_std: float
    skew: float       # popularity of the r-th most popular expert ~ 1 / r**skew
    note: str = field(default="", compare=False)

    @property
    def M(self) -> int:
        """Routed rows: tokens * top_k."""
        return self.tokens * self.top_k


MOE_WORKLOADS = {
    "moe_tiny": MoEWorkload("moe_tiny", 160, 2, 8, 256, 256, 256,
                            1.0, _fan_in(256), _fan_in(256), 1.0, skew=1.0,
                            note="correctness case; full oracle in seconds"),
    "moe": MoEWorkload("moe", 8192, 2, 16, 3584, 2048, 3584,
                       1.0, _fan_in(3584), _fan_in(2048), 1.0, skew=0.8,
                       note="16 experts of width 2048 on the target model dimension, top-2 routing"),
}


def expert_counts(tokens: int, top_k: int, experts: int, skew: float, seed: int = BASE_SEED) -> np.ndarray:
    """Routed rows per expert: each token picks top_k distinct experts, drawn
    without replacement from a Zipf-like popularity over a seeded random
    order of the experts (Gumbel top-k).  Returns int64 [experts] summing to
    tokens * top_k."""
    if not 1 <= top_k <= experts:
        raise ValueError("need 1 <= top_k <= experts")
    rng = np.random.Generator(np.random.PCG64(seed + SEED_ROUTE))
    p = 1.0 / np.arange(1, experts + 1, dtype=np.float64) ** skew
    p = p[rng.permutation(experts)]
    keys = np.log(p)[None, :] + rng.gumbel(size=(tokens, experts))
    chosen = np.argpartition(-keys, top_k - 1, axis=1)[:, :top_k]
    return np.bincount(chosen.ravel(), minlength=experts).astype(np.int64)


def group_offsets(counts) -> np.ndarray:
    """int32 [E + 1] row offsets of the expert-packed rows: 0, c0, c0 + c1, ..."""
    counts = np.asarray(counts, dtype=np.int64)
    if np.any(counts < 0):
        raise ValueError("negative count")
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def make_moe_inputs(w: MoEWorkload, seed: int = BASE_SEED, weight_sets: int | None = None, counts=None):
    """bf16 bit patterns for x [M, D], W1 [E, D, 2I], W_down [E, I, Dout],
    dy [M, Dout], and the int32 offsets [E + 1], with M = tokens * top_k.

    ``weight_sets`` < E draws that many distinct expert weight sets and gives
    expert e the set e % weight_sets (a timing shortcut: the values keep the
    same distribution); by default every expert has its own.  ``counts``
    overrides the routed rows per expert."""
    if counts is None:
        counts = expert_counts(w.tokens, w.top_k, w.experts, w.skew, seed)
    counts = np.asarray(counts, dtype=np.int64)
    if counts.shape != (w.experts,):
        raise ValueError("one count per expert")
    M = int(counts.sum())
    nsets = w.experts if weight_sets is None else max(1, min(int(weight_sets), w.experts))
    x = normal_bf16((M, w.D), w.x_std, seed + SEED_X)
    dy = normal_bf16((M, w.Dout), w.dy_std, seed + SEED_DY)
    W1 = np.empty((w.experts, w.D, 2 * w.I), dtype=np.uint16)
    Wd = np.empty((w.experts, w.I, w.Dout), dtype=np.uint16)
    for e in range(nsets):
        W1[e] = normal_bf16((w.D, 2 * w.I), w.w1_std, seed + SEED_W1 + 16 * (e + 1))
        Wd[e] = normal_bf16((w.I, w.Dout), w.wd_std, seed + SEED_WD + 16 * (e + 1))
    for e in range(nsets, w.experts):
        W1[e] = W1[e % nsets]
        Wd[e] = Wd[e % nsets]
    return x, W1, Wd, dy, group_offsets(counts)

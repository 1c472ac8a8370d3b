"""Seeded synthetic workloads for MoE dispatch/combine.

This module only draws inputs: it holds none of the routing, layout,
quantisation or combine arithmetic, and both the CPU oracle (through the tests)
and the HIP library (through the tests and the benchmark) take their inputs
from it.

The shapes are the pages' workloads:
  * DeepSeek-V3-shaped prefill, 4096 tokens x hidden 7168, top-4 groups then
    top-8 experts, FP8 dispatch and BF16 combine ("DeepSeek, DeepEP
    open-sourced", GeekNews 19421, section "Performance > Normal kernels");
  * 128-token low-latency decode (same page, "Performance > Low-latency
    kernels");
  * 8K tokens per batch (DeepEP V2 digest, section "performance measurement
    results"), here with a Zipf-skewed router to stress hot experts;
  * Mixtral-8x7B-shaped softmax top-2 (Perplexity "Efficient and Portable
    Mixture-of-Experts Communication", section "Introduction" names Mixtral
    8x7B), and a tiny case the oracle finishes instantly.
DeepSeek-V3 uses 256 routed experts in 8 groups; the pages give 4096 x 7168
top-8 with top-4 groups, the expert and group counts are the model's.

Expert-MLP workloads (the step between dispatch and combine; Mega MoE news
page): FP8 E4M3FN operands with power-of-two block scales drawn directly as
bit patterns (sign, exponent field and mantissa uniform over a range), never
by quantising real numbers, and per-expert row counts drawn multinomially.
The expert width I is not on the pages: 2048 (DeepSeek-V3's) is our choice.

Recipe: numpy ``default_rng(seed)`` streams; x ~ N(0,1) and y ~ N(0,1) drawn
in fp32 and rounded to bf16 (nearest-even on the bit pattern); router logits
~ N(0,1) fp32.  Sub-streams: x = seed, logits = seed+1, y = seed+2, Zipf
permutation = seed+3.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int                  # tokens
    H: int                  # hidden size
    E: int                  # experts
    G: int                  # expert groups
    g: int                  # groups kept per token
    k: int                  # experts per token
    score: str              # "sigmoid" | "softmax"
    R: int                  # virtual ranks (contiguous blocks of E/R experts)
    dtype: str              # dispatch dtype: "fp8" (E4M3FN, 1x128 scales) | "bf16"
    capacity: int = 0       # 0: compact receive buffer; >0: padded slots per expert
    skew: bool = False      # Zipf(1.2) per-expert bias on the logits
    seed: int = 0

    @property
    def N(self) -> int:
        return self.E * self.capacity if self.capacity > 0 else self.T * self.k

    @property
    def S(self) -> int:
        return self.H // 128

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", T=64, H=256, E=16, G=4, g=2, k=2, score="sigmoid", R=4,
                     dtype="fp8"),
    "dsv3_prefill": Workload("dsv3_prefill", T=4096, H=7168, E=256, G=8, g=4, k=8,
                             score="sigmoid", R=32, dtype="fp8"),
    "ll_decode": Workload("ll_decode", T=128, H=7168, E=256, G=8, g=4, k=8,
                          score="sigmoid", R=32, dtype="fp8", capacity=128),
    "mixtral": Workload("mixtral", T=16384, H=4096, E=8, G=1, g=1, k=2, score="softmax",
                        R=8, dtype="bf16"),
    "skewed_8k": Workload("skewed_8k", T=8192, H=7168, E=256, G=8, g=4, k=8,
                          score="sigmoid", R=32, dtype="fp8", skew=True),
}

# Bias scale for the skewed workload: chosen by bisection (tests/golden/
# calibrate_skew.py, which routes with the oracle) so that on the seed-0 draw
# the hottest expert receives 10x the mean load T*k/E.
SKEW_BETA = 0.2998046875
ZIPF_ALPHA = 1.2


def get(name: str) -> Workload:
    return WORKLOADS[name]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); uint16 patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def gen_x(wl: Workload) -> np.ndarray:
    rng = np.random.default_rng(wl.seed)
    return f32_to_bf16_bits(rng.standard_normal((wl.T, wl.H), dtype=np.float32))


def zipf_bias(wl: Workload, beta: float = SKEW_BETA) -> np.ndarray:
    """b_e = beta * ln(p_e / mean p), p_e ~ (perm(e)+1)^-alpha (float32 [E])."""
    rng = np.random.default_rng(wl.seed + 3)
    perm = rng.permutation(wl.E)
    p = (perm + 1.0) ** -ZIPF_ALPHA
    return (beta * np.log(p / p.mean())).astype(np.float32)


def gen_logits(wl: Workload, beta: float | None = None) -> np.ndarray:
    rng = np.random.default_rng(wl.seed + 1)
    logits = rng.standard_normal((wl.T, wl.E), dtype=np.float32)
    if wl.skew:
        logits = (logits + zipf_bias(wl, SKEW_BETA if beta is None else beta)[None, :]).astype(
            np.float32)
    return logits


def gen_y(wl: Workload, rows: int | None = None) -> np.ndarray:
    """Synthetic expert outputs, bf16 [N,H] (the expert MLP is not on this path)."""
    rng = np.random.default_rng(wl.seed + 2)
    n = wl.N if rows is None else rows
    return f32_to_bf16_bits(rng.standard_normal((n, wl.H), dtype=np.float32))


def tie_heavy(logits: np.ndarray) -> np.ndarray:
    """Correctness-only variant: logits rounded to multiples of 1/8 (many ties)."""
    return (np.round(logits * 8.0) / 8.0).astype(np.float32)


def custom(name: str = "custom", **kw) -> Workload:
    return Workload(name=name, **kw)


def algorithmic_bytes(wl: Workload) -> dict:
    """Bytes each step must move (inputs read once, outputs written once)."""
    T, H, k, E, S = wl.T, wl.H, wl.k, wl.E, wl.S
    pairs = T * k
    if wl.capacity > 0:
        rows = pairs  # only routed pairs are written/read (upper bound when nothing drops)
    else:
        rows = pairs
    route = T * E * 4 + pairs * 8
    layout = pairs * 4 + (E * 3 + wl.R * 2 + 2) * 4 + pairs * 4 + rows * 4 + (
        wl.N * 4 if wl.capacity > 0 else 0)
    if wl.dtype == "fp8":
        dispatch = T * H * 2 + rows * H + rows * S * 4 + pairs * 4
    else:
        dispatch = T * H * 2 + rows * H * 2 + pairs * 4
    combine = rows * H * 2 + T * H * 2 + pairs * 8
    # backward: grad_out read, y rows read, grad_y rows written, pos/w read,
    # grad_w written; dispatch's backward is a combine with unit weights
    combine_backward = T * H * 2 + 2 * rows * H * 2 + pairs * 12
    dispatch_backward = rows * H * 2 + T * H * 2 + pairs * 4
    return dict(route=route, layout=layout, dispatch=dispatch, combine=combine,
                total=route + layout + dispatch + combine,
                combine_backward=combine_backward, dispatch_backward=dispatch_backward)


def describe(wl: Workload) -> str:
    return (f"{wl.name}: T={wl.T} H={wl.H} E={wl.E} G={wl.G}/g={wl.g} k={wl.k} {wl.score} "
            f"R={wl.R} {wl.dtype} " + (f"padded C={wl.capacity}" if wl.capacity else "compact")
            + (" zipf" if wl.skew else ""))


__all__ = ["Workload", "WORKLOADS", "get", "gen_x", "gen_logits", "gen_y", "tie_heavy",
           "f32_to_bf16_bits", "bf16_bits_to_f32", "zipf_bias", "algorithmic_bytes",
           "describe", "SKEW_BETA", "custom"]


# --------------------------------------------------------------------------
# expert MLP inputs
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class MlpWorkload:
    name: str
    N: int          # receive rows
    H: int          # hidden size
    I: int          # expert intermediate size
    E: int          # experts whose rows are in the buffer
    align: int = 0  # expert regions start on multiples of this many rows (0: packed)
    seed: int = 0

    def replace(self, **kw) -> "MlpWorkload":
        return dataclasses.replace(self, **kw)


MLP_WORKLOADS = {
    "mlp_tiny": MlpWorkload("mlp_tiny", N=300, H=256, I=256, E=3),
    # one rank of a 32-rank expert-parallel DeepSeek-V3 layer: 8 local experts
    # receive 32 ranks x 4096 tokens x top-8 / 32 = 32768 rows
    "mlp_rank": MlpWorkload("mlp_rank", N=32768, H=7168, I=2048, E=8),
    # the single-GPU receive buffer of dsv3_prefill: 256 experts, 32768 rows
    "mlp_all": MlpWorkload("mlp_all", N=32768, H=7168, I=2048, E=256),
    # one rank at decode: 32 ranks x 128 tokens x top-8 / 32 = 1024 rows over the
    # 8 local experts (~128 each): the weights dominate the bytes
    "mlp_decode": MlpWorkload("mlp_decode", N=1024, H=7168, I=2048, E=8),
}


def mlp_ranges(wl: MlpWorkload):
    """Per-expert row counts (multinomial, seed+10) and region starts: (start,
    count, rows_needed) int32; with align > 1 each start is a multiple of align."""
    rng = np.random.default_rng(wl.seed + 10)
    A = wl.align if wl.align > 1 else 1
    total = wl.N - (wl.E * (A - 1) if A > 1 else 0)
    count = rng.multinomial(total, np.full(wl.E, 1.0 / wl.E)).astype(np.int32)
    span = (count + A - 1) // A * A
    start = np.concatenate([[0], np.cumsum(span)[:-1]]).astype(np.int32)
    return start, count, int(start[-1] + span[-1])


def _fp8_codes(rng, shape, emin: int, emax: int) -> np.ndarray:
    """Random E4M3FN bit patterns: sign, exponent field in [emin, emax] and
    mantissa uniform; the NaN pattern (exponent 15, mantissa 7) is avoided."""
    sign = rng.integers(0, 2, shape, dtype=np.uint8)
    ex = rng.integers(emin, emax + 1, shape, dtype=np.uint8)
    man = rng.integers(0, 8, shape, dtype=np.uint8)
    man = np.where((ex == 15) & (man == 7), np.uint8(6), man)
    return ((sign << 7) | (ex << 3) | man).astype(np.uint8)


def _pow2(rng, shape, lo: int, hi: int) -> np.ndarray:
    return np.ldexp(np.float32(1.0), rng.integers(lo, hi + 1, shape)).astype(np.float32)


def gen_mlp_x(wl: MlpWorkload):
    """FP8 activations [N,H] and power-of-two scales [N,H/128] (values up to ~1.75)."""
    rng = np.random.default_rng(wl.seed + 11)
    return _fp8_codes(rng, (wl.N, wl.H), 8, 15), _pow2(rng, (wl.N, wl.H // 128), -9, -8)


def gen_mlp_weights(wl: MlpWorkload, which: str):
    """'w1': codes [E,2I,H], scales [E,2I/128,H/128]; 'w2': codes [E,H,I], scales
    [E,H/128,I/128].  Magnitudes keep the projections of order one."""
    if which == "w1":
        rng = np.random.default_rng(wl.seed + 12)
        R, K = 2 * wl.I, wl.H
    else:
        rng = np.random.default_rng(wl.seed + 13)
        R, K = wl.H, wl.I
    return _fp8_codes(rng, (wl.E, R, K), 4, 9), _pow2(rng, (wl.E, R // 128, K // 128), -8, -7)

"""Seeded synthetic stage-boundary activations and the workload table.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the codec's arithmetic, so both the GPU path and the oracle can
take their inputs from it.

The pages train GPT2-XL, Qwen2.5-3B and LLaMA-3.2-1B over pipeline stages and
never publish activation tensors; these generators stand in for those
stage-boundary activations ([micro-batch x sequence, channels], heavy-tailed
outlier channels, near-zero rows, post-GeLU skew). Random numbers come from
numpy's counter-based Philox bit generator keyed by (seed, workload id).

Arrays are returned as ``float32`` for fp32 workloads and as ``uint16`` bf16 bit
patterns for bf16 workloads (numpy has no bf16 type).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = 0
BF16 = 1


@dataclasses.dataclass(frozen=True)
class Params:
    """Codec parameters: quantization tile G, ranking scope S in tokens (0 = all),
    average code-bit budget, candidate widths, outlier threshold tau,
    allocation tile A in channels (0 = G) and allocator (0 = top-p% between two
    widths, 1 = greedy over every candidate)."""

    tile: int = 64
    tokens_per_sample: int = 0
    bit_budget: float = 3.8
    candidates: tuple = (3, 4)
    tau: float = 2.0
    alloc_tile: int = 0
    allocator: int = 0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    hidden: int
    dtype: int
    params: Params
    recipe: str
    wid: int


def _philox(seed: int, wid: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=[int(seed), int(wid)]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _finish(x64: np.ndarray, dtype: int) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return x32 if dtype == F32 else f32_to_bf16_bits(x32)


def _count(frac: float, n: int) -> int:
    # round half up of frac * n
    return int(math.floor(frac * n + 0.5))


def gen_normal_outliers(tokens, hidden, dtype, seed, wid, n_out, mult, lognormal_mult=False):
    g = _philox(seed, wid)
    x = g.standard_normal((tokens, hidden))
    ch = g.choice(hidden, size=n_out, replace=False)
    m = np.full(n_out, float(mult))
    if lognormal_mult:
        m = m * np.exp(g.standard_normal(n_out))
    x[:, ch] *= m
    return _finish(x, dtype)


def gen_llama_like(tokens, hidden, dtype, seed, wid, n_heavy, heavy_mult):
    """Per-channel log-normal scale (sigma = 1) on N(0,1); n_heavy channels draw
    Student-t (nu = 2) values times heavy_mult instead."""
    g = _philox(seed, wid)
    sig = np.exp(g.standard_normal(hidden))
    x = g.standard_normal((tokens, hidden))
    ch = g.choice(hidden, size=n_heavy, replace=False)
    # Student-t with 2 degrees of freedom: Z / sqrt(chi2_2 / 2), chi2_2 / 2 = -ln U
    z = g.standard_normal((tokens, n_heavy))
    u = g.random((tokens, n_heavy))
    u = np.maximum(u, np.finfo(np.float64).tiny)
    x[:, ch] = heavy_mult * z / np.sqrt(-np.log(u))
    x *= sig[None, :]
    return _finish(x, dtype)


def gen_sparse_rows(tokens, hidden, dtype, seed, wid, zero_frac, n_massive, massive_mult):
    """N(0,1) with a fraction of near-zero tokens (x 1e-3) and massive channels."""
    g = _philox(seed, wid)
    x = g.standard_normal((tokens, hidden))
    rows = g.choice(tokens, size=_count(zero_frac, tokens), replace=False)
    x[rows, :] *= 1e-3
    ch = g.choice(hidden, size=n_massive, replace=False)
    x[:, ch] *= massive_mult
    return _finish(x, dtype)


def gen_gelu(tokens, hidden, dtype, seed, wid, n_out, mult, var=2.0):
    """Exact GeLU of N(0, var) plus outlier channels."""
    from scipy.special import erf

    g = _philox(seed, wid)
    u = g.standard_normal((tokens, hidden)) * math.sqrt(var)
    x = 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))
    ch = g.choice(hidden, size=n_out, replace=False)
    x[:, ch] *= mult
    return _finish(x, dtype)


def gen_gradients(tokens, hidden, dtype, seed, wid, heavy_frac=0.01, heavy_mult=100.0):
    """Activation gradients at a stage boundary (what Algorithm 1 sends back):
    N(0,1) per element times a per-token scale 1e-6 * lognormal(sigma = 1.5),
    and a few tokens (heavy_frac) x heavy_mult: most tokens carry gradients of
    order 1e-6..1e-5 (App. H speaks of 1e-5), a few carry most of the norm."""
    g = _philox(seed, wid)
    row = 1e-6 * np.exp(1.5 * g.standard_normal(tokens))
    heavy = g.choice(tokens, size=_count(heavy_frac, tokens), replace=False) if tokens else np.zeros(0, int)
    row[heavy] *= heavy_mult
    x = g.standard_normal((tokens, hidden)) * row[:, None]
    return _finish(x, dtype)


WORKLOADS = {
    "c1_256x512_f32_g32": Workload(
        "c1_256x512_f32_g32", 256, 512, F32,
        Params(tile=32, tokens_per_sample=0, bit_budget=4.0, candidates=(3, 4, 8), tau=2.0),
        "N(0,1) fp32, 4 outlier channels x50", 1),
    "c2_4096x2048_bf16_g64": Workload(
        "c2_4096x2048_bf16_g64", 4096, 2048, BF16,
        Params(tile=64, tokens_per_sample=1024, bit_budget=3.5, candidates=(2, 3, 4, 8), tau=2.0),
        "N(0,1) bf16, 1% outlier channels x30*lognormal", 2),
    "c3_16384x4096_bf16_g64": Workload(
        "c3_16384x4096_bf16_g64", 16384, 4096, BF16,
        Params(tile=64, tokens_per_sample=2048, bit_budget=3.0, candidates=(3, 4, 8), tau=2.0),
        "per-channel lognormal scale, 0.5% Student-t(2) x100 channels", 3),
    "c4_16384x5120_f32_g128": Workload(
        "c4_16384x5120_f32_g128", 16384, 5120, F32,
        Params(tile=128, tokens_per_sample=2048, bit_budget=4.0, candidates=(2, 3, 4, 8), tau=2.0),
        "N(0,1) fp32, 30% rows x1e-3, 8 massive channels x500", 4),
    "c5_8192x8192_bf16_g64": Workload(
        "c5_8192x8192_bf16_g64", 8192, 8192, BF16,
        Params(tile=64, tokens_per_sample=0, bit_budget=3.0, candidates=(3, 4, 8), tau=2.0),
        "GeLU(N(0,2)) bf16, 0.1% outlier channels x200", 5),
    # activation gradients going back across the boundary, coded by TAH-Quant at
    # 4 bits (App. H, Table 10); the same tensors feed the fixed-point compressor
    "g1_8192x8192_bf16_grad": Workload(
        "g1_8192x8192_bf16_grad", 8192, 8192, BF16,
        Params(tile=64, tokens_per_sample=0, bit_budget=4.0, candidates=(4,), tau=2.0),
        "activation gradients: N(0,1) x 1e-6 lognormal(1.5) per token, 1% tokens x100", 6),
    "g2_4096x2048_f32_grad": Workload(
        "g2_4096x2048_f32_grad", 4096, 2048, F32,
        Params(tile=64, tokens_per_sample=1024, bit_budget=3.8, candidates=(3, 4), tau=2.0),
        "activation gradients, fp32, 80/20 INT4/INT3 per 1024-token sample", 7),
}

# The fixed-point backward compressor's settings for the gradient workloads:
# bits (6-8 in the paper's runs, 10 after its NaN event, 4 in App. H) and the
# constant c of Eq. (24), here chosen so that a 1e-5 gradient is about 1/20 of
# the largest representable value.
NAIVE = {
    "g1_8192x8192_bf16_grad": dict(bits=8, c=4096.0),
    "g2_4096x2048_f32_grad": dict(bits=10, c=4096.0),
}

# Coverage variants: mixed allocations at other budgets, the tau values of
# App. F (0, 2, 4, never), allocation tiles of several quantization tiles up to
# whole tokens (Sec. 3.2: A = C is token-level allocation), and the greedy
# allocator over every candidate width.
COVERAGE = {
    "x1a_c2_budget5": ("c2_4096x2048_bf16_g64", dict(bit_budget=5.0, candidates=(3, 4, 8))),
    "x1b_c2_budget2p5": ("c2_4096x2048_bf16_g64", dict(bit_budget=2.5, candidates=(2, 3, 4, 8))),
    "x2_c5_budget3p8": ("c5_8192x8192_bf16_g64", dict(bit_budget=3.8, candidates=(3, 4, 8))),
    "x3a_c1_tau0": ("c1_256x512_f32_g32", dict(tau=0.0)),
    "x3b_c1_tauinf": ("c1_256x512_f32_g32", dict(tau=math.inf)),
    "x3c_c2_tau0": ("c2_4096x2048_bf16_g64", dict(tau=0.0)),
    "x3d_c2_tauinf": ("c2_4096x2048_bf16_g64", dict(tau=math.inf)),
    "x3e_c2_tau4": ("c2_4096x2048_bf16_g64", dict(tau=4.0)),
    "x4a_c2_alloc256": ("c2_4096x2048_bf16_g64", dict(alloc_tile=256)),
    "x4b_c5_token_level": ("c5_8192x8192_bf16_g64", dict(bit_budget=3.8, candidates=(3, 4, 8), alloc_tile=8192)),
    "x4c_c4_token_level": ("c4_16384x5120_f32_g128", dict(alloc_tile=5120)),
    # the greedy allocator over every candidate width (allocator 1)
    "x5a_c2_greedy": ("c2_4096x2048_bf16_g64", dict(allocator=1)),
    "x5b_c5_greedy": ("c5_8192x8192_bf16_g64", dict(bit_budget=3.8, candidates=(3, 4, 8), allocator=1)),
    "x5c_c4_greedy_a640": ("c4_16384x5120_f32_g128", dict(alloc_tile=640, allocator=1)),
}


def workload(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    base, over = COVERAGE[name]
    w = WORKLOADS[base]
    return dataclasses.replace(w, name=name, params=dataclasses.replace(w.params, **over))


def generate(name: str, seed: int = 0, tokens: int | None = None) -> np.ndarray:
    """Input tensor of a workload. ``tokens`` truncates the row count (a bounded
    sample of the same distribution, drawn from the same stream layout)."""
    w = workload(name)
    T = w.tokens if tokens is None else int(tokens)
    H = w.hidden
    if w.wid == 1:
        return gen_normal_outliers(T, H, w.dtype, seed, w.wid, 4, 50.0)
    if w.wid == 2:
        return gen_normal_outliers(T, H, w.dtype, seed, w.wid, _count(0.01, H), 30.0, lognormal_mult=True)
    if w.wid == 3:
        return gen_llama_like(T, H, w.dtype, seed, w.wid, _count(0.005, H), 100.0)
    if w.wid == 4:
        return gen_sparse_rows(T, H, w.dtype, seed, w.wid, 0.30, 8, 500.0)
    if w.wid == 5:
        return gen_gelu(T, H, w.dtype, seed, w.wid, _count(0.001, H), 200.0)
    if w.wid in (6, 7):
        return gen_gradients(T, H, w.dtype, seed, w.wid)
    raise KeyError(name)


def random_tensor(tokens, hidden, dtype, seed, scale=1.0, n_out=0, mult=1.0):
    """Small generic input for edge-case tests."""
    g = _philox(seed, 100)
    x = g.standard_normal((tokens, hidden)) * scale
    if n_out and hidden:
        ch = g.choice(hidden, size=min(n_out, hidden), replace=False)
        x[:, ch] *= mult
    return _finish(x, dtype)

"""Seeded synthetic inputs for the row-wise normalisation ops.

This module only draws random numbers and casts them to the storage dtypes; it holds none
of the normalisation arithmetic. Both sides of every parity check (the fp64 oracle under
``oracle/`` and the HIP library under ``transformer_row_wise_amd/``) receive the tensors
built here, and neither of them imports the other.

Recipe (the same for every workload):
  * ``numpy.random.default_rng(seed)`` (PCG64), draws taken in float64 in the order
    x, r, w, b, g (g: the output cotangent of a backward call);
  * ``N(mean, std)`` means ``rng.normal(loc=mean, scale=std)`` (std, not variance);
    ``U(lo, hi)`` is ``rng.uniform(lo, hi)``; Student-t(3) is ``rng.standard_t(3)``;
  * the "1% of rows times 1e3" outlier rows are picked after every draw, with
    ``rng.choice(rows, rows // 100, replace=False)``, and the same rows are scaled in x and r;
  * float64 -> float32 by numpy's round-to-nearest-even cast, then float32 -> bfloat16 by
    torch's round-to-nearest-even cast (CPU).

Tensors are returned on the CPU; callers move them to the device themselves.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def cast(a64: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 draws -> float32 (RNE) -> bf16 (RNE, torch) as a CPU tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float32))
    return t if dtype == "f32" else t.to(DTYPES[dtype])


def draw(rng: np.random.Generator, spec, shape):
    """One float64 draw. ``spec`` is ("normal", mean, std), ("uniform", lo, hi),
    ("t3",) or ("const", value)."""
    kind = spec[0]
    if kind == "normal":
        return rng.normal(spec[1], spec[2], size=shape)
    if kind == "uniform":
        return rng.uniform(spec[1], spec[2], size=shape)
    if kind == "t3":
        return rng.standard_t(3, size=shape)
    if kind == "const":
        return np.full(shape, float(spec[1]))
    raise ValueError(f"unknown distribution {spec!r}")


@dataclasses.dataclass
class RowInputs:
    """Inputs of one row-wise call: x (and r, g) of shape [rows, hidden]; w, b of [hidden]."""

    x: torch.Tensor
    r: torch.Tensor | None
    w: torch.Tensor | None
    b: torch.Tensor | None
    eps: float
    g: torch.Tensor | None = None


def row_inputs(rows, hidden, dtype, *, seed=0, x=("normal", 0.0, 1.0), r=None,
               w=("normal", 1.0, 0.1), b=None, g=None, w_dtype=None, eps=1e-5,
               outlier_frac=0.0, outlier_scale=1e3) -> RowInputs:
    """Draws x (and r, w, b, g when given a distribution) in the recipe's order."""
    rng = np.random.default_rng(seed)
    wd = w_dtype or dtype
    x64 = draw(rng, x, (rows, hidden))
    r64 = draw(rng, r, (rows, hidden)) if r is not None else None
    w64 = draw(rng, w, (hidden,)) if w is not None else None
    b64 = draw(rng, b, (hidden,)) if b is not None else None
    g64 = draw(rng, g, (rows, hidden)) if g is not None else None
    if outlier_frac > 0 and rows > 0:
        pick = rng.choice(rows, int(rows * outlier_frac), replace=False)
        x64[pick] *= outlier_scale
        if r64 is not None:
            r64[pick] *= outlier_scale
    return RowInputs(
        x=cast(x64, dtype),
        r=cast(r64, dtype) if r64 is not None else None,
        w=cast(w64, wd) if w64 is not None else None,
        b=cast(b64, wd) if b64 is not None else None,
        eps=eps,
        g=cast(g64, dtype) if g64 is not None else None,
    )


@dataclasses.dataclass
class RopeInputs:
    """Inputs of one NormRope call: x [B, H, L, D], w [D] and the rotation settings."""

    x: torch.Tensor
    w: torch.Tensor | None
    eps: float
    dims: int
    base: float
    scale: float
    offset: int


def rope_inputs(B, H, L, D, dtype, *, seed=0, x=("normal", 0.0, 1.0),
                w=("uniform", 0.5, 1.5), w_dtype=None, eps=1e-6, dims=None,
                base=10000.0, scale=1.0, offset=0) -> RopeInputs:
    rng = np.random.default_rng(seed)
    x64 = draw(rng, x, (B, H, L, D))
    w64 = draw(rng, w, (D,)) if w is not None else None
    return RopeInputs(
        x=cast(x64, dtype),
        w=cast(w64, w_dtype or dtype) if w64 is not None else None,
        eps=eps, dims=D if dims is None else dims, base=base, scale=scale, offset=offset,
    )


# ---------------------------------------------------------------------------------------
# The named workloads. Sizes and distributions follow the five synthetic configurations
# of the row-wise normalisation benchmark: small fp32 add-RMSNorm, bf16 add-RMSNorm at
# 4096x4096, bf16 LayerNorm at 16384x8192 (affine and not), bf16 NormRope at
# [8,32,512,128] (two pair modes, plain and cache output) and add-RMSNorm at scale with
# heavy-tailed values.
# ---------------------------------------------------------------------------------------

def cfg_add_rms_small_f32(seed=0):
    """add-RMSNorm fp32, x and r [64,512] ~N(0,1), w ~U(0.5,1.5), eps 1e-6."""
    return row_inputs(64, 512, "f32", seed=seed, x=("normal", 0.0, 1.0),
                      r=("normal", 0.0, 1.0), w=("uniform", 0.5, 1.5), eps=1e-6)


def cfg_add_rms_4k_bf16(seed=0):
    """add-RMSNorm bf16, x and r [4096,4096] ~N(0,1), w ~N(1,0.1), eps 1e-5."""
    return row_inputs(4096, 4096, "bf16", seed=seed, x=("normal", 0.0, 1.0),
                      r=("normal", 0.0, 1.0), w=("normal", 1.0, 0.1), eps=1e-5)


def cfg_layer_norm_bf16(seed=0, affine=True, rows=16384, hidden=8192):
    """LayerNorm bf16, x [16384,8192] ~N(0.5, std 2), w ~N(1,0.1), b ~N(0,0.1), eps 1e-5.
    The no-affine case draws the same x (w and b are simply not drawn after it)."""
    return row_inputs(rows, hidden, "bf16", seed=seed, x=("normal", 0.5, 2.0),
                      w=("normal", 1.0, 0.1) if affine else None,
                      b=("normal", 0.0, 0.1) if affine else None, eps=1e-5)


def cfg_norm_rope_bf16(seed=0, offset=0):
    """NormRope bf16, x [8,32,512,128] ~N(0,1), w[128] ~U(0.5,1.5), eps 1e-6, dims 128,
    base 1e4, scale 1. The cache form writes [8,32,2048,128] at offset 1024."""
    return rope_inputs(8, 32, 512, 128, "bf16", seed=seed, eps=1e-6, dims=128,
                       base=10000.0, scale=1.0, offset=offset)


NORM_ROPE_CACHE_LEN = 2048
NORM_ROPE_CACHE_OFFSET = 1024


def cfg_add_rms_scale(rows=16384, hidden=8192, dtype="bf16", seed=0):
    """add-RMSNorm at scale: x and r Student-t(3), 1% of rows times 1e3, w ~N(1,0.1),
    eps 1e-6. Shapes [16384,8192] and [65536,5120], bf16 and fp32."""
    return row_inputs(rows, hidden, dtype, seed=seed, x=("t3",), r=("t3",),
                      w=("normal", 1.0, 0.1), eps=1e-6, outlier_frac=0.01)


# The headline measurement: add-RMSNorm, bf16, 16384 x 8192.
METRIC_ROWS = 16384
METRIC_HIDDEN = 8192


# Backward workloads (RmsNormVjp, LayerNormVjp): the forward inputs of the add-RMSNorm and
# LayerNorm workloads at [16384, 8192] bf16 with a cotangent g ~ N(0, 1) of the same shape.

def cfg_rms_vjp(rows=16384, hidden=8192, dtype="bf16", seed=0):
    """RMSNorm backward: x Student-t(3) with 1% of rows x1e3, w ~N(1,0.1), g ~N(0,1),
    eps 1e-6."""
    return row_inputs(rows, hidden, dtype, seed=seed, x=("t3",), w=("normal", 1.0, 0.1),
                      g=("normal", 0.0, 1.0), eps=1e-6, outlier_frac=0.01)


def cfg_ln_vjp(rows=16384, hidden=8192, dtype="bf16", seed=0):
    """LayerNorm backward: x ~N(0.5, std 2), w ~N(1,0.1), g ~N(0,1), eps 1e-5."""
    return row_inputs(rows, hidden, dtype, seed=seed, x=("normal", 0.5, 2.0),
                      w=("normal", 1.0, 0.1), g=("normal", 0.0, 1.0), eps=1e-5)


@dataclasses.dataclass
class RopeQKInputs:
    """Query [T, Hq, D] and key [T, Hk, D] rows with their token positions [T] (int64)."""

    q: torch.Tensor
    k: torch.Tensor | None
    positions: torch.Tensor


def rope_qk_inputs(T, Hq, Hk, D, dtype, *, seed=0, positions="arange", max_position=None):
    """q then k ~ N(0, 1); positions 0 .. T-1 ("arange", a prefill) or uniform integers in
    [0, max_position) ("random", a decode batch of independent sequences)."""
    rng = np.random.default_rng(seed)
    q64 = rng.standard_normal((T, Hq, D))
    k64 = rng.standard_normal((T, Hk, D)) if Hk else None
    if positions == "arange":
        pos = np.arange(T, dtype=np.int64)
    else:
        pos = rng.integers(0, max_position, size=T, dtype=np.int64)
    return RopeQKInputs(q=cast(q64, dtype), k=cast(k64, dtype) if k64 is not None else None,
                        positions=torch.from_numpy(pos))


def rope_freqs_draw(dims, kind, seed=0):
    """Synthetic per-pair divisors for the freqs input, float32 [dims / 2]: "uniform" in
    [0.5, 5000), or "loguniform" in [1, 1e7) (the span of long-context scaled divisors)."""
    rng = np.random.default_rng(seed)
    if kind == "uniform":
        f = rng.uniform(0.5, 5000.0, dims // 2)
    else:
        f = np.exp(rng.uniform(0.0, np.log(1e7), dims // 2))
    return torch.from_numpy(f.astype(np.float32))


# Positions-form workload: a Llama-3-8B-shaped prefill of 16384 tokens, 32 query and 8 key
# heads of 128 features, bf16, Llama 3 scaled frequencies (base 500000, the MinivLLM
# defaults factor 32, low 1, high 4, original context 8192).
ROPE_QK_SHAPE = (16384, 32, 8, 128)
ROPE_QK_BASE = 500000.0


def cfg_rope_qk_bf16(seed=0):
    T, Hq, Hk, D = ROPE_QK_SHAPE
    return rope_qk_inputs(T, Hq, Hk, D, "bf16", seed=seed)


# Softmax-family workloads: scores of one attention layer's prefill ([8 * 32 heads, 512, 512]
# bf16, N(0, 3)) for the causal softmax; a [16384, 8192] bf16 softmax; and the language-model
# head's loss over a Llama-3-sized vocabulary: logits [4096, 128256] bf16 ~ N(0, 2), targets
# uniform over the vocabulary, loss cotangent 1 / 4096 (a mean over the rows).
CE_SHAPE = (4096, 128256)


@dataclasses.dataclass
class CEInputs:
    logits: torch.Tensor
    targets: torch.Tensor   # int64
    g: torch.Tensor         # float32 loss cotangent per row


def ce_inputs(rows, V, dtype, *, seed=0, std=2.0, g="mean"):
    """logits ~ N(0, std) then targets ~ U{0 .. V-1}, then g (1 / rows, or ~ N(0, 1))."""
    rng = np.random.default_rng(seed)
    x64 = rng.normal(0.0, std, size=(rows, V))
    t = rng.integers(0, V, size=rows, dtype=np.int64)
    g64 = np.full(rows, 1.0 / rows) if g == "mean" else rng.standard_normal(rows)
    return CEInputs(logits=cast(x64, dtype), targets=torch.from_numpy(t),
                    g=torch.from_numpy(g64.astype(np.float32)))


def cfg_ce_bf16(seed=0):
    return ce_inputs(*CE_SHAPE, "bf16", seed=seed)


def scores(shape, dtype, *, seed=0, std=3.0):
    """Attention-like scores ~ N(0, std)."""
    rng = np.random.default_rng(seed)
    return cast(rng.normal(0.0, std, size=shape), dtype)

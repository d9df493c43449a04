"""Frequency scalings of RoPE for long contexts (oracle; test infrastructure only).

Sources: nuvec-nn 0.4.0 ``layers.rs`` docs, ``Rope`` ("optionally with a frequency scaling,
Rope::scaled: mlx-lm's Llama3RoPE, YarnRoPE, SuScaledRoPE, ProportionalRoPE; the
frequencies are computed from the settings"), and the MinivLLM API reference, "Layers",
``RotaryEmbedding`` (Llama 3 NTK-by-parts scaling with ``factor``, ``low_freq_factor``,
``high_freq_factor`` and ``original_max_position_embeddings``; defaults 32, 1, 4, 8192).
The pages name the strategies and their settings but print no formula; each function
below follows the published method named in its docstring. ProportionalRoPE has no
definition in the pages or in a publication this module can follow, so it is absent.

Every strategy returns ``(freqs, mscale)``: freqs[i] (float32 values, as float64) is the
divisor of the position for rotated pair i (theta_i = 1 / freqs[i], the convention of the
``freqs`` input of ``Rope``), and mscale multiplies the rotated features (1 when the method
has none). Every real-valued setting enters as its float32 value (the interface takes
them as f32, like eps, base and scale); all arithmetic is float64; freqs are rounded once
to float32.
"""

import math

import numpy as np

from .rounding import f32_param, round_to


def _base_periods(dims, base):
    """base^(2i/dims), i = 0 .. dims/2 - 1: the unscaled divisors."""
    i = np.arange(dims // 2, dtype=np.float64)
    return np.power(f32_param(base), (2.0 * i) / dims)


def default_freqs(dims, base):
    """Plain RoPE: freqs[i] = base^(2i/dims), mscale 1."""
    return round_to(_base_periods(dims, base), "f32"), 1.0


def llama3_freqs(dims, base, factor=32.0, low_freq_factor=1.0, high_freq_factor=4.0,
                 original_max=8192):
    """Llama 3 NTK-by-parts scaling (Meta's Llama 3.1 RoPE frequency scaling; mlx-lm's
    Llama3RoPE). With wavelength 2*pi*f of each unscaled divisor f: pairs whose wavelength
    is below original_max / high_freq_factor keep f; pairs above original_max /
    low_freq_factor get f * factor; in between, with s = (original_max / wavelength -
    low_freq_factor) / (high_freq_factor - low_freq_factor), the inverse frequencies are
    blended, 1/f' = (1 - s) / (factor f) + s / f."""
    factor, low_freq_factor, high_freq_factor = (f32_param(v) for v in
                                                 (factor, low_freq_factor, high_freq_factor))
    f = _base_periods(dims, base)
    wavelen = 2.0 * math.pi * f
    low_wavelen = original_max / low_freq_factor
    high_wavelen = original_max / high_freq_factor
    out = f.copy()
    out[wavelen > low_wavelen] = f[wavelen > low_wavelen] * factor
    mid = (wavelen > high_wavelen) & (wavelen < low_wavelen)
    s = (original_max / wavelen[mid] - low_freq_factor) / (high_freq_factor - low_freq_factor)
    out[mid] = f[mid] / ((1.0 - s) / factor + s)
    return round_to(out, "f32"), 1.0


def yarn_freqs(dims, base, factor=4.0, original_max=4096, beta_fast=32.0, beta_slow=1.0,
               mscale=1.0, mscale_all_dim=0.0):
    """YaRN (Peng et al. 2023, "YaRN: Efficient Context Window Extension of Large Language
    Models", NTK-by-parts interpolation with a linear ramp, section 3.2, and the attention
    temperature of section 3.4; mlx-lm's YarnRoPE). The ramp runs over pair indices from
    floor(d(beta_fast)) to ceil(d(beta_slow)), clamped to [0, dims - 1], where
    d(r) = dims * ln(original_max / (2 pi r)) / (2 ln base) is the pair index whose
    wavelength fits r rotations in the original context; below the ramp pairs keep f
    (extrapolation), above it they get factor * f (interpolation), and on it the inverse
    frequencies blend linearly. mscale = g(factor, mscale) / g(factor, mscale_all_dim),
    g(s, m) = 0.1 m ln s + 1 (1 when s <= 1)."""
    factor, beta_fast, beta_slow, mscale, mscale_all_dim = (
        f32_param(v) for v in (factor, beta_fast, beta_slow, mscale, mscale_all_dim))
    f = _base_periods(dims, base)

    def corr_dim(rotations):
        return dims * math.log(original_max / (rotations * 2.0 * math.pi)) / (2.0 * math.log(f32_param(base)))

    low = max(math.floor(corr_dim(beta_fast)), 0)
    high = min(math.ceil(corr_dim(beta_slow)), dims - 1)
    if low == high:
        high += 0.001
    ramp = np.clip((np.arange(dims // 2, dtype=np.float64) - low) / (high - low), 0.0, 1.0)
    keep = 1.0 - ramp  # weight of the unscaled (extrapolated) inverse frequency
    inv = keep / f + (1.0 - keep) / (factor * f)

    def g(s, m):
        return 1.0 if s <= 1 else 0.1 * m * math.log(s) + 1.0

    return round_to(1.0 / inv, "f32"), g(factor, mscale) / g(factor, mscale_all_dim)


def su_freqs(dims, base, long_factor, max_position=131072, original_max=4096):
    """LongRoPE / "su" scaling (Ding et al. 2024, "LongRoPE"; Phi-3 technical report;
    mlx-lm's SuScaledRoPE): per-pair rescale factors multiply the divisors,
    freqs[i] = long_factor[i] * base^(2i/dims), and the rotated features are scaled by
    sqrt(1 + ln(max_position / original_max) / ln(original_max))."""
    lf = np.asarray(long_factor, dtype=np.float32).astype(np.float64)
    assert lf.shape == (dims // 2,)
    out = round_to(lf * _base_periods(dims, base), "f32")
    ms = math.sqrt(1.0 + math.log(max_position / original_max) / math.log(original_max))
    return out, ms

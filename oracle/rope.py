"""fp64 NormRope: per-row RMS normalisation followed by a rotary position embedding of the
first ``dims`` features (oracle; test infrastructure only).

Sources: nuvec-core ``fast::FastOp``, variants ``NormRope`` (each [b, h, l] row of a
[B, H, L, D] input RMS-normalised with eps, or not at all when eps is absent, then rotated
as ``Rope`` at position offset + l, and either returned or written into a cache at those
positions) and ``Rope`` (``dims`` even; ``traditional`` pairs neighbours instead of the two
halves; ``base`` and ``scale`` as f32 bits, scale applied to the position; ``forward=false``
is the inverse rotation). nuvec-nn ``layers.rs``, ``Rope``: defaults half-split, base 10000,
scale 1, frequencies computed from the settings and never loaded.

Readings where the pages print no formula (the textbook RoPE of RoFormer, Su et al. 2021,
section 3.2): pair i of the rotated features has frequency theta_i = base^(-2i/dims),
angle a = scale * position * theta_i, and the pair (u, v) turns counter-clockwise,
(u, v) -> (u cos a - v sin a, u sin a + v cos a); the inverse uses -a. The RMS statistic
spans all D features; features at index >= dims are normalised but not rotated.

``freqs`` (the optional input of ``Rope`` and ``NormRope``, which the pages say replaces
``base``): read in the convention of the fast rope the pages name (MLX's ``fast::rope``),
freqs[i] is the period divisor of pair i, theta_i = 1 / freqs[i]; with the defaults
freqs[i] = base^(2i/dims). ``mscale`` multiplies the rotated features (the attention factor
of the scaled variants: mlx-lm's YarnRoPE and SuScaledRoPE scale x[..., :dims] before the
rotation); 1 for plain RoPE.

``rope_positions`` is the positions-tensor form of the MinivLLM API reference
(``RotaryEmbedding.forward(positions, query, key)``): rows of [T, H, D] arrays, token t at
position positions[t], the same rotation for every head of the token.
"""

import numpy as np

from .rounding import f32_param, round_to


def rope_frequencies(dims, base, freqs=None):
    """theta_i for i = 0 .. dims/2 - 1 in float64: base^(-2 i / dims), or 1 / freqs[i]."""
    if freqs is not None:
        f = np.asarray(freqs, dtype=np.float64)
        assert f.shape == (dims // 2,), f.shape
        return 1.0 / f
    i = np.arange(dims // 2, dtype=np.float64)
    return np.power(f32_param(base), (-2.0 * i) / dims)


def rope_angles(positions, dims, base, scale, freqs=None):
    """Angles [len(positions), dims/2]: scale * position * theta_i."""
    p = np.asarray(positions, dtype=np.float64)
    return (f32_param(scale) * p)[:, None] * rope_frequencies(dims, base, freqs)[None, :]


def _rotate(xn, a, dims, traditional, forward, mscale):
    """Rotate the first dims features of rows xn [..., P, D] by angles a [P, dims/2]."""
    c = np.cos(a)
    s = np.sin(a)
    if not forward:
        s = -s
    iu, iv = _pair_index(dims, traditional)
    u = xn[..., iu]
    v = xn[..., iv]
    y = xn.copy()
    m = f32_param(mscale)
    y[..., iu] = m * (u * c - v * s)
    y[..., iv] = m * (u * s + v * c)
    return y


def _pair_index(dims, traditional):
    """Feature indices (u, v) of each rotated pair."""
    half = dims // 2
    i = np.arange(half)
    if traditional:
        return 2 * i, 2 * i + 1
    return i, i + half


def norm_rope(x, w, *, normalize, eps, dims, traditional, base, scale, offset, forward,
              dtype, cache=None, freqs=None, mscale=1.0):
    """x: [B, H, L, D] float64 values. Returns the rotated [B, H, L, D] array rounded to
    ``dtype``; with ``cache`` ([B, H, Lc, D] values) returns a copy of the cache with rows
    offset .. offset + L - 1 of every (b, h) replaced by the result and the rest untouched.
    """
    x = np.asarray(x, dtype=np.float64)
    B, H, L, D = x.shape
    if normalize:
        mean_sq = np.sum(x * x, axis=-1, keepdims=True) / D
        xn = x / np.sqrt(mean_sq + f32_param(eps))
        if w is not None:
            xn = xn * np.asarray(w, dtype=np.float64)
    else:
        xn = x.copy()

    a = rope_angles(offset + np.arange(L), dims, base, scale, freqs)  # [L, dims/2]
    y = round_to(_rotate(xn, a, dims, traditional, forward, mscale), dtype)

    if cache is None:
        return y
    out = np.array(cache, dtype=np.float64, copy=True)
    out[:, :, offset:offset + L, :] = y
    return out


def rope_positions(x, positions, *, dims, traditional, base, scale, forward, dtype,
                   freqs=None, mscale=1.0):
    """x: [T, H, D] float64 values, positions: [T] integers. Every head of token t turns at
    position positions[t]; returns [T, H, D] rounded to ``dtype``."""
    x = np.asarray(x, dtype=np.float64)
    a = rope_angles(np.asarray(positions), dims, base, scale, freqs)  # [T, dims/2]
    y = _rotate(x, a[:, None, :], dims, traditional, forward, mscale)
    return round_to(y, dtype)

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
"""

import numpy as np

from .rounding import f32_param, round_to


def rope_frequencies(dims, base):
    """theta_i = base^(-2 i / dims) for i = 0 .. dims/2 - 1, in float64."""
    i = np.arange(dims // 2, dtype=np.float64)
    return np.power(f32_param(base), (-2.0 * i) / dims)


def rope_angles(positions, dims, base, scale):
    """Angles [len(positions), dims/2]: scale * position * theta_i."""
    p = np.asarray(positions, dtype=np.float64)
    return (f32_param(scale) * p)[:, None] * rope_frequencies(dims, base)[None, :]


def _pair_index(dims, traditional):
    """Feature indices (u, v) of each rotated pair."""
    half = dims // 2
    i = np.arange(half)
    if traditional:
        return 2 * i, 2 * i + 1
    return i, i + half


def norm_rope(x, w, *, normalize, eps, dims, traditional, base, scale, offset, forward,
              dtype, cache=None):
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

    a = rope_angles(offset + np.arange(L), dims, base, scale)  # [L, dims/2]
    c = np.cos(a)
    s = np.sin(a)
    if not forward:
        s = -s
    iu, iv = _pair_index(dims, traditional)
    u = xn[..., iu]
    v = xn[..., iv]
    y = xn.copy()
    y[..., iu] = u * c - v * s
    y[..., iv] = u * s + v * c
    y = round_to(y, dtype)

    if cache is None:
        return y
    out = np.array(cache, dtype=np.float64, copy=True)
    out[:, :, offset:offset + L, :] = y
    return out

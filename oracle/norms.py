"""fp64 RMSNorm, residual add-RMSNorm and LayerNorm over the last axis (oracle; test
infrastructure only).

Inputs are float64 arrays holding the exact input values; ``w`` and ``b`` may be None,
which means the scalars 1 and 0. ``dtype`` ("bf16", "f32", or "f64" for no rounding) is the
output dtype; the result is rounded to it once, at the end.
"""

import numpy as np

from .rounding import f32_param, round_to


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def rms_norm(x, w, eps, dtype):
    """x / sqrt(mean(x^2) + eps) * w over the last axis.

    nuvec-core ``fast::FastOp``, variant ``RmsNorm``: the definition, ``w`` 1-D or the
    scalar 1, eps held as the bits of an f32. MinivLLM "Layers", ``LayerNorm``: the same
    formula with a learned ``gamma``.
    """
    x = _f64(x)
    w = _f64(w)
    d = x.shape[-1]
    mean_sq = np.sum(x * x, axis=-1, keepdims=True) / d
    y = x / np.sqrt(mean_sq + f32_param(eps))
    if w is not None:
        y = y * w
    return round_to(y, dtype)


def add_rms_norm(x, r, w, eps, dtype):
    """Returns (RMSNorm(h), h) with h = x + r rounded to ``dtype``.

    nuvec-core ``fast::FastOp``, variant ``AddRmsNorm``: h is x + r and the result is
    ``RmsNorm`` of h. MinivLLM "Layers", ``LayerNorm.forward`` with a residual: the updated
    residual is returned beside the normalised value. Reading taken where the pages are
    silent: the normalisation is of the returned h, i.e. after its rounding to the storage
    dtype (both pages normalise the very h that they hand back).
    """
    h = round_to(_f64(x) + _f64(r), dtype)
    return rms_norm(h, w, eps, dtype), h


def layer_norm(x, w, b, eps, dtype):
    """(x - mean) / sqrt(var + eps) * w + b over the last axis.

    nuvec-core ``fast::FastOp``, variant ``LayerNorm``: ``w`` and ``b`` 1-D or the scalars
    1 and 0. nuvec-nn ``layers.rs``, ``LayerNorm``: affine by default, ``without_bias`` drops
    b, ``affine(false)`` drops both. Reading: var is the biased (divide by D) variance,
    taken in a second pass around the mean. The mean takes one correction step (mean +
    mean(x - mean), the corrected two-pass mean), so that its float64 rounding error stays
    negligible against the spread even when |mean| / std is as large as 1e6.
    """
    x = _f64(x)
    w = _f64(w)
    b = _f64(b)
    d = x.shape[-1]
    mean = np.sum(x, axis=-1, keepdims=True) / d
    mean = mean + np.sum(x - mean, axis=-1, keepdims=True) / d
    centred = x - mean
    var = np.sum(centred * centred, axis=-1, keepdims=True) / d
    y = centred / np.sqrt(var + f32_param(eps))
    if w is not None:
        y = y * w
    if b is not None:
        y = y + b
    return round_to(y, dtype)

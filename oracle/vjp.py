"""fp64 vector-Jacobian products of RMSNorm and LayerNorm (oracle; test infrastructure only).

Sources: nuvec-core 0.5.0 ``fast::FastOp``, variants ``RmsNormVjp`` ((x, w, g): the gradients
of ``RmsNorm`` for x and w) and ``LayerNormVjp`` ((x, w, b, g): the gradients of ``LayerNorm``
for x, w and b). g is the cotangent of the output, of x's shape; w and b are 1-D and shared by
every row, so their gradients sum over all leading (row) axes.

Derivation (calculus on the forward definitions, per row of D features):
  RMSNorm   y_j = x_j r w_j,  r = (sum_k x_k^2 / D + eps)^(-1/2)
            dx_j = r g_j w_j - x_j r^3 (sum_k g_k w_k x_k) / D
            dw_j = sum over rows of g_j x_j r
  LayerNorm xh_j = (x_j - mu) r,  r = (var + eps)^(-1/2),  y_j = xh_j w_j + b_j
            with d_j = g_j w_j:  dx_j = r (d_j - mean(d) - xh_j mean(d xh))
            dw_j = sum over rows of g_j xh_j,  db_j = sum over rows of g_j
w absent means the scalar 1 (its gradient is then that of a weight of ones). Results are
rounded once, to nearest even: dx to x's dtype, dw and db to the parameters' dtype.
"""

import numpy as np

from .rounding import f32_param, round_to


def _rows(a):
    a = np.asarray(a, dtype=np.float64)
    return a.reshape(-1, a.shape[-1])


def rms_norm_vjp(x, w, g, eps, dtype, w_dtype=None):
    """Returns (dx, dw) for RMSNorm; dw is the gradient for w (a vector of ones if w is None)."""
    x2 = _rows(x)
    g2 = _rows(g)
    d = x2.shape[-1]
    wv = np.ones(d) if w is None else np.asarray(w, dtype=np.float64)
    r = 1.0 / np.sqrt(np.sum(x2 * x2, axis=-1, keepdims=True) / d + f32_param(eps))
    dot = np.sum(g2 * wv * x2, axis=-1, keepdims=True)
    dx = r * g2 * wv - x2 * (r ** 3) * dot / d
    dw = np.sum(g2 * x2 * r, axis=0)
    return (round_to(dx.reshape(np.shape(x)), dtype), round_to(dw, w_dtype or dtype))


def layer_norm_vjp(x, w, b, g, eps, dtype, w_dtype=None):
    """Returns (dx, dw, db) for LayerNorm (b does not enter the gradients).

    Two sums are written in a form that is equal by definition and stays accurate in
    float64 when a mean is large against the spread: the mean of x takes one correction
    step (mean + mean(x - mean), the corrected two-pass mean), and mean(d xh) is taken as
    mean((d - mean(d)) xh), which is the same number because mean(xh) = 0. Formed
    directly, mean(d xh) multiplies the rounding error of sum(xh) by mean(d)."""
    x2 = _rows(x)
    g2 = _rows(g)
    d = x2.shape[-1]
    wv = np.ones(d) if w is None else np.asarray(w, dtype=np.float64)
    mu = np.sum(x2, axis=-1, keepdims=True) / d
    mu = mu + np.sum(x2 - mu, axis=-1, keepdims=True) / d
    c = x2 - mu
    r = 1.0 / np.sqrt(np.sum(c * c, axis=-1, keepdims=True) / d + f32_param(eps))
    xh = c * r
    dxh = g2 * wv
    m1 = np.sum(dxh, axis=-1, keepdims=True) / d
    m2 = np.sum((dxh - m1) * xh, axis=-1, keepdims=True) / d
    dx = r * (dxh - m1 - xh * m2)
    dw = np.sum(g2 * xh, axis=0)
    db = np.sum(g2, axis=0)
    wd = w_dtype or dtype
    return (round_to(dx.reshape(np.shape(x)), dtype), round_to(dw, wd), round_to(db, wd))

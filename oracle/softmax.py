"""fp64 softmax family over the last axis (oracle; test infrastructure only).

Sources: nuvec-core 0.5.0 ``fast::FastOp`` (docs.rs), variants
  * ``Softmax``         -- (x): softmax over the last axis (the kernels accumulate in float32);
  * ``CausalSoftmax``   -- (x) with field ``rows``: Softmax of causally masked scores; row r of
                           the second-to-last axis (whose length is a multiple of ``rows``)
                           keeps the columns c <= r % rows + L - rows (L the last axis), every
                           other score is replaced by the dtype's lowest finite value;
  * ``LogSumExp``       -- (x): log(sum(exp(x))) over the last axis, which becomes size 1;
  * ``CrossEntropy``    -- (logits, targets): logsumexp(logits) - logits[target] per row, a
                           float32 result;
  * ``CrossEntropyVjp`` -- (logits, targets, loss, g): the gradient of CrossEntropy for the
                           logits, g * (softmax(logits) - onehot(target)) per row.
Every value is computed in float64 from the exact input values and rounded once: to the
input's dtype (Softmax, CausalSoftmax, LogSumExp, CrossEntropyVjp) or to float32
(CrossEntropy). A target outside [0, V) gives NaN (loss and gradient row): the pages do
not define it. ``loss`` does not enter the gradient's definition and is not read here.
"""

import numpy as np

from .rounding import round_to

# The lowest finite value of each storage dtype (what masked scores become).
LOWEST = {"bf16": -float.fromhex("0x1.fep127"), "f32": -float.fromhex("0x1.fffffep127"),
          "f64": -np.finfo(np.float64).max}


def _softmax64(x):
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def softmax(x, dtype):
    """exp(x - max) / sum over the last axis."""
    return round_to(_softmax64(x), dtype)


def causal_mask(R, L, rows):
    """[R, L] booleans: True where row r keeps column c (c <= r % rows + L - rows)."""
    assert R % rows == 0
    r = np.arange(R)[:, None] % rows
    c = np.arange(L)[None, :]
    return c <= r + L - rows


def causal_softmax(x, rows, dtype):
    """x [..., R, L]: masked scores take the dtype's lowest finite value, then softmax."""
    x = np.asarray(x, dtype=np.float64)
    keep = causal_mask(x.shape[-2], x.shape[-1], rows)
    return softmax(np.where(keep, x, LOWEST[dtype]), dtype)


def logsumexp(x, dtype):
    """log(sum(exp(x))) over the last axis, kept as an axis of size 1."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", over="ignore"):
        finite_m = np.where(np.isfinite(m), m, 0.0)
        out = finite_m + np.log(np.sum(np.exp(x - finite_m), axis=-1, keepdims=True))
    return round_to(out, dtype)


def _targets(targets, V):
    t = np.asarray(targets, dtype=np.int64).reshape(-1)
    valid = (t >= 0) & (t < V)
    return np.where(valid, t, 0), valid


def cross_entropy(logits, targets):
    """logsumexp(logits) - logits[target] per row of logits [rows, V]; float32 values."""
    x = np.asarray(logits, dtype=np.float64)
    x = x.reshape(-1, x.shape[-1])
    t, valid = _targets(targets, x.shape[-1])
    lse = logsumexp(x, "f64")[:, 0]
    loss = lse - x[np.arange(x.shape[0]), t]
    return round_to(np.where(valid, loss, np.nan), "f32")


def cross_entropy_vjp(logits, targets, g, dtype):
    """g[row] * (softmax(logits[row]) - onehot(targets[row])), rounded to dtype."""
    x = np.asarray(logits, dtype=np.float64)
    x = x.reshape(-1, x.shape[-1])
    t, valid = _targets(targets, x.shape[-1])
    d = _softmax64(x)
    d[np.arange(x.shape[0]), t] -= 1.0
    d = d * np.asarray(g, dtype=np.float64).reshape(-1, 1)
    d[~valid] = np.nan
    return round_to(d, dtype)

"""Element-by-element comparison rules for parity checks.

  * bit-exact: the residual sum h and cache placement (including untouched cache rows);
  * bf16 outputs: at most 1 apart as ordered integers (+0 and -0 equal; NaN only with NaN);
  * fp32 outputs: |got - want| <= 1e-6 + 1e-5 * |want| (NaN only with NaN; infinities equal).

Every check returns the largest distance and the count over tolerance, and raises with
both when the count is not zero.
"""

import numpy as np
import torch


def bf16_bits_of(t):
    """uint16 bit patterns of a bf16 tensor (any device) or of an array of bf16 values."""
    if isinstance(t, torch.Tensor):
        assert t.dtype == torch.bfloat16, t.dtype
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    v32 = np.asarray(t, dtype=np.float64).astype(np.float32)
    return (v32.view(np.uint32) >> 16).astype(np.uint16)


def f64_of(t):
    """float64 values of a tensor (exact for bf16 and fp32)."""
    return t.detach().cpu().to(torch.float64).numpy()


def _bf16_ordered(bits):
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _bf16_isnan(bits):
    b = bits.astype(np.int64)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def bf16_ulp_distance(got_bits, want_bits):
    g = np.asarray(got_bits, dtype=np.uint16).ravel()
    w = np.asarray(want_bits, dtype=np.uint16).ravel()
    d = np.abs(_bf16_ordered(g) - _bf16_ordered(w))
    gn, wn = _bf16_isnan(g), _bf16_isnan(w)
    d = np.where(gn & wn, 0, d)
    d = np.where(gn ^ wn, np.iinfo(np.int64).max, d)
    return d


def check_bf16(got, want, max_ulp=1, what="output"):
    d = bf16_ulp_distance(bf16_bits_of(got), bf16_bits_of(want))
    over = int(np.count_nonzero(d > max_ulp))
    worst = int(d.max()) if d.size else 0
    if over:
        idx = np.flatnonzero(d > max_ulp)[:8]
        raise AssertionError(
            f"{what}: {over} of {d.size} bf16 elements more than {max_ulp} ulp apart "
            f"(max {worst}); first flat indices {idx.tolist()}")
    return worst, over


def check_f32(got, want, rtol=1e-5, atol=1e-6, what="output"):
    g = np.asarray(got, dtype=np.float64).ravel()
    w = np.asarray(want, dtype=np.float64).ravel()
    gn, wn = np.isnan(g), np.isnan(w)
    with np.errstate(invalid="ignore"):
        err = np.abs(g - w)
        tol = atol + rtol * np.abs(w)
        bad = ~(err <= tol)
    both_inf_equal = np.isinf(g) & np.isinf(w) & (g == w)
    bad &= ~both_inf_equal
    bad = np.where(gn & wn, False, bad)
    bad |= gn ^ wn
    over = int(np.count_nonzero(bad))
    finite = np.isfinite(err)
    worst = float((err[finite] / tol[finite]).max()) if finite.any() else 0.0
    if over:
        idx = np.flatnonzero(bad)[:8]
        raise AssertionError(
            f"{what}: {over} of {g.size} fp32 elements outside {rtol} rel / {atol} abs "
            f"(worst err/tol {worst:.3g}); first flat indices {idx.tolist()}")
    return worst, over


def check_exact_bits(got, want, what="output"):
    """Bit-for-bit equality of two tensors or arrays of the same dtype."""
    if isinstance(got, torch.Tensor):
        got = got.detach().cpu().contiguous()
        g = got.view(torch.int16 if got.element_size() == 2 else torch.int32).numpy()
    else:
        g = np.asarray(got)
    if isinstance(want, torch.Tensor):
        want = want.detach().cpu().contiguous()
        w = want.view(torch.int16 if want.element_size() == 2 else torch.int32).numpy()
    else:
        w = np.asarray(want)
    bad = g.ravel() != w.ravel()
    over = int(np.count_nonzero(bad))
    if over:
        idx = np.flatnonzero(bad)[:8]
        raise AssertionError(f"{what}: {over} of {bad.size} elements differ in their bits; "
                             f"first flat indices {idx.tolist()}")
    return 0, 0


def check_output(got, want_f64, dtype, what="output"):
    """Compare a device/CPU tensor of ``dtype`` with oracle values (already rounded)."""
    if dtype == "bf16":
        return check_bf16(got, want_f64, what=what)
    return check_f32(f64_of(got), want_f64, what=what)


def bits_of_values(v, dtype):
    """Bit patterns of oracle values rounded to ``dtype`` (uint16 or uint32)."""
    if dtype == "bf16":
        return bf16_bits_of(v)
    return np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32)


def tensor_bits(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)

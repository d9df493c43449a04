"""Planted mistakes in copies of the oracle (CPU only): each must fail at least one pin.

A copy of ``oracle/`` is written to a temporary directory under a fresh package name with
one source edit, imported, and run through every pin; the test passes when some pin
raises. This shows the pins can tell a plausible mistake (a dropped term, a wrong sign or
index, a wrong divisor, a wrong rounding) from the real definition.
"""

import importlib
import os
import shutil
import sys

import pytest

import pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

# (file, text to replace, replacement, what the mistake is)
MUTANTS = [
    ("norms.py", "y = x / np.sqrt(mean_sq + f32_param(eps))", "y = x / np.sqrt(mean_sq)",
     "RmsNorm drops eps"),
    ("norms.py", "mean_sq = np.sum(x * x, axis=-1, keepdims=True) / d",
     "mean_sq = np.sum(x * x, axis=-1, keepdims=True)", "RmsNorm sums instead of averaging"),
    ("norms.py", "    if w is not None:\n        y = y * w\n    return round_to(y, dtype)\n\n\ndef add",
     "    return round_to(y, dtype)\n\n\ndef add", "RmsNorm ignores w"),
    ("norms.py", "y = x / np.sqrt(mean_sq + f32_param(eps))",
     "y = x / np.sqrt(mean_sq + eps)", "eps not taken as its float32 value"),
    ("norms.py", "h = round_to(_f64(x) + _f64(r), dtype)", "h = _f64(x) + _f64(r)",
     "residual h not rounded to the storage dtype"),
    ("norms.py", "return rms_norm(h, w, eps, dtype), h",
     "return rms_norm(_f64(x) + _f64(r), w, eps, dtype), h",
     "AddRmsNorm normalises the unrounded sum"),
    ("norms.py", "var = np.sum(centred * centred, axis=-1, keepdims=True) / d",
     "var = np.sum(centred * centred, axis=-1, keepdims=True) / (d - 1)",
     "LayerNorm uses the unbiased variance"),
    ("norms.py", "y = centred / np.sqrt(var + f32_param(eps))",
     "y = x / np.sqrt(var + f32_param(eps))", "LayerNorm does not centre the output"),
    ("norms.py", "y = centred / np.sqrt(var + f32_param(eps))",
     "y = centred / (np.sqrt(var) + f32_param(eps))", "LayerNorm adds eps outside the root"),
    ("norms.py", "y = y + b", "y = y - b", "LayerNorm subtracts the bias"),
    ("rounding.py", "np.rint(np.ldexp(y, -q))", "np.trunc(np.ldexp(y, -q))",
     "bf16 rounding truncates"),
    ("rounding.py", "np.rint(np.ldexp(y, -q))", "np.floor(np.ldexp(y, -q) + 0.5)",
     "bf16 rounding sends ties up"),
    ("rounding.py", "_BF16_MIN_QUANTUM_EXP = -133", "_BF16_MIN_QUANTUM_EXP = -126",
     "bf16 subnormals flushed"),
    ("rounding.py", "_BF16_SIG_BITS = 8", "_BF16_SIG_BITS = 7", "bf16 keeps one bit too few"),
    ("rope.py", "y[..., iu] = m * (u * c - v * s)\n    y[..., iv] = m * (u * s + v * c)",
     "y[..., iu] = m * (u * c + v * s)\n    y[..., iv] = m * (-u * s + v * c)",
     "rotation turns clockwise"),
    ("rope.py", "    if traditional:\n        return 2 * i, 2 * i + 1",
     "    if not traditional:\n        return 2 * i, 2 * i + 1", "pair modes swapped"),
    ("rope.py", "return i, i + half", "return i, i + half - 1", "half-mode partner off by one"),
    ("rope.py", "(-2.0 * i) / dims", "(-1.0 * i) / dims", "frequency exponent halved"),
    ("rope.py", "(-2.0 * i) / dims", "(-2.0 * i) / (dims - 2)", "frequency exponent over dims - 2"),
    ("rope.py", "rope_angles(offset + np.arange(L)", "rope_angles(np.arange(L)",
     "offset ignored"),
    ("rope.py", "rope_angles(offset + np.arange(L)", "rope_angles(offset + np.arange(L) + 1",
     "positions start one late"),
    ("rope.py", "return (f32_param(scale) * p)", "return (p + 0 * f32_param(scale))",
     "scale ignored"),
    ("rope.py", "        s = -s", "        s = s", "inverse rotation not inverted"),
    ("rope.py", "mean_sq = np.sum(x * x, axis=-1, keepdims=True) / D",
     "mean_sq = np.sum(x[..., :dims] ** 2, axis=-1, keepdims=True) / max(dims, 1)",
     "RMS over the rotated features only"),
    ("rope.py", "xn = xn * np.asarray(w, dtype=np.float64)", "xn = xn",
     "NormRope ignores w"),
    ("rope.py", "out[:, :, offset:offset + L, :] = y", "out[:, :, 0:L, :] = y",
     "cache written from row 0"),
    ("rope.py", "xn = x / np.sqrt(mean_sq + f32_param(eps))", "xn = x / np.sqrt(mean_sq)",
     "NormRope drops eps"),
    ("rope.py", "return 1.0 / f", "return f", "freqs taken as frequencies, not divisors"),
    ("rope.py", "m = f32_param(mscale)", "m = 1.0", "mscale ignored"),
    ("rope.py", "y[..., iv] = m * (u * s + v * c)", "y[..., iv] = u * s + v * c",
     "mscale on one half of each pair only"),
    ("rope.py", "a = rope_angles(np.asarray(positions), dims, base, scale, freqs)",
     "a = rope_angles(np.arange(len(positions)), dims, base, scale, freqs)",
     "positions tensor ignored"),
    ("rope_scaling.py", "out[wavelen > low_wavelen] = f[wavelen > low_wavelen] * factor",
     "out[wavelen > low_wavelen] = f[wavelen > low_wavelen] / factor",
     "Llama 3 low-frequency pairs divided by the factor"),
    ("rope_scaling.py", "high_wavelen = original_max / high_freq_factor",
     "high_wavelen = original_max / low_freq_factor / 2", "Llama 3 high edge misplaced"),
    ("rope_scaling.py", "out[mid] = f[mid] / ((1.0 - s) / factor + s)",
     "out[mid] = f[mid] / (s / factor + (1.0 - s))", "Llama 3 blend weights swapped"),
    ("rope_scaling.py", "keep = 1.0 - ramp", "keep = ramp", "YaRN ramp reversed"),
    ("rope_scaling.py", "inv = keep / f + (1.0 - keep) / (factor * f)",
     "inv = 1.0 / (keep * f + (1.0 - keep) * factor * f)",
     "YaRN blends the divisors instead of the inverse frequencies"),
    ("rope_scaling.py", "inv = keep / f + (1.0 - keep) / (factor * f)",
     "inv = 1.0 / (f * factor ** (1.0 - keep))",
     "YaRN blends geometrically"),
    ("rope_scaling.py", "low = max(math.floor(corr_dim(beta_fast)), 0)",
     "low = max(math.floor(corr_dim(beta_slow)), 0)", "YaRN ramp start from beta_slow"),
    ("rope_scaling.py", "return 1.0 if s <= 1 else 0.1 * m * math.log(s) + 1.0",
     "return 1.0 if s <= 1 else 0.1 * m * math.log10(s) + 1.0", "YaRN attention factor log10"),
    ("rope_scaling.py", "ms = math.sqrt(1.0 + math.log(max_position / original_max) / math.log(original_max))",
     "ms = 1.0 + math.log(max_position / original_max) / math.log(original_max)",
     "su attention factor without the root"),
    ("rope_scaling.py", "out = round_to(lf * _base_periods(dims, base), \"f32\")",
     "out = round_to(lf / _base_periods(dims, base), \"f32\")", "su factors divide"),
    ("softmax.py", "    return c <= r + L - rows", "    return c <= r + L - rows - 1",
     "causal mask one column short"),
    ("softmax.py", "    return c <= r + L - rows", "    return c <= r", "causal mask not aligned at the end"),
    ("softmax.py", "    e = np.exp(x - m)\n    return e / np.sum(e, axis=-1, keepdims=True)",
     "    e = np.exp(x)\n    return e / np.sum(e, axis=-1, keepdims=True)",
     "softmax without the maximum taken out"),
    ("softmax.py", "return softmax(np.where(keep, x, LOWEST[dtype]), dtype)",
     "return softmax(np.where(keep, x, -np.inf), dtype)", "masked scores as -inf"),
    ("softmax.py", "out = finite_m + np.log(np.sum(np.exp(x - finite_m), axis=-1, keepdims=True))",
     "out = np.log(np.sum(np.exp(x - finite_m), axis=-1, keepdims=True))",
     "logsumexp drops the maximum"),
    ("softmax.py", "loss = lse - x[np.arange(x.shape[0]), t]", "loss = x[np.arange(x.shape[0]), t] - lse",
     "cross-entropy sign"),
    ("softmax.py", "    d[np.arange(x.shape[0]), t] -= 1.0\n", "", "gradient without the one-hot"),
    ("softmax.py", "    d = d * np.asarray(g, dtype=np.float64).reshape(-1, 1)\n", "",
     "gradient ignores g"),
    ("vjp.py", "x2 * (r ** 3) * dot / d", "x2 * (r ** 2) * dot / d", "RmsNormVjp r^2 for r^3"),
    ("vjp.py", "dx = r * g2 * wv - x2 * (r ** 3) * dot / d", "dx = r * g2 * wv",
     "RmsNormVjp drops the term through the statistic"),
    ("vjp.py", "dot = np.sum(g2 * wv * x2", "dot = np.sum(g2 * x2", "RmsNormVjp dot ignores w"),
    ("vjp.py", "dw = np.sum(g2 * x2 * r, axis=0)", "dw = np.sum(g2 * x2, axis=0)",
     "RmsNormVjp dw not normalised"),
    ("vjp.py", "dw = np.sum(g2 * x2 * r, axis=0)", "dw = np.mean(g2 * x2 * r, axis=0)",
     "RmsNormVjp dw averages over rows"),
    ("vjp.py", "x2 * x2, axis=-1, keepdims=True) / d + f32_param(eps)",
     "x2 * x2, axis=-1, keepdims=True) / d", "RmsNormVjp drops eps"),
    ("vjp.py", "dx = r * (dxh - m1 - xh * m2)", "dx = r * (dxh - m1 + xh * m2)",
     "LayerNormVjp wrong sign on the variance term"),
    ("vjp.py", "dx = r * (dxh - m1 - xh * m2)", "dx = r * (dxh - xh * m2)",
     "LayerNormVjp drops the mean term"),
    ("vjp.py", "dxh = g2 * wv", "dxh = g2", "LayerNormVjp dx ignores w"),
    ("vjp.py", "dw = np.sum(g2 * xh, axis=0)", "dw = np.sum(g2 * c, axis=0)",
     "LayerNormVjp dw uses the uncentred-unscaled x"),
    ("vjp.py", "db = np.sum(g2, axis=0)", "db = np.sum(g2 * wv, axis=0)",
     "LayerNormVjp db scaled by w"),
    ("vjp.py", "np.sum(c * c, axis=-1, keepdims=True) / d", "np.sum(c * c, axis=-1, keepdims=True) / (d - 1)",
     "LayerNormVjp unbiased variance"),
    ("vjp.py", "m2 = np.sum((dxh - m1) * xh, axis=-1, keepdims=True) / d",
     "m2 = np.sum(dxh * c, axis=-1, keepdims=True) / d", "LayerNormVjp m2 not normalised"),
]


def _load_mutant(tmp_path, k, fname, old, new):
    name = f"oracle_mutant_{k}"
    dst = tmp_path / name
    shutil.copytree(ORACLE_DIR, dst, ignore=shutil.ignore_patterns("__pycache__"))
    path = dst / fname
    src = path.read_text()
    assert src.count(old) >= 1, f"mutation text not found in {fname}: {old!r}"
    path.write_text(src.replace(old, new, 1))
    sys.path.insert(0, str(tmp_path))
    try:
        return importlib.import_module(name)
    finally:
        sys.path.remove(str(tmp_path))


@pytest.mark.parametrize("k", range(len(MUTANTS)), ids=[m[3] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(tmp_path, k):
    fname, old, new, what = MUTANTS[k]
    mutant = _load_mutant(tmp_path, k, fname, old, new)
    for pin in pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError, IndexError):
            return
    pytest.fail(f"no pin caught the planted mistake: {what}")

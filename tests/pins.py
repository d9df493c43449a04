"""Pins of the fp64 oracle to things other than itself.

Every pin is a function of the oracle module, so the same pins run against the real oracle
(``test_oracle_pins.py``) and against copies of it with a planted mistake
(``test_oracle_mutants.py``, which demands that every planted mistake fails some pin).

What pins what:
  * rounding      -- torch's float32 -> bfloat16 cast (a library routine) on float32 inputs;
                     exact rational rounding (``brute.round_fraction``) on float64 inputs,
                     including the double-rounding hazards;
  * RmsNorm       -- hand-worked fixtures, the constant-row closed form, mean(out^2) =
                     ms/(ms+eps), power-of-two scale invariance (bit-exact), torch's
                     ``rms_norm`` in float64, 50-digit brute force;
  * AddRmsNorm    -- hand-worked fixtures, h against torch's float32 add + cast, out against
                     RmsNorm of the returned h, 50-digit brute force;
  * LayerNorm     -- hand-worked fixtures, constant row gives b, no-affine moments,
                     torch's ``layer_norm`` in float64, 50-digit brute force;
  * NormRope      -- hand-worked fixtures (cos 1, sin 1 ...), identity at position 0,
                     per-pair norm preservation, inverse undoes forward, half/interleaved
                     permutation, relative-position property, cache placement, RMS over
                     all D, 50-digit brute force.
  * Rope freqs /  -- 50-digit brute force with freqs and mscale, freqs = base^(2i/dims)
    positions        reproduces the base form, mscale is a plain factor, the positions form
                     equals the offset form row by row;
  * scaled freqs  -- band properties of each published method (pairs kept, pairs scaled by
                     the factor, the blend in between and its continuity at the band edges,
                     ramp ends, closed-form attention factors), identity at factor 1;
  * softmax family -- hand-worked fixtures (equal shares, underflow, causal rows with and
                     without survivors, ln 4), 50-digit brute force (the gradient by numerical
                     differentiation of the loss), torch's softmax / logsumexp /
                     cross_entropy and its autograd in float64, invariants (rows sum to 1,
                     shift invariance, LSE(x + c) = LSE(x) + c, gradient rows sum to 0);
  * RmsNormVjp /  -- hand-worked fixtures, 50-digit numerical differentiation of the
    LayerNormVjp     forward (brute force), torch autograd of ``rms_norm`` / ``layer_norm``
                     in float64, and the invariances every gradient of these maps obeys
                     (RMS: x . dx = 0 at eps = 0; LN: sum(dx) = 0, and x . dx = 0 at
                     eps = 0; db = column sums of g).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

import brute
import mpmath

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _vals(strs):
    return None if strs is None else np.array([float(Fraction(s)) for s in strs])


def _rng(seed=1234):
    return np.random.default_rng(seed)


def _bf16_values(a):
    """Round arbitrary draws onto the bf16 grid with torch (input preparation only)."""
    t = torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def _f32_values(a):
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    ok = np.abs(a - b) <= atol + rtol * np.abs(b)
    assert ok.all(), f"{what}: max abs diff {np.max(np.abs(a - b))}"


def _same_values(a, b, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    ok = (a == b) | (np.isnan(a) & np.isnan(b))
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} values differ"


# ------------------------------------------------------------------------------ rounding

def pin_round_bf16_matches_torch_on_f32(o):
    """Every float32 input (random bit patterns across all exponents, plus ties, subnormals
    and the overflow edge) rounds as torch's float32 -> bfloat16 cast does."""
    rng = _rng(1)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2**16, size=20_000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    special = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0xFF7F8000, 0x00008000, 0x00018000,
                        0x80008000, 0x00000001, 0x3F808000, 0x3F818000, 0x00000000, 0x80000000,
                        0x7F800000, 0xFF800000], dtype=np.uint32)
    allbits = np.concatenate([bits, ties, special])
    v = allbits.view(np.float32)
    v = v[~np.isnan(v)]
    want = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = o.bf16_bits(o.round_bf16(v.astype(np.float64)))
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} mismatches"


def pin_round_exact_on_f64(o):
    """float64 inputs (not float32 values) round to the nearest bf16 / fp32 value of the
    exact input, ties to even, as exact rational arithmetic decides. Includes values a hair
    past a bf16 midpoint whose float32 rounding would land on the midpoint (the double
    rounding trap) and exact midpoints."""
    rng = _rng(2)
    cases = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 130, 3000)))
    for m in range(1, 64):
        mid = 1.0 + (2 * m + 1) * 2.0 ** -8
        cases += [mid, mid + 2.0 ** -40, mid - 2.0 ** -40, -mid, -(mid + 2.0 ** -40)]
        cases += [mid * 2.0 ** -130, (mid + 2.0 ** -30) * 2.0 ** -131]
    f32mid = 1.0 + 2.0 ** -24
    cases += [f32mid, f32mid + 2.0 ** -50, 1.0 + 3 * 2.0 ** -24, 3.4e38, 3.403e38, 1e-45, 7e-46]
    for y in cases:
        for fmt, fn in (("bf16", o.round_bf16), ("f32", o.round_f32)):
            want = brute.round_fraction(Fraction(y), fmt)
            got = float(fn(np.array([y]))[0])
            assert got == want, (fmt, y, got, want)


def pin_round_specials(o):
    """NaN stays NaN, infinities stay, the sign of zero and of tiny values is kept."""
    y = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, -1e-300, 1e-300])
    for fn in (o.round_bf16, o.round_f32):
        r = fn(y)
        assert np.isnan(r[0]) and r[1] == np.inf and r[2] == -np.inf
        assert np.signbit(r[4]) and not np.signbit(r[3])
        assert r[5] == 0 and np.signbit(r[5]) and r[6] == 0 and not np.signbit(r[6])


# ------------------------------------------------------------------------------- RmsNorm

def pin_rms_golden(o):
    g = _golden("rms_norm_hand.json")
    for c in g["cases"]:
        x = _vals(c["x"])[None, :]
        w = _vals(c["w"])
        want = _vals(c["expect"])
        got = o.rms_norm(x, w, c["eps"], "f64")[0]
        _close(got, want, 1e-15, 1e-300, c["why"])
        for dt in ("bf16", "f32"):
            gr = o.rms_norm(x, w, c["eps"], dt)[0]
            exp = [brute.round_fraction(Fraction(s), dt) for s in c["expect"]]
            _same_values(gr, exp, c["why"])


def pin_rms_constant_row(o):
    """x = c everywhere: out_j = w_j c / sqrt(c^2 + eps), eps taken as its float32 value."""
    rng = _rng(3)
    for c in (1.0, -3.25, 1e-3, 7e4, 2.0 ** -20):
        for eps in (1e-6, 1e-5, 0.1):
            w = rng.uniform(0.5, 1.5, 16)
            x = np.full((1, 16), c)
            got = o.rms_norm(x, w, eps, "f64")[0]
            e = float(np.float32(eps))
            want = w * c / math.sqrt(c * c + e)
            _close(got, want, 1e-14, 0, f"c={c} eps={eps}")


def pin_rms_mean_square(o):
    """With w = 1: mean(out^2) = ms / (ms + eps)."""
    rng = _rng(4)
    x = rng.standard_normal((32, 300)) * np.exp(rng.uniform(-6, 6, (32, 1)))
    for eps in (1e-6, 1e-2, 0.5):
        out = o.rms_norm(x, None, eps, "f64")
        ms = np.mean(x * x, axis=-1)
        e = float(np.float32(eps))
        _close(np.mean(out * out, axis=-1), ms / (ms + e), 1e-12, 0, f"eps={eps}")


def pin_rms_scale_invariance(o):
    """eps = 0: RMSNorm(alpha x) == RMSNorm(x) bit for bit for alpha = 2^k (every step scales
    exactly), and to 1e-13 for other alpha."""
    rng = _rng(5)
    x = _bf16_values(rng.standard_normal((16, 256)))
    w = _bf16_values(rng.normal(1, 0.1, 256))
    for dt in ("bf16", "f32", "f64"):
        base = o.rms_norm(x, w, 0.0, dt)
        for k in (-7, -1, 1, 5, 20):
            _same_values(o.rms_norm(x * 2.0 ** k, w, 0.0, dt), base, f"2^{k} {dt}")
    base = o.rms_norm(x, w, 0.0, "f64")
    for alpha in (3.0, -0.7, 1e5):
        _close(o.rms_norm(x * alpha, w, 0.0, "f64"), np.sign(alpha) * base, 1e-13, 1e-300)


def pin_rms_torch(o):
    """torch.nn.functional.rms_norm in float64 on the CPU (an independent library routine)."""
    rng = _rng(6)
    for d in (1, 7, 64, 1000):
        x = rng.standard_normal((9, d)) * 3
        w = rng.normal(1, 0.2, d)
        for eps in (1e-6, 1e-5, 0.25):
            e = float(np.float32(eps))
            want = torch.nn.functional.rms_norm(torch.from_numpy(x), (d,), torch.from_numpy(w),
                                                eps=e).numpy()
            _close(o.rms_norm(x, w, eps, "f64"), want, 1e-13, 1e-300, f"d={d}")
            want1 = torch.nn.functional.rms_norm(torch.from_numpy(x), (d,), None, eps=e).numpy()
            _close(o.rms_norm(x, None, eps, "f64"), want1, 1e-13, 1e-300, f"d={d} no w")


def pin_rms_brute(o):
    """2 x 8 inputs against the 50-digit evaluation, rounded exactly."""
    rng = _rng(7)
    for dt, cast in (("bf16", _bf16_values), ("f32", _f32_values)):
        for eps in (1e-6, 0.3):
            x = cast(rng.standard_normal((2, 8)) * 2)
            w = cast(rng.uniform(0.5, 1.5, 8))
            got = o.rms_norm(x, w, eps, dt)
            for i in range(2):
                want = [brute.round_mp(v, dt) for v in brute.rms_row(x[i], w, eps)]
                _same_values(got[i], want, f"{dt} row {i}")


# ---------------------------------------------------------------------------- AddRmsNorm

def pin_add_golden(o):
    g = _golden("add_rms_norm_hand.json")
    for c in g["cases"]:
        x = _vals(c["x"])[None, :]
        r = _vals(c["r"])[None, :]
        out, h = o.add_rms_norm(x, r, _vals(c["w"]), c["eps"], c["dtype"])
        _same_values(h[0], _vals(c["expect_h"]), c["why"])
        if c["expect"] is not None:
            exp = [brute.round_fraction(Fraction(s), c["dtype"]) for s in c["expect"]]
            _same_values(out[0], exp, c["why"])


def pin_add_residual_torch(o):
    """h equals torch's (x.float() + r.float()).to(dtype) bit for bit: one float32 add then
    one rounding is the correctly rounded sum for these formats."""
    rng = _rng(8)
    for dt, tdt in (("bf16", torch.bfloat16), ("f32", torch.float32)):
        for scale in (1.0, 1e3, 1e-30):
            xt = torch.from_numpy(rng.standard_t(3, (64, 96)) * scale).to(tdt)
            rt = torch.from_numpy(rng.standard_t(3, (64, 96)) * scale).to(tdt)
            want = (xt.float() + rt.float()).to(tdt).to(torch.float64).numpy()
            _, h = o.add_rms_norm(xt.to(torch.float64).numpy(), rt.to(torch.float64).numpy(),
                                  None, 1e-6, dt)
            _same_values(h, want, f"{dt} scale {scale}")


def pin_add_normalises_returned_h(o):
    """out is RmsNorm of the returned (rounded) h, bit for bit."""
    rng = _rng(9)
    for dt, cast in (("bf16", _bf16_values), ("f32", _f32_values)):
        x = cast(rng.standard_normal((64, 40)))
        r = cast(rng.standard_normal((64, 40)))
        w = cast(rng.uniform(0.5, 1.5, 40))
        out, h = o.add_rms_norm(x, r, w, 1e-6, dt)
        _same_values(out, o.rms_norm(h, w, 1e-6, dt), dt)


def pin_add_brute(o):
    rng = _rng(10)
    for dt, cast in (("bf16", _bf16_values), ("f32", _f32_values)):
        x = cast(rng.standard_normal((2, 8)))
        r = cast(rng.standard_normal((2, 8)))
        w = cast(rng.normal(1, 0.1, 8))
        out, h = o.add_rms_norm(x, r, w, 1e-6, dt)
        for i in range(2):
            hs = [brute.round_fraction(Fraction(float(a)) + Fraction(float(b)), dt)
                  for a, b in zip(x[i], r[i])]
            _same_values(h[i], hs, "h")
            want = [brute.round_mp(v, dt) for v in brute.rms_row(hs, w, 1e-6)]
            _same_values(out[i], want, f"{dt} row {i}")


# ----------------------------------------------------------------------------- LayerNorm

def pin_ln_golden(o):
    g = _golden("layer_norm_hand.json")
    for c in g["cases"]:
        x = _vals(c["x"])[None, :]
        got = o.layer_norm(x, _vals(c["w"]), _vals(c["b"]), c["eps"], "f64")[0]
        if "expect" in c:
            _close(got, _vals(c["expect"]), 1e-15, 1e-300, c["why"])
        else:
            _close(got, np.array([float(s) for s in c["expect_decimal"]]), 1e-15, 0, c["why"])


def pin_ln_constant_row(o):
    """A constant row of bf16 values gives exactly b (and 0 without b)."""
    rng = _rng(11)
    for d in (1, 5, 4096, 8192):
        c = float(_bf16_values([rng.normal(0.5, 2)])[0])
        x = np.full((2, d), c)
        w = _bf16_values(rng.normal(1, 0.1, d))
        b = _bf16_values(rng.normal(0, 0.1, d))
        for dt in ("bf16", "f32"):
            _same_values(o.layer_norm(x, w, b, 1e-5, dt)[0], b, f"d={d}")
            assert np.all(o.layer_norm(x, w, None, 1e-5, dt) == 0)


def pin_ln_moments(o):
    """Without affine: mean(out) = 0 and mean(out^2) = v / (v + eps), v the biased variance."""
    rng = _rng(12)
    x = rng.normal(0.5, 2, (16, 513)) + rng.normal(0, 50, (16, 1))
    for eps in (1e-5, 0.5):
        out = o.layer_norm(x, None, None, eps, "f64")
        v = np.var(x, axis=-1)
        e = float(np.float32(eps))
        _close(np.mean(out, axis=-1), np.zeros(16), 0, 1e-13, "mean")
        _close(np.mean(out * out, axis=-1), v / (v + e), 1e-12, 0, "variance")


def pin_ln_torch(o):
    """torch.nn.functional.layer_norm in float64 on the CPU, affine, scale-only and none."""
    rng = _rng(13)
    for d in (2, 33, 1024):
        x = rng.normal(0.5, 2, (7, d))
        w = rng.normal(1, 0.1, d)
        b = rng.normal(0, 0.1, d)
        for eps in (1e-5, 0.1):
            e = float(np.float32(eps))
            for ww, bb in ((w, b), (w, None), (None, None)):
                want = torch.nn.functional.layer_norm(
                    torch.from_numpy(x), (d,),
                    None if ww is None else torch.from_numpy(ww),
                    None if bb is None else torch.from_numpy(bb), eps=e).numpy()
                _close(o.layer_norm(x, ww, bb, eps, "f64"), want, 1e-12, 1e-14, f"d={d}")


def pin_ln_brute(o):
    rng = _rng(14)
    for dt, cast in (("bf16", _bf16_values), ("f32", _f32_values)):
        x = cast(rng.normal(0.5, 2, (2, 8)))
        w = cast(rng.normal(1, 0.1, 8))
        b = cast(rng.normal(0, 0.1, 8))
        for ww, bb in ((w, b), (None, None)):
            got = o.layer_norm(x, ww, bb, 1e-5, dt)
            for i in range(2):
                want = [brute.round_mp(v, dt) for v in brute.layer_row(x[i], ww, bb, 1e-5)]
                _same_values(got[i], want, f"{dt} row {i}")


# ------------------------------------------------------------------------------ NormRope

def _rope(o, x, w=None, **kw):
    args = dict(normalize=True, eps=1e-6, dims=x.shape[-1], traditional=False, base=10000.0,
                scale=1.0, offset=0, forward=True, dtype="f64")
    args.update(kw)
    return o.norm_rope(x, w, **args)


def pin_rope_golden(o):
    g = _golden("rope_hand.json")
    for c in g["cases"]:
        x = _vals(c["x"]).reshape(1, 1, 1, -1)
        extra = {}
        if "freqs" in c:
            extra = dict(freqs=_vals(c["freqs"]), mscale=c["mscale"])
        got = _rope(o, x, None, normalize=c["normalize"], eps=c.get("eps", 0.0), dims=c["dims"],
                    traditional=c["traditional"], base=c["base"], scale=c["scale"],
                    offset=c["offset"], forward=c["forward"], **extra)[0, 0, 0]
        if "expect" in c:
            _close(got, _vals(c["expect"]), 1e-15, 1e-300, c["why"])
        else:
            _close(got, np.array([float(s) for s in c["expect_decimal"]]), 1e-14, 1e-15, c["why"])


def pin_rope_frequencies(o):
    """theta_i against 50-digit powers, and angle = scale * position * theta_i."""
    for dims, base in ((128, 10000.0), (64, 500000.0), (6, 3.0)):
        th = o.rope_frequencies(dims, base)
        assert th.shape == (dims // 2,)
        want = [float(brute.mpmath.power(brute.f32(base), brute.mpmath.mpf(-2 * i) / dims))
                for i in range(dims // 2)]
        _close(th, want, 4.5e-16, 0, f"dims={dims}")
    a = o.rope_angles([0, 5, 1535], 128, 10000.0, 0.75)
    _close(a[2], 0.75 * 1535 * o.rope_frequencies(128, 10000.0), 4.5e-16, 0, "angles")
    _close(a[:, 0], [0.0, 3.75, 0.75 * 1535], 0, 0, "pair 0 angle is scale * position")


def pin_rope_identity_at_zero(o):
    """Position 0 (offset 0, l = 0) is RmsNorm of the row; other positions are not."""
    rng = _rng(15)
    x = _bf16_values(rng.standard_normal((2, 3, 4, 64)))
    w = _bf16_values(rng.uniform(0.5, 1.5, 64))
    for trad in (False, True):
        for dt in ("bf16", "f32", "f64"):
            y = _rope(o, x, w, traditional=trad, dtype=dt)
            _same_values(y[:, :, 0], o.rms_norm(x[:, :, 0], w, 1e-6, dt), "p=0")
            assert not np.array_equal(y[:, :, 1], o.rms_norm(x[:, :, 1], w, 1e-6, dt))


def pin_rope_norm_preserving(o):
    """Each pair keeps its length: u'^2 + v'^2 = u^2 + v^2."""
    rng = _rng(16)
    x = rng.standard_normal((2, 2, 8, 32))
    for trad in (False, True):
        xn = _rope(o, x, None, normalize=False, offset=900, scale=1.5, traditional=trad)
        idx = np.arange(16)
        iu, iv = (2 * idx, 2 * idx + 1) if trad else (idx, idx + 16)
        _close(xn[..., iu] ** 2 + xn[..., iv] ** 2, x[..., iu] ** 2 + x[..., iv] ** 2, 1e-12, 1e-14)
        assert not np.allclose(xn, x)


def pin_rope_inverse(o):
    """forward=false undoes forward=true (the normalised row comes back)."""
    rng = _rng(17)
    x = rng.standard_normal((2, 2, 16, 48))
    w = rng.uniform(0.5, 1.5, 48)
    for trad in (False, True):
        for dims in (48, 32, 0):
            kw = dict(dims=dims, traditional=trad, offset=1024, base=5000.0, scale=0.9)
            y = _rope(o, x, w, **kw)
            back = _rope(o, y, None, normalize=False, forward=False, **kw)
            _close(back, _rope(o, x, w, **dict(kw, offset=0, scale=0.0)), 1e-12, 1e-13)


def pin_rope_half_vs_interleaved(o):
    """Interleaved mode equals half mode on the first dims features de-interleaved."""
    rng = _rng(18)
    D, dims = 40, 24
    x = rng.standard_normal((1, 2, 5, D))
    w = rng.uniform(0.5, 1.5, D)
    perm = np.concatenate([np.arange(0, dims, 2), np.arange(1, dims, 2), np.arange(dims, D)])
    inv = np.argsort(perm)
    a = _rope(o, x, w, dims=dims, traditional=True, offset=3)
    b = _rope(o, x[..., perm], w[perm], dims=dims, traditional=False, offset=3)[..., inv]
    _close(a, b, 1e-13, 1e-15)  # the sum of squares runs in another order


def pin_rope_relative_position(o):
    """<R_m q, R_n k> depends only on m - n (the property RoPE is built for)."""
    rng = _rng(19)
    q = rng.standard_normal((1, 1, 1, 64))
    k = rng.standard_normal((1, 1, 1, 64))
    for trad in (False, True):
        def rot(v, p):
            return _rope(o, v, None, normalize=False, offset=p, traditional=trad)[0, 0, 0]
        for m, n, s in ((5, 2, 100), (0, 40, 777), (1500, 1499, -1499)):
            a = np.dot(rot(q, m), rot(k, n))
            b = np.dot(rot(q, m + s), rot(k, n + s))
            assert abs(a - b) <= 1e-12 * (1 + abs(a)), (m, n, s, a, b)


def pin_rope_passthrough_and_span(o):
    """Features >= dims equal RmsNorm of the whole row (RMS over all D, not rotated)."""
    rng = _rng(20)
    x = rng.standard_normal((2, 2, 6, 24))
    w = rng.uniform(0.5, 1.5, 24)
    y = _rope(o, x, w, dims=8, offset=11)
    _same_values(y[..., 8:], o.rms_norm(x, w, 1e-6, "f64")[..., 8:], "passthrough")
    y0 = _rope(o, x, None, dims=8, offset=11, normalize=False)
    _same_values(y0[..., 8:], x[..., 8:], "no normalisation")


def pin_rope_cache(o):
    """Cache rows offset .. offset + L - 1 hold the plain result; the rest keep their values."""
    rng = _rng(21)
    x = _bf16_values(rng.standard_normal((2, 3, 5, 16)))
    w = _bf16_values(rng.uniform(0.5, 1.5, 16))
    cache = _bf16_values(rng.standard_normal((2, 3, 12, 16)))
    for trad in (False, True):
        kw = dict(traditional=trad, offset=6, dtype="bf16")
        y = _rope(o, x, w, **kw)
        c = _rope(o, x, w, cache=cache, **kw)
        _same_values(c[:, :, 6:11], y, "written rows")
        _same_values(c[:, :, :6], cache[:, :, :6], "rows before")
        _same_values(c[:, :, 11:], cache[:, :, 11:], "rows after")


def pin_rope_brute(o):
    """B = H = 1, L = 2, D = 8, dims 4 and 8, both modes, both directions, with and without
    normalisation, against 50-digit evaluation rounded exactly."""
    rng = _rng(22)
    for dt, cast in (("bf16", _bf16_values), ("f32", _f32_values)):
        x = cast(rng.standard_normal((1, 1, 2, 8)))
        w = cast(rng.uniform(0.5, 1.5, 8))
        for dims in (4, 8):
            for trad in (False, True):
                for fwd in (True, False):
                    for norm in (True, False):
                        kw = dict(normalize=norm, eps=1e-6, dims=dims, traditional=trad,
                                  base=10000.0, scale=1.0, forward=fwd)
                        got = o.norm_rope(x, w, offset=700, dtype=dt, **kw)
                        for l in range(2):
                            want = [brute.round_mp(v, dt) for v in
                                    brute.rope_row(x[0, 0, l], w, pos=700 + l, **kw)]
                            _same_values(got[0, 0, l], want, f"{dt} {kw} l={l}")


# ------------------------------------------------------------- Rope freqs / positions

def pin_rope_freqs_brute(o):
    """Rotation with a freqs vector and an mscale against the 50-digit evaluation."""
    rng = _rng(31)
    for dt, cast in (("bf16", _bf16_values), ("f32", _f32_values)):
        for trad in (False, True):
            x = cast(rng.standard_normal((1, 1, 2, 8)))
            freqs = _f32_values(rng.uniform(0.5, 300.0, 2))
            got = o.norm_rope(x, None, normalize=False, eps=1e-6, dims=4, traditional=trad,
                              base=10000.0, scale=0.5, offset=37, forward=True, dtype=dt,
                              freqs=freqs, mscale=1.25)
            for l in range(2):
                want = brute.rope_row(x[0, 0, l], None, normalize=False, eps=1e-6, dims=4,
                                      traditional=trad, base=10000.0, scale=0.5, pos=37 + l,
                                      forward=True, freqs=freqs.tolist(), mscale=1.25)
                _same_values(got[0, 0, l], [brute.round_mp(v, dt) for v in want], f"{dt} {l}")


def pin_rope_freqs_reproduce_base(o):
    """freqs[i] = base^(2i/dims) (rounded to f32) gives the base form, to the angle change
    that rounding makes (relative 2^-24 of an angle of at most 40 rad here)."""
    rng = _rng(32)
    x = rng.standard_normal((2, 3, 40, 16))
    f = np.power(10000.0, 2.0 * np.arange(6) / 12).astype(np.float32).astype(np.float64)
    kw = dict(normalize=False, eps=1e-6, dims=12, base=10000.0, scale=1.0, offset=0,
              forward=True, dtype="f64")
    for trad in (False, True):
        a = o.norm_rope(x, None, traditional=trad, **kw)
        b = o.norm_rope(x, None, traditional=trad, freqs=f, **kw)
        _close(b, a, 0, 40 * 2.0 ** -23 * np.max(np.abs(x)) * 2, "freqs vs base")


def pin_rope_mscale_is_a_factor(o):
    rng = _rng(33)
    x = rng.standard_normal((1, 2, 5, 10))
    kw = dict(normalize=False, eps=1e-6, dims=6, traditional=False, base=500.0, scale=1.0,
              offset=3, forward=True, dtype="f64")
    a = o.norm_rope(x, None, **kw)
    b = o.norm_rope(x, None, mscale=2.0, **kw)
    _same_values(b[..., :6], 2.0 * a[..., :6], "rotated features doubled")
    _same_values(b[..., 6:], a[..., 6:], "pass-through features unchanged")


def pin_rope_positions_form(o):
    """[T, H, D] rows with positions p[t] equal the [B, H, L, D] form at offset p[t] (one
    row each), head by head."""
    rng = _rng(34)
    T, H, D = 5, 3, 8
    x = _bf16_values(rng.standard_normal((T, H, D)))
    pos = np.array([7, 0, 3000, 7, 42])
    f = _f32_values(rng.uniform(1.0, 50.0, 3))
    for trad in (False, True):
        for freqs in (None, f):
            got = o.rope_positions(x, pos, dims=6, traditional=trad, base=100.0, scale=0.75,
                                   forward=False, dtype="bf16", freqs=freqs, mscale=1.5)
            for t in range(T):
                want = o.norm_rope(x[t][None, :, None, :], None, normalize=False, eps=1e-6,
                                   dims=6, traditional=trad, base=100.0, scale=0.75,
                                   offset=int(pos[t]), forward=False, dtype="bf16",
                                   freqs=freqs, mscale=1.5)
                _same_values(got[t], want[0, :, 0, :], f"token {t}")


# ------------------------------------------------------------------ scaled frequencies

def pin_llama3_bands(o):
    """Pairs with wavelength 2 pi f below original_max / high_freq_factor keep f, above
    original_max / low_freq_factor get factor * f, in between lie strictly between and grow
    with the wavelength; factor 1 changes nothing."""
    S = o.rope_scaling
    for dims, base, orig in ((128, 500000.0, 8192), (64, 10000.0, 2048), (8, 65536.0, 4096)):
        f = _f32_values(np.power(np.float64(np.float32(base)), 2.0 * np.arange(dims // 2) / dims))
        fexact = np.power(np.float64(np.float32(base)), 2.0 * np.arange(dims // 2) / dims)
        got, ms = S.llama3_freqs(dims, base, factor=32.0, low_freq_factor=1.0,
                                 high_freq_factor=4.0, original_max=orig)
        assert ms == 1.0
        wl = 2 * np.pi * fexact
        lo, hi = wl < orig / 4.0, wl > orig / 1.0
        _same_values(got[lo], f[lo], "high-frequency pairs kept")
        _same_values(got[hi], _f32_values(32.0 * fexact[hi]), "low-frequency pairs scaled")
        mid = ~lo & ~hi
        if mid.any():
            assert np.all(got[mid] > f[mid]) and np.all(got[mid] < 32.0 * f[mid])
            ratio = got[mid] / fexact[mid]
            assert np.all(np.diff(ratio) > 0), "blend must grow with the wavelength"
        same, _ = S.llama3_freqs(dims, base, factor=1.0, original_max=orig)
        _close(same, fexact, 2.0 ** -23, 0, "factor 1")


def pin_llama3_blend_is_continuous(o):
    """At the band edges the blend meets the two outer rules: a pair just inside the high
    edge keeps ~f, one just inside the low edge gets ~factor * f."""
    S = o.rope_scaling
    for target, want_ratio in ((8192 / 4.0 * (1 + 1e-9), 1.0), (8192 / 1.0 * (1 - 1e-9), 8.0)):
        # with dims = 4, pair 1 has f = base^(1/2): pick base so that 2 pi f = target
        base = (target / (2 * np.pi)) ** 2
        got, _ = S.llama3_freqs(4, base, factor=8.0, original_max=8192)
        fexact = np.sqrt(np.float64(np.float32(base)))
        _close(got[1] / fexact, want_ratio, 1e-5, 0, f"edge {target}")


def pin_yarn_ramp(o):
    """Pairs below floor(d(beta_fast)) keep f, pairs from ceil(d(beta_slow)) on get
    factor * f, with d(r) the pair index whose wavelength fits r turns in original_max;
    factor 1 changes nothing; the attention factor is 0.1 ln(factor) + 1 by default."""
    S = o.rope_scaling
    dims, base, orig = 64, 10000.0, 4096
    fexact = np.power(10000.0, 2.0 * np.arange(dims // 2) / dims)
    d = lambda r: dims * np.log(orig / (r * 2 * np.pi)) / (2 * np.log(base))
    lo, hi = int(np.floor(d(32.0))), int(np.ceil(d(1.0)))
    got, ms = S.yarn_freqs(dims, base, factor=8.0, original_max=orig)
    _close(got[:lo + 1], fexact[:lo + 1], 2.0 ** -23, 0, "extrapolated pairs")
    _close(got[hi:], 8.0 * fexact[hi:], 2.0 ** -23, 0, "interpolated pairs")
    assert np.all(got[lo + 1:hi] > fexact[lo + 1:hi]) and np.all(got[lo + 1:hi] < 8 * fexact[lo + 1:hi])
    _close(ms, 0.1 * np.log(8.0) + 1.0, 1e-15, 0, "attention factor")
    one, ms1 = S.yarn_freqs(dims, base, factor=1.0, original_max=orig)
    _close(one, fexact, 2.0 ** -23, 0, "factor 1")
    assert ms1 == 1.0
    _, ms2 = S.yarn_freqs(dims, base, factor=np.e ** 5, mscale=1.0, mscale_all_dim=1.0)
    assert ms2 == 1.0, "equal mscale and mscale_all_dim cancel"


def pin_yarn_ramp_interior(o):
    """A hand-worked pair on the ramp (YaRN, section 3.2: the ramp blends the two inverse
    frequencies linearly). dims 8 and base 16 give divisors f_i = 16^(i/4) = 2^i, and
    d(r) = 8 ln(64 / (2 pi r)) / (2 ln 16) = log2(64 / (2 pi r)); with original context 64,
    beta_fast 8 and beta_slow 4: d(8) = log2(4 / pi) = 0.35, so the ramp starts at pair
    floor(0.35) = 0, and d(4) = log2(8 / pi) = 1.35, so it ends at ceil(1.35) = 2. Pair 1
    sits at ramp 1/2: 1/f' = (1/2) (1/f + 1/(factor f)) = (1/2)(1/2 + 1/6) = 1/3 with
    factor 3, so f' = 3 (a linear blend of the divisors would give 4, a geometric one
    sqrt(12)). Pair 0 keeps f = 1; pairs 2 and 3 get 3 f = 12 and 24. The attention factor is
    0.1 ln 3 + 1."""
    S = o.rope_scaling
    got, ms = S.yarn_freqs(8, 16.0, factor=3.0, original_max=64, beta_fast=8.0, beta_slow=4.0)
    _same_values(got, [1.0, 3.0, 12.0, 24.0], "YaRN ramp at 0, 1/2, 1, 1")
    _close(ms, 0.1 * np.log(3.0) + 1.0, 1e-15, 0, "attention factor of factor 3")


def pin_su_scaling(o):
    S = o.rope_scaling
    dims, base = 16, 10000.0
    lf = np.linspace(1.0, 40.0, 8)
    fexact = np.power(10000.0, 2.0 * np.arange(8) / 16)
    got, ms = S.su_freqs(dims, base, lf, max_position=4096 ** 2, original_max=4096)
    _close(got / fexact, lf, 2.0 ** -23, 0, "per-pair factors")
    _close(ms, np.sqrt(2.0), 1e-15, 0, "max = original^2 gives sqrt 2")
    _, ms1 = S.su_freqs(dims, base, np.ones(8), max_position=4096, original_max=4096)
    assert ms1 == 1.0


# ---------------------------------------------------------------------- softmax family

def pin_softmax_golden(o):
    g = _golden("softmax_hand.json")
    S = o.softmax
    for c in g["softmax"]:
        x = _vals(c["x"])[None]
        _close(S.softmax(x, "f64")[0], _vals(c["expect"]), 1e-15, 1e-300, c["why"])
        for dt in ("bf16", "f32"):
            want = [brute.round_fraction(Fraction(v), dt) for v in c["expect"]]
            _same_values(S.softmax(x, dt)[0], want, c["why"])
    for c in g["causal"]:
        x = np.array([[float(Fraction(v)) for v in r] for r in c["x"]])
        want = np.array([[float(Fraction(v)) for v in r] for r in c["expect"]])
        for dt in ("bf16", "f32"):
            _close(S.causal_softmax(x, c["rows"], dt), want, 2.0 ** -7, 0, c["why"])
        _close(S.causal_softmax(x, c["rows"], "f64"), want, 1e-15, 0, c["why"])
    for c in g["logsumexp"]:
        got = S.logsumexp(_vals(c["x"])[None], "f64")[0, 0]
        _close(got, float(c["expect_decimal"]), 1e-15, 0, c["why"])
    for c in g["cross_entropy"]:
        got = S.cross_entropy(_vals(c["x"])[None], [c["t"]])[0]
        _close(got, np.float32(float(c["expect_decimal"])), 0, 0, c["why"])
    for c in g["cross_entropy_vjp"]:
        got = S.cross_entropy_vjp(_vals(c["x"])[None], [c["t"]], [float(Fraction(c["g"]))],
                                  "f64")[0]
        _close(got, _vals(c["expect"]), 1e-15, 1e-300, c["why"])


def pin_softmax_brute(o):
    """Softmax, logsumexp, cross-entropy and its gradient on short rows against 50 digits
    (the gradient by numerical differentiation of g * loss)."""
    S = o.softmax
    rng = _rng(41)
    for dt, cast in (("bf16", _bf16_values), ("f32", _f32_values)):
        x = cast(rng.standard_normal((3, 9)) * 4)
        got = S.softmax(x, dt)
        lse = S.logsumexp(x, dt)
        t = rng.integers(0, 9, 3)
        g = _f32_values(rng.standard_normal(3))
        ce = S.cross_entropy(x, t)
        dx = S.cross_entropy_vjp(x, t, g, dt)
        for i in range(3):
            _same_values(got[i], [brute.round_mp(v, dt) for v in brute.softmax_row(x[i])], "sm")
            _same_values(lse[i], [brute.round_mp(brute.logsumexp_row(x[i]), dt)], "lse")
            want = brute.logsumexp_row(x[i]) - mpmath.mpf(x[i][t[i]])
            _same_values(ce[i:i + 1], [brute.round_mp(want, "f32")], "ce")
            bd = brute.cross_entropy_vjp_row(x[i], int(t[i]), g[i])
            _same_values(dx[i], [brute.round_mp(v, dt) for v in bd], "ce vjp")


def pin_softmax_torch(o):
    """torch's softmax, logsumexp, cross_entropy (reduction none) and autograd, float64."""
    S = o.softmax
    rng = _rng(42)
    for V in (1, 7, 1000):
        x = rng.standard_normal((6, V)) * 3
        xt = torch.from_numpy(x)
        _close(S.softmax(x, "f64"), torch.softmax(xt, -1).numpy(), 1e-13, 1e-300, "softmax")
        _close(S.logsumexp(x, "f64"), torch.logsumexp(xt, -1, keepdim=True).numpy(), 1e-14,
               1e-14, "logsumexp")
        t = rng.integers(0, V, 6)
        want = torch.nn.functional.cross_entropy(xt, torch.from_numpy(t), reduction="none")
        _close(S.cross_entropy(x, t), want.numpy().astype(np.float32), 2.0 ** -23, 1e-7, "ce")
        g = rng.standard_normal(6)
        xr = xt.clone().requires_grad_(True)
        torch.nn.functional.cross_entropy(xr, torch.from_numpy(t), reduction="none").backward(
            torch.from_numpy(g))
        _close(S.cross_entropy_vjp(x, t, g, "f64"), xr.grad.numpy(), 1e-12, 1e-15, "ce vjp")


def pin_softmax_invariants(o):
    S = o.softmax
    rng = _rng(43)
    x = _bf16_values(rng.standard_normal((5, 300)) * 6)
    p = S.softmax(x, "f64")
    _close(np.sum(p, axis=-1), np.ones(5), 1e-14, 0, "rows sum to 1")
    for c in (1.0, -37.0, 1024.0):  # x + c is exact in float64 for these bf16 values
        _same_values(S.softmax(x + c, "f64"), p, f"shift {c}")
        _close(S.logsumexp(x + c, "f64"), S.logsumexp(x, "f64") + c, 1e-15, 1e-12, "lse shift")
    big = x * 100 + 1e4  # exp of these overflows unless the maximum is taken out first
    assert np.all(np.isfinite(S.softmax(big, "f64"))) and np.all(np.isfinite(S.logsumexp(big, "f64")))
    t = rng.integers(0, 300, 5)
    g = rng.standard_normal(5)
    d = S.cross_entropy_vjp(x, t, g, "f64")
    _close(np.sum(d, axis=-1), np.zeros(5), 0, 1e-13, "gradient rows sum to 0")
    assert np.all(S.cross_entropy(x, t) >= 0)
    bad = S.cross_entropy(x[:2], [-1, 300])
    assert np.all(np.isnan(bad)) and np.all(np.isnan(S.cross_entropy_vjp(x[:1], [300], [1.0], "f64")))


# --------------------------------------------------------------------- RmsNormVjp / LN

def _rows_vals(rows):
    return np.array([[float(Fraction(v)) for v in r] for r in rows])


def pin_rms_vjp_golden(o):
    g = _golden("rms_norm_vjp_hand.json")
    for c in g["cases"]:
        x, gg = _rows_vals(c["x"]), _rows_vals(c["g"])
        w = _vals(c["w"])
        want_dx, want_dw = _rows_vals(c["expect_dx"]), _vals(c["expect_dw"])
        for dt in ("f64", "bf16", "f32"):
            dx, dw = o.rms_norm_vjp(x, w, gg, c["eps"], dt)
            _same_values(dx, want_dx, c["why"] + " dx " + dt)
            _same_values(dw, want_dw, c["why"] + " dw " + dt)


def pin_ln_vjp_golden(o):
    g = _golden("layer_norm_vjp_hand.json")
    for c in g["cases"]:
        x, gg = _rows_vals(c["x"]), _rows_vals(c["g"])
        w, b = _vals(c["w"]), _vals(c["b"])
        want = (_rows_vals(c["expect_dx"]), _vals(c["expect_dw"]), _vals(c["expect_db"]))
        for dt in ("f64", "bf16", "f32"):
            got = o.layer_norm_vjp(x, w, b, gg, c["eps"], dt)
            for name, a, e in zip(("dx", "dw", "db"), got, want):
                _same_values(a, e, c["why"] + " " + name + " " + dt)


def pin_rms_vjp_brute(o):
    """2 x 8 inputs: 50-digit numerical derivatives of the brute-force forward, rounded
    exactly, equal the oracle's rounded gradients."""
    rng = _rng(21)
    for dt, cast in (("bf16", _bf16_values), ("f32", _f32_values)):
        for eps, with_w in ((1e-6, True), (0.3, False)):
            x = cast(rng.standard_normal((2, 8)) * 2)
            w = cast(rng.uniform(0.5, 1.5, 8)) if with_w else None
            g = cast(rng.standard_normal((2, 8)))
            dx, dw = o.rms_norm_vjp(x, w, g, eps, dt)
            bdx, bdw = brute.rms_vjp_rows(x.tolist(), None if w is None else w.tolist(),
                                          g.tolist(), eps)
            for i in range(2):
                _same_values(dx[i], [brute.round_mp(v, dt) for v in bdx[i]], f"{dt} dx {i}")
            _same_values(dw, [brute.round_mp(v, dt) for v in bdw], f"{dt} dw")


def pin_ln_vjp_brute(o):
    rng = _rng(22)
    for dt, cast in (("bf16", _bf16_values), ("f32", _f32_values)):
        for eps, with_w in ((1e-5, True), (0.2, False)):
            x = cast(rng.normal(0.5, 2, (2, 8)))
            w = cast(rng.normal(1, 0.1, 8)) if with_w else None
            b = cast(rng.normal(0, 0.1, 8)) if with_w else None
            g = cast(rng.standard_normal((2, 8)))
            dx, dw, db = o.layer_norm_vjp(x, w, b, g, eps, dt)
            bdx, bdw, bdb = brute.layer_vjp_rows(x.tolist(), None if w is None else w.tolist(),
                                                 None if b is None else b.tolist(), g.tolist(),
                                                 eps)
            for i in range(2):
                _same_values(dx[i], [brute.round_mp(v, dt) for v in bdx[i]], f"{dt} dx {i}")
            _same_values(dw, [brute.round_mp(v, dt) for v in bdw], f"{dt} dw")
            _same_values(db, [brute.round_mp(v, dt) for v in bdb], f"{dt} db")


def _torch_grads(fn, x, params, g):
    xt = torch.from_numpy(x).requires_grad_(True)
    ps = [None if p is None else torch.from_numpy(p).requires_grad_(True) for p in params]
    fn(xt, *ps).backward(torch.from_numpy(g))
    return [xt.grad.numpy()] + [None if p is None else p.grad.numpy() for p in ps]


def pin_rms_vjp_torch(o):
    """torch autograd of torch.nn.functional.rms_norm in float64 on the CPU."""
    rng = _rng(23)
    for d in (1, 7, 64, 1000):
        x = rng.standard_normal((9, d)) * 3
        w = rng.normal(1, 0.2, d)
        g = rng.standard_normal((9, d))
        for eps in (1e-6, 0.25):
            e = float(np.float32(eps))
            f = lambda xt, wt: torch.nn.functional.rms_norm(xt, (d,), wt, eps=e)
            tdx, tdw = _torch_grads(f, x, [w], g)
            dx, dw = o.rms_norm_vjp(x, w, g, eps, "f64")
            _close(dx, tdx, 1e-11, 1e-13, f"d={d} dx")
            _close(dw, tdw, 1e-11, 1e-13, f"d={d} dw")


def pin_ln_vjp_torch(o):
    """torch autograd of torch.nn.functional.layer_norm in float64 on the CPU."""
    rng = _rng(24)
    for d in (2, 33, 1024):
        x = rng.normal(0.5, 2, (7, d))
        w = rng.normal(1, 0.1, d)
        b = rng.normal(0, 0.1, d)
        g = rng.standard_normal((7, d))
        for eps in (1e-5, 0.1):
            e = float(np.float32(eps))
            f = lambda xt, wt, bt: torch.nn.functional.layer_norm(xt, (d,), wt, bt, eps=e)
            tdx, tdw, tdb = _torch_grads(f, x, [w, b], g)
            dx, dw, db = o.layer_norm_vjp(x, w, b, g, eps, "f64")
            _close(dx, tdx, 1e-11, 1e-13, f"d={d} dx")
            _close(dw, tdw, 1e-11, 1e-13, f"d={d} dw")
            _close(db, tdb, 1e-12, 1e-13, f"d={d} db")


def pin_vjp_invariances(o):
    """RMSNorm is scale invariant at eps = 0, so x . dx = 0 per row; LayerNorm is shift
    invariant (sum dx = 0 for any eps) and scale invariant at eps = 0 (x . dx = 0); db is
    the column sum of g. Checked relative to the sizes of the terms."""
    rng = _rng(25)
    x = rng.normal(0.3, 2, (6, 200))
    w = rng.normal(1, 0.2, 200)
    b = rng.normal(0, 0.1, 200)
    g = rng.standard_normal((6, 200))
    dx, _ = o.rms_norm_vjp(x, w, g, 0.0, "f64")
    scale = np.sum(np.abs(x * dx), axis=-1)
    assert np.all(np.abs(np.sum(x * dx, axis=-1)) <= 1e-13 * scale), "RMS x.dx"
    for eps in (0.0, 0.5):
        dx, _, db = o.layer_norm_vjp(x, w, b, g, eps, "f64")
        assert np.all(np.abs(np.sum(dx, axis=-1)) <= 1e-13 * np.sum(np.abs(dx), axis=-1)), "LN sum"
        _close(db, np.sum(g, axis=0), 1e-14, 1e-14, "db")
        if eps == 0.0:
            s = np.sum(np.abs(x * dx), axis=-1)
            assert np.all(np.abs(np.sum(x * dx, axis=-1)) <= 1e-13 * s), "LN x.dx"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

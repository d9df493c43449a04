"""Brute force for tiny inputs: every op evaluated at 50 significant digits with mpmath and
rounded to the output format with exact rational arithmetic (``fractions.Fraction``).

This is deliberately a different computation from the oracle: no numpy, no float64
intermediates, and its own round-to-nearest-even written on exact rationals (find the
binade, scale to an integer grid, compare the remainder with one half).
"""

from fractions import Fraction

import mpmath

mpmath.mp.dps = 50

# (significant bits, exponent of the smallest quantum, overflow threshold exponent)
FORMATS = {
    "bf16": (8, -133, 128),
    "f32": (24, -149, 128),
}


def _binade(a: Fraction) -> int:
    """e with 2**e <= a < 2**(e+1), for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_fraction(q: Fraction, fmt: str):
    """Nearest value of ``fmt`` to the exact rational q, ties to even; ±inf on overflow."""
    p, qmin, ovf = FORMATS[fmt]
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    qe = max(_binade(a) - (p - 1), qmin)
    scaled = a / Fraction(2) ** qe
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = Fraction(n) * Fraction(2) ** qe
    if r >= Fraction(2) ** ovf:
        return sign * float("inf")
    return sign * float(r)


def mpf_to_fraction(v) -> Fraction:
    """Exact value of an mpf: (-1)^sign * man * 2^exp from its raw tuple."""
    sign, man, exp, _ = mpmath.mpf(v)._mpf_
    q = Fraction(man) * Fraction(2) ** exp if exp >= 0 else Fraction(man, 2 ** (-exp))
    return -q if sign else q


def round_mp(v, fmt):
    return round_fraction(mpf_to_fraction(v), fmt)


def f32(v):
    import struct
    return struct.unpack("f", struct.pack("f", v))[0]


def rms_row(x, w, eps):
    d = len(x)
    xs = [mpmath.mpf(v) for v in x]
    ms = mpmath.fsum(v * v for v in xs) / d
    den = mpmath.sqrt(ms + mpmath.mpf(f32(eps)))
    return [xs[j] / den * (mpmath.mpf(w[j]) if w is not None else 1) for j in range(d)]


def layer_row(x, w, b, eps):
    d = len(x)
    xs = [mpmath.mpf(v) for v in x]
    mu = mpmath.fsum(xs) / d
    var = mpmath.fsum((v - mu) ** 2 for v in xs) / d
    den = mpmath.sqrt(var + mpmath.mpf(f32(eps)))
    out = []
    for j in range(d):
        y = (xs[j] - mu) / den
        if w is not None:
            y *= mpmath.mpf(w[j])
        if b is not None:
            y += mpmath.mpf(b[j])
        out.append(y)
    return out


def rope_row(x, w, *, normalize, eps, dims, traditional, base, scale, pos, forward,
             freqs=None, mscale=1.0):
    """One [D] row rotated at integer position ``pos`` (pair i at frequency 1 / freqs[i]
    when freqs is given; rotated features times mscale)."""
    d = len(x)
    xs = rms_row(x, w, eps) if normalize else [mpmath.mpf(v) for v in x]
    out = list(xs)
    half = dims // 2
    m = mpmath.mpf(f32(mscale))
    for i in range(half):
        if freqs is None:
            theta = mpmath.power(mpmath.mpf(f32(base)), mpmath.mpf(-2 * i) / dims)
        else:
            theta = 1 / mpmath.mpf(freqs[i])
        a = mpmath.mpf(f32(scale)) * pos * theta
        c, s = mpmath.cos(a), mpmath.sin(a)
        if not forward:
            s = -s
        iu, iv = (2 * i, 2 * i + 1) if traditional else (i, i + half)
        u, v = xs[iu], xs[iv]
        out[iu] = m * (u * c - v * s)
        out[iv] = m * (u * s + v * c)
    assert len(out) == d
    return out


def _grad(f, point, k):
    """d f / d point[k] at `point` (a list of mpf), by mpmath's high-precision numerical
    differentiation: a finite-difference derivative, independent of any closed form."""
    def fk(t):
        q = list(point)
        q[k] = t
        return f(q)
    return mpmath.diff(fk, point[k])


def rms_vjp_rows(x, w, g, eps):
    """(dx rows, dw) of RmsNorm for the rows x[i] with cotangents g[i]: the derivatives of
    L = sum_i sum_j g[i][j] * RmsNorm(x)[i][j] with respect to x and to w (w None = ones)."""
    d = len(x[0])
    wv = [mpmath.mpf(1)] * d if w is None else [mpmath.mpf(v) for v in w]
    dx = []
    for xi, gi in zip(x, g):
        gm = [mpmath.mpf(v) for v in gi]
        loss = lambda q: mpmath.fsum(a * b for a, b in zip(gm, rms_row(q, wv, eps)))
        pt = [mpmath.mpf(v) for v in xi]
        dx.append([_grad(loss, pt, k) for k in range(d)])

    def loss_w(q):
        return mpmath.fsum(mpmath.fsum(mpmath.mpf(a) * b for a, b in zip(gi, rms_row(xi, q, eps)))
                           for xi, gi in zip(x, g))
    dw = [_grad(loss_w, wv, k) for k in range(d)]
    return dx, dw


def layer_vjp_rows(x, w, b, g, eps):
    """(dx rows, dw, db) of LayerNorm, the same way (w None = ones, b None = zeros)."""
    d = len(x[0])
    wv = [mpmath.mpf(1)] * d if w is None else [mpmath.mpf(v) for v in w]
    bv = [mpmath.mpf(0)] * d if b is None else [mpmath.mpf(v) for v in b]
    dx = []
    for xi, gi in zip(x, g):
        gm = [mpmath.mpf(v) for v in gi]
        loss = lambda q: mpmath.fsum(a * c for a, c in zip(gm, layer_row(q, wv, bv, eps)))
        pt = [mpmath.mpf(v) for v in xi]
        dx.append([_grad(loss, pt, k) for k in range(d)])

    def total(wq, bq):
        return mpmath.fsum(
            mpmath.fsum(mpmath.mpf(a) * c for a, c in zip(gi, layer_row(xi, wq, bq, eps)))
            for xi, gi in zip(x, g))
    dw = [_grad(lambda q: total(q, bv), wv, k) for k in range(d)]
    db = [_grad(lambda q: total(wv, q), bv, k) for k in range(d)]
    return dx, dw, db


def softmax_row(x):
    xs = [mpmath.mpf(v) for v in x]
    e = [mpmath.exp(v) for v in xs]
    s = mpmath.fsum(e)
    return [v / s for v in e]


def logsumexp_row(x):
    return mpmath.log(mpmath.fsum(mpmath.exp(mpmath.mpf(v)) for v in x))


def cross_entropy_vjp_row(x, t, g):
    """Numerical derivatives of g * (logsumexp(x) - x[t]) with respect to each x_j."""
    gm = mpmath.mpf(g)
    loss = lambda q: gm * (mpmath.log(mpmath.fsum(mpmath.exp(v) for v in q)) - q[t])
    pt = [mpmath.mpf(v) for v in x]
    return [_grad(loss, pt, k) for k in range(len(x))]

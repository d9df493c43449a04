"""Helpers for the GPU parity tests: run an op through the C ABI (Python binding) and compare
with the fp64 oracle under the parity rules of ``compare.py``."""

import contextlib
import os
import sys

import numpy as np
import torch

import compare
import oracle

DEV = torch.device("cuda:0")
DT = {torch.bfloat16: "bf16", torch.float32: "f32"}


def f64(t):
    return None if t is None else t.detach().cpu().to(torch.float64).numpy()


def dev(t):
    return None if t is None else t.to(DEV)


def say(msg):
    """Name the case on stdout before a GPU step, so a failing run shows where it was."""
    print(msg, flush=True)
    sys.stdout.flush()


@contextlib.contextmanager
def forced_path(path):
    old = os.environ.get("NRM_FORCE_PATH")
    if path is None:
        os.environ.pop("NRM_FORCE_PATH", None)
    else:
        os.environ["NRM_FORCE_PATH"] = path
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("NRM_FORCE_PATH", None)
        else:
            os.environ["NRM_FORCE_PATH"] = old


def assert_h_exact(h_gpu, h_want, what="h"):
    """Bit-exact residual: GPU bits against the oracle's values in the same dtype."""
    got = compare.tensor_bits(h_gpu)
    want = compare.bits_of_values(h_want, DT[h_gpu.dtype])
    bad = got.ravel() != want.ravel()
    n = int(np.count_nonzero(bad))
    assert n == 0, f"{what}: {n} of {bad.size} elements differ in their bits"


def check_add(nrm, inp, rows_sel=None):
    """add-RMSNorm on the device against the oracle; rows_sel restricts the comparison."""
    x, r, w = dev(inp.x), dev(inp.r), dev(inp.w)
    out, h = nrm.add_rms_norm(x, r, w, inp.eps)
    torch.cuda.synchronize()
    dt = DT[inp.x.dtype]
    xs, rs = inp.x, inp.r
    if rows_sel is not None:
        xs, rs, out, h = xs[rows_sel], rs[rows_sel], out[rows_sel], h[rows_sel]
    want_out, want_h = oracle.add_rms_norm(f64(xs), f64(rs), f64(inp.w), inp.eps, dt)
    assert_h_exact(h, want_h)
    return compare.check_output(out, want_out, dt, what="add_rms_norm out")


def check_rms(nrm, inp, rows_sel=None):
    x, w = dev(inp.x), dev(inp.w)
    out = nrm.rms_norm(x, w, inp.eps)
    torch.cuda.synchronize()
    dt = DT[inp.x.dtype]
    xs = inp.x
    if rows_sel is not None:
        xs, out = xs[rows_sel], out[rows_sel]
    return compare.check_output(out, oracle.rms_norm(f64(xs), f64(inp.w), inp.eps, dt), dt,
                                what="rms_norm out")


def check_ln(nrm, inp, rows_sel=None):
    out = nrm.layer_norm(dev(inp.x), dev(inp.w), dev(inp.b), inp.eps)
    torch.cuda.synchronize()
    dt = DT[inp.x.dtype]
    xs = inp.x
    if rows_sel is not None:
        xs, out = xs[rows_sel], out[rows_sel]
    want = oracle.layer_norm(f64(xs), f64(inp.w), f64(inp.b), inp.eps, dt)
    return compare.check_output(out, want, dt, what="layer_norm out")


def rope_oracle(rp, *, normalize=True, traditional=False, forward=True, cache=None):
    return oracle.norm_rope(f64(rp.x), f64(rp.w), normalize=normalize, eps=rp.eps, dims=rp.dims,
                            traditional=traditional, base=rp.base, scale=rp.scale,
                            offset=rp.offset, forward=forward, dtype=DT[rp.x.dtype],
                            cache=f64(cache))


def run_rope(nrm, rp, *, normalize=True, traditional=False, forward=True, cache=None):
    out = nrm.norm_rope(dev(rp.x), dev(rp.w), eps=rp.eps if normalize else None, dims=rp.dims,
                        traditional=traditional, base=rp.base, scale=rp.scale,
                        offset=rp.offset, forward=forward, cache=dev(cache))
    torch.cuda.synchronize()
    return out


def check_rope(nrm, rp, *, normalize=True, traditional=False, forward=True, cache=None):
    got = run_rope(nrm, rp, normalize=normalize, traditional=traditional, forward=forward,
                   cache=cache)
    want = rope_oracle(rp, normalize=normalize, traditional=traditional, forward=forward,
                       cache=cache)
    dt = DT[rp.x.dtype]
    res = compare.check_output(got, want, dt, what="norm_rope out")
    if cache is not None:
        # rows outside offset .. offset + L keep their bits exactly
        L, off = rp.x.shape[2], rp.offset
        keep = np.ones(cache.shape[2], dtype=bool)
        keep[off:off + L] = False
        g = compare.tensor_bits(got)[:, :, keep]
        w = compare.tensor_bits(cache)[:, :, keep]
        assert np.array_equal(g, w), "cache rows outside the written range changed"
    return res


def run_vjp(nrm, inp, ln, want_dw=True, want_db=True):
    x, w, g = dev(inp.x), dev(inp.w), dev(inp.g)
    if ln:
        res = nrm.layer_norm_vjp(x, w, g, inp.eps, want_dw=want_dw, want_db=want_db)
    else:
        res = nrm.rms_norm_vjp(x, w, g, inp.eps, want_dw=want_dw)
    torch.cuda.synchronize()
    return res


def vjp_oracle(inp, ln, rows_sel=None, chunk=None):
    """Oracle gradients. dx for rows_sel (all rows when None). dw (and db) always sum over
    every row: with ``chunk`` the rows are taken in chunks whose unrounded float64 column
    sums are added, then rounded once (the sum over rows, in pieces that fit in memory)."""
    dt = DT[inp.x.dtype]
    wdt = DT[inp.w.dtype] if inp.w is not None else dt
    w = f64(inp.w)
    xs = inp.x if rows_sel is None else inp.x[rows_sel]
    gs = inp.g if rows_sel is None else inp.g[rows_sel]
    if ln:
        dx = oracle.layer_norm_vjp(f64(xs), w, None, f64(gs), inp.eps, dt, wdt)[0]
    else:
        dx = oracle.rms_norm_vjp(f64(xs), w, f64(gs), inp.eps, dt, wdt)[0]
    rows = inp.x.shape[0]
    step = chunk or max(rows, 1)
    sums = None
    for r0 in range(0, rows, step):
        xc, gc = f64(inp.x[r0:r0 + step]), f64(inp.g[r0:r0 + step])
        if ln:
            part = oracle.layer_norm_vjp(xc, w, None, gc, inp.eps, "f64")[1:]
        else:
            part = oracle.rms_norm_vjp(xc, w, gc, inp.eps, "f64")[1:]
        sums = list(part) if sums is None else [a + b for a, b in zip(sums, part)]
    if sums is None:
        sums = [np.zeros(inp.x.shape[-1])] * (2 if ln else 1)
    params = [oracle.round_to(s, wdt) for s in sums]
    return dx, params


def check_vjp(nrm, inp, ln, rows_sel=None, chunk=None):
    """Backward on the device against the oracle: dx (on rows_sel), dw (and db)."""
    got = run_vjp(nrm, inp, ln)
    want_dx, want_params = vjp_oracle(inp, ln, rows_sel, chunk)
    dt = DT[inp.x.dtype]
    wdt = DT[inp.w.dtype] if inp.w is not None else dt
    gdx = got[0] if rows_sel is None else got[0][rows_sel]
    res = [compare.check_output(gdx, want_dx, dt, what="dx")]
    for name, g, wv in zip(("dw", "db"), got[1:], want_params):
        res.append(compare.check_output(g, wv, wdt, what=name))
    return res

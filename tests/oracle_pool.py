"""Full-size parity: the fp64 oracle over every row of a large workload, in chunks of rows
spread over a process pool, each chunk compared in the worker with the GPU's output for it.

Test infrastructure only (it calls ``oracle/``). Inputs travel as bit patterns (bf16 as
uint16, fp32 as float32) and are decoded exactly to float64 in the worker; the comparison
rules are those of ``compare.py``: h bit-exact, bf16 outputs within 1 ulp, fp32 outputs
within 1e-5 relative + 1e-6 absolute.
"""

import multiprocessing as mp
import os

import numpy as np
import torch

import compare
import oracle

# Processes: the host's cores, at most 16 (the GPU machine's share).
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))
CHUNK_ROWS = 512


def bits(t):
    """A CPU copy of a tensor as numpy bits: bf16 -> uint16, fp32 -> float32."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    assert t.dtype == torch.float32, t.dtype
    return t.numpy()


def _decode(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _dtype_of(a):
    return "bf16" if a.dtype == np.uint16 else "f32"


def _out_stats(got, want, dt):
    """(largest distance, count over tolerance) of one output chunk."""
    if dt == "bf16":
        d = compare.bf16_ulp_distance(got, compare.bf16_bits_of(want))
        return int(d.max()) if d.size else 0, int(np.count_nonzero(d > 1))
    g = got.astype(np.float64).ravel()
    w = np.asarray(want, dtype=np.float64).ravel()
    with np.errstate(invalid="ignore"):
        err = np.abs(g - w)
        tol = 1e-6 + 1e-5 * np.abs(w)
        bad = ~(err <= tol)
    bad &= ~(np.isinf(g) & np.isinf(w) & (g == w))
    gn, wn = np.isnan(g), np.isnan(w)
    bad = np.where(gn & wn, False, bad) | (gn ^ wn)
    fin = np.isfinite(err)
    worst = float((err[fin] / tol[fin]).max()) if fin.any() else 0.0
    return worst, int(np.count_nonzero(bad))


def _h_mismatches(got, want_values, dt):
    want = compare.bits_of_values(want_values, dt)
    g = got.view(np.uint32) if got.dtype == np.float32 else got
    return int(np.count_nonzero(g.ravel() != want.ravel()))


def _worker(job):
    op, r0, args = job
    if op == "add_rms_norm":
        x, r, w, eps, out, h = args
        dt = _dtype_of(x)
        want_out, want_h = oracle.add_rms_norm(_decode(x), _decode(r), _decode(w), eps, dt)
        worst, over = _out_stats(out, want_out, dt)
        return r0, worst, over, _h_mismatches(h, want_h, dt)
    if op == "layer_norm":
        x, w, b, eps, out = args
        dt = _dtype_of(x)
        want = oracle.layer_norm(_decode(x), _decode(w), _decode(b), eps, dt)
        worst, over = _out_stats(out, want, dt)
        return r0, worst, over, 0
    raise ValueError(op)


def _run(jobs):
    ctx = mp.get_context("spawn")
    with ctx.Pool(WORKERS) as pool:
        res = pool.map(_worker, jobs, chunksize=1)
    worst = max(r[1] for r in res)
    over = sum(r[2] for r in res)
    h_bad = sum(r[3] for r in res)
    first = [r[0] for r in res if r[2] or r[3]][:4]
    return worst, over, h_bad, first


def check_add_rms_all_rows(x, r, w, eps, out, h):
    """add-RMSNorm on every row: h bit-exact, out within the bar. Tensors on any device."""
    xb, rb, wb, ob, hb = bits(x), bits(r), bits(w), bits(out), bits(h)
    rows = xb.shape[0]
    jobs = [("add_rms_norm", r0, (xb[r0:r0 + CHUNK_ROWS], rb[r0:r0 + CHUNK_ROWS], wb, eps,
                                  ob[r0:r0 + CHUNK_ROWS], hb[r0:r0 + CHUNK_ROWS]))
            for r0 in range(0, rows, CHUNK_ROWS)]
    worst, over, h_bad, first = _run(jobs)
    assert h_bad == 0, f"h: {h_bad} elements differ in their bits (chunks from rows {first})"
    assert over == 0, f"out: {over} elements over the bar, worst {worst} (chunks from rows {first})"
    return worst


def check_layer_norm_all_rows(x, w, b, eps, out):
    """LayerNorm on every row, out within the bar."""
    xb, wb, bb, ob = bits(x), bits(w), bits(b), bits(out)
    rows = xb.shape[0]
    jobs = [("layer_norm", r0, (xb[r0:r0 + CHUNK_ROWS], wb, bb, eps, ob[r0:r0 + CHUNK_ROWS]))
            for r0 in range(0, rows, CHUNK_ROWS)]
    worst, over, _, first = _run(jobs)
    assert over == 0, f"out: {over} elements over the bar, worst {worst} (chunks from rows {first})"
    return worst

"""Calls from several host threads at once, each on its own stream: add-RMSNorm on one, the
LayerNorm backward (with its workspace) and NormRope on another, repeated while they overlap;
every result is compared with the oracle afterwards."""

import threading

import pytest
import torch

import compare
import oracle
import workloads
from gpu_util import DEV, assert_h_exact, f64, say

pytestmark = pytest.mark.gpu


def test_threads_on_their_own_streams(nrm_lib):
    say("two host threads, two streams, overlapping calls")
    add_in = workloads.row_inputs(512, 4096, "bf16", seed=91, r=("normal", 0.0, 1.0), eps=1e-6)
    vjp_in = workloads.row_inputs(700, 8192, "bf16", seed=92, x=("normal", 0.5, 2.0),
                                  g=("normal", 0.0, 1.0))
    rp = workloads.rope_inputs(2, 8, 64, 128, "bf16", seed=93, offset=300)
    rounds = 30
    got, errors = {}, []
    gate = threading.Barrier(2)

    def run_add():
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            x, r, w = add_in.x.to(DEV), add_in.r.to(DEV), add_in.w.to(DEV)
            gate.wait()
            for _ in range(rounds):
                out, h = nrm_lib.add_rms_norm(x, r, w, add_in.eps)
            s.synchronize()
            got["add"] = (out.cpu(), h.cpu())

    def run_vjp_rope():
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            x, w, g = vjp_in.x.to(DEV), vjp_in.w.to(DEV), vjp_in.g.to(DEV)
            xr, wr = rp.x.to(DEV), rp.w.to(DEV)
            gate.wait()
            for _ in range(rounds):
                dx, dw, db = nrm_lib.layer_norm_vjp(x, w, g, vjp_in.eps)
                ro = nrm_lib.norm_rope(xr, wr, eps=rp.eps, dims=rp.dims, base=rp.base,
                                       scale=rp.scale, offset=rp.offset)
            s.synchronize()
            got["vjp"] = (dx.cpu(), dw.cpu(), db.cpu())
            got["rope"] = ro.cpu()

    def guarded(fn):
        def run():
            try:
                fn()
            except Exception as e:  # reported below, after the threads have joined
                errors.append(repr(e))
        return run

    threads = [threading.Thread(target=guarded(f)) for f in (run_add, run_vjp_rope)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(120)
    assert not errors, errors
    assert set(got) == {"add", "vjp", "rope"}

    out, h = got["add"]
    want_out, want_h = oracle.add_rms_norm(f64(add_in.x), f64(add_in.r), f64(add_in.w),
                                           add_in.eps, "bf16")
    assert_h_exact(h, want_h)
    compare.check_output(out, want_out, "bf16", what="add_rms_norm out")
    want = oracle.layer_norm_vjp(f64(vjp_in.x), f64(vjp_in.w), None, f64(vjp_in.g), vjp_in.eps,
                                 "bf16")
    for gt, wt, what in zip(got["vjp"], want, ("dx", "dw", "db")):
        compare.check_output(gt, wt, "bf16", what=what)
    want_rope = oracle.norm_rope(f64(rp.x), f64(rp.w), normalize=True, eps=rp.eps, dims=rp.dims,
                                 traditional=False, base=rp.base, scale=rp.scale,
                                 offset=rp.offset, forward=True, dtype="bf16")
    compare.check_output(got["rope"], want_rope, "bf16", what="norm_rope out")

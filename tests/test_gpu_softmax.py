"""GPU parity of the softmax family (Softmax, CausalSoftmax, LogSumExp, CrossEntropy and its
gradient) through the C ABI against the fp64 oracle, element by element.

Bars: bf16 outputs within 1 ulp; fp32 outputs (the loss, fp32 softmax) within 1e-5 relative
+ 1e-6 absolute; confident rows (loss near 0) are also held to 1e-5 relative alone.
"""

import numpy as np
import pytest
import torch

import compare
import oracle
import workloads
from gpu_util import DEV, dev, f64, forced_path, say

pytestmark = pytest.mark.gpu

# 5000 and 10000 (bf16): register rows whose team is 192 threads (three waves, one team per
# block); 20000 and 40000: streaming rows of one and two steps (their first step parked in LDS)
WIDTHS = [1, 2, 7, 8, 33, 64, 100, 512, 520, 4096, 5000, 8192, 10000, 16384, 20000, 40000,
          50257, 65536, 100277, 128256, 131072, 140000]
PATHS = [None, "chunked", "scalar"]


@pytest.mark.parametrize("n", WIDTHS)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_softmax_widths(nrm_lib, n, dt):
    say(f"softmax n={n} {dt}")
    x = workloads.scores((3, n), dt, seed=n)
    got = nrm_lib.softmax(dev(x))
    lse = nrm_lib.logsumexp(dev(x))
    torch.cuda.synchronize()
    compare.check_output(got, oracle.softmax.softmax(f64(x), dt), dt, what="softmax")
    compare.check_output(lse, oracle.softmax.logsumexp(f64(x), dt), dt, what="logsumexp")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("n", [512, 4096, 12345])
@pytest.mark.parametrize("rows", [1, 5, 64, 300])
def test_softmax_paths_and_rows(nrm_lib, path, n, rows):
    say(f"softmax path={path} n={n} rows={rows}")
    x = workloads.scores((rows, n), "bf16", seed=rows + n)
    with forced_path(path):
        got = nrm_lib.softmax(dev(x))
        lse = nrm_lib.logsumexp(dev(x))
        torch.cuda.synchronize()
    compare.check_output(got, oracle.softmax.softmax(f64(x), "bf16"), "bf16", what="softmax")
    compare.check_output(lse, oracle.softmax.logsumexp(f64(x), "bf16"), "bf16", what="lse")


@pytest.mark.parametrize("N,R,L,rows", [(2, 8, 8, 8), (2, 64, 512, 64), (1, 512, 512, 512),
                                        (3, 6, 4, 3), (2, 16, 1000, 8), (1, 12, 2, 12),
                                        (4, 128, 4096, 128), (1, 2048, 12000, 2048),
                                        (1, 1024, 5000, 1024), (1, 256, 16384, 256),
                                        (1, 2048, 16400, 2048), (1, 64, 70000, 64)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("path", [None, "scalar"])
def test_causal_softmax(nrm_lib, N, R, L, rows, dt, path):
    # L = 12000 and 16384 (bf16), 5000 (fp32): rows of 8 chunks per thread in registers,
    # the cut inside the last chunks of each thread and whole chunks past it never read;
    # 16400 and 70000: the streaming kernel
    say(f"causal N={N} R={R} L={L} rows={rows} {dt} path={path}")
    x = workloads.scores((N, R, L), dt, seed=R + L)
    with forced_path(path):
        got = nrm_lib.causal_softmax(dev(x), rows)
        torch.cuda.synchronize()
    compare.check_output(got, oracle.softmax.causal_softmax(f64(x), rows, dt), dt,
                         what="causal softmax")


def _ce_check(nrm, inp, dt, path=None, i32=False, sel=None):
    t = inp.targets.to(torch.int32) if i32 else inp.targets
    with forced_path(path):
        loss = nrm.cross_entropy(dev(inp.logits), dev(t))
        dl = nrm.cross_entropy_vjp(dev(inp.logits), dev(t), dev(inp.g), loss=loss)
        torch.cuda.synchronize()
    x, tt, g = inp.logits, inp.targets.numpy(), inp.g.numpy()
    if sel is not None:
        x, tt, g, loss, dl = x[sel], tt[sel], g[sel], loss[sel], dl[sel]
    want = oracle.softmax.cross_entropy(f64(x), tt)
    compare.check_f32(f64(loss), want, what="loss")
    compare.check_output(dl, oracle.softmax.cross_entropy_vjp(f64(x), tt, g, dt), dt,
                         what="dlogits")
    return loss, want


@pytest.mark.parametrize("V", [2, 100, 1000, 5000, 10000, 20000, 32000, 50257, 100277, 128256,
                               151936])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_cross_entropy_vocab(nrm_lib, V, dt):
    say(f"cross_entropy V={V} {dt}")
    _ce_check(nrm_lib, workloads.ce_inputs(6, V, dt, seed=V, g="normal"), dt)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("i32", [False, True])
def test_cross_entropy_paths(nrm_lib, path, i32):
    say(f"cross_entropy path={path} int32={i32}")
    _ce_check(nrm_lib, workloads.ce_inputs(70, 4096, "bf16", seed=3, g="normal"), "bf16",
              path, i32)


@pytest.mark.parametrize("path", [None, "scalar"])
def test_cross_entropy_confident_rows(nrm_lib, path):
    """Target logits far above the rest: losses from ~1e-2 down to ~1e-12 keep 1e-5
    relative precision, and so does the target's gradient entry (bf16, 1 ulp)."""
    say(f"cross_entropy confident path={path}")
    inp = workloads.ce_inputs(8, 1000, "bf16", seed=5, g="normal")
    x = inp.logits.float()
    for i in range(8):
        x[i, inp.targets[i]] = 4.0 + 3.0 * i
    inp.logits = x.to(torch.bfloat16)
    loss, want = _ce_check(nrm_lib, inp, "bf16", path)
    got = f64(loss)
    assert np.all(np.abs(got - want) <= 1e-5 * np.abs(want)), (got, want)


def test_cross_entropy_bad_targets(nrm_lib):
    say("cross_entropy out-of-range targets")
    inp = workloads.ce_inputs(4, 100, "bf16", seed=6, g="normal")
    inp.targets[1] = -1
    inp.targets[3] = 100
    _ce_check(nrm_lib, inp, "bf16")


def test_softmax_special_values(nrm_lib):
    say("softmax special values")
    x = workloads.scores((5, 600), "f32", seed=7)
    x[0, 10] = float("nan")
    x[1, :300] = -float("inf")
    x[2, :] = -float("inf")
    x[3, 5] = float("inf")
    x[4, :] = 1e30
    for dt in ("f32", "bf16"):
        xs = x.to(torch.bfloat16) if dt == "bf16" else x
        for path in (None, "scalar"):
            with forced_path(path):
                got = nrm_lib.softmax(dev(xs))
                lse = nrm_lib.logsumexp(dev(xs))
                torch.cuda.synchronize()
            compare.check_output(got, oracle.softmax.softmax(f64(xs), dt), dt, what="softmax")
            compare.check_output(lse, oracle.softmax.logsumexp(f64(xs), dt), dt, what="lse")


def test_causal_softmax_special_values(nrm_lib):
    """Causal rows of 512 columns (rows_per_block 640, so rows 0-127 keep no column) with
    special kept scores, in waves beside ordinary rows: kept scores all at the dtype's lowest
    value (the maximum is that value, masked scores count as much as kept ones), all -inf
    (only the masked columns remain), a NaN, a +inf, huge values; every slot of a row past
    its cut is then either skipped as a whole or computed, and both must agree."""
    R, L, rows = 640, 512, 640
    for dt in ("bf16", "f32"):
        say(f"causal softmax special values {dt}")
        x = workloads.scores((1, R, L), "f32", seed=17)
        lowest = -3.3895313892515355e38 if dt == "bf16" else float(np.finfo(np.float32).min)
        x[0, 200, :73] = lowest             # cut 72: every kept score the lowest value
        x[0, 300, :173] = -float("inf")     # cut 172: every kept score -inf
        x[0, 401, 5] = float("nan")         # cut 273
        x[0, 502, 10] = float("inf")        # cut 374
        x[0, 150, :23] = 1e30               # cut 22
        x[0, 131, 3] = -float("inf")        # cut 3: one of four kept scores -inf
        xs = x.to(torch.bfloat16) if dt == "bf16" else x
        for path in (None, "scalar"):
            with forced_path(path):
                got = nrm_lib.causal_softmax(dev(xs), rows)
                torch.cuda.synchronize()
            compare.check_output(got, oracle.softmax.causal_softmax(f64(xs), rows, dt), dt,
                                 what=f"causal softmax, path {path}")


def test_softmax_misaligned_bases(nrm_lib):
    """Rows starting 2 bytes past a 16-byte boundary (a view one element into a buffer):
    head, chunk body and tail per row, with an output of the same phase; an output of another
    phase takes the one-element-at-a-time kernel; the loss and its gradient alike."""
    say("softmax misaligned bases")
    rows, n = 6, 4096
    flat = dev(workloads.scores((1, rows * n + 8), "bf16", seed=77)).reshape(-1)
    x = flat[1:1 + rows * n].view(rows, n)
    oflat = torch.empty_like(flat)
    out_same = oflat[1:1 + rows * n].view(rows, n)
    got_same = nrm_lib.softmax(x, out=out_same)
    got_other = nrm_lib.softmax(x)
    lse = nrm_lib.logsumexp(x)
    torch.cuda.synchronize()
    want = oracle.softmax.softmax(f64(x.cpu()), "bf16")
    compare.check_output(got_same, want, "bf16", what="softmax, same phase")
    compare.check_output(got_other, want, "bf16", what="softmax, other phase")
    compare.check_output(lse, oracle.softmax.logsumexp(f64(x.cpu()), "bf16"), "bf16", what="lse")
    tg = torch.from_numpy(np.random.default_rng(78).integers(0, n, rows))
    tg[0], tg[1] = 0, n - 1  # first and last column: in a row's head and tail
    g = torch.from_numpy(np.random.default_rng(79).normal(size=rows).astype(np.float32))
    loss = nrm_lib.cross_entropy(x, dev(tg))
    dl = nrm_lib.cross_entropy_vjp(x, dev(tg), dev(g), dlogits=out_same)
    torch.cuda.synchronize()
    compare.check_f32(f64(loss), oracle.softmax.cross_entropy(f64(x.cpu()), tg.numpy()), what="loss")
    compare.check_output(dl, oracle.softmax.cross_entropy_vjp(f64(x.cpu()), tg.numpy(), g.numpy(),
                                                              "bf16"), "bf16", what="dlogits")


def test_softmax_special_values_odd_width(nrm_lib):
    say("softmax special values, odd width")
    x = workloads.scores((5, 1001), "f32", seed=17)
    x[0, 3] = float("nan")       # in the first row's body
    x[1, :500] = -float("inf")
    x[2, :] = -float("inf")
    x[3, 1000] = float("inf")    # in a tail
    x[4, :] = 1e30
    for dt in ("f32", "bf16"):
        xs = x.to(torch.bfloat16) if dt == "bf16" else x
        got = nrm_lib.softmax(dev(xs))
        lse = nrm_lib.logsumexp(dev(xs))
        torch.cuda.synchronize()
        compare.check_output(got, oracle.softmax.softmax(f64(xs), dt), dt, what="softmax")
        compare.check_output(lse, oracle.softmax.logsumexp(f64(xs), dt), dt, what="lse")


@pytest.mark.parametrize("n", [3000, 50257, 128256])
def test_softmax_in_place(nrm_lib, n):
    say(f"softmax and gradient in place n={n}")
    for path in (None, "scalar"):
        with forced_path(path):
            x = dev(workloads.scores((40, n), "bf16", seed=8))
            ref = nrm_lib.softmax(x)
            nrm_lib.softmax(x, out=x)
            inp = workloads.ce_inputs(40, n, "bf16", seed=9, g="normal")
            lg = dev(inp.logits)
            dref = nrm_lib.cross_entropy_vjp(lg, dev(inp.targets), dev(inp.g))
            nrm_lib.cross_entropy_vjp(lg, dev(inp.targets), dev(inp.g), dlogits=lg)
            torch.cuda.synchronize()
        compare.check_exact_bits(x, ref, "softmax in place")
        compare.check_exact_bits(lg, dref, "gradient in place")


def test_softmax_deterministic(nrm_lib):
    say("softmax determinism")
    inp = workloads.ce_inputs(64, 128256, "bf16", seed=10, g="normal")
    a = nrm_lib.cross_entropy(dev(inp.logits), dev(inp.targets))
    b = nrm_lib.cross_entropy(dev(inp.logits), dev(inp.targets))
    torch.cuda.synchronize()
    compare.check_exact_bits(a, b, "second run")


@pytest.mark.slow
def test_cross_entropy_full_size(nrm_lib):
    """[4096, 128256] bf16 in the benchmark's launch: loss and gradient on 48 sampled rows,
    logsumexp on the same rows."""
    say("cross_entropy full size")
    inp = workloads.cfg_ce_bf16()
    sel = np.sort(np.random.default_rng(11).choice(workloads.CE_SHAPE[0], 48, replace=False))
    _ce_check(nrm_lib, inp, "bf16", sel=sel)
    lse = nrm_lib.logsumexp(dev(inp.logits))
    torch.cuda.synchronize()
    compare.check_output(lse[sel], oracle.softmax.logsumexp(f64(inp.logits[sel]), "bf16"),
                         "bf16", what="lse")

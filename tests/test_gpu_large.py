"""Arrays past 2^31 elements (4 GiB of bf16), and rows of 2^23 to 2^25 elements.

Past 2^31 elements every element offset overflows 32 bits somewhere in the array. Each input is
K distinct rows drawn by the workload recipe and repeated on the device
until the array is that large, so every output row must equal the output of its base row bit for
bit (the kernels are deterministic, and a repeated row meets the same arithmetic: with K even the
two-row LayerNorm blocks keep each base row in the same slot). The test checks that for every
row on the device, and checks the base rows against the fp64 oracle. Column sums (dw, db) over
rows repeated 2^12 times are 2^12 times the base rows' sums, which rounding keeps exact, so the
oracle of the base rows gives them too. NormRope rows differ by position: every (b, h) holds the
same [L, D] block, so each must equal (0, 0) bit for bit, and (0, 0) is compared with the
oracle at all L positions (also into a cache). The very wide rows are compared with the oracle
on every element."""

import pytest
import torch

import compare
import oracle
import workloads
from gpu_util import DEV, assert_h_exact, f64, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

K = 66            # distinct base rows (even)
REPS = 4096       # repeats of the base rows: [K * REPS, 8192] has 2,214,592,512 elements
BIG = 2 ** 31


@pytest.fixture(autouse=True)
def _free_device_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def tile(t, reps):
    """Host tensor [K, ...] -> device tensor [K * reps, ...] whose row i is row i % K."""
    d = t.to(DEV)
    return d.repeat(reps, *([1] * (d.dim() - 1)))


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def assert_rows_repeat(t, what, k=K):
    """Row i of t (first axis) equals row i % k bit for bit, for every row."""
    assert t.shape[0] % k == 0
    v = _bits(t.contiguous()).reshape(t.shape[0] // k, k, -1)
    base = v[0]
    step = max(1, (1 << 27) // base.numel())
    for s in range(1, v.shape[0], step):
        blk = v[s:s + step]
        if not torch.equal(blk, base.unsqueeze(0).expand_as(blk)):
            bad = (blk != base.unsqueeze(0)).reshape(blk.shape[0], -1).any(dim=1).nonzero()
            raise AssertionError(f"{what}: repeat {s + int(bad[0])} of the base rows differs "
                                 f"from the first")


def test_large_add_rms_norm_bf16(nrm_lib):
    say(f"large add-RMSNorm bf16 [{K * REPS}, 8192]")
    inp = workloads.row_inputs(K, 8192, "bf16", seed=71, r=("normal", 0.0, 1.0), eps=1e-6)
    x, r = tile(inp.x, REPS), tile(inp.r, REPS)
    assert x.numel() > BIG
    out, h = nrm_lib.add_rms_norm(x, r, inp.w.to(DEV), inp.eps)
    torch.cuda.synchronize()
    del x, r
    assert_rows_repeat(h, "h")
    assert_rows_repeat(out, "out")
    want_out, want_h = oracle.add_rms_norm(f64(inp.x), f64(inp.r), f64(inp.w), inp.eps, "bf16")
    assert_h_exact(h[:K], want_h)
    compare.check_output(out[:K], want_out, "bf16", what="add_rms_norm out")


def test_large_rms_norm_narrow_f32(nrm_lib):
    reps = 2 ** 19
    say(f"large RMSNorm fp32 [{K * reps}, 64]")
    inp = workloads.row_inputs(K, 64, "f32", seed=72, eps=1e-6)
    x = tile(inp.x, reps)
    assert x.numel() > BIG
    out = nrm_lib.rms_norm(x, inp.w.to(DEV), inp.eps)
    torch.cuda.synchronize()
    del x
    assert_rows_repeat(out, "out")
    compare.check_output(out[:K], oracle.rms_norm(f64(inp.x), f64(inp.w), inp.eps, "f32"),
                         "f32", what="rms_norm out")


def test_large_layer_norm_bf16(nrm_lib):
    say(f"large LayerNorm bf16 [{K * REPS}, 8192] with w and b")
    inp = workloads.row_inputs(K, 8192, "bf16", seed=73, x=("normal", 0.5, 2.0),
                               b=("normal", 0.0, 0.1))
    x = tile(inp.x, REPS)
    out = nrm_lib.layer_norm(x, inp.w.to(DEV), inp.b.to(DEV), inp.eps)
    torch.cuda.synchronize()
    del x
    assert_rows_repeat(out, "out")
    want = oracle.layer_norm(f64(inp.x), f64(inp.w), f64(inp.b), inp.eps, "bf16")
    compare.check_output(out[:K], want, "bf16", what="layer_norm out")


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
def test_large_vjp_bf16(nrm_lib, ln):
    say(f"large {'LayerNorm' if ln else 'RMSNorm'} backward bf16 [{K * REPS}, 8192]")
    inp = workloads.row_inputs(K, 8192, "bf16", seed=74 + ln, g=("normal", 0.0, 1.0),
                               x=("normal", 0.5, 2.0) if ln else ("normal", 0.0, 1.0))
    x, g, w = tile(inp.x, REPS), tile(inp.g, REPS), inp.w.to(DEV)
    if ln:
        dx, dw, db = nrm_lib.layer_norm_vjp(x, w, g, inp.eps)
    else:
        dx, dw = nrm_lib.rms_norm_vjp(x, w, g, inp.eps)
    torch.cuda.synchronize()
    del x, g
    assert_rows_repeat(dx, "dx")
    if ln:
        want = oracle.layer_norm_vjp(f64(inp.x), f64(inp.w), None, f64(inp.g), inp.eps, "bf16")
    else:
        want = oracle.rms_norm_vjp(f64(inp.x), f64(inp.w), f64(inp.g), inp.eps, "bf16")
    compare.check_output(dx[:K], want[0], "bf16", what="dx")
    # the base rows' column sums, rounded to bf16, times 2^12: exactly the rounded sums over
    # every row
    compare.check_output(dw, want[1] * REPS, "bf16", what="dw")
    if ln:
        compare.check_output(db, want[2] * REPS, "bf16", what="db")


def test_large_softmax_bf16(nrm_lib):
    say(f"large Softmax bf16 [{K * REPS}, 8192]")
    s = workloads.scores((K, 8192), "bf16", seed=76)
    x = tile(s, REPS)
    out = nrm_lib.softmax(x)
    torch.cuda.synchronize()
    del x
    assert_rows_repeat(out, "out")
    compare.check_output(out[:K], oracle.softmax.softmax(f64(s), "bf16"), "bf16",
                         what="softmax out")


def test_large_cross_entropy_bf16(nrm_lib):
    reps = 256
    V = workloads.CE_SHAPE[1]
    say(f"large CrossEntropy bf16 [{K * reps}, {V}] and its gradient")
    inp = workloads.ce_inputs(K, V, "bf16", seed=77, g="normal")
    logits, tgt, g = tile(inp.logits, reps), tile(inp.targets, reps), tile(inp.g, reps)
    assert logits.numel() > BIG
    loss = nrm_lib.cross_entropy(logits, tgt)
    dl = nrm_lib.cross_entropy_vjp(logits, tgt, g)
    torch.cuda.synchronize()
    del logits
    assert_rows_repeat(loss.reshape(-1, 1), "loss")
    assert_rows_repeat(dl, "dlogits")
    x = f64(inp.logits)
    t = inp.targets.numpy()
    compare.check_f32(f64(loss[:K]), oracle.softmax.cross_entropy(x, t), what="loss")
    compare.check_output(dl[:K], oracle.softmax.cross_entropy_vjp(x, t, f64(inp.g), "bf16"),
                         "bf16", what="dlogits")


def test_large_rope_positions_bf16(nrm_lib):
    reps = 8192
    say(f"large Rope positions form bf16 q [{K * reps}, 32, 128], k [{K * reps}, 8, 128]")
    qk = workloads.rope_qk_inputs(K, 32, 8, 128, "bf16", seed=78, positions="random",
                                  max_position=131072)
    q, k, pos = tile(qk.q, reps), tile(qk.k, reps), tile(qk.positions, reps)
    assert q.numel() > BIG
    qo, ko = nrm_lib.rope_positions(pos, q, k, base=500000.0)
    torch.cuda.synchronize()
    del q, k
    assert_rows_repeat(qo, "q out")
    assert_rows_repeat(ko, "k out")
    p = qk.positions.numpy()
    for got, src, what in ((qo, qk.q, "q out"), (ko, qk.k, "k out")):
        want = oracle.rope_positions(f64(src), p, dims=128, traditional=False, base=500000.0,
                                     scale=1.0, forward=True, dtype="bf16")
        compare.check_output(got[:K], want, "bf16", what=what)


@pytest.mark.parametrize("traditional", [False, True])
def test_large_norm_rope_bf16(nrm_lib, traditional):
    B, H, L, D = 8, 32, 65600, 128
    say(f"large NormRope bf16 [{B}, {H}, {L}, {D}] traditional={traditional} (and cache)")
    rp = workloads.rope_inputs(1, 1, L, D, "bf16", seed=79)
    x = rp.x.to(DEV).expand(B, H, L, D).contiguous()
    assert x.numel() > BIG
    w = rp.w.to(DEV)
    off = 64
    kw = dict(eps=rp.eps, dims=D, traditional=traditional, base=rp.base, scale=rp.scale)
    out = nrm_lib.norm_rope(x, w, offset=off, **kw)
    cache = None
    if not traditional:
        cache = torch.zeros(B, H, L + off, D, dtype=torch.bfloat16, device=DEV)
        nrm_lib.norm_rope(x, w, offset=off, cache=cache, **kw)
    torch.cuda.synchronize()
    del x
    assert_rows_repeat(out.reshape(B * H, L * D), "out", k=1)
    want = oracle.norm_rope(f64(rp.x), f64(rp.w), normalize=True, eps=rp.eps, dims=D,
                            traditional=traditional, base=rp.base, scale=rp.scale, offset=off,
                            forward=True, dtype="bf16")
    compare.check_output(out[0:1, 0:1], want, "bf16", what="norm_rope out")
    if cache is not None:
        # the written rows are the plain output bit for bit; the rows before offset stay zero
        assert torch.equal(_bits(cache[:, :, off:]), _bits(out)), "cache rows differ from out"
        assert not bool(_bits(cache[:, :, :off]).any()), "cache rows before offset changed"


@pytest.mark.parametrize("op,dt,n", [("rms", "bf16", 2 ** 25 + 8), ("rms", "bf16", 2 ** 25 + 3),
                                     ("add", "f32", 2 ** 24 + 4), ("ln", "bf16", 2 ** 25 + 8)],
                         ids=lambda v: str(v))
def test_very_wide_rows(nrm_lib, op, dt, n):
    """A few rows of 2^24 to 2^25 elements (the looping kernels; 2^25 + 3 one element at a
    time), every element against the oracle."""
    say(f"very wide rows {op} {dt} [3, {n}]")
    inp = workloads.row_inputs(3, n, dt, seed=80, r=("normal", 0.0, 1.0) if op == "add" else None,
                               x=("normal", 0.5, 2.0) if op == "ln" else ("normal", 0.0, 1.0),
                               b=("normal", 0.0, 0.1) if op == "ln" else None)
    x, w = inp.x.to(DEV), inp.w.to(DEV)
    if op == "rms":
        got = nrm_lib.rms_norm(x, w, inp.eps)
        want = oracle.rms_norm(f64(inp.x), f64(inp.w), inp.eps, dt)
    elif op == "add":
        got, h = nrm_lib.add_rms_norm(x, inp.r.to(DEV), w, inp.eps)
        want, want_h = oracle.add_rms_norm(f64(inp.x), f64(inp.r), f64(inp.w), inp.eps, dt)
        assert_h_exact(h, want_h)
    else:
        got = nrm_lib.layer_norm(x, w, inp.b.to(DEV), inp.eps)
        want = oracle.layer_norm(f64(inp.x), f64(inp.w), f64(inp.b), inp.eps, dt)
    compare.check_output(got, want, dt, what=f"{op} out")


@pytest.mark.parametrize("dt,n", [("bf16", 2 ** 25 + 3), ("f32", 2 ** 24)], ids=str)
def test_very_wide_softmax_family(nrm_lib, dt, n):
    """Softmax, LogSumExp, CrossEntropy and its gradient over rows of 2^24 to 2^25 columns."""
    say(f"very wide softmax family {dt} [2, {n}]")
    inp = workloads.ce_inputs(2, n, dt, seed=81, g="normal")
    x, tgt, g = inp.logits.to(DEV), inp.targets.to(DEV), inp.g.to(DEV)
    xs = f64(inp.logits)
    compare.check_output(nrm_lib.softmax(x), oracle.softmax.softmax(xs, dt), dt, what="softmax")
    compare.check_output(nrm_lib.logsumexp(x), oracle.softmax.logsumexp(xs, dt), dt,
                         what="logsumexp")
    t = inp.targets.numpy()
    compare.check_f32(f64(nrm_lib.cross_entropy(x, tgt)), oracle.softmax.cross_entropy(xs, t),
                      what="loss")
    compare.check_output(nrm_lib.cross_entropy_vjp(x, tgt, g),
                         oracle.softmax.cross_entropy_vjp(xs, t, f64(inp.g), dt), dt,
                         what="dlogits")


@pytest.mark.parametrize("ln,dt,n", [(False, "bf16", 2 ** 24 + 8), (True, "f32", 2 ** 23 + 4)],
                         ids=str)
def test_very_wide_vjp(nrm_lib, ln, dt, n):
    """The backward over a few rows of 2^23 to 2^24 elements (the looping kernel): dx, dw and db
    on every element."""
    say(f"very wide {'LayerNorm' if ln else 'RMSNorm'} backward {dt} [3, {n}]")
    inp = workloads.row_inputs(3, n, dt, seed=82, g=("normal", 0.0, 1.0))
    x, w, g = inp.x.to(DEV), inp.w.to(DEV), inp.g.to(DEV)
    if ln:
        got = nrm_lib.layer_norm_vjp(x, w, g, inp.eps)
        want = oracle.layer_norm_vjp(f64(inp.x), f64(inp.w), None, f64(inp.g), inp.eps, dt)
    else:
        got = nrm_lib.rms_norm_vjp(x, w, g, inp.eps)
        want = oracle.rms_norm_vjp(f64(inp.x), f64(inp.w), f64(inp.g), inp.eps, dt)
    for gt, wt, what in zip(got, want, ("dx", "dw", "db")):
        compare.check_output(gt, wt, dt, what=what)


def test_launch_pieces_layer_norm(nrm_lib):
    """A LayerNorm call over more than 1 GiB runs as pieces of whole rows: [65539, 8192] bf16
    is two pieces of 32768 rows (two-row kernel) and a tail of 3 (one row per block). Every
    row before the tail equals its base row bit for bit; the base rows and the tail match the
    oracle."""
    reps = 993
    n = K * reps + 1
    say(f"LayerNorm bf16 [{n}, 8192] in launch pieces")
    inp = workloads.row_inputs(K, 8192, "bf16", seed=83, x=("normal", 0.5, 2.0),
                               b=("normal", 0.0, 0.1))
    x = tile(inp.x, reps + 1)[:n].contiguous()
    assert x.shape[0] == n and x.shape[0] * 8192 * 2 * 2 > 2 ** 30
    out = nrm_lib.layer_norm(x, inp.w.to(DEV), inp.b.to(DEV), inp.eps)
    torch.cuda.synchronize()
    del x
    head = 2 * 32768
    assert_rows_repeat(out[:head - head % K], "out")
    want = oracle.layer_norm(f64(inp.x), f64(inp.w), f64(inp.b), inp.eps, "bf16")
    compare.check_output(out[:K], want, "bf16", what="base rows")
    tail = list(range(head - head % K, n))
    compare.check_output(out[tail], want[[i % K for i in tail]], "bf16",
                         what="rows after the last whole repeat, the tail included")

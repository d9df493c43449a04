"""GPU parity of the backward operations (RmsNormVjp, LayerNormVjp) through the C ABI against
the fp64 oracle: dx element by element, dw and db (sums over every row) element by element.

Bars as for the forward operations: bf16 within 1 ulp, fp32 within 1e-5 relative + 1e-6
absolute, of the oracle's once-rounded values. The parameter gradients are the same bits on
every run.
"""

import numpy as np
import pytest
import torch

import compare
import workloads
from gpu_util import DEV, check_vjp, dev, f64, forced_path, run_vjp, say, vjp_oracle

pytestmark = pytest.mark.gpu

HIDDEN = [1, 2, 7, 8, 64, 100, 512, 520, 1000, 4096, 5120, 8192, 8200, 12288, 16384]
WEIGHTS = [("bf16", "bf16"), ("bf16", "f32"), ("bf16", None), ("f32", "f32"), ("f32", None)]


def _inp(rows, hidden, dt, wdt, seed, ln, **kw):
    x = ("normal", 0.5, 2.0) if ln else ("t3",)
    return workloads.row_inputs(rows, hidden, dt, seed=seed, x=x,
                                w=("normal", 1.0, 0.1) if wdt else None,
                                g=("normal", 0.0, 1.0), w_dtype=wdt or None,
                                eps=1e-5 if ln else 1e-6, **kw)


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
@pytest.mark.parametrize("hidden", HIDDEN)
@pytest.mark.parametrize("dt,wdt", WEIGHTS)
def test_vjp_shapes(nrm_lib, ln, hidden, dt, wdt):
    say(f"vjp {'ln' if ln else 'rms'} rows=6 hidden={hidden} {dt} w={wdt}")
    check_vjp(nrm_lib, _inp(6, hidden, dt, wdt, hidden + 40, ln), ln)


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
@pytest.mark.parametrize("rows", [1, 2, 3, 7, 255, 256, 257, 513, 1000, 4097])
@pytest.mark.parametrize("hidden", [64, 512, 4096])
def test_vjp_row_counts(nrm_lib, ln, rows, hidden):
    """Row counts around the partial-row grid (256 blocks) and the teams per block."""
    say(f"vjp {'ln' if ln else 'rms'} rows={rows} hidden={hidden}")
    check_vjp(nrm_lib, _inp(rows, hidden, "bf16", "bf16", rows, ln), ln)


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
@pytest.mark.parametrize("rows", [512, 768, 1277, 1536, 1792, 2048, 2301, 2816])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_vjp_rows_per_block(nrm_lib, ln, rows, dt):
    """One 1024-thread team per row (hidden 8192) with 2, 3, 5, 6, 7, 8, 9 and 11 rows per
    block (256 blocks, rows strided): every mix of the row ring's start, its unrolled loop
    and its last rows, and of the two-chunk loop for fp32."""
    say(f"vjp {'ln' if ln else 'rms'} rows={rows} hidden=8192 {dt}")
    sel = np.r_[0:4, rows // 2 - 2:rows // 2 + 2, rows - 4:rows]
    check_vjp(nrm_lib, _inp(rows, 8192, dt, dt, rows + 3, ln), ln, rows_sel=sel, chunk=1024)


@pytest.mark.parametrize("path", ["chunked", "scalar"])
@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
@pytest.mark.parametrize("hidden", [512, 4096, 8192])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_vjp_generic_kernel(nrm_lib, path, ln, hidden, dt):
    """The looping kernel (16-byte chunks, or one element at a time) on rows the register
    kernel would take."""
    say(f"vjp forced {path} {'ln' if ln else 'rms'} hidden={hidden} {dt}")
    with forced_path(path):
        check_vjp(nrm_lib, _inp(300, hidden, dt, dt, 5, ln), ln)


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
def test_vjp_optional_gradients(nrm_lib, ln):
    """Asking for fewer gradients leaves dx's bits unchanged, and each parameter gradient is
    the same alone as together."""
    say(f"vjp optional gradients {'ln' if ln else 'rms'}")
    inp = _inp(700, 4096, "bf16", "bf16", 11, ln)
    full = run_vjp(nrm_lib, inp, ln)
    none = run_vjp(nrm_lib, inp, ln, want_dw=False, want_db=False)
    compare.check_exact_bits(none[0], full[0], "dx without parameter gradients")
    assert all(t is None for t in none[1:])
    if ln:
        only_w = run_vjp(nrm_lib, inp, ln, want_dw=True, want_db=False)
        only_b = run_vjp(nrm_lib, inp, ln, want_dw=False, want_db=True)
        compare.check_exact_bits(only_w[1], full[1], "dw alone")
        compare.check_exact_bits(only_b[2], full[2], "db alone")
        assert only_w[2] is None and only_b[1] is None


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
@pytest.mark.parametrize("hidden,dt,wdt", [(8000, "bf16", "bf16"), (8000, "bf16", "f32"),
                                           (8000, "bf16", None), (4000, "f32", "f32"),
                                           (4000, "f32", None)])
def test_vjp_ragged_rows_many(nrm_lib, ln, hidden, dt, wdt):
    """Rows of 1000 chunks (a 1024-thread team, the last 24 lanes past the row's end) with
    2301 rows: 256 blocks of up to 9 rows each, so every team runs the register ring's steady
    state and its tail with clamped chunks."""
    say(f"vjp ragged many rows {'ln' if ln else 'rms'} hidden={hidden} {dt} w={wdt}")
    check_vjp(nrm_lib, _inp(2301, hidden, dt, wdt, 23, ln), ln)


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
@pytest.mark.parametrize("hidden,dt,wdt", [(12000, "bf16", "bf16"), (12288, "bf16", "bf16"),
                                           (16384, "bf16", "bf16"), (16384, "bf16", "f32"),
                                           (12000, "bf16", None), (10000, "f32", "f32"),
                                           (16384, "f32", "f32")])
def test_vjp_wide_rows(nrm_lib, ln, hidden, dt, wdt):
    """Rows of 8193 to 16384 elements: 16 per thread, one team of up to 1024 threads per row,
    the dw column sums accumulated in LDS; 700 rows (256 blocks of up to 3 rows), exact and
    ragged widths."""
    say(f"vjp wide rows {'ln' if ln else 'rms'} hidden={hidden} {dt} w={wdt}")
    check_vjp(nrm_lib, _inp(700, hidden, dt, wdt, 29, ln), ln)


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
@pytest.mark.parametrize("hidden,dt,wdt", [(8, "bf16", "bf16"), (64, "bf16", "bf16"),
                                           (120, "bf16", "bf16"), (128, "bf16", "f32"),
                                           (128, "bf16", None), (256, "bf16", "bf16"),
                                           (16, "f32", "f32"), (100, "f32", None),
                                           (128, "f32", "f32")])
def test_vjp_narrow_rows_many(nrm_lib, ln, hidden, dt, wdt):
    """Rows of at most 32 chunks: teams of 8, 16 or 32 lanes, 256 / team rows in flight per
    block. 30001 rows give every team several rows (the two-buffer loop and a ragged last
    step) and leave some teams with none in the last step."""
    say(f"vjp narrow rows {'ln' if ln else 'rms'} rows=30001 hidden={hidden} {dt} w={wdt}")
    check_vjp(nrm_lib, _inp(30001, hidden, dt, wdt, 31, ln), ln)


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
@pytest.mark.parametrize("hidden,dt,wdt", [(1001, "bf16", "bf16"), (2047, "bf16", "f32"),
                                           (3001, "bf16", None), (4100, "bf16", "bf16"),
                                           (6150, "bf16", "bf16"), (8191, "bf16", "bf16"),
                                           (7000, "bf16", "f32"), (1001, "f32", "f32"),
                                           (4097, "f32", None), (6145, "f32", "f32"),
                                           (100, "bf16", "bf16"), (33, "f32", "f32")])
def test_vjp_element_rows(nrm_lib, ln, hidden, dt, wdt):
    """Widths that are not whole 16-byte chunks: 1 (33), 2 (100), 4 (up to 4096), 6 or 8
    elements per thread in one block per run of rows (8 only with bf16 weights; wider rows,
    and 7000 with fp32 weights, take the generic kernel). 2301 rows: runs of 9 rows (whole
    and partial trips of the 2-, 3- and 4-deep register rings) and a last run of 6."""
    say(f"vjp element rows {'ln' if ln else 'rms'} rows=2301 hidden={hidden} {dt} w={wdt}")
    check_vjp(nrm_lib, _inp(2301, hidden, dt, wdt, 37, ln), ln)


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_vjp_misaligned_bases(nrm_lib, ln, dt):
    """x, g and dx one element past a 16-byte boundary (views into larger buffers), with a
    width of whole chunks: the single-element kernel."""
    say(f"vjp misaligned bases {'ln' if ln else 'rms'} {dt}")
    rows, n = 300, 4096
    inp = _inp(rows, n, dt, dt, 41, ln)

    def shifted(t):
        buf = torch.zeros(rows * n + 8, dtype=t.dtype, device=DEV)
        v = buf[1:1 + rows * n].view(rows, n)
        v.copy_(dev(t))
        return v

    x, g = shifted(inp.x), shifted(inp.g)
    dxo = torch.empty(rows * n + 8, dtype=x.dtype, device=DEV)[1:1 + rows * n].view(rows, n)
    w = dev(inp.w)
    if ln:
        got = nrm_lib.layer_norm_vjp(x, w, g, inp.eps, dx=dxo)
    else:
        got = nrm_lib.rms_norm_vjp(x, w, g, inp.eps, dx=dxo)
    torch.cuda.synchronize()
    assert got[0].data_ptr() == dxo.data_ptr()
    want_dx, want_params = vjp_oracle(inp, ln)
    compare.check_output(got[0], want_dx, dt, what="dx")
    for name, gv, wv in zip(("dw", "db"), got[1:], want_params):
        compare.check_output(gv, wv, dt, what=name)


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
def test_vjp_zero_rows_zero_parameter_gradients(nrm_lib, ln):
    say(f"vjp zero rows {'ln' if ln else 'rms'}")
    x = torch.empty(0, 256, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(256, dtype=torch.bfloat16, device=DEV)
    dw = torch.full((256,), float("nan"), dtype=torch.bfloat16, device=DEV)
    if ln:
        db = torch.full((256,), float("nan"), dtype=torch.bfloat16, device=DEV)
        dx, dw, db = nrm_lib.layer_norm_vjp(x, w, x, 1e-5, dw=dw, db=db)
        torch.cuda.synchronize()
        assert torch.all(db == 0)
    else:
        dx, dw = nrm_lib.rms_norm_vjp(x, w, x, 1e-5, dw=dw)
        torch.cuda.synchronize()
    assert dx.numel() == 0 and torch.all(dw == 0)


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
@pytest.mark.parametrize("into", ["x", "g"])
def test_vjp_in_place(nrm_lib, ln, into):
    """dx written over x or over g gives the out-of-place bits (fast, single-element and
    generic kernels)."""
    for path, hidden in ((None, 4096), (None, 1000), (None, 4100), ("chunked", 4096),
                         ("scalar", 1000)):
        say(f"vjp in place into {into} {'ln' if ln else 'rms'} path={path}")
        inp = _inp(300, hidden, "bf16", "bf16", 12, ln)
        with forced_path(path):
            ref = run_vjp(nrm_lib, inp, ln)
            x, w, g = dev(inp.x), dev(inp.w), dev(inp.g)
            target = x if into == "x" else g
            if ln:
                got = nrm_lib.layer_norm_vjp(x, w, g, inp.eps, dx=target)
            else:
                got = nrm_lib.rms_norm_vjp(x, w, g, inp.eps, dx=target)
            torch.cuda.synchronize()
        compare.check_exact_bits(target, ref[0], f"dx in place over {into}")
        for a, b in zip(got[1:], ref[1:]):
            compare.check_exact_bits(a, b, "parameter gradient with dx in place")


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
def test_vjp_deterministic(nrm_lib, ln):
    say(f"vjp determinism {'ln' if ln else 'rms'}")
    inp = _inp(3000, 8192, "bf16", "bf16", 13, ln)
    a = run_vjp(nrm_lib, inp, ln)
    b = run_vjp(nrm_lib, inp, ln)
    for u, v in zip(a, b):
        compare.check_exact_bits(u, v, "second run")


def test_vjp_special_rows(nrm_lib):
    """Constant rows (LayerNorm: x - mean is exactly 0, so they add nothing to dw) and
    all-zero rows (RMSNorm: dx = g w / sqrt(eps), nothing to dw)."""
    say("vjp special rows")
    for ln in (False, True):
        inp = _inp(40, 4096, "bf16", "bf16", 14, ln)
        inp.x[::3] = 0.0
        inp.x[1::3] = 2.5
        check_vjp(nrm_lib, inp, ln)


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
@pytest.mark.parametrize("hidden", [4096, 8191])
def test_vjp_graph_replays(nrm_lib, ln, hidden):
    """Captured in a HIP graph (row kernel + column sum), every replay matches eager; 8191
    takes the single-element kernel with its column sums in LDS."""
    say(f"vjp graph {'ln' if ln else 'rms'} hidden={hidden}")
    inp = _inp(1024, hidden, "bf16", "bf16", 15, ln)
    x, w, g = dev(inp.x), dev(inp.w), dev(inp.g)
    eager = run_vjp(nrm_lib, inp, ln)
    dx = torch.empty_like(x)
    dw = torch.empty_like(w)
    db = torch.empty_like(w) if ln else None
    ws = torch.empty(nrm_lib.vjp_workspace_bytes(1024, hidden, ln), dtype=torch.uint8,
                     device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            if ln:
                nrm_lib.layer_norm_vjp(x, w, g, inp.eps, dx=dx, dw=dw, db=db, workspace=ws)
            else:
                nrm_lib.rms_norm_vjp(x, w, g, inp.eps, dx=dx, dw=dw, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        dx.fill_(float("nan"))
        dw.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        compare.check_exact_bits(dx, eager[0], f"replay {rep} dx")
        compare.check_exact_bits(dw, eager[1], f"replay {rep} dw")
        if ln:
            compare.check_exact_bits(db, eager[2], f"replay {rep} db")


@pytest.mark.slow
@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
def test_vjp_full_size(nrm_lib, ln):
    """[16384, 8192] bf16 in the benchmark's launch: dx on sampled rows, dw and db over all
    rows (the oracle's float64 column sums taken in chunks of rows, rounded once)."""
    say(f"vjp full size {'ln' if ln else 'rms'}")
    inp = workloads.cfg_ln_vjp() if ln else workloads.cfg_rms_vjp()
    rng = np.random.default_rng(99)
    sel = torch.from_numpy(np.sort(rng.choice(inp.x.shape[0], 64, replace=False)))
    check_vjp(nrm_lib, inp, ln, rows_sel=sel, chunk=1024)

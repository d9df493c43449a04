"""LayerNorm and LayerNormVjp on rows whose mean is large against their spread, where a
variance formed from raw moments (sum x^2 / n - mean^2) loses every bit even in fp64: fp32
rows 1e4 + N(0, 0.01) (|mean| / sigma = 1e6) and -3e5 + N(0, 0.5) (6e5), and bf16 rows
1024 + N(0, 16) whose values differ by a few units in the last place. Every kernel shape is
reached: teams (narrow rows), one block per row, two rows per block (4097 rows with a scale
or shift), single-element rows (widths that are not whole 16-byte chunks), the looping and
register kernels (forced), and for the backward the narrow teams, the register-row kernel
(one and two chunks per thread, exact and ragged), the single-element kernel and the generic
kernel (forced). Backward cotangents are N(0, 1), or 1e3 + N(0, 1) so that d = g w has a
large mean too. Compared with the oracle element by element (bf16 within 1 ulp, fp32 within
1e-5 relative + 1e-6 absolute)."""

import numpy as np
import pytest

import workloads
from gpu_util import check_ln, check_vjp, forced_path, say

pytestmark = pytest.mark.gpu

MEANS = [("f32", ("normal", 1e4, 0.01)), ("f32", ("normal", -3e5, 0.5)),
         ("bf16", ("normal", 1024.0, 16.0))]
MEAN_IDS = ["f32-1e4", "f32-3e5", "bf16-1024"]


def _ln_inputs(rows, hidden, dt, xd, affine, seed):
    inp = workloads.row_inputs(rows, hidden, dt, seed=seed, x=xd, w=("normal", 1.0, 0.1),
                               b=("normal", 0.0, 0.1), eps=1e-5)
    if "w" not in affine:
        inp.w = None
    if "b" not in affine:
        inp.b = None
    return inp


@pytest.mark.parametrize("dt,xd", MEANS, ids=MEAN_IDS)
@pytest.mark.parametrize("hidden", [256, 4096, 4100, 8192, 8200])
@pytest.mark.parametrize("affine", ["wb", "none"])
def test_layer_norm_large_mean(nrm_lib, dt, xd, hidden, affine):
    say(f"layer_norm large mean rows=64 hidden={hidden} {dt} {xd} {affine}")
    check_ln(nrm_lib, _ln_inputs(64, hidden, dt, xd, affine, seed=hidden))


@pytest.mark.parametrize("dt,xd", MEANS, ids=MEAN_IDS)
@pytest.mark.parametrize("hidden", [4096, 8192, 8200])
def test_layer_norm_large_mean_row_pairs(nrm_lib, dt, xd, hidden):
    say(f"layer_norm large mean row pairs rows=4097 hidden={hidden} {dt} {xd}")
    inp = _ln_inputs(4097, hidden, dt, xd, "wb", seed=hidden + 1)
    check_ln(nrm_lib, inp, rows_sel=np.r_[0:3, 2047:2050, 4093:4097])


@pytest.mark.parametrize("dt,xd", MEANS, ids=MEAN_IDS)
@pytest.mark.parametrize("path", ["wave", "block", "chunked", "scalar"])
def test_layer_norm_large_mean_forced(nrm_lib, dt, xd, path):
    say(f"layer_norm large mean forced={path} rows=16 hidden=4096 {dt} {xd}")
    with forced_path(path):
        check_ln(nrm_lib, _ln_inputs(16, 4096, dt, xd, "wb", seed=7))


@pytest.mark.parametrize("dt,xd", MEANS, ids=MEAN_IDS)
@pytest.mark.parametrize("gmean", [0.0, 1e3])
@pytest.mark.parametrize("hidden", [128, 4096, 4100, 8192, 8200, 12000])
def test_layer_norm_vjp_large_mean(nrm_lib, dt, xd, gmean, hidden):
    say(f"layer_norm_vjp large mean rows=300 hidden={hidden} {dt} {xd} g mean {gmean}")
    inp = workloads.row_inputs(300, hidden, dt, seed=hidden + 3, x=xd, w=("normal", 1.0, 0.1),
                               g=("normal", gmean, 1.0), eps=1e-5)
    check_vjp(nrm_lib, inp, ln=True)


@pytest.mark.parametrize("dt,xd", MEANS, ids=MEAN_IDS)
@pytest.mark.parametrize("path", ["chunked", "scalar"])
def test_layer_norm_vjp_large_mean_forced(nrm_lib, dt, xd, path):
    say(f"layer_norm_vjp large mean forced={path} rows=40 hidden=4096 {dt} {xd}")
    inp = workloads.row_inputs(40, 4096, dt, seed=11, x=xd, w=("normal", 1.0, 0.1),
                               g=("normal", 1e3, 1.0), eps=1e-5)
    with forced_path(path):
        check_vjp(nrm_lib, inp, ln=True)

"""The full-size comparison harness (oracle_pool) on the CPU: the oracle's own outputs pass,
and a planted error in h or out is caught. No GPU involved."""

import numpy as np
import torch

import oracle
import oracle_pool
import pytest
import workloads


def _bf16_tensor(values):
    return torch.from_numpy(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)


def _add_case(dt):
    inp = workloads.row_inputs(1100, 64, dt, seed=5, x=("t3",), r=("t3",), eps=1e-6,
                               outlier_frac=0.01)
    f = lambda t: t.to(torch.float64).numpy()
    out, h = oracle.add_rms_norm(f(inp.x), f(inp.r), f(inp.w), inp.eps, dt)
    cast = _bf16_tensor if dt == "bf16" else (lambda v: torch.from_numpy(v.astype(np.float32)))
    return inp, cast(out), cast(h)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_add_rms_all_rows_passes_and_catches(dt):
    inp, out, h = _add_case(dt)
    oracle_pool.check_add_rms_all_rows(inp.x, inp.r, inp.w, inp.eps, out, h)
    bad_h = h.clone()
    bad_h.view(torch.int16 if dt == "bf16" else torch.int32)[1037, 5] ^= 1
    with pytest.raises(AssertionError, match="h: 1 elements"):
        oracle_pool.check_add_rms_all_rows(inp.x, inp.r, inp.w, inp.eps, out, bad_h)
    bad_out = out.clone()
    if dt == "bf16":
        bad_out.view(torch.int16)[600, 3] += 2  # two units in the last place
    else:
        bad_out[600, 3] *= 1.0 + 3e-5
    with pytest.raises(AssertionError, match="out: 1 elements"):
        oracle_pool.check_add_rms_all_rows(inp.x, inp.r, inp.w, inp.eps, bad_out, h)


def test_layer_norm_all_rows_passes_and_catches():
    inp = workloads.row_inputs(700, 96, "bf16", seed=6, x=("normal", 0.5, 2.0),
                               b=("normal", 0.0, 0.1), eps=1e-5)
    f = lambda t: t.to(torch.float64).numpy()
    out = _bf16_tensor(oracle.layer_norm(f(inp.x), f(inp.w), f(inp.b), inp.eps, "bf16"))
    oracle_pool.check_layer_norm_all_rows(inp.x, inp.w, inp.b, inp.eps, out)
    out.view(torch.int16)[699, 95] -= 2
    with pytest.raises(AssertionError, match="out: 1 elements"):
        oracle_pool.check_layer_norm_all_rows(inp.x, inp.w, inp.b, inp.eps, out)

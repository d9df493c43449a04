"""nrm_layer_norm_vjp_noalloc (partial column sums in the library's static device scratch)
against nrm_layer_norm_vjp with a caller workspace, both through the C ABI: the same kernels,
so dx, dw and db must agree bit for bit. Two calls in a row, the second smaller than the
first, so the second runs over the first call's leftover scratch contents."""

import numpy as np
import pytest
import torch

import compare
import workloads
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu

F32, BF16 = 0, 1


def _codes(t):
    return BF16 if t.dtype == torch.bfloat16 else F32


def _run(L, inp, noalloc):
    x, w, g = inp.x.to(DEV), inp.w.to(DEV), inp.g.to(DEV)
    rows, hidden = x.shape
    dx = torch.empty_like(x)
    dw = torch.full_like(w, float("nan"))
    db = torch.full_like(w, float("nan"))
    if noalloc:
        st = L.nrm_layer_norm_vjp_noalloc(x.data_ptr(), w.data_ptr(), g.data_ptr(), dx.data_ptr(),
                                          dw.data_ptr(), db.data_ptr(), rows, hidden, inp.eps,
                                          _codes(x), _codes(w), None)
    else:
        need = L.nrm_norm_vjp_workspace_bytes(rows, hidden, 1)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
        st = L.nrm_layer_norm_vjp(x.data_ptr(), w.data_ptr(), g.data_ptr(), dx.data_ptr(),
                                  dw.data_ptr(), db.data_ptr(), rows, hidden, inp.eps, _codes(x),
                                  _codes(w), ws.data_ptr(), need, None)
    assert st == 0, L.nrm_last_error().decode()
    torch.cuda.synchronize()
    return dx, dw, db


def test_noalloc_matches_workspace_twice(nrm_lib):
    L = nrm_lib.load()
    cases = [
        # the largest partial-sum set the scratch holds: 256 partial rows of 8192 for dw and db
        ("bf16 [4096, 8192]", workloads.row_inputs(4096, 8192, "bf16", seed=31,
                                                   x=("normal", 0.5, 2.0), w=("normal", 1.0, 0.1),
                                                   g=("normal", 0.0, 1.0), eps=1e-5)),
        # smaller, another dtype and a ragged width, over the first call's leftover contents
        ("f32 [300, 4100]", workloads.row_inputs(300, 4100, "f32", seed=32,
                                                 x=("normal", 1e4, 0.01), w=("normal", 1.0, 0.1),
                                                 g=("normal", 1e3, 1.0), eps=1e-5)),
    ]
    for name, inp in cases:
        say(f"layer_norm_vjp_noalloc {name}")
        got = _run(L, inp, noalloc=True)
        want = _run(L, inp, noalloc=False)
        for what, gt, wt in zip(("dx", "dw", "db"), got, want):
            compare.check_exact_bits(gt, wt, what=f"{name} {what}")


def test_noalloc_rejects_beyond_the_scratch(nrm_lib):
    L = nrm_lib.load()
    x = torch.zeros(4096, 8200, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(8200, dtype=torch.bfloat16, device=DEV)
    dx, dw, db = torch.empty_like(x), torch.empty_like(w), torch.empty_like(w)
    st = L.nrm_layer_norm_vjp_noalloc(x.data_ptr(), w.data_ptr(), x.data_ptr(), dx.data_ptr(),
                                      dw.data_ptr(), db.data_ptr(), 4096, 8200, 1e-5, BF16, BF16,
                                      None)
    assert st == 2 and "at most 33554432 scratch bytes" in L.nrm_last_error().decode()

"""The five synthetic workloads at full size, through the same calls the bench times, every
output element compared with the oracle: the small ones in this process, the [16384, 8192]
and [65536, 5120] ones in chunks of rows over a process pool (oracle_pool), h bit for bit on
every row."""

import numpy as np
import pytest
import torch

import compare
import workloads
import oracle_pool
from gpu_util import DEV, check_add, check_ln, check_rope, dev, f64, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def test_cfg1_add_rms_fp32_small(nrm_lib):
    say("cfg1 add-RMSNorm fp32 [64,512]")
    check_add(nrm_lib, workloads.cfg_add_rms_small_f32())


def test_cfg2_add_rms_bf16_4k(nrm_lib):
    say("cfg2 add-RMSNorm bf16 [4096,4096]")
    check_add(nrm_lib, workloads.cfg_add_rms_4k_bf16())


@pytest.mark.parametrize("affine", [True, False])
def test_cfg3_layer_norm_bf16(nrm_lib, affine):
    say(f"cfg3 LayerNorm bf16 [16384,8192] affine={affine}")
    inp = workloads.cfg_layer_norm_bf16(affine=affine)
    out = nrm_lib.layer_norm(dev(inp.x), dev(inp.w), dev(inp.b), inp.eps)
    torch.cuda.synchronize()
    oracle_pool.check_layer_norm_all_rows(inp.x, inp.w, inp.b, inp.eps, out)


@pytest.mark.parametrize("traditional", [False, True])
@pytest.mark.parametrize("cache", [False, True])
def test_cfg4_norm_rope_bf16(nrm_lib, traditional, cache):
    say(f"cfg4 NormRope bf16 [8,32,512,128] traditional={traditional} cache={cache}")
    if cache:
        rp = workloads.cfg_norm_rope_bf16(offset=workloads.NORM_ROPE_CACHE_OFFSET)
        c = torch.zeros(8, 32, workloads.NORM_ROPE_CACHE_LEN, 128, dtype=torch.bfloat16)
        check_rope(nrm_lib, rp, traditional=traditional, cache=c)
    else:
        check_rope(nrm_lib, workloads.cfg_norm_rope_bf16(), traditional=traditional)


@pytest.fixture(scope="module")
def scale_inputs():
    """The fp32 draws of the at-scale workloads; bf16 inputs are their RNE casts."""
    return {shape: workloads.cfg_add_rms_scale(*shape, dtype="f32")
            for shape in ((16384, 8192), (65536, 5120))}


@pytest.mark.parametrize("shape", [(16384, 8192), (65536, 5120)], ids=["16384x8192", "65536x5120"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_cfg5_add_rms_at_scale(nrm_lib, scale_inputs, shape, dt):
    say(f"cfg5 add-RMSNorm {dt} {shape}")
    inp = scale_inputs[shape]
    if dt == "bf16":
        inp = workloads.RowInputs(x=inp.x.to(torch.bfloat16), r=inp.r.to(torch.bfloat16),
                                  w=inp.w.to(torch.bfloat16), b=None, eps=inp.eps)
    out, h = nrm_lib.add_rms_norm(dev(inp.x), dev(inp.r), dev(inp.w), inp.eps)
    torch.cuda.synchronize()
    oracle_pool.check_add_rms_all_rows(inp.x, inp.r, inp.w, inp.eps, out, h)

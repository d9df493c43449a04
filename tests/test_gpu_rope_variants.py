"""GPU parity of the Rope variants through the C ABI against the fp64 oracle: standalone Rope
with base or a freqs vector and an attention factor, NormRope with freqs, and the
positions form on query and key rows (one launch), including the scaled frequencies of
the host generators. Bars: bf16 within 1 ulp, fp32 within 1e-5 relative + 1e-6 absolute.
"""

import numpy as np
import pytest
import torch

import compare
import oracle
import workloads
from gpu_util import DEV, DT, dev, f64, forced_path, say

pytestmark = pytest.mark.gpu


def _freqs(kind, dims, rng):
    """freqs input and mscale: none, or seeded synthetic divisors (the scaled-frequency
    generators themselves are checked against the oracle on the host)."""
    if kind is None:
        return None, 1.0
    seed = int(rng.integers(1 << 30))
    return workloads.rope_freqs_draw(dims, kind, seed), (1.0 if kind == "uniform" else 1.2079)


def _rope_case(nrm, N, L, D, dims, dt, trad, offset, fkind, forward, seed, path=None):
    rng = np.random.default_rng(seed)
    x = workloads.cast(rng.standard_normal((N, L, D)), dt)
    freqs, ms = _freqs(fkind, dims, rng)
    with forced_path(path):
        got = nrm.rope(dev(x), dims=dims, traditional=trad, base=10000.0, scale=0.5,
                       offset=offset, forward=forward, freqs=dev(freqs), mscale=ms)
        torch.cuda.synchronize()
    want = oracle.norm_rope(f64(x)[:, None], None, normalize=False, eps=0.0, dims=dims,
                            traditional=trad, base=10000.0, scale=0.5, offset=offset,
                            forward=forward, dtype=dt, freqs=f64(freqs), mscale=ms)[:, 0]
    compare.check_output(got, want, dt, what="rope out")


@pytest.mark.parametrize("D,dims", [(128, 128), (128, 64), (64, 64), (96, 32), (80, 80),
                                    (16, 0), (130, 128), (6, 4)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("trad", [False, True])
@pytest.mark.parametrize("fkind", [None, "uniform", "loguniform"])
def test_rope_shapes(nrm_lib, D, dims, dt, trad, fkind):
    say(f"rope D={D} dims={dims} {dt} trad={trad} freqs={fkind}")
    _rope_case(nrm_lib, 5, 33, D, dims, dt, trad, 1000, fkind, True, D + dims)


@pytest.mark.parametrize("path", [None, "scalar"])
@pytest.mark.parametrize("forward", [True, False])
def test_rope_paths_and_inverse(nrm_lib, path, forward):
    say(f"rope path={path} forward={forward}")
    _rope_case(nrm_lib, 300, 40, 128, 128, "bf16", False, 70000, "uniform", forward, 3, path)


def test_rope_in_place(nrm_lib):
    say("rope in place")
    rng = np.random.default_rng(4)
    x = dev(workloads.cast(rng.standard_normal((16, 64, 128)), "bf16"))
    ref = nrm_lib.rope(x, offset=5)
    y = x.clone()
    nrm_lib.rope(y, offset=5, out=y)
    torch.cuda.synchronize()
    compare.check_exact_bits(y, ref, "rope in place")


@pytest.mark.parametrize("fkind", ["uniform", "loguniform"])
@pytest.mark.parametrize("trad", [False, True])
def test_norm_rope_with_freqs(nrm_lib, fkind, trad):
    say(f"norm_rope freqs={fkind} trad={trad}")
    rp = workloads.rope_inputs(2, 4, 50, 128, "bf16", seed=6, offset=1024)
    freqs, _ = _freqs(fkind, 128, np.random.default_rng(7))
    cache = torch.zeros(2, 4, 2048, 128, dtype=torch.bfloat16)
    got = nrm_lib.norm_rope(dev(rp.x), dev(rp.w), eps=rp.eps, traditional=trad, offset=1024,
                            freqs=dev(freqs), cache=dev(cache))
    torch.cuda.synchronize()
    want = oracle.norm_rope(f64(rp.x), f64(rp.w), normalize=True, eps=rp.eps, dims=128,
                            traditional=trad, base=rp.base, scale=rp.scale, offset=1024,
                            forward=True, dtype="bf16", cache=f64(cache), freqs=f64(freqs))
    compare.check_output(got, want, "bf16", what="norm_rope cache with freqs")


def _qk_case(nrm, T, Hq, Hk, D, dims, dt, trad, pos_kind, fkind, seed, path=None, i32=False,
             in_place=False):
    inp = workloads.rope_qk_inputs(T, Hq, Hk, D, dt, seed=seed, positions=pos_kind,
                                   max_position=1 << 20)
    rng = np.random.default_rng(seed + 1)
    freqs, ms = _freqs(fkind, dims, rng)
    pos = inp.positions.to(torch.int32) if i32 else inp.positions
    q, k = dev(inp.q), dev(inp.k)
    with forced_path(path):
        if in_place:
            qo, ko = nrm.rope_positions(dev(pos), q, k, dims=dims, traditional=trad,
                                        base=10000.0, scale=1.0, freqs=dev(freqs), mscale=ms,
                                        q_out=q, k_out=k)
            assert qo is q and (k is None or ko is k)
        else:
            qo, ko = nrm.rope_positions(dev(pos), q, k, dims=dims, traditional=trad,
                                        base=10000.0, scale=1.0, freqs=dev(freqs), mscale=ms)
        torch.cuda.synchronize()
    kw = dict(dims=dims, traditional=trad, base=10000.0, scale=1.0, forward=True, dtype=dt,
              freqs=f64(freqs), mscale=ms)
    p = inp.positions.numpy()
    compare.check_output(qo, oracle.rope_positions(f64(inp.q), p, **kw), dt, what="q")
    if Hk:
        compare.check_output(ko, oracle.rope_positions(f64(inp.k), p, **kw), dt, what="k")


@pytest.mark.parametrize("Hq,Hk", [(8, 2), (32, 8), (1, 1), (3, 0), (40, 40)])
@pytest.mark.parametrize("D,dims", [(128, 128), (64, 64), (128, 64), (96, 96)])
@pytest.mark.parametrize("trad", [False, True])
def test_rope_positions_shapes(nrm_lib, Hq, Hk, D, dims, trad):
    say(f"rope_positions Hq={Hq} Hk={Hk} D={D} dims={dims} trad={trad}")
    _qk_case(nrm_lib, 37, Hq, Hk, D, dims, "bf16", trad, "random", "loguniform", Hq * 7 + Hk)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("path", [None, "scalar"])
@pytest.mark.parametrize("i32", [False, True])
def test_rope_positions_dtypes_paths(nrm_lib, dt, path, i32):
    say(f"rope_positions {dt} path={path} int32={i32}")
    _qk_case(nrm_lib, 200, 8, 2, 128, 128, dt, False, "random", "loguniform", 11, path, i32)


@pytest.mark.parametrize("fkind", [None, "uniform", "loguniform"])
def test_rope_positions_in_place(nrm_lib, fkind):
    say(f"rope_positions in place freqs={fkind}")
    _qk_case(nrm_lib, 300, 32, 8, 128, 128, "bf16", False, "arange", fkind, 12, in_place=True)


def test_rope_positions_batched_repeat(nrm_lib):
    """[B, L, H, D] query and key with one sequence's positions [L]: the binding repeats the
    positions per sequence; every sequence equals the single-sequence result."""
    say("rope_positions batched")
    rng = np.random.default_rng(13)
    q = dev(workloads.cast(rng.standard_normal((3, 20, 8, 64)), "bf16"))
    k = dev(workloads.cast(rng.standard_normal((3, 20, 2, 64)), "bf16"))
    pos = torch.arange(100, 120, device=DEV)
    qo, ko = nrm_lib.rope_positions(pos, q, k)
    for b in range(3):
        q1, k1 = nrm_lib.rope_positions(pos, q[b].contiguous(), k[b].contiguous())
        torch.cuda.synchronize()
        compare.check_exact_bits(qo[b], q1, f"sequence {b} q")
        compare.check_exact_bits(ko[b], k1, f"sequence {b} k")


def test_rope_positions_matches_offset_form(nrm_lib):
    """positions offset + t on [T, H, D] rows give the bits of Rope on the [H, T, D]
    transpose at that offset (both kernels compute the same angles and products)."""
    say("rope_positions vs rope")
    rng = np.random.default_rng(14)
    q = dev(workloads.cast(rng.standard_normal((64, 4, 128)), "bf16"))
    pos = torch.arange(64, device=DEV) + 777
    qo, _ = nrm_lib.rope_positions(pos, q)
    r = nrm_lib.rope(q.transpose(0, 1).contiguous(), offset=777)
    torch.cuda.synchronize()
    compare.check_exact_bits(qo, r.transpose(0, 1).contiguous(), "positions vs offset form")


@pytest.mark.parametrize("Hq,Hk", [(8, 2), (1, 1), (3, 0), (40, 40)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("trad", [False, True])
@pytest.mark.parametrize("fkind", [None, "loguniform"])
@pytest.mark.parametrize("D", [128, 64])
def test_rope_positions_many_tokens(nrm_lib, Hq, Hk, dt, trad, fkind, D):
    """4099 tokens (not a multiple of the positions a block takes) of 128 or 64 rotated
    features: the several-positions-per-block kernel (lane groups of 4, 8 or 16), with 1 to 80
    rows per position, bf16 and fp32, both pair layouts and both frequency forms; the oracle
    checks sampled tokens, the first and last ones among them."""
    T = 4099
    say(f"rope_positions T={T} D={D} Hq={Hq} Hk={Hk} {dt} trad={trad} freqs={fkind}")
    inp = workloads.rope_qk_inputs(T, Hq, Hk, D, dt, seed=Hq + 3 * Hk, positions="random",
                                   max_position=1 << 20)
    freqs, ms = _freqs(fkind, D, np.random.default_rng(Hq))
    qo, ko = nrm_lib.rope_positions(dev(inp.positions), dev(inp.q),
                                    dev(inp.k) if Hk else None, dims=D, traditional=trad,
                                    base=10000.0, freqs=dev(freqs), mscale=ms)
    torch.cuda.synchronize()
    sel = np.unique(np.r_[0:5, T - 5:T, np.random.default_rng(T).choice(T, 40, replace=False)])
    kw = dict(dims=D, traditional=trad, base=10000.0, scale=1.0, forward=True, dtype=dt,
              freqs=f64(freqs), mscale=ms)
    p = inp.positions.numpy()[sel]
    compare.check_output(qo[sel], oracle.rope_positions(f64(inp.q[sel]), p, **kw), dt, "q")
    if Hk:
        compare.check_output(ko[sel], oracle.rope_positions(f64(inp.k[sel]), p, **kw), dt, "k")


@pytest.mark.parametrize("i32", [False, True])
def test_rope_positions_many_tokens_inverse(nrm_lib, i32):
    """The inverse rotation, int64 or int32 positions and a position scale on the
    several-positions kernel, against the oracle on sampled tokens."""
    T, Hq, Hk, D = 4103, 8, 2, 128
    say(f"rope_positions inverse T={T} int32={i32}")
    inp = workloads.rope_qk_inputs(T, Hq, Hk, D, "bf16", seed=21, positions="random",
                                   max_position=1 << 20)
    pos = inp.positions.to(torch.int32) if i32 else inp.positions
    qo, ko = nrm_lib.rope_positions(dev(pos), dev(inp.q), dev(inp.k), base=10000.0, scale=0.5,
                                    forward=False)
    torch.cuda.synchronize()
    sel = np.unique(np.r_[0:3, T - 3:T, np.random.default_rng(22).choice(T, 30, replace=False)])
    kw = dict(dims=D, traditional=False, base=10000.0, scale=0.5, forward=False, dtype="bf16",
              freqs=None, mscale=1.0)
    p = inp.positions.numpy()[sel]
    compare.check_output(qo[sel], oracle.rope_positions(f64(inp.q[sel]), p, **kw), "bf16", "q")
    compare.check_output(ko[sel], oracle.rope_positions(f64(inp.k[sel]), p, **kw), "bf16", "k")


@pytest.mark.slow
def test_rope_positions_full_size(nrm_lib):
    """The benchmark's prefill shape ([16384, 32 + 8, 128] bf16, base 500000, divisors
    spanning the scaled range) in its launch; the oracle checks 48 sampled tokens."""
    say("rope_positions full size")
    inp = workloads.cfg_rope_qk_bf16()
    T, Hq, Hk, D = workloads.ROPE_QK_SHAPE
    freqs = workloads.rope_freqs_draw(D, "loguniform", seed=16)
    qo, ko = nrm_lib.rope_positions(dev(inp.positions), dev(inp.q), dev(inp.k),
                                    base=workloads.ROPE_QK_BASE, freqs=dev(freqs))
    torch.cuda.synchronize()
    sel = np.sort(np.random.default_rng(15).choice(T, 48, replace=False))
    kw = dict(dims=D, traditional=False, base=workloads.ROPE_QK_BASE, scale=1.0, forward=True,
              dtype="bf16", freqs=f64(freqs), mscale=1.0)
    p = inp.positions.numpy()[sel]
    compare.check_output(qo[sel], oracle.rope_positions(f64(inp.q[sel]), p, **kw), "bf16", "q")
    compare.check_output(ko[sel], oracle.rope_positions(f64(inp.k[sel]), p, **kw), "bf16", "k")

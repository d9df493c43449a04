"""GPU parity: the HIP library through its C ABI against the fp64 oracle, element by element,
on shapes that span several tiles and ragged tails, with every kernel shape forced in turn.

Bars: h and cache placement bit-exact; bf16 outputs within 1 ulp; fp32 outputs within
1e-5 relative + 1e-6 absolute.
"""

import numpy as np
import pytest
import torch

import compare
import workloads
import oracle
from gpu_util import (DEV, assert_h_exact, check_add, check_ln, check_rms, check_rope, dev, f64,
                      forced_path, run_rope, say)

pytestmark = pytest.mark.gpu

# widths: tiny, not a 16-byte multiple, one wave per row, one block per row, looping kernel;
# 20000, 28000 and 57352 are ragged widths of the six- and eight-chunk row_block kernels (fp32
# 5000 and 7000 chunks, bf16 7169 chunks: the last thread's chunks are clamped)
HIDDEN = [1, 2, 7, 8, 64, 100, 512, 520, 1000, 4096, 5120, 8192, 8200, 12288, 16384, 20000,
          24576, 28000, 32768, 40000, 49152, 57352, 65536, 70000]
WEIGHTS = [("bf16", "bf16"), ("bf16", "f32"), ("bf16", None), ("f32", "f32"), ("f32", None)]


def _row(rows, hidden, dt, wdt, seed, **kw):
    return workloads.row_inputs(rows, hidden, dt, seed=seed,
                                w=("normal", 1.0, 0.1) if wdt else None,
                                w_dtype=wdt if wdt else None, **kw)


@pytest.mark.parametrize("hidden", HIDDEN)
@pytest.mark.parametrize("dt,wdt", WEIGHTS)
def test_add_rms_norm_shapes(nrm_lib, hidden, dt, wdt):
    say(f"add_rms_norm rows=5 hidden={hidden} {dt} w={wdt}")
    inp = _row(5, hidden, dt, wdt, seed=hidden, r=("normal", 0.0, 1.0), eps=1e-6)
    check_add(nrm_lib, inp)


@pytest.mark.parametrize("hidden", HIDDEN)
@pytest.mark.parametrize("dt,wdt", WEIGHTS)
def test_rms_norm_shapes(nrm_lib, hidden, dt, wdt):
    say(f"rms_norm rows=5 hidden={hidden} {dt} w={wdt}")
    inp = _row(5, hidden, dt, wdt, seed=hidden + 1, x=("t3",), eps=1e-5)
    check_rms(nrm_lib, inp)


@pytest.mark.parametrize("hidden", HIDDEN)
@pytest.mark.parametrize("dt,wdt", WEIGHTS)
@pytest.mark.parametrize("affine", ["wb", "w", "b", "none"])
def test_layer_norm_shapes(nrm_lib, hidden, dt, wdt, affine):
    say(f"layer_norm rows=5 hidden={hidden} {dt} w={wdt} {affine}")
    inp = workloads.row_inputs(5, hidden, dt, seed=hidden + 2, x=("normal", 0.5, 2.0),
                               w=("normal", 1.0, 0.1), b=("normal", 0.0, 0.1),
                               w_dtype=wdt or dt, eps=1e-5)
    if "w" not in affine:
        inp.w = None
    if "b" not in affine:
        inp.b = None
    check_ln(nrm_lib, inp)


# Narrow rows take teams of 4 .. 64 lanes with several rows per block: 1001 rows leave the last
# block partly empty; chunk counts 1, 2, 3, 8, 15, 16, 32, 64, 125, 128 (bf16) and 2, 16, 25,
# 32, 64, 128 (fp32) cover every team size, exact and ragged.
NARROW = [("bf16", 8), ("bf16", 16), ("bf16", 24), ("bf16", 64), ("bf16", 120), ("bf16", 128),
          ("bf16", 256), ("bf16", 512), ("bf16", 1000), ("bf16", 1024), ("f32", 8), ("f32", 64),
          ("f32", 100), ("f32", 128), ("f32", 256), ("f32", 512)]


@pytest.mark.parametrize("dt,hidden", NARROW)
@pytest.mark.parametrize("wkind", ["same", "f32", None])
def test_narrow_rows_many(nrm_lib, dt, hidden, wkind):
    wdt = None if wkind is None else ("f32" if wkind == "f32" else dt)
    say(f"narrow rows=1001 hidden={hidden} {dt} w={wdt}")
    check_add(nrm_lib, _row(1001, hidden, dt, wdt, seed=hidden + 7, r=("normal", 0.0, 1.0),
                            eps=1e-6))
    check_rms(nrm_lib, _row(1001, hidden, dt, wdt, seed=hidden + 8, x=("t3",), eps=1e-5))
    inp = workloads.row_inputs(1001, hidden, dt, seed=hidden + 9, x=("normal", 0.5, 2.0),
                               w=("normal", 1.0, 0.1), b=("normal", 0.0, 0.1),
                               w_dtype=wdt or dt, eps=1e-5)
    if wkind is None:
        inp.w = inp.b = None
    check_ln(nrm_lib, inp)


@pytest.mark.parametrize("dt,wdt,hidden", [("bf16", "bf16", 8192), ("bf16", "bf16", 4000),
                                           ("bf16", "bf16", 6000), ("bf16", "f32", 2048),
                                           ("bf16", "f32", 1000), ("f32", "f32", 8192),
                                           ("f32", "f32", 1000), ("bf16", "f32", 20000),
                                           ("f32", "f32", 20000)])
@pytest.mark.parametrize("affine", ["wb", "w", "b"])
def test_layer_norm_row_pairs(nrm_lib, dt, wdt, hidden, affine):
    """LayerNorm with w and / or b over 4096 rows or more: two rows per block (2, 3 or 4 chunks
    per thread, exact and ragged widths). 4097 rows: the last block's second row is past the
    end. Compared on the first, middle and last rows. Width 20000 stays on one row per block
    (fp32 parameters beside bf16 data at 4 chunks per thread, fp32 at 6)."""
    say(f"layer_norm row pairs rows=4097 hidden={hidden} {dt} w={wdt} {affine}")
    inp = workloads.row_inputs(4097, hidden, dt, seed=hidden + 17, x=("normal", 0.5, 2.0),
                               w=("normal", 1.0, 0.1), b=("normal", 0.0, 0.1), w_dtype=wdt,
                               eps=1e-5)
    if "w" not in affine:
        inp.w = None
    if "b" not in affine:
        inp.b = None
    check_ln(nrm_lib, inp, rows_sel=np.r_[0:3, 2047:2050, 4093:4097])


@pytest.mark.parametrize("dt,wdt,hidden", [("f32", "f32", 8192), ("f32", "f32", 12000),
                                           ("f32", "f32", 16384), ("bf16", "f32", 4096),
                                           ("bf16", "f32", 5000), ("bf16", "f32", 24000)])
def test_rms_norm_row_pairs(nrm_lib, dt, wdt, hidden):
    """RMSNorm with fp32 weights over 4096 rows or more: two rows per block (2, 3 or 4 chunks
    per thread, exact and ragged). 4097 rows: the last block's second row is past the end."""
    say(f"rms_norm row pairs rows=4097 hidden={hidden} {dt} w={wdt}")
    inp = _row(4097, hidden, dt, wdt, seed=hidden + 19, x=("t3",), eps=1e-5)
    check_rms(nrm_lib, inp, rows_sel=np.r_[0:3, 2047:2050, 4093:4097])


# Widths that are not whole 16-byte chunks: one block per row of at most 256 threads with 1
# (33, 100), 2 (300, 521: 320 threads for RMSNorm and LayerNorm) or 4 (1001) elements per
# thread, and ceil(hidden / 256) from 1025 to 4096 (1100: 5, 1300: 6, 1537: 7, 2047: 8,
# 2500: 10, 3000: 12, 3500: 14, 4095: 16; add-RMSNorm up to 2048 in bf16); RMSNorm and
# LayerNorm rows of 4097 to 8192 with ceil(hidden / 512) per thread in blocks of 512 (4100
# and 4097: 9, 6500: 13, 8191: 16), rows up to 12288 with ceil(hidden / 768) in blocks of up
# to 768 (10001: 14, 12285 and 12287: 16); add-RMSNorm rows otherwise, and 12289, take the
# looping kernel.
ELEMS = [("bf16", 33), ("bf16", 100), ("bf16", 300), ("bf16", 521), ("bf16", 1001),
         ("bf16", 1100), ("bf16", 1300), ("bf16", 1537), ("bf16", 2047), ("bf16", 2500),
         ("bf16", 3000), ("bf16", 3500), ("bf16", 4095), ("bf16", 4100), ("bf16", 6500), ("bf16", 8191),
         ("bf16", 10001), ("bf16", 12287), ("bf16", 12289), ("f32", 1001), ("f32", 2047),
         ("f32", 3333), ("f32", 4097), ("f32", 12285)]


@pytest.mark.parametrize("dt,hidden", ELEMS)
@pytest.mark.parametrize("wkind", ["same", "f32", None])
def test_element_rows(nrm_lib, dt, hidden, wkind):
    if wkind == "f32" and dt == "f32":
        pytest.skip("same as 'same' for fp32 data")
    wdt = None if wkind is None else ("f32" if wkind == "f32" else dt)
    say(f"element rows=300 hidden={hidden} {dt} w={wdt}")
    check_add(nrm_lib, _row(300, hidden, dt, wdt, seed=hidden + 11, r=("normal", 0.0, 1.0),
                            eps=1e-6))
    check_rms(nrm_lib, _row(300, hidden, dt, wdt, seed=hidden + 12, x=("t3",), eps=1e-5))
    for affine in ("wb", "w", "b", "none"):
        inp = workloads.row_inputs(300, hidden, dt, seed=hidden + 13, x=("normal", 0.5, 2.0),
                                   w=("normal", 1.0, 0.1), b=("normal", 0.0, 0.1),
                                   w_dtype=wdt or dt, eps=1e-5)
        if wkind is None or "w" not in affine:
            inp.w = None
        if wkind is None or "b" not in affine:
            inp.b = None
        check_ln(nrm_lib, inp)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_misaligned_bases(nrm_lib, dt):
    """x, r, h and out one element past a 16-byte boundary (views into larger buffers) with a
    width of whole chunks: the single-element kernel, for all three forward operations."""
    say(f"forward misaligned bases {dt}")
    rows, n = 300, 4096

    def shifted(t=None, like=None):
        src = t if t is not None else like
        buf = torch.zeros(rows * n + 8, dtype=src.dtype, device=DEV)
        v = buf[1:1 + rows * n].view(rows, n)
        if t is not None:
            v.copy_(dev(t))
        return v

    inp = _row(rows, n, dt, dt, seed=51, r=("normal", 0.0, 1.0), eps=1e-6)
    x, r = shifted(inp.x), shifted(inp.r)
    out, h = shifted(like=x), shifted(like=x)
    got, gh = nrm_lib.add_rms_norm(x, r, dev(inp.w), inp.eps, out=out, h=h)
    got2 = nrm_lib.rms_norm(x, dev(inp.w), inp.eps, out=shifted(like=x))
    lin = workloads.row_inputs(rows, n, dt, seed=52, x=("normal", 0.5, 2.0),
                               w=("normal", 1.0, 0.1), b=("normal", 0.0, 0.1), eps=1e-5)
    got3 = nrm_lib.layer_norm(shifted(lin.x), dev(lin.w), dev(lin.b), lin.eps,
                              out=shifted(like=x))
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr() and gh.data_ptr() == h.data_ptr()
    want_out, want_h = oracle.add_rms_norm(f64(inp.x), f64(inp.r), f64(inp.w), inp.eps, dt)
    assert_h_exact(gh, want_h)
    compare.check_output(got, want_out, dt, what="add_rms_norm out")
    compare.check_output(got2, oracle.rms_norm(f64(inp.x), f64(inp.w), inp.eps, dt), dt,
                         what="rms_norm out")
    compare.check_output(got3, oracle.layer_norm(f64(lin.x), f64(lin.w), f64(lin.b), lin.eps,
                                                 dt), dt, what="layer_norm out")


@pytest.mark.parametrize("path", ["wave", "block", "rowblock", "chunked", "scalar"])
@pytest.mark.parametrize("hidden", [512, 4096, 5120, 8192, 16384, 24576])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_forced_kernel_shapes(nrm_lib, path, hidden, dt):
    """Every kernel shape gives oracle-parity results on the same inputs."""
    say(f"forced path={path} hidden={hidden} {dt}")
    with forced_path(path):
        check_add(nrm_lib, _row(37, hidden, dt, dt, seed=7, r=("t3",), eps=1e-6))
        check_rms(nrm_lib, _row(37, hidden, dt, dt, seed=8, eps=1e-6))
        check_ln(nrm_lib, workloads.row_inputs(37, hidden, dt, seed=9, x=("normal", 0.5, 2.0),
                                               b=("normal", 0.0, 0.1), eps=1e-5))


@pytest.mark.parametrize("rows", [1, 3, 4, 5, 63, 257])
def test_ragged_row_counts(nrm_lib, rows):
    say(f"ragged rows={rows}")
    check_add(nrm_lib, _row(rows, 4096, "bf16", "bf16", seed=rows, r=("normal", 0, 1)))


# ------------------------------------------------------------------------------ NormRope

ROPE_SHAPES = [
    # (B, H, L, D, dims)
    (2, 3, 5, 128, 128),
    (1, 2, 7, 64, 64),
    (2, 2, 4, 128, 64),
    (1, 1, 3, 128, 32),
    (1, 2, 3, 256, 256),
    (1, 1, 2, 1024, 1024),
    (1, 1, 2, 2048, 2048),
    (2, 1, 3, 96, 96),
    (1, 2, 4, 80, 80),
    (1, 1, 3, 72, 72),
    (1, 1, 3, 8, 4),
    (1, 1, 2, 6, 6),
    (1, 1, 2, 7, 6),
    (1, 2, 3, 128, 0),
    (3, 5, 33, 128, 128),
    (2, 16, 33, 64, 64),     # 4-lane groups (bf16), 32 rows per position
    (1, 4, 9, 64, 32),       # 4-lane groups with pass-through chunks
    (8, 32, 3, 128, 128),    # four rows per lane group, two positions per block, odd L
    (4, 33, 5, 128, 96),     # the same with a partial last step and pass-through chunks
]


@pytest.mark.parametrize("shape", ROPE_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("traditional", [False, True])
def test_norm_rope_shapes(nrm_lib, shape, dt, traditional):
    B, H, L, D, dims = shape
    say(f"norm_rope {shape} {dt} traditional={traditional}")
    rp = workloads.rope_inputs(B, H, L, D, dt, seed=D + L, dims=dims, offset=1021)
    check_rope(nrm_lib, rp, traditional=traditional)


@pytest.mark.parametrize("traditional", [False, True])
@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("forward", [True, False])
@pytest.mark.parametrize("path", [None, "scalar"])
def test_norm_rope_modes(nrm_lib, traditional, normalize, forward, path):
    say(f"norm_rope modes trad={traditional} norm={normalize} fwd={forward} path={path}")
    with forced_path(path):
        for dt, wdt in (("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")):
            rp = workloads.rope_inputs(2, 4, 9, 128, dt, seed=11, w_dtype=wdt, offset=1530,
                                       base=500000.0, scale=0.25)
            check_rope(nrm_lib, rp, normalize=normalize, traditional=traditional, forward=forward)


@pytest.mark.parametrize("offset", [0, 1, 4096, 100000, 3000000])
@pytest.mark.parametrize("scale", [1.0, 0.125, 37.5])
def test_norm_rope_positions(nrm_lib, offset, scale):
    """Angles from 0 to ~1e8 rad: the in-kernel sin/cos range reduction across many
    quadrants, in both kernels."""
    say(f"norm_rope offset={offset} scale={scale}")
    rp = workloads.rope_inputs(1, 2, 16, 128, "bf16", seed=offset % 1000, offset=offset,
                               scale=scale)
    for path in (None, "scalar"):
        with forced_path(path):
            check_rope(nrm_lib, rp)
            check_rope(nrm_lib, rp, traditional=True)


@pytest.mark.parametrize("shape", [(1, 4, 4099, 128), (2, 3, 4100, 64), (1, 16, 4097, 64),
                                   (1, 4, 16411, 128), (1, 2, 8195, 256)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("traditional", [False, True])
@pytest.mark.parametrize("wkind", ["bf16", "f32", None])
@pytest.mark.parametrize("cache", [False, True])
def test_norm_rope_many_positions(nrm_lib, shape, traditional, wkind, cache):
    """Few heads at thousands of positions with every feature rotated: several positions
    per block (lane groups of 4, 8 or 16; 4 to 16 positions per block, the last block
    partial), normalised, with bf16, fp32 or no weight, into an output or rows
    offset .. offset + L of a cache."""
    B, H, L, D = shape
    say(f"norm_rope many positions {shape} trad={traditional} w={wkind} cache={cache}")
    rp = workloads.rope_inputs(B, H, L, D, "bf16", seed=L + D, w_dtype=wkind,
                               w=None if wkind is None else ("uniform", 0.5, 1.5),
                               offset=37 if cache else 0)
    c = torch.zeros(B, H, L + 50, D, dtype=torch.bfloat16) if cache else None
    check_rope(nrm_lib, rp, traditional=traditional, cache=c)


@pytest.mark.parametrize("traditional", [False, True])
@pytest.mark.parametrize("path", [None, "scalar"])
def test_norm_rope_cache(nrm_lib, traditional, path):
    """Cache mode: rows offset .. offset + L - 1 written, every other element keeps its bits."""
    say(f"norm_rope cache trad={traditional} path={path}")
    with forced_path(path):
        rp = workloads.rope_inputs(2, 3, 6, 128, "bf16", seed=5, offset=9)
        cache = workloads.cast(np.random.default_rng(3).standard_normal((2, 3, 20, 128)), "bf16")
        check_rope(nrm_lib, rp, traditional=traditional, cache=cache)


# ------------------------------------------------------------------------------ edge cases

def test_in_place(nrm_lib):
    """out == x for RMSNorm and LayerNorm; h == r and out == x for add-RMSNorm; out == x for
    NormRope."""
    say("in-place")
    inp = _row(9, 4096, "bf16", "bf16", seed=1, r=("normal", 0, 1), eps=1e-6)
    import oracle

    x, r, w = dev(inp.x), dev(inp.r), dev(inp.w)
    want_out, want_h = oracle.add_rms_norm(f64(inp.x), f64(inp.r), f64(inp.w), inp.eps, "bf16")
    out, h = nrm_lib.add_rms_norm(x, r, w, inp.eps, out=x, h=r)
    torch.cuda.synchronize()
    assert out.data_ptr() == x.data_ptr() and h.data_ptr() == r.data_ptr()
    compare.check_bf16(x, want_out)
    compare.check_exact_bits(r, compare.bits_of_values(want_h, "bf16").view(np.int16))

    x = dev(inp.x)
    nrm_lib.rms_norm(x, w, inp.eps, out=x)
    torch.cuda.synchronize()
    compare.check_bf16(x, oracle.rms_norm(f64(inp.x), f64(inp.w), inp.eps, "bf16"))

    x = dev(inp.x)
    nrm_lib.layer_norm(x, w, None, 1e-5, out=x)
    torch.cuda.synchronize()
    compare.check_bf16(x, oracle.layer_norm(f64(inp.x), f64(inp.w), None, 1e-5, "bf16"))

    rp = workloads.rope_inputs(2, 2, 5, 128, "bf16", seed=4, offset=77)
    for path in (None, "scalar"):
        with forced_path(path):
            xr = dev(rp.x)
            nrm_lib.norm_rope(xr, dev(rp.w), eps=rp.eps, offset=rp.offset, out=xr)
            torch.cuda.synchronize()
            want = oracle.norm_rope(f64(rp.x), f64(rp.w), normalize=True, eps=rp.eps, dims=128,
                                    traditional=False, base=1e4, scale=1.0, offset=77,
                                    forward=True, dtype="bf16")
            compare.check_bf16(xr, want)


def _guarded(like, pad=4096):
    """A contiguous view into a larger buffer whose margins hold a canary pattern."""
    n = like.numel()
    buf = torch.empty(n + 2 * pad, dtype=like.dtype, device=DEV)
    buf.view(torch.int16 if like.element_size() == 2 else torch.int32).fill_(0x5A5A)
    return buf, buf[pad:pad + n].view(like.shape), pad


def _canary_ok(buf, pad, n):
    b = buf.view(torch.int16 if buf.element_size() == 2 else torch.int32).cpu().numpy()
    return np.all(b[:pad] == 0x5A5A) and np.all(b[pad + n:] == 0x5A5A)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("hidden", [100, 4096, 5120, 40000])
def test_guard_bands(nrm_lib, dt, hidden):
    """No kernel writes outside its output."""
    say(f"guard bands {dt} hidden={hidden}")
    inp = _row(7, hidden, dt, dt, seed=2, r=("normal", 0, 1), b=("normal", 0, 0.1))
    x, r, w, b = dev(inp.x), dev(inp.r), dev(inp.w), dev(inp.b)
    bo, out, pad = _guarded(x)
    bh, h, _ = _guarded(x)
    nrm_lib.add_rms_norm(x, r, w, 1e-6, out=out, h=h)
    nrm_lib.rms_norm(x, w, 1e-6, out=out)
    nrm_lib.layer_norm(x, w, b, 1e-5, out=out)
    torch.cuda.synchronize()
    assert _canary_ok(bo, pad, x.numel()) and _canary_ok(bh, pad, x.numel())


@pytest.mark.parametrize("shape", [(2, 3, 5, 128, 128), (1, 1, 3, 72, 72)])
def test_norm_rope_guard_bands(nrm_lib, shape):
    B, H, L, D, dims = shape
    say(f"norm_rope guard bands {shape}")
    rp = workloads.rope_inputs(B, H, L, D, "bf16", seed=1, dims=dims)
    x = dev(rp.x)
    for trad in (False, True):
        bo, out, pad = _guarded(x)
        nrm_lib.norm_rope(x, dev(rp.w), dims=dims, traditional=trad, out=out)
        torch.cuda.synchronize()
        assert _canary_ok(bo, pad, x.numel())


def test_deterministic(nrm_lib):
    """Two runs give the same bits (fixed reduction order)."""
    say("determinism")
    inp = _row(64, 8192, "bf16", "bf16", seed=3, r=("t3",), eps=1e-6)
    x, r, w = dev(inp.x), dev(inp.r), dev(inp.w)
    o1, h1 = nrm_lib.add_rms_norm(x, r, w, inp.eps)
    o2, h2 = nrm_lib.add_rms_norm(x, r, w, inp.eps)
    l1 = nrm_lib.layer_norm(x, w, w, 1e-5)
    l2 = nrm_lib.layer_norm(x, w, w, 1e-5)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(l1.view(torch.int16), l2.view(torch.int16))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("path", [None, "wave", "block", "scalar"])
def test_scale_invariance_bit_exact(nrm_lib, dt, path):
    """eps = 0 and alpha = 2^k: RMSNorm(alpha x) has the same bits as RMSNorm(x) (every step,
    including the row scalar, scales exactly)."""
    say(f"scale invariance {dt} path={path}")
    inp = _row(16, 4096, dt, dt, seed=4)
    x, w = dev(inp.x), dev(inp.w)
    with forced_path(path):
        base = nrm_lib.rms_norm(x, w, 0.0)
        for k in (-9, -1, 3, 12):
            got = nrm_lib.rms_norm(x * 2.0 ** k, w, 0.0)
            torch.cuda.synchronize()
            compare.check_exact_bits(got, base, what=f"2^{k}")


def test_rope_identity_and_inverse(nrm_lib):
    """Position 0 gives RMSNorm of the row; the inverse rotation undoes the forward one."""
    say("rope identity / inverse")
    rp = workloads.rope_inputs(2, 2, 4, 128, "bf16", seed=6, offset=0)
    y = run_rope(nrm_lib, rp)
    r0 = nrm_lib.rms_norm(dev(rp.x)[:, :, 0].contiguous(), dev(rp.w), rp.eps)
    torch.cuda.synchronize()
    compare.check_bf16(y[:, :, 0], f64(r0), what="position 0 vs rms_norm")
    rp2 = workloads.rope_inputs(2, 2, 4, 128, "f32", seed=6, offset=1000)
    y = run_rope(nrm_lib, rp2)
    back = nrm_lib.norm_rope(y, eps=None, offset=1000, forward=False)
    plain = nrm_lib.norm_rope(dev(rp2.x), dev(rp2.w), eps=rp2.eps, scale=0.0)
    torch.cuda.synchronize()
    compare.check_f32(f64(back), f64(plain), rtol=1e-5, atol=1e-6, what="inverse")


def test_special_values(nrm_lib):
    """NaN / inf stay in their row; an all-zero row gives 0 (eps > 0) or NaN (eps = 0)."""
    say("special values")
    import oracle

    x = torch.randn(6, 4096, dtype=torch.float32).to(torch.bfloat16)
    x[1, 17] = float("nan")
    x[2, 5] = float("inf")
    x[3] = 0
    x[4, 4095] = -float("inf")
    w = torch.ones(4096, dtype=torch.bfloat16)
    for eps in (1e-6, 0.0):
        got = nrm_lib.rms_norm(dev(x), dev(w), eps)
        torch.cuda.synchronize()
        want = oracle.rms_norm(f64(x), f64(w), eps, "bf16")
        compare.check_bf16(got, want, what=f"rms eps={eps}")
        got = nrm_lib.layer_norm(dev(x), dev(w), None, eps)
        torch.cuda.synchronize()
        with np.errstate(invalid="ignore"):
            want = oracle.layer_norm(f64(x), f64(w), None, eps, "bf16")
        compare.check_bf16(got, want, what=f"ln eps={eps}")


def test_error_writes_nothing(nrm_lib):
    """A rejected call (partial overlap) raises and leaves the output untouched."""
    say("error path writes nothing")
    buf = torch.zeros(2 * 4096 + 8, dtype=torch.bfloat16, device=DEV)
    x = torch.randn(2, 4096, device=DEV).to(torch.bfloat16)
    out = buf[8:8 + 2 * 4096].view(2, 4096)
    h = buf[:2 * 4096].view(2, 4096)
    with pytest.raises(nrm_lib.NrmError, match="NRM_ERR_ALIAS"):
        nrm_lib.add_rms_norm(x, x, None, 1e-5, out=out, h=h)
    torch.cuda.synchronize()
    assert torch.count_nonzero(buf.view(torch.int16)) == 0


def test_zero_rows(nrm_lib):
    say("zero rows")
    x = torch.empty(0, 4096, dtype=torch.bfloat16, device=DEV)
    assert nrm_lib.rms_norm(x).shape == (0, 4096)
    o, h = nrm_lib.add_rms_norm(x, x)
    assert o.numel() == 0 and h.numel() == 0
    assert nrm_lib.norm_rope(torch.empty(2, 0, 5, 128, dtype=torch.bfloat16, device=DEV)).numel() == 0


@pytest.mark.parametrize("path", [None, "wave", "block", "chunked"])
def test_in_place_many_rows(nrm_lib, path):
    """In place over many rows, so persistent blocks prefetch the next row while writing the
    current one: h == r and out == x for add-RMSNorm, out == x for LayerNorm."""
    say(f"in-place many rows path={path}")
    import oracle

    inp = _row(3000, 4096, "bf16", "bf16", seed=12, r=("t3",), b=("normal", 0, 0.1), eps=1e-6)
    want_out, want_h = oracle.add_rms_norm(f64(inp.x), f64(inp.r), f64(inp.w), inp.eps, "bf16")
    want_ln = oracle.layer_norm(f64(inp.x), f64(inp.w), f64(inp.b), 1e-5, "bf16")
    with forced_path(path):
        x, r, w, b = dev(inp.x), dev(inp.r), dev(inp.w), dev(inp.b)
        nrm_lib.add_rms_norm(x, r, w, inp.eps, out=x, h=r)
        torch.cuda.synchronize()
        compare.check_bf16(x, want_out, what="out in x")
        compare.check_exact_bits(r, compare.bits_of_values(want_h, "bf16").view(np.int16),
                                 what="h in r")
        x = dev(inp.x)
        nrm_lib.layer_norm(x, w, b, 1e-5, out=x)
        torch.cuda.synchronize()
        compare.check_bf16(x, want_ln, what="layer_norm in x")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_in_place_element_rows(nrm_lib, dt):
    """out == x for RMSNorm and LayerNorm on rows of single elements (width 4100)."""
    say(f"in-place element rows {dt}")
    import oracle

    inp = _row(300, 4100, dt, dt, seed=13, x=("t3",), b=("normal", 0, 0.1), eps=1e-6)
    x, w, b = dev(inp.x), dev(inp.w), dev(inp.b)
    nrm_lib.rms_norm(x, w, inp.eps, out=x)
    torch.cuda.synchronize()
    compare.check_output(x, oracle.rms_norm(f64(inp.x), f64(inp.w), inp.eps, dt), dt,
                         what="rms_norm in x")
    x = dev(inp.x)
    nrm_lib.layer_norm(x, w, b, 1e-5, out=x)
    torch.cuda.synchronize()
    compare.check_output(x, oracle.layer_norm(f64(inp.x), f64(inp.w), f64(inp.b), 1e-5, dt), dt,
                         what="layer_norm in x")


def test_hip_graph_replays(nrm_lib):
    """The library's launches capture into a HIP graph (torch.cuda.CUDAGraph) and every
    replay matches the eager call on the inputs present at that replay; the inputs change
    eagerly, with synchronisations, between replays."""
    say("hip graph capture and replays")
    import oracle

    inp = _row(96, 4096, "bf16", "bf16", seed=21, r=("normal", 0, 1), b=("normal", 0, 0.1))
    rp = workloads.rope_inputs(2, 4, 8, 128, "bf16", seed=22, offset=300)
    x, r, w, b = dev(inp.x), dev(inp.r), dev(inp.w), dev(inp.b)
    xr, wr = dev(rp.x), dev(rp.w)
    out, h, ln_out = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    rope_out = torch.empty_like(xr)

    def calls():
        nrm_lib.add_rms_norm(x, r, w, 1e-6, out=out, h=h)
        nrm_lib.layer_norm(x, w, b, 1e-5, out=ln_out)
        nrm_lib.norm_rope(xr, wr, eps=rp.eps, offset=rp.offset, out=rope_out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    gen = torch.Generator().manual_seed(5)
    for rep in range(4):
        xs = torch.randn(x.shape, generator=gen).to(torch.bfloat16)
        rs = torch.randn(r.shape, generator=gen).to(torch.bfloat16)
        xrs = torch.randn(xr.shape, generator=gen).to(torch.bfloat16)
        x.copy_(xs)
        r.copy_(rs)
        xr.copy_(xrs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want_out, want_h = oracle.add_rms_norm(f64(xs), f64(rs), f64(inp.w), 1e-6, "bf16")
        compare.check_bf16(out, want_out, what=f"replay {rep} out")
        compare.check_exact_bits(h, compare.bits_of_values(want_h, "bf16").view(np.int16),
                                 what=f"replay {rep} h")
        compare.check_bf16(ln_out, oracle.layer_norm(f64(xs), f64(inp.w), f64(inp.b), 1e-5,
                                                     "bf16"), what=f"replay {rep} layer_norm")
        want_rope = oracle.norm_rope(f64(xrs), f64(rp.w), normalize=True, eps=rp.eps, dims=128,
                                     traditional=False, base=1e4, scale=1.0, offset=300,
                                     forward=True, dtype="bf16")
        compare.check_bf16(rope_out, want_rope, what=f"replay {rep} norm_rope")
        # eager work between replays
        e_out, _ = nrm_lib.add_rms_norm(x, r, w, 1e-6)
        torch.cuda.synchronize()
        compare.check_exact_bits(e_out, out, what=f"eager after replay {rep}")

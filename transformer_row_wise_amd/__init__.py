"""Fused row-wise normalisation on AMD Instinct MI355X: the Python binding of libnrm.so.

Every function here only marshals arguments (checks devices, dtypes, shapes and
contiguity, allocates outputs with torch, passes raw device pointers and torch's current
HIP stream) and calls the C ABI declared in ``include/nrm.h``; every step of the
computation runs in the library's HIP kernels. There is no fallback: if the library is not
built, ``load()`` raises.

    rms_norm(x, w=None, eps=1e-5)                -> out
    add_rms_norm(x, r, w=None, eps=1e-5)         -> (out, h)   h = x + r
    layer_norm(x, w=None, b=None, eps=1e-5)      -> out
    norm_rope(x, w=None, eps=1e-6, dims=None, traditional=False, base=10000.0, scale=1.0,
              offset=0, forward=True, cache=None, freqs=None)
                                                 -> out (or the cache, written in place)
    rope(x, dims=None, traditional=False, base=10000.0, scale=1.0, offset=0, forward=True,
         freqs=None, mscale=1.0)                 -> out
    rope_positions(positions, q, k=None, ...)    -> (q_out, k_out)
    rope_freqs_llama3 / rope_freqs_yarn / rope_freqs_su(...) -> (freqs, mscale) on the host
    softmax(x) / causal_softmax(x, rows)         -> out
    logsumexp(x)                                 -> [..., 1]
    cross_entropy(logits, targets)               -> fp32 loss per row
    cross_entropy_vjp(logits, targets, g)        -> dlogits
    rms_norm_vjp(x, w, g, eps=1e-5)              -> (dx, dw)
    layer_norm_vjp(x, w, g, eps=1e-5)            -> (dx, dw, db)
"""

import ctypes
import os

import torch

__all__ = [
    "NrmError", "load", "lib", "rms_norm", "add_rms_norm", "layer_norm", "norm_rope",
    "rms_norm_vjp", "layer_norm_vjp", "vjp_workspace_bytes", "rope", "rope_positions",
    "rope_freqs_llama3", "rope_freqs_yarn", "rope_freqs_su", "softmax", "causal_softmax",
    "logsumexp", "cross_entropy", "cross_entropy_vjp", "bench_copy", "bench_copy2",
    "bench_copy2_row", "layer_norm_vjp_noalloc", "NRM_F32",
    "NRM_BF16", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnrm.so")
NRM_F32, NRM_BF16 = 0, 1
_DTYPES = {torch.float32: NRM_F32, torch.bfloat16: NRM_BF16}
_lib = None

_i64, _f32, _int, _vp = ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_void_p
_sz = ctypes.c_size_t
_SIGNATURES = {
    "nrm_rms_norm": [_vp, _vp, _vp, _i64, _i64, _f32, _int, _int, _vp],
    "nrm_add_rms_norm": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _int, _int, _vp],
    "nrm_layer_norm": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _int, _int, _vp],
    "nrm_norm_rope": [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _f32, _i64, _int, _f32, _f32,
                      _i64, _int, _vp, _int, _i64, _int, _int, _vp],
    "nrm_rope": [_vp, _vp, _i64, _i64, _i64, _i64, _int, _f32, _f32, _i64, _int, _vp, _f32, _int,
                 _vp],
    "nrm_rope_positions": [_vp, _vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, _i64, _i64, _int,
                           _f32, _f32, _int, _vp, _f32, _int, _vp],
    "nrm_rope_freqs_llama3": [_i64, _f32, _f32, _f32, _f32, _i64, _vp, _vp],
    "nrm_rope_freqs_yarn": [_i64, _f32, _f32, _i64, _f32, _f32, _f32, _f32, _vp, _vp],
    "nrm_rope_freqs_su": [_i64, _f32, _vp, _i64, _i64, _vp, _vp],
    "nrm_norm_vjp_workspace_bytes": [_i64, _i64, _int],
    "nrm_rms_norm_vjp": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _int, _int, _vp, _sz, _vp],
    "nrm_layer_norm_vjp": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _int, _int, _vp, _sz,
                           _vp],
    "nrm_layer_norm_vjp_noalloc": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _int, _int,
                                   _vp],
    "nrm_softmax": [_vp, _vp, _i64, _i64, _int, _vp],
    "nrm_causal_softmax": [_vp, _vp, _i64, _i64, _i64, _i64, _int, _vp],
    "nrm_logsumexp": [_vp, _vp, _i64, _i64, _int, _vp],
    "nrm_cross_entropy": [_vp, _vp, _int, _vp, _i64, _i64, _int, _vp],
    "nrm_cross_entropy_vjp": [_vp, _vp, _int, _vp, _vp, _vp, _i64, _i64, _int, _vp],
    "nrm_bench_copy": [_vp, _vp, _i64, _vp],
    "nrm_bench_copy2": [_vp, _vp, _vp, _vp, _i64, _vp],
    "nrm_bench_copy2_row": [_vp, _vp, _vp, _vp, _i64, _i64, _vp],
    "nrm_last_error": [],
    "nrm_status_name": [_int],
    "nrm_version": [],
}
_RESTYPES = {"nrm_last_error": ctypes.c_char_p, "nrm_status_name": ctypes.c_char_p,
             "nrm_norm_vjp_workspace_bytes": ctypes.c_size_t}


class NrmError(RuntimeError):
    """A failed nrm_* call: ``status`` is the nrm_status code, ``name`` its name."""

    def __init__(self, status, name, message):
        super().__init__(f"{name}: {message}")
        self.status = status
        self.name = name


def load(path=None):
    """Load libnrm.so (once) and declare its C signatures. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is not built; run `python -m transformer_row_wise_amd.build`")
    lib = ctypes.CDLL(p)
    for name, args in _SIGNATURES.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = _RESTYPES.get(name, ctypes.c_int)
    _lib = lib
    return lib


def lib():
    return load()


def _raise(status):
    L = load()
    raise NrmError(status, L.nrm_status_name(status).decode(), L.nrm_last_error().decode())


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream():
    """The current device's current stream, as a raw handle (torch's direct accessor where it
    exists: a fraction of a microsecond against ~3 for torch.cuda.current_stream())."""
    if _raw_stream is not None and _cur_device is not None:
        return _raw_stream(_cur_device())
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t, what):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"{what} must be float32 or bfloat16, got {t.dtype}") from None


def _check_act(t, what, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{what} must be on a HIP device, got {t.device}")
    if device is not None and t.get_device() != device.index:
        raise ValueError(f"{what} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _check_param(p, what, n, x):
    if p is None:
        return None, _DTYPES[x.dtype]
    _check_act(p, what, x.device)
    if p.dim() != 1 or p.shape[0] != n:
        raise ValueError(f"{what} must have shape [{n}], got {list(p.shape)}")
    if p.dtype not in (x.dtype, torch.float32):
        raise TypeError(f"{what} must be {x.dtype} or float32, got {p.dtype}")
    return p, _DTYPES[p.dtype]


def _out_like(out, x, what):
    if out is None:
        return torch.empty_like(x)
    _check_act(out, what, x.device)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError(f"{what} must be {x.dtype} of shape {list(x.shape)}, "
                         f"got {out.dtype} {list(out.shape)}")
    return out


def _rows(x):
    hidden = x.shape[-1] if x.dim() else 1
    rows = x.numel() // hidden if hidden else 0
    return rows, hidden


def rms_norm(x, w=None, eps=1e-5, out=None):
    """x / sqrt(mean(x^2) + eps) * w over the last axis (nrm_rms_norm)."""
    _check_act(x, "x")
    dt = _dtype_code(x, "x")
    rows, hidden = _rows(x)
    w, wdt = _check_param(w, "w", hidden, x)
    out = _out_like(out, x, "out")
    st = load().nrm_rms_norm(_ptr(x), _ptr(w), _ptr(out), rows, hidden, eps, dt, wdt, _stream())
    if st:
        _raise(st)
    return out


def add_rms_norm(x, r, w=None, eps=1e-5, out=None, h=None):
    """(RMSNorm(x + r), x + r) in one pass (nrm_add_rms_norm). ``h`` may be ``x`` or ``r``
    for an in-place residual update."""
    _check_act(x, "x")
    _check_act(r, "r", x.device)
    dt = _dtype_code(x, "x")
    if r.shape != x.shape or r.dtype != x.dtype:
        raise ValueError(f"r must be {x.dtype} of shape {list(x.shape)}, got {r.dtype} "
                         f"{list(r.shape)}")
    rows, hidden = _rows(x)
    w, wdt = _check_param(w, "w", hidden, x)
    out = _out_like(out, x, "out")
    h = _out_like(h, x, "h")
    st = load().nrm_add_rms_norm(_ptr(x), _ptr(r), _ptr(w), _ptr(out), _ptr(h), rows, hidden,
                                 eps, dt, wdt, _stream())
    if st:
        _raise(st)
    return out, h


def layer_norm(x, w=None, b=None, eps=1e-5, out=None):
    """(x - mean) / sqrt(var + eps) * w + b over the last axis (nrm_layer_norm)."""
    _check_act(x, "x")
    dt = _dtype_code(x, "x")
    rows, hidden = _rows(x)
    w, wdt = _check_param(w, "w", hidden, x)
    b, bdt = _check_param(b, "b", hidden, x)
    if w is not None and b is not None and wdt != bdt:
        raise TypeError(f"w and b must share a dtype, got {w.dtype} and {b.dtype}")
    pdt = wdt if w is not None else bdt
    out = _out_like(out, x, "out")
    st = load().nrm_layer_norm(_ptr(x), _ptr(w), _ptr(b), _ptr(out), rows, hidden, eps, dt,
                               pdt, _stream())
    if st:
        _raise(st)
    return out


def _freqs_arg(freqs, dims, x):
    """Device float32 [dims / 2] divisors, or None."""
    if freqs is None:
        return None
    _check_act(freqs, "freqs", x.device)
    if freqs.dtype != torch.float32 or freqs.dim() != 1 or freqs.shape[0] != dims // 2:
        raise ValueError(f"freqs must be float32 of shape [{dims // 2}], got {freqs.dtype} "
                         f"{list(freqs.shape)}")
    return freqs


def norm_rope(x, w=None, eps=1e-6, dims=None, traditional=False, base=10000.0, scale=1.0,
              offset=0, forward=True, cache=None, out=None, freqs=None):
    """NormRope over x [B, H, L, D] (nrm_norm_rope). ``eps=None`` skips the normalisation.
    With ``cache`` ([B, H, cache_len, D]) rows offset .. offset + L - 1 of the cache are
    written and the cache is returned; otherwise a new (or the given) [B, H, L, D] array."""
    _check_act(x, "x")
    dt = _dtype_code(x, "x")
    if x.dim() != 4:
        raise ValueError(f"x must be [B, H, L, D], got {list(x.shape)}")
    B, H, L, D = x.shape
    dims = D if dims is None else int(dims)
    normalize = eps is not None
    w, wdt = _check_param(w, "w", D, x)
    freqs = _freqs_arg(freqs, dims, x)
    if cache is not None:
        _check_act(cache, "cache", x.device)
        if cache.dim() != 4 or list(cache.shape[:2]) != [B, H] or cache.shape[3] != D \
                or cache.dtype != x.dtype:
            raise ValueError(f"cache must be {x.dtype} [{B}, {H}, cache_len, {D}], got "
                             f"{cache.dtype} {list(cache.shape)}")
        dst, cache_len = cache, cache.shape[2]
    else:
        dst, cache_len = _out_like(out, x, "out"), 0
    st = load().nrm_norm_rope(_ptr(x), _ptr(w), _ptr(dst), B, H, L, D, int(normalize),
                              0.0 if eps is None else eps, dims, int(bool(traditional)), base,
                              scale, int(offset), int(bool(forward)), _ptr(freqs),
                              int(cache is not None), cache_len, dt, wdt, _stream())
    if st:
        _raise(st)
    return dst


def vjp_workspace_bytes(rows, hidden, layer_norm):
    """Workspace bytes for a backward call that computes a parameter gradient."""
    return load().nrm_norm_vjp_workspace_bytes(rows, hidden, int(bool(layer_norm)))


def _param_grad(want, given, n, x, pdtype, what):
    if given is not None:
        _check_act(given, what, x.device)
        if given.dim() != 1 or given.shape[0] != n or given.dtype != pdtype:
            raise ValueError(f"{what} must be {pdtype} of shape [{n}], got {given.dtype} "
                             f"{list(given.shape)}")
        return given
    return torch.empty(n, dtype=pdtype, device=x.device) if want else None


def _workspace(workspace, need, x):
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check_act(workspace, "workspace", x.device)
    return workspace, workspace.numel() * workspace.element_size()


def _vjp_common(x, w, g):
    _check_act(x, "x")
    _check_act(g, "g", x.device)
    dt = _dtype_code(x, "x")
    if g.shape != x.shape or g.dtype != x.dtype:
        raise ValueError(f"g must be {x.dtype} of shape {list(x.shape)}, got {g.dtype} "
                         f"{list(g.shape)}")
    rows, hidden = _rows(x)
    w, wdt = _check_param(w, "w", hidden, x)
    pdtype = x.dtype if w is None else w.dtype
    return dt, rows, hidden, w, wdt, pdtype


def rms_norm_vjp(x, w, g, eps=1e-5, want_dw=True, dx=None, dw=None, workspace=None):
    """Gradients of RMSNorm for x and w given the output cotangent g (nrm_rms_norm_vjp):
    returns (dx, dw); dw is None when neither ``want_dw`` nor ``dw`` asks for it."""
    dt, rows, hidden, w, wdt, pdtype = _vjp_common(x, w, g)
    dx = _out_like(dx, x, "dx")
    dw = _param_grad(want_dw, dw, hidden, x, pdtype, "dw")
    need = vjp_workspace_bytes(rows, hidden, False) if dw is not None else 0
    ws, ws_bytes = _workspace(workspace, need, x)
    st = load().nrm_rms_norm_vjp(_ptr(x), _ptr(w), _ptr(g), _ptr(dx), _ptr(dw), rows, hidden,
                                 eps, dt, wdt, _ptr(ws), ws_bytes, _stream())
    if st:
        _raise(st)
    return dx, dw


def layer_norm_vjp(x, w, g, eps=1e-5, want_dw=True, want_db=True, dx=None, dw=None, db=None,
                   workspace=None):
    """Gradients of LayerNorm for x, w and b given the output cotangent g
    (nrm_layer_norm_vjp): returns (dx, dw, db), None for a gradient not asked for."""
    dt, rows, hidden, w, wdt, pdtype = _vjp_common(x, w, g)
    dx = _out_like(dx, x, "dx")
    dw = _param_grad(want_dw, dw, hidden, x, pdtype, "dw")
    db = _param_grad(want_db, db, hidden, x, pdtype, "db")
    need = vjp_workspace_bytes(rows, hidden, True) if (dw is not None or db is not None) else 0
    ws, ws_bytes = _workspace(workspace, need, x)
    st = load().nrm_layer_norm_vjp(_ptr(x), _ptr(w), _ptr(g), _ptr(dx), _ptr(dw), _ptr(db), rows,
                                   hidden, eps, dt, wdt, _ptr(ws), ws_bytes, _stream())
    if st:
        _raise(st)
    return dx, dw, db


def layer_norm_vjp_noalloc(x, w, g, eps=1e-5, want_dw=True, want_db=True, dx=None, dw=None,
                           db=None):
    """layer_norm_vjp through nrm_layer_norm_vjp_noalloc: the partial column sums go to the
    library's static device scratch, so the call allocates no workspace (pass dx, dw and db
    to allocate nothing at all). Calls that may overlap on one GPU must be ordered."""
    dt, rows, hidden, w, wdt, pdtype = _vjp_common(x, w, g)
    dx = _out_like(dx, x, "dx")
    dw = _param_grad(want_dw, dw, hidden, x, pdtype, "dw")
    db = _param_grad(want_db, db, hidden, x, pdtype, "db")
    st = load().nrm_layer_norm_vjp_noalloc(_ptr(x), _ptr(w), _ptr(g), _ptr(dx), _ptr(dw),
                                           _ptr(db), rows, hidden, eps, dt, wdt, _stream())
    if st:
        _raise(st)
    return dx, dw, db


def rope(x, dims=None, traditional=False, base=10000.0, scale=1.0, offset=0, forward=True,
         freqs=None, mscale=1.0, out=None):
    """Rope over x [..., L, D] (nrm_rope): row l of every leading index at offset + l."""
    _check_act(x, "x")
    dt = _dtype_code(x, "x")
    if x.dim() < 2:
        raise ValueError(f"x must be [..., L, D], got {list(x.shape)}")
    L, D = x.shape[-2], x.shape[-1]
    N = x.numel() // (L * D) if L * D else 0
    dims = D if dims is None else int(dims)
    freqs = _freqs_arg(freqs, dims, x)
    out = _out_like(out, x, "out")
    st = load().nrm_rope(_ptr(x), _ptr(out), N, L, D, dims, int(bool(traditional)), base, scale,
                         int(offset), int(bool(forward)), _ptr(freqs), mscale, dt, _stream())
    if st:
        _raise(st)
    return out


def rope_positions(positions, q, k=None, dims=None, traditional=False, base=10000.0, scale=1.0,
                   forward=True, freqs=None, mscale=1.0, q_out=None, k_out=None):
    """Rotate query [..., Hq, D] and key [..., Hk, D] rows at per-token positions in one
    launch (nrm_rope_positions). The leading axes flatten to T tokens; positions holds T
    integers, or one sequence's positions (repeated for every sequence of a batch)."""
    _check_act(q, "q")
    dt = _dtype_code(q, "q")
    if q.dim() < 3:
        raise ValueError(f"q must be [..., T, Hq, D], got {list(q.shape)}")
    Hq, D = q.shape[-2], q.shape[-1]
    T = q.numel() // (Hq * D) if Hq * D else 0
    Hk = 0
    if k is not None:
        _check_act(k, "k", q.device)
        if k.dtype != q.dtype or k.shape[:-2] != q.shape[:-2] or k.shape[-1] != D:
            raise ValueError(f"k must be {q.dtype} [..., Hk, {D}] with q's leading axes, got "
                             f"{k.dtype} {list(k.shape)}")
        Hk = k.shape[-2]
    _check_act(positions, "positions", q.device)
    if positions.dtype not in (torch.int32, torch.int64) or positions.dim() != 1:
        raise ValueError(f"positions must be a 1-D int32 or int64 tensor, got {positions.dtype} "
                         f"{list(positions.shape)}")
    if positions.shape[0] != T:
        if T and positions.shape[0] and T % positions.shape[0] == 0:
            positions = positions.repeat(T // positions.shape[0])
        else:
            raise ValueError(f"positions must hold {T} positions (or one sequence's), got "
                             f"{positions.shape[0]}")
    dims = D if dims is None else int(dims)
    freqs = _freqs_arg(freqs, dims, q)
    q_out = _out_like(q_out, q, "q_out")
    k_out = _out_like(k_out, k, "k_out") if k is not None else None
    st = load().nrm_rope_positions(_ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), _ptr(positions),
                                   int(positions.dtype == torch.int64), T, Hq, Hk, D, dims,
                                   int(bool(traditional)), base, scale, int(bool(forward)),
                                   _ptr(freqs), mscale, dt, _stream())
    if st:
        _raise(st)
    return q_out, k_out


def _host_freqs(fn, dims, *args):
    out = torch.empty(dims // 2, dtype=torch.float32)
    ms = ctypes.c_float(0.0)
    st = fn(dims, *args, ctypes.c_void_p(out.data_ptr()), ctypes.byref(ms))
    if st:
        _raise(st)
    return out, ms.value


def rope_freqs_llama3(dims, base, factor=32.0, low_freq_factor=1.0, high_freq_factor=4.0,
                      original_max=8192):
    """Llama 3 scaled divisors (nrm_rope_freqs_llama3): (CPU float32 [dims / 2], mscale)."""
    return _host_freqs(load().nrm_rope_freqs_llama3, dims, base, factor, low_freq_factor,
                       high_freq_factor, original_max)


def rope_freqs_yarn(dims, base, factor=4.0, original_max=4096, beta_fast=32.0, beta_slow=1.0,
                    mscale=1.0, mscale_all_dim=0.0):
    """YaRN scaled divisors and attention factor (nrm_rope_freqs_yarn)."""
    return _host_freqs(load().nrm_rope_freqs_yarn, dims, base, factor, original_max, beta_fast,
                       beta_slow, mscale, mscale_all_dim)


def rope_freqs_su(dims, base, long_factor, max_position=131072, original_max=4096):
    """LongRoPE ("su") scaled divisors and attention factor (nrm_rope_freqs_su)."""
    lf = torch.as_tensor(long_factor, dtype=torch.float32).contiguous()
    if lf.dim() != 1 or lf.shape[0] != dims // 2:
        raise ValueError(f"long_factor must hold {dims // 2} values, got {list(lf.shape)}")
    return _host_freqs(load().nrm_rope_freqs_su, dims, base, ctypes.c_void_p(lf.data_ptr()),
                       max_position, original_max)


def softmax(x, out=None):
    """Softmax over the last axis (nrm_softmax); ``out`` may be ``x``."""
    _check_act(x, "x")
    dt = _dtype_code(x, "x")
    rows, n = _rows(x)
    out = _out_like(out, x, "out")
    st = load().nrm_softmax(_ptr(x), _ptr(out), rows, n, dt, _stream())
    if st:
        _raise(st)
    return out


def causal_softmax(x, rows, out=None):
    """Softmax of x [..., R, L] with MLX's blocked causal mask of ``rows`` rows per block
    (nrm_causal_softmax)."""
    _check_act(x, "x")
    dt = _dtype_code(x, "x")
    if x.dim() < 2:
        raise ValueError(f"x must be [..., R, L], got {list(x.shape)}")
    R, L = x.shape[-2], x.shape[-1]
    N = x.numel() // (R * L) if R * L else 0
    out = _out_like(out, x, "out")
    st = load().nrm_causal_softmax(_ptr(x), _ptr(out), N, R, L, int(rows), dt, _stream())
    if st:
        _raise(st)
    return out


def logsumexp(x, out=None):
    """log(sum(exp(x))) over the last axis, kept as a size-1 axis (nrm_logsumexp)."""
    _check_act(x, "x")
    dt = _dtype_code(x, "x")
    rows, n = _rows(x)
    shape = list(x.shape[:-1]) + [1]
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    _check_act(out, "out", x.device)
    if list(out.shape) != shape or out.dtype != x.dtype:
        raise ValueError(f"out must be {x.dtype} {shape}, got {out.dtype} {list(out.shape)}")
    st = load().nrm_logsumexp(_ptr(x), _ptr(out), rows, n, dt, _stream())
    if st:
        _raise(st)
    return out


def _ce_common(logits, targets):
    _check_act(logits, "logits")
    dt = _dtype_code(logits, "logits")
    rows, V = _rows(logits)
    _check_act(targets, "targets", logits.device)
    if targets.dtype not in (torch.int32, torch.int64) or targets.numel() != rows:
        raise ValueError(f"targets must hold {rows} int32 or int64 values, got "
                         f"{targets.dtype} {list(targets.shape)}")
    return dt, rows, V, int(targets.dtype == torch.int64)


def cross_entropy(logits, targets, loss=None):
    """logsumexp(logits) - logits[target] per row, float32 (nrm_cross_entropy)."""
    dt, rows, V, i64 = _ce_common(logits, targets)
    shape = list(logits.shape[:-1])
    if loss is None:
        loss = torch.empty(shape, dtype=torch.float32, device=logits.device)
    _check_act(loss, "loss", logits.device)
    if loss.dtype != torch.float32 or loss.numel() != rows:
        raise ValueError(f"loss must be float32 with {rows} values")
    st = load().nrm_cross_entropy(_ptr(logits), _ptr(targets), i64, _ptr(loss), rows, V, dt,
                                  _stream())
    if st:
        _raise(st)
    return loss


def cross_entropy_vjp(logits, targets, g, loss=None, dlogits=None):
    """Gradient of cross_entropy for the logits given the loss cotangent g (float32 per
    row) (nrm_cross_entropy_vjp); ``dlogits`` may be ``logits``."""
    dt, rows, V, i64 = _ce_common(logits, targets)
    _check_act(g, "g", logits.device)
    if g.dtype != torch.float32 or g.numel() != rows:
        raise ValueError(f"g must be float32 with {rows} values")
    dlogits = _out_like(dlogits, logits, "dlogits")
    st = load().nrm_cross_entropy_vjp(_ptr(logits), _ptr(targets), i64, _ptr(loss), _ptr(g),
                                      _ptr(dlogits), rows, V, dt, _stream())
    if st:
        _raise(st)
    return dlogits


def bench_copy(src, dst):
    """16-byte copy of src into dst (nrm_bench_copy): the bandwidth ceiling."""
    _check_act(src, "src")
    _check_act(dst, "dst", src.device)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst is smaller than src")
    st = load().nrm_bench_copy(_ptr(src), _ptr(dst), n, _stream())
    if st:
        _raise(st)
    return dst


def bench_copy2(src1, src2, dst1, dst2):
    """dst1 = src1 and dst2 = src2 with 16-byte chunks (nrm_bench_copy2): the bandwidth
    ceiling of two arrays in and two out."""
    for t, what in ((src1, "src1"), (src2, "src2"), (dst1, "dst1"), (dst2, "dst2")):
        _check_act(t, what, src1.device)
    n = src1.numel() * src1.element_size()
    if any(t.numel() * t.element_size() < n for t in (src2, dst1, dst2)):
        raise ValueError("src2, dst1 and dst2 must hold at least as many bytes as src1")
    st = load().nrm_bench_copy2(_ptr(src1), _ptr(src2), _ptr(dst1), _ptr(dst2), n, _stream())
    if st:
        _raise(st)
    return dst1, dst2


def bench_copy2_row(src1, src2, dst1, dst2, unit_bytes=16384):
    """dst1 = src1 and dst2 = src2 in the row kernels' work unit (nrm_bench_copy2_row): each
    block loads unit_bytes of each source and stores nothing until all of it has arrived."""
    for t, what in ((src1, "src1"), (src2, "src2"), (dst1, "dst1"), (dst2, "dst2")):
        _check_act(t, what, src1.device)
    n = src1.numel() * src1.element_size()
    if any(t.numel() * t.element_size() < n for t in (src2, dst1, dst2)):
        raise ValueError("src2, dst1 and dst2 must hold at least as many bytes as src1")
    st = load().nrm_bench_copy2_row(_ptr(src1), _ptr(src2), _ptr(dst1), _ptr(dst2), n,
                                    int(unit_bytes), _stream())
    if st:
        _raise(st)
    return dst1, dst2

"""Python binding of libgla (include/gla.h): argument marshalling only.

Every step of the mixer runs in the HIP kernels of libgla.so; this module only
checks tensor metadata, allocates outputs/workspace with torch, and passes raw
device pointers plus torch's current HIP stream through ctypes.  There is no
fallback: if libgla.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgla.so")

GLA_OK, GLA_ERR_INVALID_ARG, GLA_ERR_UNSUPPORTED, GLA_ERR_WORKSPACE, GLA_ERR_DEVICE = range(5)
GLA_F32, GLA_BF16 = 0, 1

SYMBOLS = (
    "gla_abi_version",
    "gla_status_str",
    "gla_fwd_workspace_bytes",
    "gla_fwd_chunked",
    "gla_bwd_workspace_bytes",
    "gla_bwd_chunked",
    "gla_fwd_states_bytes",
    "gla_fwd_chunked_states",
    "gla_bwd_chunked_states",
    "gla_decode_step",
    "gla_decode_step_pool",
    "gla_mixer_epilogue",
    "gla_fwd_chunked_epilogue",
    "gla_decode_step_epilogue",
    "gla_conv1d_silu",
    "gla_conv1d_silu_decode",
)

_lib = None


class EpilogueParams(ctypes.Structure):
    """gla_epilogue_params: device aug_a / norm_w, host head_tier."""
    _fields_ = [("aug_a", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("head_tier", ctypes.POINTER(ctypes.c_int)), ("n_tiers", ctypes.c_int),
                ("eps", ctypes.c_float)]


class GlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


def load():
    """Load libgla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libgla.so not built at {LIB_PATH}; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.gla_abi_version.restype = i
        lib.gla_status_str.restype = ctypes.c_char_p
        lib.gla_status_str.argtypes = [i]
        lib.gla_fwd_workspace_bytes.restype = sz
        lib.gla_fwd_workspace_bytes.argtypes = [i] * 7
        lib.gla_fwd_chunked.restype = i
        lib.gla_fwd_chunked.argtypes = [i] * 7 + [vp, vp, vp, vp, vp, f, vp, vp, vp, sz, vp]
        lib.gla_bwd_workspace_bytes.restype = sz
        lib.gla_bwd_workspace_bytes.argtypes = [i] * 7
        lib.gla_bwd_chunked.restype = i
        lib.gla_bwd_chunked.argtypes = [i] * 7 + [vp, vp, vp, vp, vp, f, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.gla_fwd_states_bytes.restype = sz
        lib.gla_fwd_states_bytes.argtypes = [i] * 7
        lib.gla_fwd_chunked_states.restype = i
        lib.gla_fwd_chunked_states.argtypes = [i] * 7 + [vp, vp, vp, vp, vp, f, vp, vp, vp, vp, sz, vp]
        lib.gla_bwd_chunked_states.restype = i
        lib.gla_bwd_chunked_states.argtypes = [i] * 7 + [vp] * 5 + [f] + [vp] * 9 + [sz, vp]
        lib.gla_decode_step.restype = i
        lib.gla_decode_step.argtypes = [i] * 5 + [vp, vp, vp, vp, vp, f, vp, vp]
        lib.gla_decode_step_pool.restype = i
        lib.gla_decode_step_pool.argtypes = [i] * 5 + [vp, vp, vp, vp, vp, i, vp, f, vp, vp]
        ep = ctypes.POINTER(EpilogueParams)
        lib.gla_mixer_epilogue.restype = i
        lib.gla_mixer_epilogue.argtypes = [i] * 5 + [vp, vp, vp, vp, vp, ep, vp, vp]
        lib.gla_fwd_chunked_epilogue.restype = i
        lib.gla_fwd_chunked_epilogue.argtypes = [i] * 7 + [vp, vp, vp, vp, vp, f, vp, ep, vp, vp, vp, sz, vp]
        lib.gla_decode_step_epilogue.restype = i
        lib.gla_decode_step_epilogue.argtypes = [i] * 5 + [vp, vp, vp, vp, vp, vp, i, vp, f, ep, vp, vp]
        lib.gla_conv1d_silu.restype = i
        lib.gla_conv1d_silu.argtypes = [i] * 5 + [vp] * 7
        lib.gla_conv1d_silu_decode.restype = i
        lib.gla_conv1d_silu_decode.argtypes = [i] * 4 + [vp, vp, vp, vp, i, vp, vp, vp]
        _lib = lib
    return _lib


def status_str(status: int) -> str:
    return load().gla_status_str(int(status)).decode()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GLA_BF16
    if t.dtype == torch.float32:
        return GLA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(t, name, shape, dtype, device):
    if t.device != device or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def fwd_workspace_bytes(dtype: int, B, T, H, dk, dv, chunk) -> int:
    return int(load().gla_fwd_workspace_bytes(dtype, B, T, H, dk, dv, chunk))


def fwd_chunked(q, k, v, lam, S0=None, scale=1.0, chunk=128, o=None, S_final=True,
                workspace=None, stream=None):
    """o, S_final = gla_fwd_chunked(...).  S_final=False skips the final state;
    a tensor passed as `o`/`S_final` is written in place."""
    lib = load()
    B, T, H, dk = q.shape
    dv = v.shape[3]
    dev = q.device
    _check(q, "q", (B, T, H, dk), q.dtype, dev)
    _check(k, "k", (B, T, H, dk), q.dtype, dev)
    _check(v, "v", (B, T, H, dv), q.dtype, dev)
    _check(lam, "lambda", (H,), torch.float32, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _check(o, "o", (B, T, H, dv), q.dtype, dev)
    if S_final is True:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_final is False:
        S_final = None
    if S_final is not None:
        _check(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    dt = _dt(q)
    need = lib.gla_fwd_workspace_bytes(dt, B, T, H, dk, dv, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gla_fwd_chunked(dt, B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(lam),
                             _ptr(S0), float(scale), _ptr(o), _ptr(S_final), _ptr(workspace),
                             ws_bytes, _stream(stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_fwd_chunked")
    return o, S_final


def bwd_workspace_bytes(dtype: int, B, T, H, dk, dv, chunk) -> int:
    return int(load().gla_bwd_workspace_bytes(dtype, B, T, H, dk, dv, chunk))


def bwd_chunked(q, k, v, lam, d_o, S0=None, dS_final=None, scale=1.0, chunk=128,
                dlambda=True, dS0=True, workspace=None, stream=None):
    """dq, dk, dv, dlambda ([H] or None), dS0 ([B,H,dk,dv] or None) = gla_bwd_chunked(...)."""
    lib = load()
    B, T, H, dk = q.shape
    dv = v.shape[3]
    dev = q.device
    _check(q, "q", (B, T, H, dk), q.dtype, dev)
    _check(k, "k", (B, T, H, dk), q.dtype, dev)
    _check(v, "v", (B, T, H, dv), q.dtype, dev)
    _check(d_o, "do", (B, T, H, dv), q.dtype, dev)
    _check(lam, "lambda", (H,), torch.float32, dev)
    for t, name in ((S0, "S0"), (dS_final, "dS_final")):
        if t is not None:
            _check(t, name, (B, H, dk, dv), torch.float32, dev)
    dq = torch.empty_like(q)
    dkk = torch.empty_like(k)
    dvv = torch.empty_like(v)
    dl = torch.empty(H, dtype=torch.float32, device=dev) if dlambda else None
    ds0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if dS0 else None
    dt = _dt(q)
    need = lib.gla_bwd_workspace_bytes(dt, B, T, H, dk, dv, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gla_bwd_chunked(dt, B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(S0),
                             float(scale), _ptr(d_o), _ptr(dS_final), _ptr(dq), _ptr(dkk), _ptr(dvv),
                             _ptr(dl), _ptr(ds0), _ptr(workspace), ws_bytes, _stream(stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_bwd_chunked")
    return dq, dkk, dvv, dl, ds0


def decode_step(q, k, v, lam, S, scale=1.0, o=None, stream=None):
    """In place on S: S <- lam S + k v^T, o = scale S^T q.  Returns o."""
    lib = load()
    N, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    _check(q, "q", (N, H, dk), q.dtype, dev)
    _check(k, "k", (N, H, dk), q.dtype, dev)
    _check(v, "v", (N, H, dv), q.dtype, dev)
    _check(lam, "lambda", (H,), torch.float32, dev)
    _check(S, "S", (N, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _check(o, "o", (N, H, dv), q.dtype, dev)
    st = lib.gla_decode_step(_dt(q), N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(S),
                             float(scale), _ptr(o), _stream(stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_decode_step")
    return o


def decode_step_pool(q, k, v, lam, pool, slots, scale=1.0, o=None, stream=None):
    """Decode on a page pool: row n uses page slots[n] of pool [P, H, dk, dv] (in place);
    a slot outside [0, P) (-1: padding row) gives a zero output row.  Returns o."""
    lib = load()
    N, H, dk = q.shape
    dv = v.shape[2]
    P = pool.shape[0]
    dev = q.device
    _check(q, "q", (N, H, dk), q.dtype, dev)
    _check(k, "k", (N, H, dk), q.dtype, dev)
    _check(v, "v", (N, H, dv), q.dtype, dev)
    _check(lam, "lambda", (H,), torch.float32, dev)
    _check(pool, "pool", (P, H, dk, dv), torch.float32, dev)
    _check(slots, "slots", (N,), torch.int32, dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _check(o, "o", (N, H, dv), q.dtype, dev)
    st = lib.gla_decode_step_pool(_dt(q), N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(pool), P,
                                  _ptr(slots), float(scale), _ptr(o), _stream(stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_decode_step_pool")
    return o


def _epi_params(H, dk, dv, aug_a, norm_w, head_tier, eps, dev):
    if aug_a is not None:
        _check(aug_a, "aug_a", (H, dk), torch.float32, dev)
    n_tiers = norm_w.shape[0]
    _check(norm_w, "norm_w", (n_tiers, dv), torch.float32, dev)
    tiers = [int(t) for t in head_tier]
    if len(tiers) != H:
        raise ValueError(f"head_tier: expected {H} entries, got {len(tiers)}")
    tier_arr = (ctypes.c_int * H)(*tiers)
    p = EpilogueParams(None if aug_a is None else aug_a.data_ptr(), norm_w.data_ptr(),
                       ctypes.cast(tier_arr, ctypes.POINTER(ctypes.c_int)), n_tiers, float(eps))
    return p, tier_arr


def mixer_epilogue(q, k, v, o, g, norm_w, head_tier, aug_a=None, eps=1e-6, y=None, stream=None):
    """y = silu(g) * RMSNorm_tier(o + sigmoid(q.(a*k)) v) per (row, head).
    q, k [..., H, dk]; v, o, g [..., H, dv]; norm_w [n_tiers, dv] fp32; head_tier: H ints;
    aug_a [H, dk] fp32 or None.  `y` may be `o` (in place).  Returns y."""
    lib = load()
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    lead = tuple(q.shape[:-2])
    M = 1
    for d in lead:
        M *= int(d)
    dev = q.device
    _check(q, "q", lead + (H, dk), q.dtype, dev)
    _check(k, "k", lead + (H, dk), q.dtype, dev)
    for t, name in ((v, "v"), (o, "o"), (g, "g")):
        _check(t, name, lead + (H, dv), q.dtype, dev)
    if y is None:
        y = torch.empty(lead + (H, dv), dtype=q.dtype, device=dev)
    _check(y, "y", lead + (H, dv), q.dtype, dev)
    p, _keep = _epi_params(H, dk, dv, aug_a, norm_w, head_tier, eps, dev)
    st = lib.gla_mixer_epilogue(_dt(q), M, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(g),
                                ctypes.byref(p), _ptr(y), _stream(stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_mixer_epilogue")
    return y


def decode_step_epilogue(q, k, v, g, lam, S, norm_w, head_tier, aug_a=None, eps=1e-6, scale=1.0,
                         slots=None, y=None, stream=None):
    """Decode step with the epilogue fused: S (pages [N, H, dk, dv], or a pool [P, H, dk, dv]
    indexed by int32 `slots`) is updated in place; returns y [N, H, dv]."""
    lib = load()
    N, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    _check(q, "q", (N, H, dk), q.dtype, dev)
    _check(k, "k", (N, H, dk), q.dtype, dev)
    _check(v, "v", (N, H, dv), q.dtype, dev)
    _check(g, "g", (N, H, dv), q.dtype, dev)
    _check(lam, "lambda", (H,), torch.float32, dev)
    P = S.shape[0]
    if slots is None:
        _check(S, "S", (N, H, dk, dv), torch.float32, dev)
    else:
        _check(S, "pool", (P, H, dk, dv), torch.float32, dev)
        _check(slots, "slots", (N,), torch.int32, dev)
    if y is None:
        y = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _check(y, "y", (N, H, dv), q.dtype, dev)
    p, _keep = _epi_params(H, dk, dv, aug_a, norm_w, head_tier, eps, dev)
    st = lib.gla_decode_step_epilogue(_dt(q), N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(lam),
                                      _ptr(S), P, _ptr(slots), float(scale), ctypes.byref(p), _ptr(y),
                                      _stream(stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_decode_step_epilogue")
    return y


def conv1d_silu(x, w, bias=None, win_in=None, win_out=True, y=None, stream=None):
    """Depth-wise causal conv (width 4) + SiLU: x [B, T, D]; w [D, 4] fp32; bias [D] or None;
    win_in [B, 4, D] fp32 or None (zeros).  Returns (y, win_out): win_out=True allocates the
    window after the last token, False skips it, a tensor (win_in itself allowed) is written."""
    lib = load()
    B, T, D = x.shape
    K = w.shape[1]
    dev = x.device
    _check(x, "x", (B, T, D), x.dtype, dev)
    _check(w, "w", (D, K), torch.float32, dev)
    if bias is not None:
        _check(bias, "bias", (D,), torch.float32, dev)
    if win_in is not None:
        _check(win_in, "win_in", (B, K, D), torch.float32, dev)
    if win_out is True:
        win_out = torch.empty((B, K, D), dtype=torch.float32, device=dev)
    elif win_out is False:
        win_out = None
    if win_out is not None:
        _check(win_out, "win_out", (B, K, D), torch.float32, dev)
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", (B, T, D), x.dtype, dev)
    st = lib.gla_conv1d_silu(_dt(x), B, T, D, K, _ptr(x), _ptr(w), _ptr(bias), _ptr(win_in), _ptr(y),
                             _ptr(win_out), _stream(stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_conv1d_silu")
    return y, win_out


def conv1d_silu_decode(x, w, bias, win, slots=None, y=None, stream=None):
    """One token per row: x [N, D]; win [N, 4, D] fp32 (or a pool [P, 4, D] indexed by
    int32 `slots`), updated in place.  Returns y [N, D]."""
    lib = load()
    N, D = x.shape
    K = w.shape[1]
    dev = x.device
    _check(x, "x", (N, D), x.dtype, dev)
    _check(w, "w", (D, K), torch.float32, dev)
    if bias is not None:
        _check(bias, "bias", (D,), torch.float32, dev)
    P = win.shape[0]
    if slots is None:
        _check(win, "win", (N, K, D), torch.float32, dev)
    else:
        _check(win, "win", (P, K, D), torch.float32, dev)
        _check(slots, "slots", (N,), torch.int32, dev)
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", (N, D), x.dtype, dev)
    st = lib.gla_conv1d_silu_decode(_dt(x), N, D, K, _ptr(x), _ptr(w), _ptr(bias), _ptr(win), P, _ptr(slots),
                                    _ptr(y), _stream(stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_conv1d_silu_decode")
    return y


def fwd_chunked_epilogue(q, k, v, lam, g, norm_w, head_tier, aug_a=None, eps=1e-6, S0=None, scale=1.0,
                         chunk=128, y=None, S_final=True, workspace=None, stream=None):
    """y, S_final: the forward followed by the mixer epilogue (y in place of o)."""
    lib = load()
    B, T, H, dk = q.shape
    dv = v.shape[3]
    dev = q.device
    _check(q, "q", (B, T, H, dk), q.dtype, dev)
    _check(k, "k", (B, T, H, dk), q.dtype, dev)
    _check(v, "v", (B, T, H, dv), q.dtype, dev)
    _check(g, "g", (B, T, H, dv), q.dtype, dev)
    _check(lam, "lambda", (H,), torch.float32, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if y is None:
        y = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _check(y, "y", (B, T, H, dv), q.dtype, dev)
    if S_final is True:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_final is False:
        S_final = None
    if S_final is not None:
        _check(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    dt = _dt(q)
    need = lib.gla_fwd_workspace_bytes(dt, B, T, H, dk, dv, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    p, _keep = _epi_params(H, dk, dv, aug_a, norm_w, head_tier, eps, dev)
    st = lib.gla_fwd_chunked_epilogue(dt, B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(S0),
                                      float(scale), _ptr(g), ctypes.byref(p), _ptr(y), _ptr(S_final),
                                      _ptr(workspace), ws_bytes, _stream(stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_fwd_chunked_epilogue")
    return y, S_final


def fwd_chunked_states(q, k, v, lam, S0=None, scale=1.0, chunk=128, S_final=True, workspace=None, stream=None):
    """o, S_final, states = the forward, also saving every chunk's start state for the backward."""
    lib = load()
    B, T, H, dk = q.shape
    dv = v.shape[3]
    dev = q.device
    _check(q, "q", (B, T, H, dk), q.dtype, dev)
    _check(k, "k", (B, T, H, dk), q.dtype, dev)
    _check(v, "v", (B, T, H, dv), q.dtype, dev)
    _check(lam, "lambda", (H,), torch.float32, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if S_final else None
    nc = (T + chunk - 1) // chunk
    states = torch.empty((B, H, nc, dk, dv), dtype=q.dtype, device=dev)
    dt = _dt(q)
    need = lib.gla_fwd_workspace_bytes(dt, B, T, H, dk, dv, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gla_fwd_chunked_states(dt, B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(S0),
                                    float(scale), _ptr(o), _ptr(S_final), _ptr(states), _ptr(workspace), ws_bytes,
                                    _stream(stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_fwd_chunked_states")
    return o, S_final, states


def bwd_chunked_states(q, k, v, lam, d_o, states, S0=None, dS_final=None, scale=1.0, chunk=128,
                       dlambda=True, dS0=True, workspace=None, stream=None):
    """dq, dk, dv, dlambda, dS0 from the chunk start states saved by fwd_chunked_states."""
    lib = load()
    B, T, H, dk = q.shape
    dv = v.shape[3]
    dev = q.device
    nc = (T + chunk - 1) // chunk
    for t, name, shape in ((q, "q", (B, T, H, dk)), (k, "k", (B, T, H, dk)), (v, "v", (B, T, H, dv)),
                           (d_o, "do", (B, T, H, dv)), (states, "states", (B, H, nc, dk, dv))):
        _check(t, name, shape, q.dtype, dev)
    _check(lam, "lambda", (H,), torch.float32, dev)
    for t, name in ((S0, "S0"), (dS_final, "dS_final")):
        if t is not None:
            _check(t, name, (B, H, dk, dv), torch.float32, dev)
    dq, dkk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dl = torch.empty(H, dtype=torch.float32, device=dev) if dlambda else None
    ds0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if dS0 else None
    dt = _dt(q)
    need = lib.gla_bwd_workspace_bytes(dt, B, T, H, dk, dv, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gla_bwd_chunked_states(dt, B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(S0),
                                    float(scale), _ptr(d_o), _ptr(dS_final), _ptr(states), _ptr(dq), _ptr(dkk),
                                    _ptr(dvv), _ptr(dl), _ptr(ds0), _ptr(workspace), ws_bytes, _stream(stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_bwd_chunked_states")
    return dq, dkk, dvv, dl, ds0

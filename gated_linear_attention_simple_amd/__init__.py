"""Python binding of libgla (include/gla.h, include/gla_plan.h): argument marshalling only.

Every step of the mixer runs in the HIP kernels of libgla.so; this module only
checks tensor metadata, allocates outputs/workspace with torch, and passes raw
device pointers plus a HIP stream through ctypes.  There is no fallback: if
libgla.so is missing or fails to load, every call raises, and tensors that are
not on the current GPU are rejected before the library is called.

Streams: a call runs on `stream` (default: torch's current stream).  Outputs and
workspace are allocated on that stream, so the caching allocator orders their
reuse after the call's kernels.

Token-major tensors of the chunked calls ([B, T, H, d]) may be strided views,
e.g. q, k, v, g sliced out of one fused [B, T, H (2 dk + 2 dv)] projection: the
head and feature dimensions must be packed; the batch and token strides are
passed to the library, which validates them.
"""
from __future__ import annotations

import contextlib
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
    "gla_bwd_states_workspace_bytes",
    "gla_bwd_chunked_states",
    "gla_decode_step",
    "gla_decode_step_pool",
    "gla_mixer_epilogue",
    "gla_fwd_chunked_epilogue",
    "gla_decode_step_epilogue",
    "gla_conv1d_silu",
    "gla_conv1d_silu_decode",
    "gla_plan_resolve",
    "gla_fwd_workspace_bytes_planned",
    "gla_bwd_workspace_bytes_planned",
    "gla_fwd_chunked_planned",
    "gla_bwd_chunked_planned",
    "gla_fwd_chunked_noalloc",
)

# the allocation-free forward's workspace limit (GLA_NOALLOC_WORKSPACE_MAX in gla.h)
NOALLOC_WORKSPACE_MAX = 32 << 20

_lib = None


class EpilogueParams(ctypes.Structure):
    """gla_epilogue_params: device aug_a / norm_w, host head_tier."""
    _fields_ = [("aug_a", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("head_tier", ctypes.POINTER(ctypes.c_int)), ("n_tiers", ctypes.c_int),
                ("eps", ctypes.c_float)]


class Stride(ctypes.Structure):
    """gla_stride: element strides of a token-major tensor (0 = packed)."""
    _fields_ = [("batch", ctypes.c_longlong), ("token", ctypes.c_longlong)]


class Strides(ctypes.Structure):
    """gla_strides: one gla_stride per token-major tensor of the chunked calls."""
    _fields_ = [(name, Stride) for name in ("q", "k", "v", "o", "d_o", "dq", "dk", "dv", "g")]


class Plan(ctypes.Structure):
    """gla_plan: segments (0 = library), chain (-1 = library, 0, 1), psub (0 = library, 1),
    scan (-1 = library, 0 = scan launch, 1 = folded into the segments)."""
    _fields_ = [("segments", ctypes.c_int), ("chain", ctypes.c_int), ("psub", ctypes.c_int),
                ("scan", ctypes.c_int)]


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
        stp, pp, ep = ctypes.POINTER(Strides), ctypes.POINTER(Plan), ctypes.POINTER(EpilogueParams)
        lib.gla_abi_version.restype = i
        lib.gla_status_str.restype = ctypes.c_char_p
        lib.gla_status_str.argtypes = [i]
        for name in ("gla_fwd_workspace_bytes", "gla_bwd_workspace_bytes", "gla_fwd_states_bytes",
                     "gla_bwd_states_workspace_bytes"):
            getattr(lib, name).restype = sz
            getattr(lib, name).argtypes = [i] * 7
        lib.gla_fwd_chunked.argtypes = [i] * 7 + [vp] * 5 + [f, vp, vp, stp, vp, sz, vp]
        lib.gla_bwd_chunked.argtypes = [i] * 7 + [vp] * 5 + [f] + [vp] * 7 + [stp, vp, sz, vp]
        lib.gla_fwd_chunked_states.argtypes = [i] * 7 + [vp] * 5 + [f, vp, vp, vp, stp, vp, sz, vp]
        lib.gla_bwd_chunked_states.argtypes = [i] * 7 + [vp] * 5 + [f] + [vp] * 8 + [stp, vp, sz, vp]
        lib.gla_decode_step.argtypes = [i] * 5 + [vp, vp, vp, vp, vp, f, vp, vp]
        lib.gla_decode_step_pool.argtypes = [i] * 5 + [vp, vp, vp, vp, vp, i, vp, f, vp, vp]
        lib.gla_mixer_epilogue.argtypes = [i] * 5 + [vp, vp, vp, vp, vp, ep, vp, vp]
        lib.gla_fwd_chunked_epilogue.argtypes = [i] * 7 + [vp] * 5 + [f, vp, ep, vp, vp, stp, vp, sz, vp]
        lib.gla_decode_step_epilogue.argtypes = [i] * 5 + [vp, vp, vp, vp, vp, vp, i, vp, f, ep, vp, vp]
        lib.gla_conv1d_silu.argtypes = [i] * 5 + [vp] * 7
        lib.gla_conv1d_silu_decode.argtypes = [i] * 4 + [vp, vp, vp, vp, i, vp, vp, vp]
        lib.gla_plan_resolve.argtypes = [i] * 7 + [pp, pp]
        lib.gla_fwd_workspace_bytes_planned.restype = sz
        lib.gla_fwd_workspace_bytes_planned.argtypes = [i] * 7 + [pp]
        lib.gla_bwd_workspace_bytes_planned.restype = sz
        lib.gla_bwd_workspace_bytes_planned.argtypes = [i] * 8 + [pp]
        lib.gla_fwd_chunked_planned.argtypes = [i] * 7 + [vp] * 5 + [f, vp, vp, vp, vp, ep, stp, pp, vp, sz, vp]
        lib.gla_bwd_chunked_planned.argtypes = [i] * 7 + [vp] * 5 + [f] + [vp] * 8 + [stp, pp, vp, sz, vp]
        lib.gla_fwd_chunked_noalloc.argtypes = [i] * 7 + [vp] * 5 + [f, vp, vp, stp, vp]
        for name in SYMBOLS:   # every call that computes returns a gla_status
            if name not in ("gla_status_str", "gla_abi_version") and not name.endswith("bytes"):
                getattr(lib, name).restype = i
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


def _device(t: torch.Tensor) -> torch.device:
    """The device every tensor of a call must be on: the current CUDA (HIP) device."""
    if t.device.type != "cuda":
        raise ValueError(f"libgla runs on the GPU: got a tensor on {t.device}")
    cur = torch.cuda.current_device()
    if t.device.index != cur:
        raise ValueError(f"tensors must be on the current device cuda:{cur}, got {t.device}")
    return t.device


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s, ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocate on the call's stream (a no-op when it is the current one)."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _check(t, name, shape, dtype, device):
    if t.device != device or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _check_tok(t, name, shape, dtype, device):
    """A token-major [B, T, H, d] tensor: packed heads and features, any batch/token strides."""
    if t.device != device or t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected {dtype} {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    _, _, H, d = shape
    if t.numel() > 0 and (t.stride(3) != 1 or (H > 1 and t.stride(2) != d)):
        raise ValueError(f"{name}: heads and features must be packed (strides [..., {d}, 1]), got {t.stride()}")


def _strides(**tensors) -> Strides:
    """Batch and token strides of [B, T, H, d] tensors; a dimension of size 1 is never
    stepped over, so its stride is left packed (0)."""
    s = Strides()
    for name, t in tensors.items():
        if t is not None and t.numel() > 0:
            getattr(s, name).batch = t.stride(0) if t.shape[0] > 1 else 0
            getattr(s, name).token = t.stride(1) if t.shape[1] > 1 else 0
    return s


def _plan(plan):
    """A gla_plan from a dict {segments, chain, psub, scan} (missing keys: the library's choice)."""
    if plan is None:
        return None
    return Plan(int(plan.get("segments", 0)), int(plan.get("chain", -1)), int(plan.get("psub", 0)),
                int(plan.get("scan", -1)))


def _ref(p):
    return None if p is None else ctypes.byref(p)


def _raise(st, where):
    if st != GLA_OK:
        raise GlaError(st, where)


def plan_resolve(dtype: int, B, T, H, dk, dv, chunk, plan=None) -> dict:
    """The launch plan the library runs for these sizes (with an optional hint dict)."""
    out = Plan()
    _raise(load().gla_plan_resolve(dtype, B, T, H, dk, dv, chunk, _ref(_plan(plan)), ctypes.byref(out)),
           "gla_plan_resolve")
    return {"segments": out.segments, "chain": out.chain, "psub": out.psub, "scan": out.scan}


def fwd_workspace_bytes(dtype: int, B, T, H, dk, dv, chunk, plan=None) -> int:
    lib = load()
    if plan is None:
        return int(lib.gla_fwd_workspace_bytes(dtype, B, T, H, dk, dv, chunk))
    return int(lib.gla_fwd_workspace_bytes_planned(dtype, B, T, H, dk, dv, chunk, ctypes.byref(_plan(plan))))


def bwd_workspace_bytes(dtype: int, B, T, H, dk, dv, chunk, saved_states=False, plan=None) -> int:
    lib = load()
    if plan is None:
        fn = lib.gla_bwd_states_workspace_bytes if saved_states else lib.gla_bwd_workspace_bytes
        return int(fn(dtype, B, T, H, dk, dv, chunk))
    return int(lib.gla_bwd_workspace_bytes_planned(dtype, B, T, H, dk, dv, chunk, int(bool(saved_states)),
                                                   ctypes.byref(_plan(plan))))


def _workspace(need, workspace, dev):
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    return workspace, (0 if workspace is None else workspace.numel() * workspace.element_size())


def _fwd_common(q, k, v, lam, S0, g, name):
    B, T, H, dk = q.shape
    dv = v.shape[3]
    dev = _device(q)
    _check_tok(q, "q", (B, T, H, dk), q.dtype, dev)
    _check_tok(k, "k", (B, T, H, dk), q.dtype, dev)
    _check_tok(v, "v", (B, T, H, dv), q.dtype, dev)
    if g is not None:
        _check_tok(g, "g", (B, T, H, dv), q.dtype, dev)
    _check(lam, "lambda", (H,), torch.float32, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    return B, T, H, dk, dv, dev


def _final_state(S_final, B, H, dk, dv, dev):
    if S_final is True:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_final is False:
        S_final = None
    if S_final is not None:
        _check(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    return S_final


def _fwd_call(q, k, v, lam, S0, scale, chunk, o, S_final, states, g, ep, workspace, stream, plan, where):
    lib = load()
    B, T, H, dk, dv, dev = _fwd_common(q, k, v, lam, S0, g, where)
    s, sp = _stream(stream)
    dt = _dt(q)
    with _on(stream):
        if o is None:
            o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
        _check_tok(o, "y" if ep is not None else "o", (B, T, H, dv), q.dtype, dev)
        S_final = _final_state(S_final, B, H, dk, dv, dev)
        if states is True:
            nc = (T + chunk - 1) // chunk
            states = torch.empty((B, H, nc, dk, dv), dtype=q.dtype, device=dev)
        workspace, ws_bytes = _workspace(fwd_workspace_bytes(dt, B, T, H, dk, dv, chunk, plan), workspace, dev)
    st = _strides(q=q, k=k, v=v, o=o, g=g)
    if plan is not None:
        rc = lib.gla_fwd_chunked_planned(dt, B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(S0),
                                         float(scale), _ptr(o), _ptr(S_final), _ptr(states), _ptr(g), ep,
                                         ctypes.byref(st), ctypes.byref(_plan(plan)), _ptr(workspace), ws_bytes, sp)
    elif states is not None:
        rc = lib.gla_fwd_chunked_states(dt, B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(S0),
                                        float(scale), _ptr(o), _ptr(S_final), _ptr(states), ctypes.byref(st),
                                        _ptr(workspace), ws_bytes, sp)
    elif ep is not None:
        rc = lib.gla_fwd_chunked_epilogue(dt, B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(S0),
                                          float(scale), _ptr(g), ep, _ptr(o), _ptr(S_final), ctypes.byref(st),
                                          _ptr(workspace), ws_bytes, sp)
    else:
        rc = lib.gla_fwd_chunked(dt, B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(S0),
                                 float(scale), _ptr(o), _ptr(S_final), ctypes.byref(st), _ptr(workspace), ws_bytes,
                                 sp)
    _raise(rc, where)
    return o, S_final, states


def fwd_chunked(q, k, v, lam, S0=None, scale=1.0, chunk=128, o=None, S_final=True, workspace=None, stream=None,
                plan=None):
    """o, S_final = gla_fwd_chunked(...).  S_final=False skips the final state; a tensor
    passed as `o`/`S_final` is written in place.  `plan` (dict, tests and sweeps) runs
    gla_fwd_chunked_planned with that launch plan."""
    o, S_final, _ = _fwd_call(q, k, v, lam, S0, scale, chunk, o, S_final, None, None, None, workspace, stream, plan,
                              "gla_fwd_chunked")
    return o, S_final


def fwd_chunked_noalloc(q, k, v, lam, o, S_final=None, S0=None, scale=1.0, chunk=128, stream=None):
    """gla_fwd_chunked_noalloc: the forward with its workspace in the library's fixed
    per-GPU scratch array (no allocation in the call; outputs are the caller's)."""
    lib = load()
    B, T, H, dk, dv, dev = _fwd_common(q, k, v, lam, S0, None, "gla_fwd_chunked_noalloc")
    _check_tok(o, "o", (B, T, H, dv), q.dtype, dev)
    if S_final is not None:
        _check(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    _, sp = _stream(stream)
    st = _strides(q=q, k=k, v=v, o=o)
    _raise(lib.gla_fwd_chunked_noalloc(_dt(q), B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(lam),
                                       _ptr(S0), float(scale), _ptr(o), _ptr(S_final), ctypes.byref(st), sp),
           "gla_fwd_chunked_noalloc")
    return o, S_final


def fwd_chunked_states(q, k, v, lam, S0=None, scale=1.0, chunk=128, S_final=True, workspace=None, stream=None,
                       plan=None):
    """o, S_final, states = the forward, also saving every chunk's start state for the backward."""
    return _fwd_call(q, k, v, lam, S0, scale, chunk, None, S_final, True, None, None, workspace, stream, plan,
                     "gla_fwd_chunked_states")


def _bwd_call(q, k, v, lam, d_o, states, S0, dS_final, scale, chunk, dlambda, dS0, workspace, stream, plan, where,
              grads=None):
    lib = load()
    B, T, H, dk = q.shape
    dv = v.shape[3]
    dev = _device(q)
    for t, name, shape in ((q, "q", (B, T, H, dk)), (k, "k", (B, T, H, dk)), (v, "v", (B, T, H, dv)),
                           (d_o, "do", (B, T, H, dv))):
        _check_tok(t, name, shape, q.dtype, dev)
    if states is not None:
        nc = (T + chunk - 1) // chunk
        _check(states, "states", (B, H, nc, dk, dv), q.dtype, dev)
    _check(lam, "lambda", (H,), torch.float32, dev)
    for t, name in ((S0, "S0"), (dS_final, "dS_final")):
        if t is not None:
            _check(t, name, (B, H, dk, dv), torch.float32, dev)
    s, sp = _stream(stream)
    dt = _dt(q)
    with _on(stream):
        if grads is None:
            grads = (torch.empty((B, T, H, dk), dtype=q.dtype, device=dev),
                     torch.empty((B, T, H, dk), dtype=q.dtype, device=dev),
                     torch.empty((B, T, H, dv), dtype=q.dtype, device=dev))
        dq, dkk, dvv = grads
        for t, name, shape in ((dq, "dq", (B, T, H, dk)), (dkk, "dk", (B, T, H, dk)), (dvv, "dv", (B, T, H, dv))):
            _check_tok(t, name, shape, q.dtype, dev)
        dl = torch.empty(H, dtype=torch.float32, device=dev) if dlambda else None
        ds0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if dS0 else None
        need = bwd_workspace_bytes(dt, B, T, H, dk, dv, chunk, states is not None, plan)
        workspace, ws_bytes = _workspace(need, workspace, dev)
    st = _strides(q=q, k=k, v=v, d_o=d_o, dq=dq, dk=dkk, dv=dvv)
    args = (dt, B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(S0), float(scale), _ptr(d_o),
            _ptr(dS_final))
    outs = (_ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dl), _ptr(ds0), ctypes.byref(st))
    if plan is not None:
        rc = lib.gla_bwd_chunked_planned(*args, _ptr(states), *outs, ctypes.byref(_plan(plan)), _ptr(workspace),
                                         ws_bytes, sp)
    elif states is not None:
        rc = lib.gla_bwd_chunked_states(*args, _ptr(states), *outs, _ptr(workspace), ws_bytes, sp)
    else:
        rc = lib.gla_bwd_chunked(*args, *outs, _ptr(workspace), ws_bytes, sp)
    _raise(rc, where)
    return dq, dkk, dvv, dl, ds0


def bwd_chunked(q, k, v, lam, d_o, S0=None, dS_final=None, scale=1.0, chunk=128, dlambda=True, dS0=True,
                workspace=None, stream=None, plan=None, grads=None):
    """dq, dk, dv, dlambda ([H] or None), dS0 ([B,H,dk,dv] or None) = gla_bwd_chunked(...).
    `grads` = (dq, dk, dv) tensors (views allowed) to write in place."""
    return _bwd_call(q, k, v, lam, d_o, None, S0, dS_final, scale, chunk, dlambda, dS0, workspace, stream, plan,
                     "gla_bwd_chunked", grads)


def bwd_chunked_states(q, k, v, lam, d_o, states, S0=None, dS_final=None, scale=1.0, chunk=128,
                       dlambda=True, dS0=True, workspace=None, stream=None, plan=None, grads=None):
    """dq, dk, dv, dlambda, dS0 from the chunk start states saved by fwd_chunked_states."""
    return _bwd_call(q, k, v, lam, d_o, states, S0, dS_final, scale, chunk, dlambda, dS0, workspace, stream, plan,
                     "gla_bwd_chunked_states", grads)


def decode_step(q, k, v, lam, S, scale=1.0, o=None, stream=None):
    """In place on S: S <- lam S + k v^T, o = scale S^T q.  Returns o."""
    lib = load()
    N, H, dk = q.shape
    dv = v.shape[2]
    dev = _device(q)
    _check(q, "q", (N, H, dk), q.dtype, dev)
    _check(k, "k", (N, H, dk), q.dtype, dev)
    _check(v, "v", (N, H, dv), q.dtype, dev)
    _check(lam, "lambda", (H,), torch.float32, dev)
    _check(S, "S", (N, H, dk, dv), torch.float32, dev)
    s, sp = _stream(stream)
    with _on(stream):
        if o is None:
            o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _check(o, "o", (N, H, dv), q.dtype, dev)
    _raise(lib.gla_decode_step(_dt(q), N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(S), float(scale),
                               _ptr(o), sp), "gla_decode_step")
    return o


def decode_step_pool(q, k, v, lam, pool, slots, scale=1.0, o=None, stream=None):
    """Decode on a page pool: row n uses page slots[n] of pool [P, H, dk, dv] (in place);
    a slot outside [0, P) (-1: padding row) gives a zero output row.  Returns o."""
    lib = load()
    N, H, dk = q.shape
    dv = v.shape[2]
    P = pool.shape[0]
    dev = _device(q)
    _check(q, "q", (N, H, dk), q.dtype, dev)
    _check(k, "k", (N, H, dk), q.dtype, dev)
    _check(v, "v", (N, H, dv), q.dtype, dev)
    _check(lam, "lambda", (H,), torch.float32, dev)
    _check(pool, "pool", (P, H, dk, dv), torch.float32, dev)
    _check(slots, "slots", (N,), torch.int32, dev)
    s, sp = _stream(stream)
    with _on(stream):
        if o is None:
            o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _check(o, "o", (N, H, dv), q.dtype, dev)
    _raise(lib.gla_decode_step_pool(_dt(q), N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(pool), P,
                                    _ptr(slots), float(scale), _ptr(o), sp), "gla_decode_step_pool")
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
    dev = _device(q)
    _check(q, "q", lead + (H, dk), q.dtype, dev)
    _check(k, "k", lead + (H, dk), q.dtype, dev)
    for t, name in ((v, "v"), (o, "o"), (g, "g")):
        _check(t, name, lead + (H, dv), q.dtype, dev)
    s, sp = _stream(stream)
    with _on(stream):
        if y is None:
            y = torch.empty(lead + (H, dv), dtype=q.dtype, device=dev)
    _check(y, "y", lead + (H, dv), q.dtype, dev)
    p, _keep = _epi_params(H, dk, dv, aug_a, norm_w, head_tier, eps, dev)
    _raise(lib.gla_mixer_epilogue(_dt(q), M, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(g),
                                  ctypes.byref(p), _ptr(y), sp), "gla_mixer_epilogue")
    return y


def decode_step_epilogue(q, k, v, g, lam, S, norm_w, head_tier, aug_a=None, eps=1e-6, scale=1.0,
                         slots=None, y=None, stream=None):
    """Decode step with the epilogue fused: S (pages [N, H, dk, dv], or a pool [P, H, dk, dv]
    indexed by int32 `slots`) is updated in place; returns y [N, H, dv]."""
    lib = load()
    N, H, dk = q.shape
    dv = v.shape[2]
    dev = _device(q)
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
    s, sp = _stream(stream)
    with _on(stream):
        if y is None:
            y = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _check(y, "y", (N, H, dv), q.dtype, dev)
    p, _keep = _epi_params(H, dk, dv, aug_a, norm_w, head_tier, eps, dev)
    _raise(lib.gla_decode_step_epilogue(_dt(q), N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(lam),
                                        _ptr(S), P, _ptr(slots), float(scale), ctypes.byref(p), _ptr(y), sp),
           "gla_decode_step_epilogue")
    return y


def conv1d_silu(x, w, bias=None, win_in=None, win_out=True, y=None, stream=None):
    """Depth-wise causal conv (width 4) + SiLU: x [B, T, D]; w [D, 4] fp32; bias [D] or None;
    win_in [B, 4, D] fp32 or None (zeros).  Returns (y, win_out): win_out=True allocates the
    window after the last token, False skips it, a tensor (win_in itself allowed) is written."""
    lib = load()
    B, T, D = x.shape
    K = w.shape[1]
    dev = _device(x)
    _check(x, "x", (B, T, D), x.dtype, dev)
    _check(w, "w", (D, K), torch.float32, dev)
    if bias is not None:
        _check(bias, "bias", (D,), torch.float32, dev)
    if win_in is not None:
        _check(win_in, "win_in", (B, K, D), torch.float32, dev)
    s, sp = _stream(stream)
    with _on(stream):
        if win_out is True:
            win_out = torch.empty((B, K, D), dtype=torch.float32, device=dev)
        elif win_out is False:
            win_out = None
        if y is None:
            y = torch.empty_like(x)
    if win_out is not None:
        _check(win_out, "win_out", (B, K, D), torch.float32, dev)
    _check(y, "y", (B, T, D), x.dtype, dev)
    _raise(lib.gla_conv1d_silu(_dt(x), B, T, D, K, _ptr(x), _ptr(w), _ptr(bias), _ptr(win_in), _ptr(y),
                               _ptr(win_out), sp), "gla_conv1d_silu")
    return y, win_out


def conv1d_silu_decode(x, w, bias, win, slots=None, y=None, stream=None):
    """One token per row: x [N, D]; win [N, 4, D] fp32 (or a pool [P, 4, D] indexed by
    int32 `slots`), updated in place.  Returns y [N, D]."""
    lib = load()
    N, D = x.shape
    K = w.shape[1]
    dev = _device(x)
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
    s, sp = _stream(stream)
    with _on(stream):
        if y is None:
            y = torch.empty_like(x)
    _check(y, "y", (N, D), x.dtype, dev)
    _raise(lib.gla_conv1d_silu_decode(_dt(x), N, D, K, _ptr(x), _ptr(w), _ptr(bias), _ptr(win), P, _ptr(slots),
                                      _ptr(y), sp), "gla_conv1d_silu_decode")
    return y


def fwd_chunked_epilogue(q, k, v, lam, g, norm_w, head_tier, aug_a=None, eps=1e-6, S0=None, scale=1.0,
                         chunk=128, y=None, S_final=True, workspace=None, stream=None, plan=None):
    """y, S_final: the forward followed by the mixer epilogue (y in place of o)."""
    H, dk = q.shape[2], q.shape[3]
    dv = v.shape[3]
    dev = _device(q)
    p, _keep = _epi_params(H, dk, dv, aug_a, norm_w, head_tier, eps, dev)
    y, S_final, _ = _fwd_call(q, k, v, lam, S0, scale, chunk, y, S_final, None, g, ctypes.byref(p), workspace, stream,
                              plan, "gla_fwd_chunked_epilogue")
    return y, S_final

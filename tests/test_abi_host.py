"""CPU-only checks of the C ABI: the library loads, exports every symbol that
include/gla.h declares, and rejects invalid arguments on the host before any
HIP call (no device is touched by these calls)."""
import ctypes
import os
import re

import pytest

import gated_linear_attention_simple_amd as gla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(gla_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_loads_and_exports_header_symbols():
    lib = gla.load()
    decl = declared_functions()
    assert "gla_fwd_chunked" in decl and "gla_decode_step" in decl
    for name in decl:
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
    assert set(gla.SYMBOLS) == set(decl)
    assert lib.gla_abi_version() == 4


def test_status_strings():
    for s in range(5):
        assert gla.status_str(s).startswith("GLA_")
    assert "UNKNOWN" in gla.status_str(99)


P = ctypes.c_void_p(16)  # non-null, 16-byte aligned dummy (never dereferenced: validation fails first)
MIS = ctypes.c_void_p(18)


def fwd(dtype=1, B=1, T=256, H=16, dk=96, dv=192, C=128, q=P, k=P, v=P, lam=P, S0=None, o=P, Sf=None,
        ws=None, wsb=0, st=None):
    return gla.load().gla_fwd_chunked(dtype, B, T, H, dk, dv, C, q, k, v, lam, S0, 1.0, o, Sf,
                                      None if st is None else ctypes.byref(st), ws, wsb, None)


def test_fwd_rejects_bad_arguments_before_touching_the_device():
    E = gla
    assert fwd(dtype=7) == E.GLA_ERR_INVALID_ARG
    assert fwd(B=0) == E.GLA_ERR_INVALID_ARG
    assert fwd(T=-1) == E.GLA_ERR_INVALID_ARG
    assert fwd(H=0) == E.GLA_ERR_INVALID_ARG
    assert fwd(dk=64) == E.GLA_ERR_UNSUPPORTED
    assert fwd(C=512) == E.GLA_ERR_UNSUPPORTED
    assert fwd(C=96) == E.GLA_ERR_UNSUPPORTED
    assert fwd(dtype=0, C=256) == E.GLA_ERR_UNSUPPORTED          # 256-token chunks: bf16 only
    assert fwd(dtype=0, C=128) == E.GLA_ERR_UNSUPPORTED          # fp32 stops at chunk 64
    assert fwd(dtype=1, dk=16, dv=32, C=32) == E.GLA_ERR_UNSUPPORTED
    assert fwd(q=None) == E.GLA_ERR_INVALID_ARG
    assert fwd(v=MIS) == E.GLA_ERR_INVALID_ARG
    assert fwd(lam=None) == E.GLA_ERR_INVALID_ARG
    assert fwd(S0=MIS) == E.GLA_ERR_INVALID_ARG
    assert fwd(B=70000, T=1) == E.GLA_ERR_UNSUPPORTED               # grid limit on B*H


def test_fwd_workspace_contract():
    lib = gla.load()
    need = lib.gla_fwd_workspace_bytes(1, 1, 2048, 16, 96, 192, 128)
    assert need > 0 and need % (96 * 192 * 4) == 0
    assert fwd(T=2048) == gla.GLA_ERR_WORKSPACE
    assert fwd(T=2048, ws=P, wsb=need - 1) == gla.GLA_ERR_WORKSPACE
    assert lib.gla_fwd_workspace_bytes(1, 1, 2048, 16, 64, 192, 128) == 0   # unsupported -> 0
    # a large batch fills the GPU without splitting the sequence: no workspace
    assert lib.gla_fwd_workspace_bytes(1, 32, 2048, 16, 96, 192, 128) == 0


def test_decode_rejects_bad_arguments():
    lib = gla.load()
    d = lambda dtype=1, N=4, H=16, dk=96, dv=192, q=P, S=P: lib.gla_decode_step(
        dtype, N, H, dk, dv, q, P, P, P, S, 1.0, P, None)
    assert d(dtype=5) == gla.GLA_ERR_INVALID_ARG
    assert d(N=-1) == gla.GLA_ERR_INVALID_ARG
    assert d(dk=80) == gla.GLA_ERR_UNSUPPORTED
    assert d(q=None) == gla.GLA_ERR_INVALID_ARG
    assert d(S=MIS) == gla.GLA_ERR_INVALID_ARG
    assert d(N=0, q=None) == gla.GLA_OK        # nothing to do, nothing enqueued


def test_decode_pool_rejects_bad_arguments():
    lib = gla.load()
    d = lambda dtype=1, N=4, H=16, dk=96, dv=192, pool=P, Pn=8, slots=P: lib.gla_decode_step_pool(
        dtype, N, H, dk, dv, P, P, P, P, pool, Pn, slots, 1.0, P, None)
    assert d(dtype=5) == gla.GLA_ERR_INVALID_ARG
    assert d(N=-1) == gla.GLA_ERR_INVALID_ARG
    assert d(Pn=-1) == gla.GLA_ERR_INVALID_ARG
    assert d(dk=80) == gla.GLA_ERR_UNSUPPORTED
    assert d(slots=None) == gla.GLA_ERR_INVALID_ARG
    assert d(slots=MIS) == gla.GLA_ERR_INVALID_ARG
    assert d(pool=None) == gla.GLA_ERR_INVALID_ARG
    assert d(N=0, slots=None) == gla.GLA_OK


def _epi(H=16, n_tiers=4, tiers=None, eps=1e-6, w=P, a=None):
    tiers = [h % n_tiers for h in range(H)] if tiers is None else tiers
    arr = (ctypes.c_int * max(len(tiers), 1))(*tiers)
    val = lambda x: None if x is None else x.value
    return gla.EpilogueParams(val(a), val(w), ctypes.cast(arr, ctypes.POINTER(ctypes.c_int)), n_tiers, eps), arr


def test_mixer_epilogue_rejects_bad_arguments():
    lib = gla.load()

    def e(dtype=1, M=8, H=16, dk=96, dv=192, q=P, g=P, y=P, **kw):
        p, keep = _epi(H=H, **kw)
        return lib.gla_mixer_epilogue(dtype, M, H, dk, dv, q, P, P, P, g, ctypes.byref(p), y, None)

    assert e(dtype=7) == gla.GLA_ERR_INVALID_ARG
    assert e(M=-1) == gla.GLA_ERR_INVALID_ARG
    assert e(dk=64) == gla.GLA_ERR_UNSUPPORTED
    assert e(H=65) == gla.GLA_ERR_UNSUPPORTED
    assert e(tiers=[0] * 15 + [4]) == gla.GLA_ERR_INVALID_ARG      # tier out of range
    assert e(tiers=[-1] + [0] * 15) == gla.GLA_ERR_INVALID_ARG
    assert e(n_tiers=0, tiers=[0] * 16) == gla.GLA_ERR_INVALID_ARG
    assert e(n_tiers=65, tiers=[0] * 16) == gla.GLA_ERR_INVALID_ARG
    assert e(eps=-1.0) == gla.GLA_ERR_INVALID_ARG
    assert e(eps=float("nan")) == gla.GLA_ERR_INVALID_ARG
    assert e(eps=float("inf")) == gla.GLA_ERR_INVALID_ARG
    assert e(w=None) == gla.GLA_ERR_INVALID_ARG
    assert e(w=MIS) == gla.GLA_ERR_INVALID_ARG
    assert e(a=MIS) == gla.GLA_ERR_INVALID_ARG
    assert e(q=None) == gla.GLA_ERR_INVALID_ARG
    assert e(g=MIS) == gla.GLA_ERR_INVALID_ARG
    assert e(y=None) == gla.GLA_ERR_INVALID_ARG
    assert e(M=0, q=None) == gla.GLA_OK
    assert lib.gla_mixer_epilogue(1, 8, 16, 96, 192, P, P, P, P, P, None, P, None) == gla.GLA_ERR_INVALID_ARG


def test_decode_epilogue_rejects_bad_arguments():
    lib = gla.load()

    def d(dtype=1, N=4, H=16, dk=96, dv=192, S=P, Pn=8, slots=None, g=P, y=P, **kw):
        p, keep = _epi(H=H, **kw)
        return lib.gla_decode_step_epilogue(dtype, N, H, dk, dv, P, P, P, g, P, S, Pn, slots, 1.0,
                                            ctypes.byref(p), y, None)

    assert d(dtype=2) == gla.GLA_ERR_INVALID_ARG
    assert d(N=-3) == gla.GLA_ERR_INVALID_ARG
    assert d(dk=32) == gla.GLA_ERR_UNSUPPORTED
    assert d(H=70) == gla.GLA_ERR_UNSUPPORTED
    assert d(slots=P, Pn=-1) == gla.GLA_ERR_INVALID_ARG
    assert d(slots=MIS) == gla.GLA_ERR_INVALID_ARG
    assert d(S=None) == gla.GLA_ERR_INVALID_ARG
    assert d(slots=P, Pn=0, S=None, N=0) == gla.GLA_OK
    assert d(g=None) == gla.GLA_ERR_INVALID_ARG
    assert d(y=MIS) == gla.GLA_ERR_INVALID_ARG
    assert d(tiers=[9] * 16) == gla.GLA_ERR_INVALID_ARG
    assert d(N=0, g=None) == gla.GLA_OK


def test_conv_rejects_bad_arguments():
    lib = gla.load()

    def c(dtype=1, B=2, T=10, D=3072, K=4, x=P, w=P, bias=None, wi=None, y=P, wo=None):
        return lib.gla_conv1d_silu(dtype, B, T, D, K, x, w, bias, wi, y, wo, None)

    assert c(dtype=4) == gla.GLA_ERR_INVALID_ARG
    assert c(B=-1) == gla.GLA_ERR_INVALID_ARG
    assert c(T=-2) == gla.GLA_ERR_INVALID_ARG
    assert c(K=3) == gla.GLA_ERR_UNSUPPORTED
    assert c(D=3070) == gla.GLA_ERR_UNSUPPORTED
    assert c(w=None) == gla.GLA_ERR_INVALID_ARG
    assert c(x=MIS) == gla.GLA_ERR_INVALID_ARG
    assert c(bias=MIS) == gla.GLA_ERR_INVALID_ARG
    assert c(wo=MIS) == gla.GLA_ERR_INVALID_ARG
    assert c(B=0, x=None) == gla.GLA_OK
    assert c(T=0, x=None, y=None) == gla.GLA_OK          # nothing to write
    assert c(B=65536, T=1, D=8) == gla.GLA_ERR_UNSUPPORTED            # grid limits
    assert c(B=1, T=2_097_121, D=8) == gla.GLA_ERR_UNSUPPORTED

    def d(dtype=1, N=3, D=3072, K=4, x=P, w=P, win=P, Pn=0, slots=None, y=P):
        return lib.gla_conv1d_silu_decode(dtype, N, D, K, x, w, None, win, Pn, slots, y, None)

    assert d(N=-1) == gla.GLA_ERR_INVALID_ARG
    assert d(K=5) == gla.GLA_ERR_UNSUPPORTED
    assert d(win=None) == gla.GLA_ERR_INVALID_ARG
    assert d(slots=P, Pn=-1) == gla.GLA_ERR_INVALID_ARG
    assert d(slots=MIS, Pn=4) == gla.GLA_ERR_INVALID_ARG
    assert d(y=None) == gla.GLA_ERR_INVALID_ARG
    assert d(N=0, x=None) == gla.GLA_OK
    assert d(N=65536, D=8) == gla.GLA_ERR_UNSUPPORTED


def test_saved_state_entry_points_validate():
    lib = gla.load()
    assert lib.gla_fwd_states_bytes(1, 8, 2048, 16, 96, 192, 128) == 8 * 16 * 16 * 96 * 192 * 2
    assert lib.gla_fwd_states_bytes(0, 1, 33, 2, 16, 32, 32) == 1 * 2 * 2 * 16 * 32 * 4
    assert lib.gla_fwd_states_bytes(1, 1, 100, 16, 80, 192, 128) == 0

    def f(dtype=1, B=1, T=256, dk=96, dv=192, C=128, states=P, ws=P, wsb=1 << 30):
        return lib.gla_fwd_chunked_states(dtype, B, T, 16, dk, dv, C, P, P, P, P, None, 1.0, P, None, states, None,
                                          ws, wsb, None)

    assert f(dtype=0) == gla.GLA_ERR_UNSUPPORTED           # fp32 96/192: no backward, so no saved states
    assert f(C=512) == gla.GLA_ERR_UNSUPPORTED
    assert f(states=None) == gla.GLA_ERR_INVALID_ARG
    assert f(states=MIS) == gla.GLA_ERR_INVALID_ARG
    assert f(ws=None) == gla.GLA_ERR_WORKSPACE

    def b(states=P, ws=None, wsb=0, T=256):
        return lib.gla_bwd_chunked_states(1, 1, T, 16, 96, 192, 128, P, P, P, P, None, 1.0, P, None, states, P, P, P,
                                          None, None, None, ws, wsb, None)

    assert b(states=None) == gla.GLA_ERR_INVALID_ARG
    assert b() == gla.GLA_ERR_WORKSPACE
    # the saved-state backward's workspace holds no state snapshots of its own
    full = lib.gla_bwd_workspace_bytes(1, 8, 2048, 16, 96, 192, 128)
    saved = lib.gla_bwd_states_workspace_bytes(1, 8, 2048, 16, 96, 192, 128)
    assert full - saved == 8 * 16 * 16 * 96 * 192 * 2
    # (one byte short of the call's own size: rejected before any launch)
    assert b(ws=P, wsb=lib.gla_bwd_states_workspace_bytes(1, 1, 256, 16, 96, 192, 128) - 1) == gla.GLA_ERR_WORKSPACE


def bwd(dtype=1, B=1, T=256, H=16, dk=96, dv=192, C=128, q=P, k=P, v=P, lam=P, S0=None, do=P, dST=None,
        dq=P, dk_=P, dv_=P, dl=None, dS0=None, ws=None, wsb=0, st=None):
    return gla.load().gla_bwd_chunked(dtype, B, T, H, dk, dv, C, q, k, v, lam, S0, 1.0, do, dST, dq, dk_, dv_,
                                      dl, dS0, None if st is None else ctypes.byref(st), ws, wsb, None)


def test_bwd_rejects_bad_arguments_before_touching_the_device():
    E = gla
    assert bwd(dtype=3) == E.GLA_ERR_INVALID_ARG
    assert bwd(T=-5) == E.GLA_ERR_INVALID_ARG
    assert bwd(dk=64) == E.GLA_ERR_UNSUPPORTED
    assert bwd(dtype=0) == E.GLA_ERR_UNSUPPORTED                  # fp32 backward: tiny shape only
    assert bwd(dtype=0, dk=16, dv=32, C=64) == E.GLA_ERR_UNSUPPORTED
    assert bwd(C=512) == E.GLA_ERR_UNSUPPORTED
    assert bwd(dtype=0, dk=16, dv=32, C=256) == E.GLA_ERR_UNSUPPORTED   # 256-token chunks: bf16 only
    assert bwd(do=None) == E.GLA_ERR_INVALID_ARG
    assert bwd(dv_=MIS) == E.GLA_ERR_INVALID_ARG
    assert bwd(dl=MIS) == E.GLA_ERR_INVALID_ARG
    assert bwd(dST=MIS) == E.GLA_ERR_INVALID_ARG
    need = gla.load().gla_bwd_workspace_bytes(1, 1, 256, 16, 96, 192, 128)
    assert need > 0
    assert bwd() == E.GLA_ERR_WORKSPACE
    assert bwd(ws=P, wsb=need - 1) == E.GLA_ERR_WORKSPACE


def test_strides_validated_on_the_host():
    """gla_strides: zero fields mean packed; token strides below H*d, not a multiple of
    16 bytes or at 2^22 and above are rejected, as are misaligned batch strides and
    output batch strides that make sequences overlap -- all before any HIP call."""
    E = gla

    def st(**kw):
        s = gla.Strides()
        for name, (b, t) in kw.items():
            getattr(s, name).batch, getattr(s, name).token = b, t
        return s

    fused = 16 * (2 * 96 + 2 * 192)                 # the fused QKVG projection's width
    ok = st(q=(256 * fused, fused), k=(256 * fused, fused), v=(256 * fused, fused), o=(0, 0))
    # with no workspace the call gets past the stride checks to the workspace check
    assert fwd(B=2, T=256, st=ok) == E.GLA_ERR_WORKSPACE
    assert fwd(st=st(q=(0, 16 * 96 - 8))) == E.GLA_ERR_INVALID_ARG          # token < H dk
    assert fwd(st=st(k=(0, 16 * 96 + 4))) == E.GLA_ERR_INVALID_ARG          # not 16 bytes
    assert fwd(st=st(v=(0, 1 << 22))) == E.GLA_ERR_INVALID_ARG              # too large
    assert fwd(st=st(v=(-8, 0))) == E.GLA_ERR_INVALID_ARG
    assert fwd(st=st(q=(12, 0))) == E.GLA_ERR_INVALID_ARG                   # batch not 16 bytes
    assert fwd(B=2, st=st(o=(255 * 16 * 192, 0))) == E.GLA_ERR_INVALID_ARG  # output sequences overlap
    assert fwd(B=2, st=st(q=(8, 0))) == E.GLA_ERR_WORKSPACE                 # overlapping inputs are fine
    assert bwd(st=st(dq=(0, 16 * 96 - 8))) == E.GLA_ERR_INVALID_ARG
    assert bwd(B=2, st=st(dv=(16 * 192, 0))) == E.GLA_ERR_INVALID_ARG
    assert bwd(st=st(d_o=(0, 3))) == E.GLA_ERR_INVALID_ARG


def test_plan_controls_validate_and_resolve():
    lib = gla.load()
    r = lambda **kw: gla.plan_resolve(1, *kw.pop("shape", (8, 2048, 16, 96, 192, 128)), kw or None)
    assert r() == {"segments": 2, "chain": 0, "psub": 2, "scan": 1}       # the training step's plan
    assert r(shape=(1, 2048, 16, 96, 192, 128)) == {"segments": 16, "chain": 1, "psub": 1, "scan": 0}   # layer
    assert r(shape=(1, 65536, 16, 96, 192, 128)) == {"segments": 16, "chain": 0, "psub": 1, "scan": 0}  # 64k
    assert r(chain=0, shape=(1, 2048, 16, 96, 192, 128))["chain"] == 0
    # a requested chain runs up to 64 chunks; a longer sequence keeps the segment form
    assert r(chain=1, shape=(1, 8192, 16, 96, 192, 128))["chain"] == 1
    assert r(chain=1, shape=(1, 8193, 16, 96, 192, 128))["chain"] == 0
    assert r(chain=1, shape=(1, 4096, 16, 96, 192, 64))["chain"] == 1
    assert r(psub=1) == {"segments": 2, "chain": 0, "psub": 1, "scan": 1}
    assert r(scan=0)["scan"] == 0
    assert r(segments=4, scan=1)["scan"] == 0          # six local states before the last segment: a scan
    assert r(segments=8)["segments"] == 8
    assert r(segments=5)["segments"] == 4          # 16 chunks in segments of 4
    # 256-token chunks run in the chain form whatever the hint (their tiles exceed LDS)
    assert r(shape=(8, 2048, 16, 96, 192, 256))["chain"] == 1
    assert r(chain=0, shape=(1, 300, 16, 96, 192, 256))["chain"] == 1
    assert lib.gla_fwd_workspace_bytes(1, 2, 1000, 16, 96, 192, 256) == 2 * 16 * 4 * 96 * 192 * 2
    for bad in ({"segments": 17}, {"chain": 2}, {"psub": 2}, {"segments": -1}, {"scan": 2}):
        with pytest.raises(gla.GlaError):
            r(**bad)
        assert lib.gla_fwd_workspace_bytes_planned(1, 8, 2048, 16, 96, 192, 128,
                                                   ctypes.byref(gla._plan(bad))) == 0
    # planned workspace sizes match the plain ones when nothing is fixed
    assert gla.fwd_workspace_bytes(1, 1, 2048, 16, 96, 192, 128, plan={}) == \
        lib.gla_fwd_workspace_bytes(1, 1, 2048, 16, 96, 192, 128)
    assert gla.bwd_workspace_bytes(1, 8, 2048, 16, 96, 192, 64, saved_states=True, plan={}) == \
        lib.gla_bwd_states_workspace_bytes(1, 8, 2048, 16, 96, 192, 64)


def test_noalloc_forward_limits_checked_on_the_host():
    """gla_fwd_chunked_noalloc: the usual argument errors, and a size whose workspace
    exceeds the fixed scratch array is refused with GLA_ERR_WORKSPACE, all before any
    HIP call (no device is touched here)."""
    lib = gla.load()

    def n(dtype=1, B=1, T=256, H=16, C=128, q=P, o=P):
        return lib.gla_fwd_chunked_noalloc(dtype, B, T, H, 96, 192, C, q, P, P, P, None, 1.0, o, None, None, None)

    assert n(dtype=9) == gla.GLA_ERR_INVALID_ARG
    assert n(C=512) == gla.GLA_ERR_UNSUPPORTED
    assert n(q=None) == gla.GLA_ERR_INVALID_ARG
    assert n(o=MIS) == gla.GLA_ERR_INVALID_ARG
    # B=6, H=20, T=2048: four segments, 39.8 MB of workspace > 32 MiB
    need = lib.gla_fwd_workspace_bytes(1, 6, 2048, 20, 96, 192, 128)
    assert need > gla.NOALLOC_WORKSPACE_MAX
    assert n(B=6, T=2048, H=20) == gla.GLA_ERR_WORKSPACE
    # the workloads it is for fit: the layer, the training width, the 64k prefill
    for B, T in ((1, 2048), (8, 2048), (1, 65536)):
        assert 0 < lib.gla_fwd_workspace_bytes(1, B, T, 16, 96, 192, 128) <= gla.NOALLOC_WORKSPACE_MAX


def test_binding_rejects_cpu_tensors_before_the_library():
    """A host tensor handed to a GPU kernel would fault the device: the binding raises
    before any library call."""
    import torch
    q = torch.zeros(1, 4, 16, 96, dtype=torch.bfloat16)
    v = torch.zeros(1, 4, 16, 192, dtype=torch.bfloat16)
    lam = torch.full((16,), 0.9)
    with pytest.raises(ValueError, match="GPU"):
        gla.fwd_chunked(q, q, v, lam)
    with pytest.raises(ValueError, match="GPU"):
        gla.bwd_chunked(q, q, v, lam, v)
    with pytest.raises(ValueError, match="GPU"):
        gla.decode_step(q[:, 0], q[:, 0], v[:, 0], lam, torch.zeros(1, 16, 96, 192))
    with pytest.raises(ValueError, match="GPU"):
        gla.conv1d_silu(torch.zeros(1, 4, 3072, dtype=torch.bfloat16), torch.zeros(3072, 4))


def test_bwd_workspace_holds_both_snapshot_sets():
    lib = gla.load()
    B, T, H, C = 8, 2048, 16, 128
    need = lib.gla_bwd_workspace_bytes(1, B, T, H, 96, 192, C)
    snaps = 2 * B * H * (T // C) * 96 * 192 * 2
    assert snaps <= need <= snaps + 16 * 1024 * 1024


def _excluded(rel, patterns):
    """tar-style exclusion: './x' anchors at the top, other patterns match any path component run."""
    import fnmatch
    parts = rel.split("/")
    for p in patterns:
        if p.startswith("./"):
            anchored = p[2:].rstrip("/")
            if rel == anchored or rel.startswith(anchored + "/"):
                return True
        elif any(fnmatch.fnmatch("/".join(parts[i:]), p) or fnmatch.fnmatch(parts[i], p) for i in range(len(parts))):
            return True
    return False


def test_gpu_snapshot_keeps_what_gpu_runs_load():
    """Files the GPU tests, smoke() and bench.py read (the built library, its sources, the
    committed counter summaries, the golden fixtures, the input generator) must not be
    listed in .gpurunignore, or a GPU run would go without them."""
    path = os.path.join(ROOT, ".gpurunignore")
    if not os.path.exists(path):
        return
    patterns = [l.strip() for l in open(path) if l.strip() and not l.startswith("#")]
    needed = ["gated_linear_attention_simple_amd/libgla.so", "profiles/counters.json", "bench.py",
              "__graft_entry__.py", "gla_inputs.py", "include/gla.h"]
    csrc = os.path.join(ROOT, "gated_linear_attention_simple_amd", "csrc")
    needed += [f"gated_linear_attention_simple_amd/csrc/{f}" for f in os.listdir(csrc)]
    needed += [f"tests/golden/{f}" for f in os.listdir(os.path.join(ROOT, "tests", "golden"))]
    needed += [f"tests/{f}" for f in os.listdir(os.path.join(ROOT, "tests")) if f.endswith(".py")]
    for rel in needed:
        assert not _excluded(rel, patterns), f"{rel} is excluded from GPU runs by .gpurunignore"
    # the check itself catches the pattern that excluded the counter summaries before
    assert _excluded("profiles/counters.json", ["./profiles"])

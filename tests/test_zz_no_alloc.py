"""gla_fwd_chunked_noalloc (the forward for callers that cannot allocate: its workspace
is the library's fixed per-GPU scratch array) against gla_fwd_chunked, through the C
ABI: three calls in a row on the same GPU, each smaller than the one before, so every
call runs over scratch contents the previous call left.  The two entry points run the
same kernels on the same plan, so outputs must agree bit for bit (stronger than the
oracle tolerance); the first call is also checked against the oracle."""
import ctypes
import sys

import pytest
import torch

import gated_linear_attention_simple_amd as gla
import gla_inputs as gi
import oracle
from parity_util import assert_close, f64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _noalloc(x, chunk, o, S):
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[3]
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    return gla.load().gla_fwd_chunked_noalloc(
        gla.GLA_BF16, B, T, H, dk, dv, chunk, p(x["q"]), p(x["k"]), p(x["v"]), p(x["lam"]), p(x["S0"]),
        ctypes.c_float(x["scale"]), p(o), p(S), None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


# largest first: the training width (two segments, 28.3 MB of scratch), the Laplace layer
# (tiled chain, 9.4 MB), a ragged two-sequence case at chunk 64 (three segments), and
# 256-token chunks (tiled chain, 2.4 MB)
CALLS = [(2, 8, 2048, 128, 0.0), (1, 1, 2048, 128, 0.01), (1, 2, 700, 64, 0.01), (1, 2, 500, 256, 0.01)]


def test_noalloc_forward_matches_the_workspace_forward():
    for i, (wi, B, T, chunk, s0) in enumerate(CALLS):
        w = gi.workloads()[wi]
        x = gi.fwd_inputs(w, DEV, 8100 + i, B=B, T=T, s0_var=s0)
        need = gla.fwd_workspace_bytes(gla.GLA_BF16, B, T, 16, 96, 192, chunk)
        assert 0 < need <= gla.NOALLOC_WORKSPACE_MAX
        _say(f"noalloc call {i}: B={B} T={T} C={chunk} workspace {need} bytes")
        o = torch.full((B, T, 16, 192), float("nan"), dtype=torch.bfloat16, device=DEV)
        S = torch.full((B, 16, 96, 192), float("nan"), device=DEV)
        assert _noalloc(x, chunk, o, S) == gla.GLA_OK
        o_ref, S_ref = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"], chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"call {i}: o differs from gla_fwd_chunked"
        assert torch.equal(S, S_ref), f"call {i}: S_final differs from gla_fwd_chunked"
        if i == 1:
            ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), S0=f64(x["S0"]),
                                scale=x["scale"])
            assert_close(f64(o), ro, "bf16", "o")
            assert_close(f64(S), rS, "bf16", "S_final")
        del x, o, S, o_ref, S_ref
        torch.cuda.empty_cache()


def test_noalloc_refuses_oversized_workspace():
    """B=6, H=20, T=2048 would need 39.8 MB of workspace: refused, nothing launched."""
    w = gi.workloads()[1]
    w = gi.Workload(w.name, 6, 2048, 20, 96, 192, 128, "bf16", tuple(gi.laplace_lambdas(20)), w.scale)
    x = gi.fwd_inputs(w, DEV, 8200)
    o = torch.zeros((6, 2048, 20, 192), dtype=torch.bfloat16, device=DEV)
    assert _noalloc(x, 128, o, None) == gla.GLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not o.any()

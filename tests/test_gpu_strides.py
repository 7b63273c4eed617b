"""Strided views at the boundary (gla_strides): q, k, v and the output gate g read in
place from one fused projection output, as the Laplace 3B post's paragraph "QKVG
projection" produces them (width H (2 dk + 2 dv) = 9,216 for the Laplace layer), and
gradients written in place into a fused gradient buffer.

Every case is compared bit for bit with the same call on packed copies (the kernels
only address differently) and with the fp64 oracle.
"""
import sys

import numpy as np
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


def _fused(x, g=None, pad_tokens=0):
    """One [B, T + pad, H (2 dk + 2 dv)] buffer holding q, k, v, g side by side per token
    (pad_tokens extra rows per sequence make the batch stride differ from T * token);
    returns views q, k, v, g of the first T rows and the buffer."""
    q, k, v = x["q"], x["k"], x["v"]
    B, T, H, dk = q.shape
    dv = v.shape[3]
    width = H * (2 * dk + 2 * dv)
    X = torch.full((B, T + pad_tokens, width), float("nan"), dtype=q.dtype, device=DEV)
    offs = [0, H * dk, 2 * H * dk, 2 * H * dk + H * dv, width]
    views = []
    for i, (t, d) in enumerate(((q, dk), (k, dk), (v, dv), (g, dv))):
        view = X[:, :T, offs[i]:offs[i + 1]].view(B, T, H, d) if T > 0 else None
        if t is not None:
            view.copy_(t)
        views.append(view)
    return views, X


FWD_CASES = {
    "layer_chain": (1, 1, 2048, 128, None, {"chain": 1}),
    "layer_segments": (1, 1, 2048, 128, 0.01, {"chain": 0}),
    "ragged_c64": (1, 2, 1000, 64, 0.01, None),
    "ragged_c32": (1, 2, 1000, 32, 0.01, None),
    "ragged_c256": (1, 2, 1000, 256, 0.01, None),
    "train_width": (2, 8, 2048, 128, None, None),
    "fp32_wide_c64": (1, 2, 300, 64, 0.01, None),
    "fp32_tiny": (0, 3, 250, 32, 0.5, None),
}


@pytest.mark.parametrize("case", sorted(FWD_CASES))
def test_forward_reads_fused_projection(case):
    wi, B, T, chunk, s0, plan = FWD_CASES[case]
    w = gi.workloads()[wi]
    if case.startswith("fp32"):
        w = gi.Workload(w.name, w.B, w.T, w.H, w.dk, w.dv, chunk, "f32", w.lambdas, w.scale)
    x = gi.fwd_inputs(w, DEV, 7000 + T + chunk, B=B, T=T, s0_var=s0)
    (q, k, v, _), X = _fused(x)
    # the output into a wider buffer as well: 40 elements of padding after each token
    H, dv = w.H, w.dv
    O = torch.full((B, T, H * dv + 40), float("nan"), dtype=q.dtype, device=DEV)
    o_view = O[..., :H * dv].view(B, T, H, dv)
    _say(f"fused projection {case} B={B} T={T} C={chunk} plan={plan}")
    o_ref, S_ref = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"], chunk=chunk,
                                   plan=plan)
    o, S = gla.fwd_chunked(q, k, v, x["lam"], S0=x["S0"], scale=x["scale"], chunk=chunk, o=o_view, plan=plan)
    torch.cuda.synchronize()
    assert o.data_ptr() == O.data_ptr()
    assert torch.equal(o, o_ref), "strided forward differs from the packed one"
    assert torch.equal(S, S_ref)
    assert bool(torch.isnan(O[..., H * dv:]).all()), "the output's padding was written"
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]),
                        S0=None if x["S0"] is None else f64(x["S0"]), scale=x["scale"])
    assert_close(f64(o), ro, w.dtype, "o")
    assert_close(f64(S), rS, w.dtype, "S_final")


BWD_CASES = {"c128": (1, 2, 1000, 128, False), "c64_saved": (1, 2, 700, 64, True), "train_c128": (2, 8, 2048, 128, True),
             "c32_saved": (1, 2, 900, 32, True), "c256_saved": (1, 2, 1000, 256, True),
             "fp32_tiny": (0, 2, 200, 32, False)}


@pytest.mark.parametrize("case", sorted(BWD_CASES))
def test_backward_fused_in_and_out(case):
    """q, k, v from the fused projection; dq, dk, dv written into one fused gradient buffer
    of the same layout (the projection's input gradient), d_o packed."""
    wi, B, T, chunk, saved = BWD_CASES[case]
    w = gi.workloads()[wi]
    x = gi.fwd_inputs(w, DEV, 7100 + T + chunk, B=B, T=T, with_do=True, with_dS=True, s0_var=0.01)
    (q, k, v, _), X = _fused(x)
    (dq, dk, dv, _), dX = _fused({"q": x["q"] * 0, "k": x["k"] * 0, "v": x["v"] * 0})
    dX.fill_(float("nan"))
    args = dict(S0=x["S0"], dS_final=x["dS"], scale=x["scale"], chunk=chunk)
    _say(f"fused backward {case} B={B} T={T} C={chunk} saved={saved}")
    if saved:
        _, _, st_ref = gla.fwd_chunked_states(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"],
                                              chunk=chunk)
        _, _, st = gla.fwd_chunked_states(q, k, v, x["lam"], S0=x["S0"], scale=x["scale"], chunk=chunk)
        ref = gla.bwd_chunked_states(x["q"], x["k"], x["v"], x["lam"], x["do"], st_ref, **args)
        got = gla.bwd_chunked_states(q, k, v, x["lam"], x["do"], st, grads=(dq, dk, dv), **args)
    else:
        ref = gla.bwd_chunked(x["q"], x["k"], x["v"], x["lam"], x["do"], **args)
        got = gla.bwd_chunked(q, k, v, x["lam"], x["do"], grads=(dq, dk, dv), **args)
    torch.cuda.synchronize()
    if saved:
        assert torch.equal(st, st_ref)
    for a, b, name in zip(got, ref, ("dq", "dk", "dv", "dlambda", "dS0")):
        assert torch.equal(a, b), f"{name}: strided backward differs from the packed one"
    assert got[0].data_ptr() == dX.data_ptr()
    assert bool(torch.isnan(dX[..., -w.H * w.dv:]).all()), "the g slot of the gradient buffer was written"
    r = oracle.bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), f64(x["do"]), S0=f64(x["S0"]),
                   dS_T=f64(x["dS"]), scale=x["scale"])
    for g_, ref_, name in zip(got[:3] + got[4:], (r[0], r[1], r[2], r[4]), ("dq", "dk", "dv", "dS0")):
        assert_close(f64(g_), ref_, w.dtype, name)
    assert_close(f64(got[3]), r[3], w.dtype, "dlambda", batch_axis=None)


@pytest.mark.parametrize("plan,pad", [({"chain": 1}, 0), ({"chain": 0}, 0), ({"chain": 0}, 5), (None, 3)])
def test_forward_epilogue_reads_fused_projection(plan, pad):
    """gla_fwd_chunked_epilogue with q, k, v and the gate g all read from the fused
    projection: the epilogue in the output kernel (tiled chain), and the forward then the
    epilogue pass over rows a token stride apart (segments), also with a batch stride that
    is not T tokens (pad rows per sequence: one pass per sequence)."""
    w = gi.workloads()[1]
    B, T = (1, 2048) if plan is not None and pad == 0 else (3, 700)
    x = gi.fwd_inputs(w, DEV, 7200 + pad, B=B, T=T, s0_var=0.01)
    e = gi.epilogue_inputs(w, DEV, 7200 + pad, (B, T))
    (q, k, v, g), X = _fused(x, e["g"], pad_tokens=pad)
    _say(f"fused epilogue forward B={B} T={T} plan={plan} pad={pad}")
    kw = dict(aug_a=e["aug_a"], S0=x["S0"], scale=x["scale"], chunk=128, plan=plan)
    y_ref, S_ref = gla.fwd_chunked_epilogue(x["q"], x["k"], x["v"], x["lam"], e["g"], e["norm_w"], e["tier"], **kw)
    y, S = gla.fwd_chunked_epilogue(q, k, v, x["lam"], g, e["norm_w"], e["tier"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(S, S_ref)
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), S0=f64(x["S0"]), scale=x["scale"])
    ry = oracle.epilogue(f64(x["q"]), f64(x["k"]), f64(x["v"]), ro, f64(e["g"]), f64(e["aug_a"]), f64(e["norm_w"]),
                         e["tier"])
    assert_close(f64(y), ry, "bf16", "y")
    assert_close(f64(S), rS, "bf16", "S_final")

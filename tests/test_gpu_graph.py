"""HIP-graph capture of the library calls (the bench times the forward as graph replays).

The forward and backward record only kernel launches on the caller's stream (no
allocation, no memset), so they can be captured.  Each replay, with unrelated
eager work and synchronisation between replays, must reproduce the eager
results bit for bit (the kernels are deterministic).
"""
import sys

import pytest
import torch

import gated_linear_attention_simple_amd as gla
import gla_inputs as gi

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("chunk,chain", [(128, "0"), (64, "0"), (128, "1")])
def test_graph_replays_match_eager(chunk, chain, monkeypatch):
    """Also with the forward's tiled state chain (two launches, a chunk start
    state workspace) in the captured sequence."""
    monkeypatch.setenv("GLA_FWD_CHAIN", chain)
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, 41 + chunk, B=2, T=700, with_do=True, s0_var=0.01)
    y = gi.fwd_inputs(w, DEV, 43 + chunk, B=2, T=700, with_do=True, s0_var=0.01)
    _say(f"graph capture fwd+bwd B=2 T=700 C={chunk} chain={chain}")
    args = (x["q"], x["k"], x["v"], x["lam"])
    o_ref, S_ref = gla.fwd_chunked(*args, S0=x["S0"], scale=x["scale"], chunk=chunk)
    g_ref = gla.bwd_chunked(*args, x["do"], S0=x["S0"], scale=x["scale"], chunk=chunk)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gla.fwd_chunked(*args, S0=x["S0"], scale=x["scale"], chunk=chunk)
        gla.bwd_chunked(*args, x["do"], S0=x["S0"], scale=x["scale"], chunk=chunk)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o, S = gla.fwd_chunked(*args, S0=x["S0"], scale=x["scale"], chunk=chunk)
        grads = gla.bwd_chunked(*args, x["do"], S0=x["S0"], scale=x["scale"], chunk=chunk)
    torch.cuda.synchronize()

    for rep in range(3):
        # unrelated eager work on the same buffers' neighbours between replays
        gla.fwd_chunked(y["q"], y["k"], y["v"], y["lam"], S0=y["S0"], scale=y["scale"], chunk=chunk)
        gla.bwd_chunked(y["q"], y["k"], y["v"], y["lam"], y["do"], S0=y["S0"], scale=y["scale"], chunk=chunk)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: o"
        assert torch.equal(S, S_ref), f"replay {rep}: S_final"
        for name, a, b in zip(("dq", "dk", "dv", "dlambda", "dS0"), grads, g_ref):
            assert torch.equal(a, b), f"replay {rep}: {name}"

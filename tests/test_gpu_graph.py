"""HIP-graph capture of the library calls (for callers that replay a captured step;
the bench itself times eager calls).

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


@pytest.mark.parametrize("chunk,chain", [(128, 0), (64, 0), (128, 1)])
def test_graph_replays_match_eager(chunk, chain):
    """Also with the forward's tiled state chain (two launches, a chunk start
    state workspace) in the captured sequence."""
    plan = {"chain": chain}
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, 41 + chunk, B=2, T=700, with_do=True, s0_var=0.01)
    y = gi.fwd_inputs(w, DEV, 43 + chunk, B=2, T=700, with_do=True, s0_var=0.01)
    _say(f"graph capture fwd+bwd B=2 T=700 C={chunk} chain={chain}")
    args = (x["q"], x["k"], x["v"], x["lam"])
    o_ref, S_ref = gla.fwd_chunked(*args, S0=x["S0"], scale=x["scale"], chunk=chunk, plan=plan)
    g_ref = gla.bwd_chunked(*args, x["do"], S0=x["S0"], scale=x["scale"], chunk=chunk, plan=plan)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gla.fwd_chunked(*args, S0=x["S0"], scale=x["scale"], chunk=chunk, plan=plan)
        gla.bwd_chunked(*args, x["do"], S0=x["S0"], scale=x["scale"], chunk=chunk, plan=plan)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o, S = gla.fwd_chunked(*args, S0=x["S0"], scale=x["scale"], chunk=chunk, plan=plan)
        grads = gla.bwd_chunked(*args, x["do"], S0=x["S0"], scale=x["scale"], chunk=chunk, plan=plan)
    torch.cuda.synchronize()

    for rep in range(3):
        # unrelated eager work on the same buffers' neighbours between replays
        gla.fwd_chunked(y["q"], y["k"], y["v"], y["lam"], S0=y["S0"], scale=y["scale"], chunk=chunk, plan=plan)
        gla.bwd_chunked(y["q"], y["k"], y["v"], y["lam"], y["do"], S0=y["S0"], scale=y["scale"], chunk=chunk,
                        plan=plan)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: o"
        assert torch.equal(S, S_ref), f"replay {rep}: S_final"
        for name, a, b in zip(("dq", "dk", "dv", "dlambda", "dS0"), grads, g_ref):
            assert torch.equal(a, b), f"replay {rep}: {name}"


def test_graph_prefill_and_decode_with_conv_and_epilogue():
    """A captured prefill (conv, forward, epilogue) and a captured decode step (conv
    window step, decode with the fused epilogue on a slot pool): every replay, with
    eager work and synchronisation between replays, equals the eager calls bit for bit."""
    w = gi.workloads()[1]
    B, T, D = 2, 300, 3072
    x = gi.fwd_inputs(w, DEV, 61, B=B, T=T)
    e = gi.epilogue_inputs(w, DEV, 61, (B, T))
    cv = gi.conv_inputs(B, T, D, "bf16", DEV, seed=62)
    _say("graph capture prefill conv+fwd+epilogue")

    def prefill():
        yc, wo = gla.conv1d_silu(cv["x"], cv["w"], cv["bias"], cv["win"])
        o, S = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], scale=x["scale"], chunk=128)
        y = gla.mixer_epilogue(x["q"], x["k"], x["v"], o, e["g"], e["norm_w"], e["tier"], aug_a=e["aug_a"])
        return yc, wo, S, y

    ref = prefill()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prefill()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = prefill()
    torch.cuda.synchronize()
    for rep in range(3):
        prefill()                                   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b, name in zip(out, ref, ("conv y", "window", "S_final", "epilogue y")):
            assert torch.equal(a, b), f"prefill replay {rep}: {name}"

    _say("graph capture decode step conv+decode-epilogue on a pool")
    wd = gi.workloads()[4]
    N, P = 6, 9
    lam = torch.tensor(wd.lambdas, device=DEV)
    pool0 = gi.decode_state(wd, DEV, seed=63, layer=0, N=P)
    cwin0 = gi.conv_inputs(P, 1, D, "bf16", DEV, seed=64)["win"]
    slots = torch.tensor([7, 0, -1, 3, 8, 2], dtype=torch.int32, device=DEV)
    d = gi.decode_token_inputs(wd, DEV, seed=63, layer=0, step=0, N=N)
    ed = gi.epilogue_inputs(wd, DEV, 63, (N,))
    xc = gi.conv_inputs(N, 1, D, "bf16", DEV, seed=65)["x"][:, 0].contiguous()
    pool, cwin = pool0.clone(), cwin0.clone()

    def step():
        yc = gla.conv1d_silu_decode(xc, cv["w"], cv["bias"], cwin, slots=slots)
        y = gla.decode_step_epilogue(d["q"], d["k"], d["v"], ed["g"], lam, pool, ed["norm_w"], ed["tier"],
                                     aug_a=ed["aug_a"], scale=wd.scale, slots=slots)
        return yc, y

    ref = step()
    torch.cuda.synchronize()
    ref_pool, ref_cwin = pool.clone(), cwin.clone()
    pool.copy_(pool0)
    cwin.copy_(cwin0)
    with torch.cuda.stream(side):
        step()
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        out = step()
    torch.cuda.synchronize()
    for rep in range(3):
        pool.copy_(pool0)
        cwin.copy_(cwin0)
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(out[0], ref[0]) and torch.equal(out[1], ref[1]), f"decode replay {rep}"
        assert torch.equal(pool, ref_pool) and torch.equal(cwin, ref_cwin), f"decode replay {rep}: state"

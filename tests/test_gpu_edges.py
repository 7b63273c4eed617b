"""GPU parity at the method's closed-form edges, lambda = 0 and lambda = 1, and with
per-head mixes of 0, 1 and interior decays (Laplace 3B post, section "i14 and the
Laplace 3B architecture", paragraph "GLA mixer": a fixed per-head decay and a rank-1
write).  lambda = 1 is causal cumulative linear attention (the state is never
decayed, over up to 2,048 tokens here); lambda = 0 keeps only the current token,
o_t = scale (q_t . k_t) v_t, and exercises 0^0 = 1 in every decay table, lambda^C = 0
in the chunk chains and segment scans, and d(lambda^n)/d lambda at 0 in dlambda.

Every case runs the HIP kernels through the C ABI and compares element by element
with the fp64 oracle on the exact bits the kernels consumed; dlambda is compared as
an H-vector and on each lambda group on its own.
"""
import sys

import numpy as np
import pytest
import torch

import gated_linear_attention_simple_amd as gla
import gla_inputs as gi
import oracle
from parity_util import assert_close, assert_close_groups, f64, lambda_groups

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

LAMBDA_SETS = {
    "zero": [0.0] * 16,
    "one": [1.0] * 16,
    "mixed": [0.0, 1.0, 0.5, 0.9, 0.99, 0.999, 0.0, 1.0, 0.25, 0.75, 0.9997, 1.0, 0.0, 0.95, 0.999, 1.0],
}
TINY_SETS = {"zero": [0.0, 0.0], "one": [1.0, 1.0], "mixed": [0.0, 1.0]}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _wl(wi, lams, chunk=None, dtype=None):
    w = gi.workloads()[wi]
    return gi.Workload(w.name, w.B, w.T, w.H, w.dk, w.dv, chunk or w.chunk, dtype or w.dtype, tuple(lams),
                       w.scale, w.s0_var)


PLANS = {None: None, "chain": {"chain": 1}, "segments": {"chain": 0}}


# (workload, B, T, chunk, dtype, S0 variance, plan): the Laplace layer through the tiled
# chain and through 16 segments, a ragged two-sequence case at chunk 64, the training
# width (two segments, sub-segment prologue), and both fp32 shapes.
FWD_CASES = {
    "layer_chain": (1, 1, 2048, 128, None, 0.01, "chain"),
    "layer_segments": (1, 1, 2048, 128, None, 0.01, "segments"),
    "ragged_c64": (1, 2, 1000, 64, None, 0.01, None),
    "ragged_c32": (1, 2, 1000, 32, None, 0.01, None),
    "layer_c256": (1, 1, 2048, 256, None, 0.01, None),
    "ragged_c256": (1, 2, 1000, 256, None, 0.01, None),
    "train_width": (2, 8, 2048, 128, None, 0.0, None),
    "fp32_tiny": (0, 2, 250, 32, None, 0.5, None),
    "fp32_wide_c64": (1, 2, 300, 64, "f32", 0.01, None),
}


@pytest.mark.parametrize("lset", sorted(LAMBDA_SETS))
@pytest.mark.parametrize("case", sorted(FWD_CASES))
def test_forward_edges(case, lset):
    wi, B, T, chunk, dtype, s0, plan = FWD_CASES[case]
    lams = (TINY_SETS if wi == 0 else LAMBDA_SETS)[lset]
    w = _wl(wi, lams, chunk, dtype)
    x = gi.fwd_inputs(w, DEV, 4000 + len(case) + T, B=B, T=T, s0_var=s0)
    _say(f"fwd edges {case} lambda={lset} B={B} T={T} C={chunk} {w.dtype} plan={plan}")
    o, S = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"], chunk=chunk,
                           plan=PLANS[plan])
    torch.cuda.synchronize()
    S0r = None if x["S0"] is None else f64(x["S0"])
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), S0=S0r, scale=x["scale"])
    assert_close(f64(o), ro, w.dtype, "o")
    assert_close(f64(S), rS, w.dtype, "S_final")


BWD_CASES = {
    "c128": (1, 2, 1000, 128, "recompute"),
    "c64": (1, 2, 700, 64, "recompute"),
    "c128_saved": (1, 2, 1000, 128, "saved"),
    "c64_saved": (1, 2, 1500, 64, "saved"),
    "c32": (1, 2, 700, 32, "recompute"),
    "c32_saved": (1, 2, 1000, 32, "saved"),
    "c256": (1, 2, 1000, 256, "recompute"),
    "c256_saved": (1, 2, 1000, 256, "saved"),
    "fp32_tiny": (0, 2, 200, 32, "recompute"),
}


@pytest.mark.parametrize("lset", sorted(LAMBDA_SETS))
@pytest.mark.parametrize("case", sorted(BWD_CASES))
def test_backward_edges(case, lset):
    wi, B, T, chunk, form = BWD_CASES[case]
    lams = (TINY_SETS if wi == 0 else LAMBDA_SETS)[lset]
    w = _wl(wi, lams, chunk)
    x = gi.fwd_inputs(w, DEV, 5000 + len(case) + T, B=B, T=T, with_do=True, with_dS=True, s0_var=0.01)
    _say(f"bwd edges {case} lambda={lset} B={B} T={T} C={chunk} {w.dtype} {form}")
    args = (x["q"], x["k"], x["v"], x["lam"])
    if form == "saved":
        _, _, st = gla.fwd_chunked_states(*args, S0=x["S0"], scale=x["scale"], chunk=chunk)
        dq, dk, dv, dl, dS0 = gla.bwd_chunked_states(*args, x["do"], st, S0=x["S0"], dS_final=x["dS"],
                                                     scale=x["scale"], chunk=chunk)
    else:
        dq, dk, dv, dl, dS0 = gla.bwd_chunked(*args, x["do"], S0=x["S0"], dS_final=x["dS"], scale=x["scale"],
                                              chunk=chunk)
    torch.cuda.synchronize()
    r = oracle.bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), f64(x["do"]), S0=f64(x["S0"]),
                   dS_T=f64(x["dS"]), scale=x["scale"])
    for got, ref, name in zip((dq, dk, dv, dS0), (r[0], r[1], r[2], r[4]), ("dq", "dk", "dv", "dS0")):
        assert_close(f64(got), ref, w.dtype, name)
    assert_close_groups(f64(dl), r[3], lambda_groups(lams), w.dtype, "dlambda")


@pytest.mark.parametrize("lset", sorted(LAMBDA_SETS))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_edges(lset, dtype):
    """Plain decode, the page pool (shuffled slots, a padding row) and the decode with
    the fused epilogue, 6 steps each, every step against the oracle."""
    w = gi.workloads()[4]
    w = gi.Workload(w.name, 9, 1, 16, 96, 192, 0, dtype, tuple(LAMBDA_SETS[lset]), 96 ** -0.5, w.s0_var, 24)
    lam = torch.tensor(w.lambdas, dtype=torch.float32, device=DEV)
    S = gi.decode_state(w, DEV, seed=61, layer=0)
    pool = torch.zeros(12, 16, 96, 192, device=DEV)
    slots = torch.tensor([3, 11, 0, 7, -1, 5, 9, 1, 4, 8], dtype=torch.int32, device=DEV)
    live = [r for r in range(10) if int(slots[r]) >= 0]
    pool[slots[live].long()] = S
    S_epi = S.clone()
    Sref = f64(S)
    e = gi.epilogue_inputs(w, DEV, 61, (w.B,))
    _say(f"decode edges lambda={lset} {dtype} N=9, 6 steps (plain, pool, epilogue)")
    for step in range(6):
        d = gi.decode_token_inputs(w, DEV, seed=61, layer=0, step=step)
        o = gla.decode_step(d["q"], d["k"], d["v"], lam, S, scale=w.scale)
        rows = {name: torch.zeros((10,) + tuple(t.shape[1:]), dtype=t.dtype, device=DEV) for name, t in d.items()}
        for name in rows:
            rows[name][live] = d[name]
        op = gla.decode_step_pool(rows["q"], rows["k"], rows["v"], lam, pool, slots, scale=w.scale)
        g = gi.epilogue_inputs(w, DEV, 61, (w.B,), step=step)["g"]
        y = gla.decode_step_epilogue(d["q"], d["k"], d["v"], g, lam, S_epi, e["norm_w"], e["tier"],
                                     aug_a=e["aug_a"], scale=w.scale)
        torch.cuda.synchronize()
        ro, Sref = oracle.decode(f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(lam), Sref, scale=w.scale)
        ry = oracle.epilogue(f64(d["q"]), f64(d["k"]), f64(d["v"]), ro, f64(g), f64(e["aug_a"]),
                             f64(e["norm_w"]), e["tier"])
        assert_close(f64(o), ro, dtype, f"o step {step}")
        assert_close(f64(S), Sref, dtype, f"S step {step}")
        assert_close(f64(op[live]), ro, dtype, f"pool o step {step}")
        assert torch.count_nonzero(op[4]) == 0, "padding row"
        assert_close(f64(pool[slots[live].long()]), Sref, dtype, f"pool pages step {step}")
        assert_close(f64(y), ry, dtype, f"epilogue y step {step}")
        assert_close(f64(S_epi), Sref, dtype, f"epilogue S step {step}")


@pytest.mark.parametrize("lset", sorted(LAMBDA_SETS))
@pytest.mark.parametrize("plan", ["chain", "segments"])
def test_forward_epilogue_edges(lset, plan):
    """The forward with the epilogue fused into its output kernel (tiled chain) and
    the forward followed by the epilogue pass (segments), Laplace-layer shape."""
    w = _wl(1, LAMBDA_SETS[lset])
    x = gi.fwd_inputs(w, DEV, seed=71, s0_var=0.01)
    e = gi.epilogue_inputs(w, DEV, 71, (w.B, w.T))
    _say(f"fwd+epilogue edges lambda={lset} plan={plan}")
    y, S = gla.fwd_chunked_epilogue(x["q"], x["k"], x["v"], x["lam"], e["g"], e["norm_w"], e["tier"],
                                    aug_a=e["aug_a"], S0=x["S0"], scale=x["scale"], chunk=128, plan=PLANS[plan])
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), S0=f64(x["S0"]), scale=x["scale"])
    ry = oracle.epilogue(f64(x["q"]), f64(x["k"]), f64(x["v"]), ro, f64(e["g"]), f64(e["aug_a"]), f64(e["norm_w"]),
                         e["tier"])
    assert_close(f64(y), ry, "bf16", "y")
    assert_close(f64(S), rS, "bf16", "S_final")

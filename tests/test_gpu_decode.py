"""GPU parity of gla_decode_step against the fp64 oracle (through the C ABI)."""
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


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 96, 192), ("f32", 96, 192), ("bf16", 16, 32), ("f32", 16, 32)])
def test_decode_steps_match_oracle(dtype, dk, dv):
    w = gi.workloads()[4]
    w = gi.Workload(w.name, 7, 1, 16, dk, dv, 0, dtype, w.lambdas, dk ** -0.5, w.s0_var, 24)
    S = gi.decode_state(w, DEV, seed=9, layer=0)
    Sref = f64(S)
    _say(f"decode {dtype} dk={dk} dv={dv} N=7, 6 steps")
    for step in range(6):
        d = gi.decode_token_inputs(w, DEV, seed=9, layer=0, step=step)
        o = gla.decode_step(d["q"], d["k"], d["v"], torch.tensor(w.lambdas, device=DEV), S, scale=w.scale)
        torch.cuda.synchronize()
        ro, Sref = oracle.decode(f64(d["q"]), f64(d["k"]), f64(d["v"]), np.array(w.lambdas), Sref, scale=w.scale)
        assert_close(f64(o), ro, dtype, f"o step {step}")
        assert_close(f64(S), Sref, dtype, f"S step {step}")


def test_decode_equals_forward_over_same_tokens():
    """k decode steps from S0 equal one forward call over those k tokens (both on GPU,
    each checked against the oracle's forward)."""
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, seed=12, B=3, T=20, s0_var=0.1)
    S = x["S0"].clone()
    outs = []
    for t in range(20):
        outs.append(gla.decode_step(x["q"][:, t].contiguous(), x["k"][:, t].contiguous(),
                                    x["v"][:, t].contiguous(), x["lam"], S, scale=x["scale"]))
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), S0=f64(x["S0"]), scale=x["scale"])
    assert_close(f64(torch.stack(outs, 1)), ro, "bf16", "decode outputs vs forward")
    assert_close(f64(S), rS, "bf16", "decode state vs forward")


def test_decode_full_width_sampled():
    """The bench's launch configuration (N=1,280 sequences, H=16, one layer's
    1.5 GB page pool): 3 steps, checked on a seeded sample of 64 sequences."""
    w = gi.workloads()[4]
    lam = torch.tensor(w.lambdas, device=DEV)
    S = gi.decode_state(w, DEV, seed=4, layer=5)
    rng = np.random.default_rng(4)
    idx = np.sort(rng.choice(w.B, 64, replace=False))
    Sref = f64(S[idx])
    _say("decode N=1280 full width, 3 steps")
    for step in range(3):
        d = gi.decode_token_inputs(w, DEV, seed=4, layer=5, step=step)
        o = gla.decode_step(d["q"], d["k"], d["v"], lam, S, scale=w.scale)
        torch.cuda.synchronize()
        ro, Sref = oracle.decode(f64(d["q"][idx]), f64(d["k"][idx]), f64(d["v"][idx]), f64(lam), Sref,
                                 scale=w.scale)
        assert_close(f64(o[idx]), ro, "bf16", f"o step {step}")
        assert_close(f64(S[idx]), Sref, "bf16", f"S step {step}")
    del S
    torch.cuda.empty_cache()


def test_decode_batch_position_invariant():
    w = gi.workloads()[4]
    lam = torch.tensor(w.lambdas, device=DEV)
    S = gi.decode_state(w, DEV, seed=8, layer=0, N=9)
    d = gi.decode_token_inputs(w, DEV, seed=8, layer=0, step=0, N=9)
    S1 = S[4:5].clone()
    o_all = gla.decode_step(d["q"], d["k"], d["v"], lam, S, scale=w.scale)
    o_one = gla.decode_step(d["q"][4:5].contiguous(), d["k"][4:5].contiguous(), d["v"][4:5].contiguous(),
                            lam, S1, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_all[4:5], o_one) and torch.equal(S[4:5], S1)

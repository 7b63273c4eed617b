"""GPU parity of gla_bwd_chunked against the fp64 oracle's reverse mode (through the C ABI).

Loss L = <do, o> + <dS_T, S_final>; gradients dq, dk, dv, dlambda (per head,
summed over the batch) and dS0 are compared with the oracle on the exact bits
the kernels consumed, per tensor and per sequence.
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


def _run(w, seed, B=None, T=None, chunk=None, s0_var=None, with_dS=True, plan=None):
    chunk = chunk or w.chunk
    x = gi.fwd_inputs(w, DEV, seed, B=B, T=T, with_do=True, with_dS=with_dS, s0_var=s0_var)
    _say(f"bwd {w.name} dtype={w.dtype} B={x['q'].shape[0]} T={x['q'].shape[1]} C={chunk} "
         f"S0={'yes' if x['S0'] is not None else 'no'} dS_T={'yes' if with_dS else 'no'} seed={seed}")
    dq, dk, dv, dl, dS0 = gla.bwd_chunked(x["q"], x["k"], x["v"], x["lam"], x["do"], S0=x["S0"],
                                          dS_final=x.get("dS"), scale=x["scale"], chunk=chunk, plan=plan)
    torch.cuda.synchronize()
    r = oracle.bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), f64(x["do"]),
                   S0=None if x["S0"] is None else f64(x["S0"]),
                   dS_T=f64(x["dS"]) if with_dS else None, scale=x["scale"])
    for got, ref, name in zip((dq, dk, dv, dS0), (r[0], r[1], r[2], r[4]), ("dq", "dk", "dv", "dS0")):
        assert_close(f64(got), ref, w.dtype, name)
    assert_close(f64(dl), r[3], w.dtype, "dlambda", batch_axis=None)
    return x, (dq, dk, dv, dl, dS0)


def test_tiny_fp32():
    _run(gi.workloads()[0], seed=50, with_dS=False)


@pytest.mark.parametrize("T", [1, 31, 33, 256])
def test_tiny_fp32_ragged_with_states(T):
    _run(gi.workloads()[0], seed=60 + T, B=2, T=T, s0_var=0.5)


@pytest.mark.parametrize("chunk", [128, 64, 32, 256])
@pytest.mark.parametrize("T", [1, 100, 300, 1000])
def test_bf16_ragged_with_states(chunk, T):
    _run(gi.workloads()[1], seed=70 + T + chunk, B=2, T=T, chunk=chunk, s0_var=0.01)


@pytest.mark.parametrize("chunk", [128, 64, 32, 256])
@pytest.mark.parametrize("T", [40, 2048])
def test_single_partial_chunk_and_full_length(chunk, T):
    """T = 40: one partial chunk with no second query half (chunks 128, 64), one full
    and one partial chunk (32); and the full 2,048-token sequence, with S0 and dS_T."""
    _run(gi.workloads()[1], seed=1500 + T + chunk, B=2, T=T, chunk=chunk, s0_var=0.01)


@pytest.mark.parametrize("nseg", [1, 3, 5])
def test_bf16_segment_split(nseg):
    _run(gi.workloads()[1], seed=90 + nseg, B=1, T=1000, chunk=64, s0_var=0.01, plan={"segments": nseg})


@pytest.mark.parametrize("chunk", [128, 64, 32, 256])
def test_train_step_config(chunk):
    """B=8, H=16, T=2048, dk=96, dv=192, bf16, do ~ N(0,1); C=128, 64, 32 and 256."""
    _run(gi.workloads()[2], seed=2, chunk=chunk, with_dS=False)


def test_empty_sequence():
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, 5, B=2, T=0, with_do=True, with_dS=True)
    dq, dk, dv, dl, dS0 = gla.bwd_chunked(x["q"], x["k"], x["v"], x["lam"], x["do"], dS_final=x["dS"],
                                          scale=x["scale"])
    torch.cuda.synchronize()
    assert torch.equal(dS0, x["dS"]) and not dl.any()


def test_bwd_deterministic():
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, 44, B=2, T=700, with_do=True, s0_var=0.01)
    a = gla.bwd_chunked(x["q"], x["k"], x["v"], x["lam"], x["do"], S0=x["S0"], scale=x["scale"])
    b = gla.bwd_chunked(x["q"], x["k"], x["v"], x["lam"], x["do"], S0=x["S0"], scale=x["scale"])
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("chunk", [128, 64])
def test_page_decay_schedule(chunk):
    """The pages' geometric half-life schedule (head 0: lambda = 0.5, whose
    powers leave fp32's normal range inside a 128-token chunk) as a stress set
    for the backward, dlambda included."""
    w = gi.workloads()[1]
    w = gi.Workload(w.name + "-page-decay", w.B, w.T, w.H, w.dk, w.dv, w.chunk, w.dtype,
                    tuple(gi.page_lambdas(w.H)), w.scale)
    _run(w, seed=90 + chunk, B=2, T=600, chunk=chunk, s0_var=0.01)


def _states_case(w, seed, B, T, chunk, s0_var, chain=None):
    plan = None if chain is None else {"chain": chain}
    x = gi.fwd_inputs(w, DEV, seed, B=B, T=T, with_do=True, with_dS=True, s0_var=s0_var)
    _say(f"fwd/bwd with saved states {w.name} B={B} T={T} C={chunk} chain={chain}")
    o, S, states = gla.fwd_chunked_states(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"],
                                          chunk=chunk, plan=plan)
    g = gla.bwd_chunked_states(x["q"], x["k"], x["v"], x["lam"], x["do"], states, S0=x["S0"], dS_final=x["dS"],
                               scale=x["scale"], chunk=chunk)
    torch.cuda.synchronize()
    return x, o, S, states, g


@pytest.mark.parametrize("wi,B,T,chunk,chain", [(1, 2, 700, 128, None), (1, 2, 700, 64, None),
                                                (1, 1, 2048, 128, 1), (1, 1, 2048, 128, 0),
                                                (1, 1, 300, 128, 1), (0, 2, 200, 32, None),
                                                (1, 2, 1000, 256, None), (1, 1, 2048, 256, None),
                                                (1, 3, 200, 256, None)])
def test_saved_states_and_backward_match_oracle(wi, B, T, chunk, chain):
    """gla_fwd_chunked_states writes the state before every chunk (checked against the
    oracle's state after each prefix of whole chunks), and gla_bwd_chunked_states'
    gradients from them match the oracle's reverse mode."""
    w = gi.workloads()[wi]
    x, o, S, states, (dq, dk, dv, dl, dS0) = _states_case(w, 90 + T + chunk, B, T, chunk, 0.01, chain)
    nc = (T + chunk - 1) // chunk
    c64 = lambda name: f64(x[name])
    for c in range(nc):
        if c == 0:
            ref = c64("S0")
        else:
            _, ref = oracle.fwd(c64("q")[:, :c * chunk], c64("k")[:, :c * chunk], c64("v")[:, :c * chunk],
                                c64("lam"), S0=c64("S0"), scale=x["scale"])
        assert_close(f64(states[:, :, c]), ref, w.dtype, f"state before chunk {c}")
    ro, rS = oracle.fwd(c64("q"), c64("k"), c64("v"), c64("lam"), S0=c64("S0"), scale=x["scale"])
    assert_close(f64(o), ro, w.dtype, "o")
    assert_close(f64(S), rS, w.dtype, "S_final")
    r = oracle.bwd(c64("q"), c64("k"), c64("v"), c64("lam"), c64("do"), S0=c64("S0"), dS_T=c64("dS"),
                   scale=x["scale"])
    for got, ref, name in zip((dq, dk, dv, dS0), (r[0], r[1], r[2], r[4]), ("dq", "dk", "dv", "dS0")):
        assert_close(f64(got), ref, w.dtype, name)
    assert_close(f64(dl), r[3], w.dtype, "dlambda", batch_axis=None)


@pytest.mark.parametrize("chunk", [128, 64, 32])
def test_saved_states_training_width(chunk):
    """The bench's training legs exactly: gla_fwd_chunked_states + gla_bwd_chunked_states
    at B=8, H=16, T=2048 (two sequence segments; the state-only prologue over half-length
    sub-segments; the forward storing every chunk's start state).  Every sequence's o,
    dq, dk, dv and dS0, and dlambda (a sum over the batch), against the oracle; the
    gradients also agree with the recomputing backward's within the bf16 bar."""
    w = gi.workloads()[2]
    plan = gla.plan_resolve(gla.GLA_BF16, 8, 2048, 16, 96, 192, chunk)
    assert plan == {"segments": 2, "chain": 0, "psub": 2, "scan": 1}, plan   # the plan the bench times
    x, o, S, states, (dq, dk, dv, dl, dS0) = _states_case(w, 7 + chunk, 8, 2048, chunk, 0.0)
    g2 = gla.bwd_chunked(x["q"], x["k"], x["v"], x["lam"], x["do"], S0=x["S0"], dS_final=x["dS"], scale=x["scale"],
                         chunk=chunk)
    torch.cuda.synchronize()
    for a, b, name in zip((dq, dk, dv, dl, dS0), g2, ("dq", "dk", "dv", "dlambda", "dS0")):
        assert_close(f64(a), f64(b), "bf16", f"{name} vs recomputing backward", batch_axis=None)
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), scale=x["scale"])
    assert_close(f64(o), ro, "bf16", "o")
    assert_close(f64(S), rS, "bf16", "S_final")
    r = oracle.bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), f64(x["do"]), dS_T=f64(x["dS"]),
                   scale=x["scale"])
    for got, ref, name in zip((dq, dk, dv, dS0), (r[0], r[1], r[2], r[4]), ("dq", "dk", "dv", "dS0")):
        assert_close(f64(got), ref, "bf16", name)
    assert_close(f64(dl), r[3], "bf16", "dlambda", batch_axis=None)


def test_saved_states_training_width_c256():
    """The bench's 256-token training leg exactly: the forward in the tiled-chain form
    (256-token chunks run only so) storing every chunk's start state, the backward's
    chains over two sequence segments and the four-workgroup gradient kernel; every
    sequence's o, dq, dk, dv and dS0 and dlambda against the oracle."""
    w = gi.workloads()[2]
    plan = gla.plan_resolve(gla.GLA_BF16, 8, 2048, 16, 96, 192, 256)
    assert plan["chain"] == 1, plan
    x, o, S, states, (dq, dk, dv, dl, dS0) = _states_case(w, 263, 8, 2048, 256, 0.0)
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), scale=x["scale"])
    assert_close(f64(o), ro, "bf16", "o")
    assert_close(f64(S), rS, "bf16", "S_final")
    r = oracle.bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), f64(x["do"]), dS_T=f64(x["dS"]),
                   scale=x["scale"])
    for got, ref, name in zip((dq, dk, dv, dS0), (r[0], r[1], r[2], r[4]), ("dq", "dk", "dv", "dS0")):
        assert_close(f64(got), ref, "bf16", name)
    assert_close(f64(dl), r[3], "bf16", "dlambda", batch_axis=None)


@pytest.mark.parametrize("chunk", [128, 64, 32, 256])
def test_bwd_batch_position_invariant(chunk):
    """Each (batch, head) unit's gradients are computed alone: permuting the batch
    permutes dq, dk, dv and dS0 bit for bit (saved-state pair and recomputing form);
    dlambda, a sum over the batch, agrees to fp32 rounding."""
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, 46 + chunk, B=4, T=650, with_do=True, with_dS=True, s0_var=0.01)
    perm = torch.tensor([2, 0, 3, 1], device=DEV)
    xp = {k: (v[perm].contiguous() if isinstance(v, torch.Tensor) and k != "lam" else v) for k, v in x.items()}
    _say(f"bwd batch permutation B=4 T=650 C={chunk}")
    outs = []
    for y in (x, xp):
        _, _, st = gla.fwd_chunked_states(y["q"], y["k"], y["v"], y["lam"], S0=y["S0"], scale=y["scale"], chunk=chunk)
        outs.append(gla.bwd_chunked_states(y["q"], y["k"], y["v"], y["lam"], y["do"], st, S0=y["S0"],
                                           dS_final=y["dS"], scale=y["scale"], chunk=chunk))
        outs.append(gla.bwd_chunked(y["q"], y["k"], y["v"], y["lam"], y["do"], S0=y["S0"], dS_final=y["dS"],
                                    scale=y["scale"], chunk=chunk))
    torch.cuda.synchronize()
    for base, permuted in ((outs[0], outs[2]), (outs[1], outs[3])):
        for i, name in ((0, "dq"), (1, "dk"), (2, "dv"), (4, "dS0")):
            assert torch.equal(permuted[i], base[i][perm]), f"{name} depends on batch position"
        a, b = f64(base[3]), f64(permuted[3])
        assert np.linalg.norm(a - b) <= 1e-6 * np.linalg.norm(a), "dlambda: batch order changed more than rounding"


@pytest.mark.parametrize("case", range(8))
def test_fwd_bwd_shape_sweep(case):
    """Seeded sweep of head counts, batch sizes, lengths (ragged and chunk-aligned),
    chunk sizes and optional S0 / dS_T through the forward and the backward, against
    the oracle: plans with one or many segments, the tiled chain, few units."""
    rng = np.random.default_rng(9000 + case)
    H = int(rng.choice([1, 3, 5, 16]))
    B = int(rng.choice([1, 2, 3]))
    chunk = int(rng.choice([32, 64, 128]))
    T = int(rng.choice([1, 63, 64, 129, 255, 384, 513, 777]))
    s0 = 0.01 if rng.random() < 0.5 else None
    lam = tuple(gi.laplace_lambdas(16))[:H] if H < 16 else tuple(gi.laplace_lambdas(16))
    w1 = gi.workloads()[1]
    w = gi.Workload(w1.name, B, T, H, 96, 192, chunk, "bf16", lam, w1.scale)
    x = gi.fwd_inputs(w, DEV, 9100 + case, B=B, T=T, with_do=True, with_dS=rng.random() < 0.5, s0_var=s0)
    _say(f"sweep case {case}: B={B} H={H} T={T} C={chunk} S0={s0 is not None} dS_T={'dS' in x}")
    o, S = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"], chunk=chunk)
    dq, dk, dv, dl, dS0 = gla.bwd_chunked(x["q"], x["k"], x["v"], x["lam"], x["do"], S0=x["S0"],
                                          dS_final=x.get("dS"), scale=x["scale"], chunk=chunk)
    torch.cuda.synchronize()
    S0r = None if x["S0"] is None else f64(x["S0"])
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), S0=S0r, scale=x["scale"])
    assert_close(f64(o), ro, "bf16", "o")
    assert_close(f64(S), rS, "bf16", "S_final")
    r = oracle.bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), f64(x["do"]), S0=S0r,
                   dS_T=f64(x["dS"]) if "dS" in x else None, scale=x["scale"])
    for got, ref, name in zip((dq, dk, dv, dS0), (r[0], r[1], r[2], r[4]), ("dq", "dk", "dv", "dS0")):
        assert_close(f64(got), ref, "bf16", name)
    assert_close(f64(dl), r[3], "bf16", "dlambda", batch_axis=None)


@pytest.mark.parametrize("B,T,chunk,saved,plan", [(8, 2048, 128, True, {}), (8, 2048, 128, False, {}),
                                                  (8, 1000, 64, True, {}), (8, 2048, 32, False, {}),
                                                  (2, 1000, 64, False, {"segments": 3, "psub": 1})])
def test_folded_chain_scans_are_bitwise_the_scans(B, T, chunk, saved, plan):
    """The backward's state passes with the segment scans folded into the emit passes
    (forward from S0, reverse from dS_T) equal the launched scans bit for bit."""
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, 2700 + T + chunk + B, B=B, T=T, with_do=True, with_dS=True, s0_var=0.01)
    _say(f"folded vs launched backward scans B={B} T={T} C={chunk} saved={saved} plan={plan}")
    args = (x["q"], x["k"], x["v"], x["lam"])
    kw = dict(S0=x["S0"], dS_final=x["dS"], scale=x["scale"], chunk=chunk)
    outs = []
    for sc in (1, 0):
        p = dict(plan, scan=sc)
        if saved:
            _, _, st = gla.fwd_chunked_states(*args, S0=x["S0"], scale=x["scale"], chunk=chunk, plan=p)
            outs.append(gla.bwd_chunked_states(*args, x["do"], st, plan=p, **kw))
        else:
            outs.append(gla.bwd_chunked(*args, x["do"], plan=p, **kw))
    torch.cuda.synchronize()
    for a_, b_, name in zip(outs[0], outs[1], ("dq", "dk", "dv", "dlambda", "dS0")):
        assert torch.equal(a_, b_), f"{name}: folded scans differ from launched scans"
    if B <= 2:
        r = oracle.bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), f64(x["do"]), S0=f64(x["S0"]),
                       dS_T=f64(x["dS"]), scale=x["scale"])
        for got, ref, name in zip(outs[0][:3] + outs[0][4:], (r[0], r[1], r[2], r[4]), ("dq", "dk", "dv", "dS0")):
            assert_close(f64(got), ref, "bf16", name)
        assert_close(f64(outs[0][3]), r[3], "bf16", "dlambda", batch_axis=None)

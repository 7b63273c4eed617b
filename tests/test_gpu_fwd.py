"""GPU parity of gla_fwd_chunked against the fp64 oracle (through the C ABI).

Inputs come from gla_inputs on the GPU; the oracle reads the exact bits the
kernel consumed.  Sizes span several chunks, several sequence segments and a
ragged tail; the Laplace-layer shape (B=1, H=16, T=2048, dk=96, dv=192, C=128)
and the 64k-token long prefill run at full size.
"""
import os
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


def _run_and_check(w, seed, B=None, T=None, chunk=None, s0_var=None, dtype=None, plan=None):
    chunk = chunk or w.chunk
    if dtype is not None:
        w = gi.Workload(w.name, w.B, w.T, w.H, w.dk, w.dv, chunk, dtype, w.lambdas, w.scale, w.s0_var)
    x = gi.fwd_inputs(w, DEV, seed, B=B, T=T, s0_var=s0_var)
    _say(f"{w.name} dtype={w.dtype} B={x['q'].shape[0]} T={x['q'].shape[1]} C={chunk} "
         f"S0={'yes' if x['S0'] is not None else 'no'} plan={plan} seed={seed}")
    o, S = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"], chunk=chunk, plan=plan)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]),
                        S0=None if x["S0"] is None else f64(x["S0"]), scale=x["scale"])
    assert_close(f64(o), ro, w.dtype, "o")
    assert_close(f64(S), rS, w.dtype, "S_final")
    return x, o, S


def test_tiny_fp32_config():
    """B=1, H=2, T=256, dk=16, dv=32, C=32, fp32, lambda={0.9,0.99}, scale 1."""
    _run_and_check(gi.workloads()[0], seed=0)


@pytest.mark.parametrize("T", [1, 31, 32, 250, 256])
def test_tiny_fp32_ragged(T):
    _run_and_check(gi.workloads()[0], seed=10 + T, B=3, T=T, s0_var=0.5)


def test_laplace_layer_config():
    """B=1, H=16, T=2048, dk=96, dv=192, C=128, bf16, lambda log-spaced, scale dk^-1/2."""
    _run_and_check(gi.workloads()[1], seed=1)


@pytest.mark.parametrize("chunk", [128, 64, 32, 256])
@pytest.mark.parametrize("T", [1, 100, 300, 1000])
def test_bf16_ragged_with_state(chunk, T):
    _run_and_check(gi.workloads()[1], seed=100 + T + chunk, B=2, T=T, chunk=chunk, s0_var=0.01)


@pytest.mark.parametrize("B,T,s0", [(1, 2048, None), (1, 2048, 0.01), (3, 513, 0.01), (2, 200, None),
                                    (1, 128, 0.01), (1, 129, None), (2, 256, 0.01), (1, 257, None),
                                    (1, 384, 0.01), (1, 4096, None)])
def test_chunk256(B, T, s0):
    """256-token chunks (the tiled chain in two 128-token passes per chunk, then one
    output workgroup per 128 query rows, the second with the cross-half score blocks):
    the Laplace layer, and lengths that end inside the first or the second half of a
    chunk or on its boundaries."""
    _run_and_check(gi.workloads()[1], seed=900 + T + B, B=B, T=T, chunk=256, s0_var=s0)


def test_fp32_laplace_shape_chunk64():
    _run_and_check(gi.workloads()[1], seed=7, B=2, T=700, chunk=64, s0_var=0.01, dtype="f32")


@pytest.mark.parametrize("nseg", [1, 2, 3, 5, 16])
def test_segment_split_equivalence(nseg):
    """Forcing different sequence-segment counts gives the oracle's result."""
    _run_and_check(gi.workloads()[1], seed=200 + nseg, B=1, T=2000, chunk=64, s0_var=0.01,
                   plan={"segments": nseg, "chain": 0})


PLANS = {"seg1": {"segments": 1, "chain": 0}, "seg3": {"segments": 3, "chain": 0}, "chain": {"chain": 1}}


@pytest.mark.parametrize("chunk,mode", [(c, m) for c in (128, 64, 32) for m in sorted(PLANS)
                                        if not (c == 32 and m == "chain")])
def test_bf16_plans(chunk, mode):
    """The bf16 launch plans: unsplit, with sequence segments, and the tiled state
    chain feeding one output workgroup per chunk (built for 64- and 128-token
    chunks); ragged tail, S0."""
    _run_and_check(gi.workloads()[1], seed=314 + chunk + len(mode), B=2, T=1000, chunk=chunk, s0_var=0.01,
                   plan=PLANS[mode])


@pytest.mark.parametrize("chunk,T", [(128, 8192), (64, 4096), (128, 8100)])
def test_chain_at_its_longest(chunk, T):
    """The tiled chain at the most chunks it runs (64; a longer sequence keeps the
    segment form), S0 given: its snapshot workspace at full size, and at 8,192
    tokens the output kernel's chunk-major order (the unit's k and v exceed an
    XCD's L2 share); 8,100 tokens end in a partial chunk."""
    assert gla.plan_resolve(gla.GLA_BF16, 1, T, 16, 96, 192, chunk, {"chain": 1})["chain"] == 1
    _run_and_check(gi.workloads()[1], seed=5150 + chunk + T, B=1, T=T, chunk=chunk, s0_var=0.01, plan={"chain": 1})


@pytest.mark.parametrize("chunk,T,s0", [(128, 2048, None), (64, 1000, None), (128, 700, 0.01), (64, 700, 0.01)])
@pytest.mark.parametrize("want_final", [True, False])
def test_chain_matches_one_chunk_segments_bitwise(chunk, T, s0, want_final):
    """The tiled state chain forms each chunk's contribution on its own and folds
    it in with the segment scan's fma, i.e. the arithmetic of the segment split
    with one chunk per segment: the outputs agree bit for bit, the final states
    (rounded in a different order by the segment path's last workgroup) to fp32
    accuracy.  Both also meet the oracle."""
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, 900 + chunk + T, B=1, T=T, s0_var=s0)
    nc = (T + chunk - 1) // chunk
    _say(f"chain vs {nc} one-chunk segments C={chunk} T={T} S0={s0 is not None} S_final={want_final}")
    outs = []
    for plan in ({"segments": nc, "chain": 0}, {"segments": 1, "chain": 1}):
        o, S = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"], chunk=chunk,
                               S_final=want_final, plan=plan)
        outs.append((o, S))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]), "o differs between the segment and chain paths"
    if want_final:
        a, b = f64(outs[0][1]), f64(outs[1][1])
        assert np.linalg.norm(a - b) <= 1e-6 * np.linalg.norm(a), "S_final: segment and chain paths disagree"
        ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]),
                            S0=None if x["S0"] is None else f64(x["S0"]), scale=x["scale"])
        assert_close(f64(outs[1][0]), ro, w.dtype, "o")
        assert_close(b, rS, w.dtype, "S_final")


@pytest.mark.parametrize("chunk,T,segs,s0", [(64, 1500, 2, 0.01), (128, 2048, 3, None), (128, 1000, 2, 0.01)])
def test_prologue_sub_segments(chunk, T, segs, s0):
    """When the state-only prologue would fill at most half the compute units it runs
    over half-length sub-segments and the scan combines their states: the start states
    differ from one prologue workgroup per segment only by fp32 rounding, which can
    flip the bf16 rounding of a state operand, so the outputs agree to rel L2 1e-3
    (a tenth of the oracle tolerance); both meet the oracle."""
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, 1700 + T + chunk, B=2, T=T, s0_var=s0)
    _say(f"prologue sub-segments B=2 T={T} C={chunk} segments={segs}")
    base = {"chain": 0, "segments": segs}
    assert gla.plan_resolve(gla.GLA_BF16, 2, T, 16, 96, 192, chunk, base)["psub"] == 2
    outs = []
    for plan in (dict(base, psub=1), base):
        outs.append(gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"], chunk=chunk,
                                    plan=plan))
    torch.cuda.synchronize()
    a, b = f64(outs[0][0]), f64(outs[1][0])
    rel = np.linalg.norm(a - b) / np.linalg.norm(a)
    assert rel <= 1e-3, f"o: prologue forms differ, rel L2 {rel:.3e}"
    a, b = f64(outs[0][1]), f64(outs[1][1])
    assert np.linalg.norm(a - b) <= 1e-5 * np.linalg.norm(a), "S_final: prologue forms disagree"
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]),
                        S0=None if x["S0"] is None else f64(x["S0"]), scale=x["scale"])
    for o, S in outs:
        assert_close(f64(o), ro, w.dtype, "o")
        assert_close(f64(S), rS, w.dtype, "S_final")


@pytest.mark.parametrize("chunk", [128, 64, 32])
def test_train_batch_forward(chunk):
    """The training width (B=8, H=16, T=2048) forward at each chunk size."""
    _run_and_check(gi.workloads()[2], seed=2, chunk=chunk)


def test_long_prefill_split_carry():
    """T = 65,536 with S0 ~ N(0, 0.01): one call == two calls carrying the state,
    and both match the oracle (checked on the final state and sampled heads' outputs)."""
    w = gi.workloads()[3]
    x = gi.fwd_inputs(w, DEV, seed=3)
    _say("long prefill T=65536 one call")
    o, S = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"], chunk=128)
    half = 32768
    _say("long prefill two calls carrying state")
    o1, S1 = gla.fwd_chunked(x["q"][:, :half].contiguous(), x["k"][:, :half].contiguous(),
                             x["v"][:, :half].contiguous(), x["lam"], S0=x["S0"], scale=x["scale"], chunk=128)
    o2, S2 = gla.fwd_chunked(x["q"][:, half:].contiguous(), x["k"][:, half:].contiguous(),
                             x["v"][:, half:].contiguous(), x["lam"], S0=S1, scale=x["scale"], chunk=128)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), S0=f64(x["S0"]),
                        scale=x["scale"])
    assert_close(f64(S), rS, "bf16", "S_final (one call)")
    assert_close(f64(S2), rS, "bf16", "S_final (two calls)")
    assert_close(f64(o), ro, "bf16", "o (one call)")
    assert_close(f64(torch.cat([o1, o2], 1)), ro, "bf16", "o (two calls)")


def test_non_chunk_aligned_split():
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, seed=33, B=2, T=1500, s0_var=0.01)
    cut = 777
    o, S = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"])
    o1, S1 = gla.fwd_chunked(x["q"][:, :cut].contiguous(), x["k"][:, :cut].contiguous(),
                             x["v"][:, :cut].contiguous(), x["lam"], S0=x["S0"], scale=x["scale"])
    o2, S2 = gla.fwd_chunked(x["q"][:, cut:].contiguous(), x["k"][:, cut:].contiguous(),
                             x["v"][:, cut:].contiguous(), x["lam"], S0=S1, scale=x["scale"])
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), S0=f64(x["S0"]),
                        scale=x["scale"])
    assert_close(f64(torch.cat([o1, o2], 1)), ro, "bf16", "o (split at 777)")
    assert_close(f64(S2), rS, "bf16", "S_final (split at 777)")


def test_empty_sequence_copies_state():
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, seed=5, B=2, T=0, s0_var=0.01)
    o, S = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"])
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 16, 192)
    assert torch.equal(S, x["S0"])
    _, Sz = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], scale=x["scale"])
    torch.cuda.synchronize()
    assert not Sz.any()


# ---------------------------------------------------------------- exact invariants

def _fwd(x, **kw):
    args = dict(S0=x.get("S0"), scale=x["scale"], chunk=128)
    args.update(kw)
    return gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], **args)


def test_deterministic_and_batch_position_invariant():
    """Same inputs -> same bits; permuting the batch permutes the results bit for bit."""
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, seed=41, B=4, T=1100, s0_var=0.01)
    o1, S1 = _fwd(x)
    o2, S2 = _fwd(x)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2), "run-to-run results differ"
    perm = torch.tensor([2, 0, 3, 1], device=DEV)
    xp = {k: (v[perm].contiguous() if isinstance(v, torch.Tensor) and k != "lam" else v) for k, v in x.items()}
    op, Sp = _fwd(xp)
    torch.cuda.synchronize()
    assert torch.equal(op, o1[perm]) and torch.equal(Sp, S1[perm]), "results depend on batch position"


def test_power_of_two_scaling_exact():
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, seed=42, B=1, T=600, s0_var=0.01)
    o, S = _fwd(x)
    x2 = dict(x)
    x2["v"] = x["v"] * 2
    x2["S0"] = x["S0"] * 2
    o2, S2 = _fwd(x2)
    torch.cuda.synchronize()
    assert torch.equal(o2, o * 2) and torch.equal(S2, S * 2)


def test_causality():
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, seed=43, B=1, T=900)
    o, _ = _fwd(x)
    cut = 333
    y = dict(x)
    for name in ("q", "k", "v"):
        t = x[name].clone()
        t[:, cut:] = -t[:, cut:]
        y[name] = t
    o2, _ = _fwd(y)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :cut], o2[:, :cut])


@pytest.mark.parametrize("chunk,chain", [(128, 0), (128, 1), (64, 0), (32, 0)])
def test_page_decay_schedule(chunk, chain):
    """The pages' geometric half-life schedule (head 0: lambda = 0.5, so lambda^C
    underflows fp32's normal range at C = 128) on the Laplace-layer shape, through
    the segment split and the tiled chain."""
    w = gi.workloads()[1]
    w = gi.Workload(w.name + "-page-decay", w.B, w.T, w.H, w.dk, w.dv, chunk, w.dtype,
                    tuple(gi.page_lambdas(w.H)), w.scale)
    _run_and_check(w, seed=95 + chunk, chunk=chunk, s0_var=0.01, plan={"chain": chain})


@pytest.mark.parametrize("B,T,chunk,s0,plan", [(8, 2048, 128, None, {}), (8, 1000, 128, 0.01, {}),
                                               (8, 2048, 64, 0.01, {}), (8, 2048, 32, None, {}),
                                               (2, 1000, 64, 0.01, {"segments": 3, "psub": 1, "chain": 0})])
def test_folded_segment_scan_is_bitwise_the_scan(B, T, chunk, s0, plan):
    """With at most two local states before the last segment the segments fold them into
    their start states themselves (no scan launch), in the scan kernel's order: outputs
    and final states equal the launched scan's bit for bit, and meet the oracle."""
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, 2600 + T + chunk + B, B=B, T=T, s0_var=s0)
    assert gla.plan_resolve(gla.GLA_BF16, B, T, 16, 96, 192, chunk, plan)["scan"] == 1
    _say(f"folded vs launched segment scan B={B} T={T} C={chunk} plan={plan}")
    outs = [gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"], chunk=chunk,
                            plan=dict(plan, scan=sc)) for sc in (1, 0)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]),
                        S0=None if x["S0"] is None else f64(x["S0"]), scale=x["scale"])
    assert_close(f64(outs[0][0]), ro, "bf16", "o")
    assert_close(f64(outs[0][1]), rS, "bf16", "S_final")

"""GPU parity at head counts other than the Laplace 3B post's 16 ("i14 and the Laplace
3B architecture": the mixer is per head, so nothing in the method fixes H).  The
launches group (batch, head) units eight to a group, one per XCD (the tiled chain, its
output kernel, the 256-token gradient), and the epilogue walks batches of (row, head)
units with a grid that is a multiple of H; head counts that are not multiples of 8
leave groups partly empty and batches that straddle rows, paths no 16-head case runs.

Every case calls the HIP kernels through the C ABI and compares element by element
with the fp64 oracle on the exact bits the kernels consumed.  dlambda is compared as an
H-vector: one head's dlambda is a sum over every token of terms of both signs and can
nearly cancel (for some seeds an interior head's value is ~1% of the terms it sums, at
any head count and in both backward forms), so its error is bounded relative to the
vector, not to that head's own value.
"""
import sys

import pytest
import torch

import gated_linear_attention_simple_amd as gla
import gla_inputs as gi
import oracle
from parity_util import assert_close, f64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

HEADS = [1, 3, 5, 12, 20]


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _lams(H):
    """The Laplace decay spread over H heads, with lambda = 0 and 1 on two of them."""
    lams = gi.laplace_lambdas(H)
    if H >= 3:
        lams[1], lams[H - 1] = 0.0, 1.0
    return lams


def _wl(H, chunk=128, dtype="bf16", B=1, T=1000):
    return gi.Workload(f"heads-{H}", B, T, H, 96, 192, chunk, dtype, tuple(_lams(H)), 96 ** -0.5, 0.01)


# (B, T, chunk, plan): the tiled chain (units <= 16 by default; forced above), the
# segment form with a ragged tail, 64-, 256- and 32-token chunks
FWD_CASES = {
    "c128_chain": (1, 1000, 128, {"chain": 1}),
    "c128_segments": (2, 700, 128, {"chain": 0}),
    "c64_chain": (1, 1000, 64, {"chain": 1}),
    "c256": (1, 1000, 256, None),
    "c32": (3, 300, 32, None),
}


@pytest.mark.parametrize("case", sorted(FWD_CASES))
@pytest.mark.parametrize("H", HEADS)
def test_forward_heads(H, case):
    B, T, chunk, plan = FWD_CASES[case]
    w = _wl(H, chunk, B=B, T=T)
    x = gi.fwd_inputs(w, DEV, 7000 + 31 * H + T, s0_var=0.01)
    _say(f"fwd heads H={H} {case} B={B} T={T} C={chunk} plan={plan}")
    o, S = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"], chunk=chunk, plan=plan)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), S0=f64(x["S0"]), scale=x["scale"])
    assert_close(f64(o), ro, "bf16", "o")
    assert_close(f64(S), rS, "bf16", "S_final")


# (B, T, chunk, form)
BWD_CASES = {
    "c128_saved": (1, 700, 128, "saved"),
    "c64_recompute": (2, 500, 64, "recompute"),
    "c32_saved": (1, 600, 32, "saved"),
    "c256_recompute": (1, 700, 256, "recompute"),
}


@pytest.mark.parametrize("case", sorted(BWD_CASES))
@pytest.mark.parametrize("H", HEADS)
def test_backward_heads(H, case):
    B, T, chunk, form = BWD_CASES[case]
    w = _wl(H, chunk, B=B, T=T)
    x = gi.fwd_inputs(w, DEV, 7100 + 31 * H + T, with_do=True, with_dS=True, s0_var=0.01)
    _say(f"bwd heads H={H} {case} B={B} T={T} C={chunk} {form}")
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
        assert_close(f64(got), ref, "bf16", name)
    assert_close(f64(dl), r[3], "bf16", "dlambda", batch_axis=None)


@pytest.mark.parametrize("H", HEADS)
def test_decode_heads(H):
    """Plain decode, the page pool (shuffled slots, a padding row) and the decode with
    the fused epilogue, 3 steps each, every step against the oracle."""
    N = 7
    w = gi.Workload(f"heads-{H}", N, 1, H, 96, 192, 0, "bf16", tuple(_lams(H)), 96 ** -0.5, 0.5, 1)
    lam = torch.tensor(w.lambdas, dtype=torch.float32, device=DEV)
    S = gi.decode_state(w, DEV, seed=81 + H, layer=0)
    pool = torch.zeros(10, H, 96, 192, device=DEV)
    slots = torch.tensor([6, 2, -1, 9, 0, 4, 7, 1], dtype=torch.int32, device=DEV)
    live = [r for r in range(8) if int(slots[r]) >= 0]
    pool[slots[live].long()] = S
    S_epi = S.clone()
    Sref = f64(S)
    e = gi.epilogue_inputs(w, DEV, 81 + H, (N,))
    _say(f"decode heads H={H} N={N}, 3 steps (plain, pool, epilogue)")
    for step in range(3):
        d = gi.decode_token_inputs(w, DEV, seed=81 + H, layer=0, step=step)
        o = gla.decode_step(d["q"], d["k"], d["v"], lam, S, scale=w.scale)
        rows = {name: torch.zeros((8,) + tuple(t.shape[1:]), dtype=t.dtype, device=DEV) for name, t in d.items()}
        for name in rows:
            rows[name][live] = d[name]
        op = gla.decode_step_pool(rows["q"], rows["k"], rows["v"], lam, pool, slots, scale=w.scale)
        g = gi.epilogue_inputs(w, DEV, 81 + H, (N,), step=step)["g"]
        y = gla.decode_step_epilogue(d["q"], d["k"], d["v"], g, lam, S_epi, e["norm_w"], e["tier"],
                                     aug_a=e["aug_a"], scale=w.scale)
        torch.cuda.synchronize()
        ro, Sref = oracle.decode(f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(lam), Sref, scale=w.scale)
        ry = oracle.epilogue(f64(d["q"]), f64(d["k"]), f64(d["v"]), ro, f64(g), f64(e["aug_a"]),
                             f64(e["norm_w"]), e["tier"])
        assert_close(f64(o), ro, "bf16", f"o step {step}")
        assert_close(f64(S), Sref, "bf16", f"S step {step}")
        assert_close(f64(op[live]), ro, "bf16", f"pool o step {step}")
        assert torch.count_nonzero(op[2]) == 0, "padding row"
        assert_close(f64(pool[slots[live].long()]), Sref, "bf16", f"pool pages step {step}")
        assert_close(f64(y), ry, "bf16", f"epilogue y step {step}")
        assert_close(f64(S_epi), Sref, "bf16", f"epilogue S step {step}")


@pytest.mark.parametrize("H", HEADS)
@pytest.mark.parametrize("rows", [(1, 1), (1, 333), (3, 250)])
def test_epilogue_pass_heads(H, rows):
    """The standalone epilogue over B x T rows of H heads (row counts that leave the
    last batch of units partial and batches that straddle rows)."""
    B, T = rows
    w = _wl(H, B=B, T=T)
    x = gi.fwd_inputs(w, DEV, 7200 + 31 * H + T)
    o = gi.fwd_inputs(w, DEV, 7300 + 31 * H + T)["v"]   # any bf16 [B, T, H, dv] stands for the output
    e = gi.epilogue_inputs(w, DEV, 7200 + H, (B, T))
    _say(f"epilogue pass heads H={H} B={B} T={T}")
    y = gla.mixer_epilogue(x["q"], x["k"], x["v"], o, e["g"], e["norm_w"], e["tier"], aug_a=e["aug_a"])
    torch.cuda.synchronize()
    ry = oracle.epilogue(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(o), f64(e["g"]), f64(e["aug_a"]),
                         f64(e["norm_w"]), e["tier"])
    assert_close(f64(y), ry, "bf16", "y")


@pytest.mark.parametrize("H", HEADS)
@pytest.mark.parametrize("plan", ["chain", "segments"])
def test_forward_epilogue_heads(H, plan):
    """The forward with the epilogue fused into its output kernel (tiled chain) and the
    forward followed by the epilogue pass (segments)."""
    w = _wl(H, B=1, T=700)
    x = gi.fwd_inputs(w, DEV, 7400 + H, s0_var=0.01)
    e = gi.epilogue_inputs(w, DEV, 7400 + H, (1, 700))
    _say(f"fwd+epilogue heads H={H} plan={plan}")
    y, S = gla.fwd_chunked_epilogue(x["q"], x["k"], x["v"], x["lam"], e["g"], e["norm_w"], e["tier"],
                                    aug_a=e["aug_a"], S0=x["S0"], scale=x["scale"], chunk=128,
                                    plan={"chain": 1 if plan == "chain" else 0})
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), S0=f64(x["S0"]), scale=x["scale"])
    ry = oracle.epilogue(f64(x["q"]), f64(x["k"]), f64(x["v"]), ro, f64(e["g"]), f64(e["aug_a"]), f64(e["norm_w"]),
                         e["tier"])
    assert_close(f64(y), ry, "bf16", "y")
    assert_close(f64(S), rS, "bf16", "S_final")


# ---------------------------------------------------------------- head permutation
# Each (batch, head) unit is computed on its own with its own lambda, whatever its
# place in the launch (its XCD group, its slot in an epilogue batch): permuting the
# heads of every input together with lambda (and the epilogue's per-head parameters)
# permutes every output bit for bit.

PERM = [5, 0, 11, 3, 14, 9, 1, 7, 15, 2, 12, 6, 10, 4, 13, 8]


def _perm_heads(t, axis):
    return None if t is None else t.index_select(axis, torch.tensor(PERM, device=t.device)).contiguous()


@pytest.mark.parametrize("chunk,plan", [(128, {"chain": 1}), (128, {"chain": 0}), (64, None), (256, None),
                                        (32, None)])
def test_head_permutation_forward(chunk, plan):
    w = _wl(16, chunk, B=2, T=500)
    x = gi.fwd_inputs(w, DEV, 7500 + chunk, s0_var=0.01)
    _say(f"fwd head permutation C={chunk} plan={plan}")
    kw = dict(scale=x["scale"], chunk=chunk, plan=plan)
    o, S = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], **kw)
    op, Sp = gla.fwd_chunked(_perm_heads(x["q"], 2), _perm_heads(x["k"], 2), _perm_heads(x["v"], 2),
                             _perm_heads(x["lam"], 0), S0=_perm_heads(x["S0"], 1), **kw)
    torch.cuda.synchronize()
    assert torch.equal(op, _perm_heads(o, 2)), "o"
    assert torch.equal(Sp, _perm_heads(S, 1)), "S_final"


@pytest.mark.parametrize("chunk,form", [(128, "saved"), (128, "recompute"), (64, "saved"), (256, "recompute"),
                                        (32, "recompute")])
def test_head_permutation_backward(chunk, form):
    w = _wl(16, chunk, B=2, T=500)
    x = gi.fwd_inputs(w, DEV, 7600 + chunk, with_do=True, with_dS=True, s0_var=0.01)
    _say(f"bwd head permutation C={chunk} {form}")

    def run(q, k, v, lam, d_o, S0, dS):
        if form == "saved":
            _, _, st = gla.fwd_chunked_states(q, k, v, lam, S0=S0, scale=x["scale"], chunk=chunk)
            return gla.bwd_chunked_states(q, k, v, lam, d_o, st, S0=S0, dS_final=dS, scale=x["scale"], chunk=chunk)
        return gla.bwd_chunked(q, k, v, lam, d_o, S0=S0, dS_final=dS, scale=x["scale"], chunk=chunk)

    base = run(x["q"], x["k"], x["v"], x["lam"], x["do"], x["S0"], x["dS"])
    perm = run(*(_perm_heads(x[n], 2) for n in ("q", "k", "v")), _perm_heads(x["lam"], 0), _perm_heads(x["do"], 2),
               _perm_heads(x["S0"], 1), _perm_heads(x["dS"], 1))
    torch.cuda.synchronize()
    for got, ref, axis, name in zip(perm, base, (2, 2, 2, 0, 1), ("dq", "dk", "dv", "dlambda", "dS0")):
        assert torch.equal(got, _perm_heads(ref, axis)), name


def test_head_permutation_decode_and_epilogue():
    """Decode (plain and with the fused epilogue) and the forward with the fused
    epilogue: heads permuted with lambda, the gate weights a_h and the tier map."""
    N = 9
    w = gi.Workload("heads-perm", N, 1, 16, 96, 192, 0, "bf16", tuple(_lams(16)), 96 ** -0.5, 0.5, 1)
    lam = torch.tensor(w.lambdas, dtype=torch.float32, device=DEV)
    S = gi.decode_state(w, DEV, seed=77, layer=0)
    d = gi.decode_token_inputs(w, DEV, seed=77, layer=0, step=0)
    e = gi.epilogue_inputs(w, DEV, 77, (N,))
    tier_p = [e["tier"][h] for h in PERM]
    _say("decode / epilogue head permutation N=9")
    Sa, Sb = S.clone(), _perm_heads(S, 1)
    o = gla.decode_step(d["q"], d["k"], d["v"], lam, Sa, scale=w.scale)
    op = gla.decode_step(*(_perm_heads(d[n], 1) for n in ("q", "k", "v")), _perm_heads(lam, 0), Sb, scale=w.scale)
    Se, Sf = S.clone(), _perm_heads(S, 1)
    y = gla.decode_step_epilogue(d["q"], d["k"], d["v"], e["g"], lam, Se, e["norm_w"], e["tier"],
                                 aug_a=e["aug_a"], scale=w.scale)
    yp = gla.decode_step_epilogue(*(_perm_heads(d[n], 1) for n in ("q", "k", "v")), _perm_heads(e["g"], 1),
                                  _perm_heads(lam, 0), Sf, e["norm_w"], tier_p, aug_a=_perm_heads(e["aug_a"], 0),
                                  scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(op, _perm_heads(o, 1)) and torch.equal(Sb, _perm_heads(Sa, 1)), "decode"
    assert torch.equal(yp, _perm_heads(y, 1)) and torch.equal(Sf, _perm_heads(Se, 1)), "decode with epilogue"

    wf = _wl(16, B=1, T=700)
    x = gi.fwd_inputs(wf, DEV, 7700, s0_var=0.01)
    ef = gi.epilogue_inputs(wf, DEV, 7700, (1, 700))
    for plan in ({"chain": 1}, {"chain": 0}):
        yf, Sf_ = gla.fwd_chunked_epilogue(x["q"], x["k"], x["v"], x["lam"], ef["g"], ef["norm_w"], ef["tier"],
                                           aug_a=ef["aug_a"], S0=x["S0"], scale=x["scale"], chunk=128, plan=plan)
        yfp, Sfp = gla.fwd_chunked_epilogue(*(_perm_heads(x[n], 2) for n in ("q", "k", "v")), _perm_heads(x["lam"], 0),
                                            _perm_heads(ef["g"], 2), ef["norm_w"], [ef["tier"][h] for h in PERM],
                                            aug_a=_perm_heads(ef["aug_a"], 0), S0=_perm_heads(x["S0"], 1),
                                            scale=x["scale"], chunk=128, plan=plan)
        torch.cuda.synchronize()
        assert torch.equal(yfp, _perm_heads(yf, 2)), f"forward with epilogue y, plan {plan}"
        assert torch.equal(Sfp, _perm_heads(Sf_, 1)), f"forward with epilogue S_final, plan {plan}"

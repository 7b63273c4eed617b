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
    lam = torch.tensor(w.lambdas, dtype=torch.float32, device=DEV)
    _say(f"decode {dtype} dk={dk} dv={dv} N=7, 6 steps")
    for step in range(6):
        d = gi.decode_token_inputs(w, DEV, seed=9, layer=0, step=step)
        o = gla.decode_step(d["q"], d["k"], d["v"], lam, S, scale=w.scale)
        torch.cuda.synchronize()
        ro, Sref = oracle.decode(f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(lam), Sref, scale=w.scale)
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
    """The bench's launch configuration (N=1,280 sequences, H=16, 96x192 fp32 pages, one
    1.5 GB pool slice per layer): 2 layers x 16 steps, the layers' launches interleaved
    as in a decode step, every step checked on a seeded sample of 64 sequences per layer
    against the oracle run from the regenerated initial pages."""
    w = gi.workloads()[4]
    lam = torch.tensor(w.lambdas, dtype=torch.float32, device=DEV)
    layers = (5, 17)
    pools = {L: gi.decode_state(w, DEV, seed=4, layer=L) for L in layers}
    rng = np.random.default_rng(4)
    idx = {L: np.sort(rng.choice(w.B, 64, replace=False)) for L in layers}
    Sref = {L: f64(pools[L][idx[L]]) for L in layers}
    _say("decode N=1280 full width, 2 layers x 16 steps")
    for step in range(16):
        for L in layers:
            d = gi.decode_token_inputs(w, DEV, seed=4, layer=L, step=step)
            o = gla.decode_step(d["q"], d["k"], d["v"], lam, pools[L], scale=w.scale)
            torch.cuda.synchronize()
            i = idx[L]
            ro, Sref[L] = oracle.decode(f64(d["q"][i]), f64(d["k"][i]), f64(d["v"][i]), f64(lam), Sref[L],
                                        scale=w.scale)
            assert_close(f64(o[i]), ro, "bf16", f"o layer {L} step {step}")
            assert_close(f64(pools[L][i]), Sref[L], "bf16", f"S layer {L} step {step}")
    del pools
    torch.cuda.empty_cache()


def test_decode_serving_run_64_steps_sampled_pairs():
    """The whole serving workload as the decode benchmark runs it: the 24-layer pool of
    1,280 sequences (36.2 GB fp32), 64 steps of one launch per layer.  A seeded sample of
    64 (layer, sequence) pairs, all 16 heads each, follows the oracle from the regenerated
    initial pages through every step: the outputs at each step, the pages at steps 16, 32,
    48 and 64."""
    w = gi.workloads()[4]
    L, N, STEPS = w.decode_layers, w.B, 64
    lam = torch.tensor(w.lambdas, dtype=torch.float32, device=DEV)
    pool = torch.empty((L, N, w.H, w.dk, w.dv), dtype=torch.float32, device=DEV)
    for layer in range(L):
        gi.decode_state(w, DEV, seed=4, layer=layer, out=pool[layer])
    rng = np.random.default_rng(404)
    flat = np.sort(rng.choice(L * N, 64, replace=False))
    rows = {layer: flat[flat // N == layer] % N for layer in range(L)}
    rows = {layer: r for layer, r in rows.items() if len(r)}
    Sref = {layer: f64(pool[layer][r]) for layer, r in rows.items()}
    _say(f"decode serving run: {L} layers x {N} sequences x {STEPS} steps, pairs in {len(rows)} layers")
    for step in range(STEPS):
        outs = {}
        for layer in range(L):
            d = gi.decode_token_inputs(w, DEV, seed=4, layer=layer, step=step)
            o = gla.decode_step(d["q"], d["k"], d["v"], lam, pool[layer], scale=w.scale)
            if layer in rows:
                r = torch.as_tensor(rows[layer], device=DEV)
                outs[layer] = (f64(o[r]), f64(d["q"][r]), f64(d["k"][r]), f64(d["v"][r]))
        for layer, (o, q, k, v) in outs.items():
            ro, Sref[layer] = oracle.decode(q, k, v, f64(lam), Sref[layer], scale=w.scale)
            assert_close(o, ro, "bf16", f"o layer {layer} step {step}")
        if step % 16 == 15:
            torch.cuda.synchronize()
            for layer, r in rows.items():
                assert_close(f64(pool[layer][r]), Sref[layer], "bf16", f"pages layer {layer} step {step}")
    del pool
    torch.cuda.empty_cache()


def test_decode_batch_position_invariant():
    w = gi.workloads()[4]
    lam = torch.tensor(w.lambdas, dtype=torch.float32, device=DEV)
    S = gi.decode_state(w, DEV, seed=8, layer=0, N=9)
    d = gi.decode_token_inputs(w, DEV, seed=8, layer=0, step=0, N=9)
    S1 = S[4:5].clone()
    o_all = gla.decode_step(d["q"], d["k"], d["v"], lam, S, scale=w.scale)
    o_one = gla.decode_step(d["q"][4:5].contiguous(), d["k"][4:5].contiguous(), d["v"][4:5].contiguous(),
                            lam, S1, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_all[4:5], o_one) and torch.equal(S[4:5], S1)


# ---------------------------------------------------------------- page pool


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_pool_matches_oracle_with_padding(dtype):
    """gla_decode_step_pool over a 23-page pool: a fixed-width batch of 16 rows
    holding 11 live sequences at shuffled page slots and 5 padding rows (slot -1,
    and out-of-range slots 23 and -7).  Live rows follow the oracle step by step
    on their own pages; padding rows give zero outputs; pages no row names stay
    bit-identical."""
    w = gi.workloads()[4]
    w = gi.Workload(w.name, 23, 1, 16, 96, 192, 0, dtype, w.lambdas, 96 ** -0.5, w.s0_var, 24)
    lam = torch.tensor(w.lambdas, dtype=torch.float32, device=DEV)
    pool = gi.decode_state(w, DEV, seed=31, layer=0)                      # [23, H, dk, dv]
    untouched = pool.clone()
    rng = np.random.default_rng(31)
    live = rng.permutation(23)[:11]                                       # 11 distinct pages
    rows = np.full(16, -1, dtype=np.int32)
    pos = rng.permutation(16)[:11]
    rows[pos] = live
    pad = [p for p in range(16) if p not in pos]
    rows[pad[0]] = 23                                                     # out of range -> padding
    rows[pad[1]] = -7
    slots = torch.tensor(rows, device=DEV)
    Sref = {int(s): f64(pool[int(s)]) for s in live}
    _say(f"decode pool {dtype} P=23 N=16 (11 live), 4 steps")
    for step in range(4):
        d = gi.decode_token_inputs(w, DEV, seed=31, layer=0, step=step, N=16)
        o = gla.decode_step_pool(d["q"], d["k"], d["v"], lam, pool, slots, scale=w.scale)
        torch.cuda.synchronize()
        for r in range(16):
            s = int(rows[r])
            if not 0 <= s < 23:
                assert torch.count_nonzero(o[r]) == 0, f"padding row {r} step {step}"
                continue
            ro, Sref[s] = oracle.decode(f64(d["q"][r:r + 1]), f64(d["k"][r:r + 1]), f64(d["v"][r:r + 1]),
                                        f64(lam), Sref[s][None], scale=w.scale)
            Sref[s] = Sref[s][0]
            assert_close(f64(o[r:r + 1]), ro, dtype, f"o row {r} step {step}")
            assert_close(f64(pool[s]), Sref[s], dtype, f"page {s} step {step}")
    others = [p for p in range(23) if p not in set(int(s) for s in live)]
    assert torch.equal(pool[others], untouched[others]), "pages not in the batch changed"


def test_decode_pool_batch_invariant_bitwise():
    """A sequence's output row and page after one pool step are bit-identical to
    decoding it alone with gla_decode_step, whatever its row, its page slot and
    the padding around it."""
    w = gi.workloads()[4]
    lam = torch.tensor(w.lambdas, dtype=torch.float32, device=DEV)
    S = gi.decode_state(w, DEV, seed=33, layer=1, N=12)
    d = gi.decode_token_inputs(w, DEV, seed=33, layer=1, step=0, N=12)
    solo_S = S.clone()
    solo_o = gla.decode_step(d["q"], d["k"], d["v"], lam, solo_S, scale=w.scale)  # row n on page n
    # the same 12 sequences in a 16-wide batch, reversed order, pages shuffled into a 20-page pool
    perm = np.random.default_rng(33).permutation(20)[:12]
    pool = torch.zeros(20, 16, 96, 192, device=DEV)
    pool[torch.tensor(perm, device=DEV)] = S
    order = list(range(11, -1, -1))
    rows = np.full(16, -1, dtype=np.int32)
    q = torch.zeros(16, 16, 96, dtype=d["q"].dtype, device=DEV)
    k = torch.zeros_like(q)
    v = torch.zeros(16, 16, 192, dtype=d["v"].dtype, device=DEV)
    for r, n in enumerate(order):
        rows[r + 2] = perm[n]
        q[r + 2], k[r + 2], v[r + 2] = d["q"][n], d["k"][n], d["v"][n]
    o = gla.decode_step_pool(q, k, v, lam, pool, torch.tensor(rows, device=DEV), scale=w.scale)
    torch.cuda.synchronize()
    for r, n in enumerate(order):
        assert torch.equal(o[r + 2], solo_o[n]), f"output of sequence {n}"
        assert torch.equal(pool[int(perm[n])], solo_S[n]), f"page of sequence {n}"


def test_prefill_hands_over_into_pool_then_decodes():
    """Prefill -> decode handoff: gla_fwd_chunked writes its final states straight
    into a page range of the pool (S_final pointer = page `first`), then pool
    decode steps continue the sequences; the result equals one forward over
    prompt + generated tokens (oracle)."""
    w = gi.workloads()[1]
    B, Tp, Tg = 3, 300, 5
    x = gi.fwd_inputs(w, DEV, seed=35, B=B, T=Tp + Tg, s0_var=0.1)
    pool = torch.zeros(8, 16, 96, 192, device=DEV)
    first = 4
    _say("prefill into pool pages 4..6, then 5 pool decode steps")
    gla.fwd_chunked(x["q"][:, :Tp].contiguous(), x["k"][:, :Tp].contiguous(), x["v"][:, :Tp].contiguous(),
                    x["lam"], S0=x["S0"], scale=x["scale"], chunk=128, S_final=pool[first:first + B])
    slots = torch.tensor([first + b for b in range(B)], dtype=torch.int32, device=DEV)
    outs = []
    for t in range(Tp, Tp + Tg):
        outs.append(gla.decode_step_pool(x["q"][:, t].contiguous(), x["k"][:, t].contiguous(),
                                         x["v"][:, t].contiguous(), x["lam"], pool, slots, scale=x["scale"]))
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), S0=f64(x["S0"]), scale=x["scale"])
    assert_close(f64(torch.stack(outs, 1)), ro[:, Tp:], "bf16", "decoded outputs")
    assert_close(f64(pool[first:first + B]), rS, "bf16", "pages after decode")


def test_decode_page_decay_schedule():
    """Decode steps under the pages' geometric half-life schedule (lambda_0 = 0.5)."""
    w = gi.workloads()[4]
    w = gi.Workload(w.name, 9, 1, 16, 96, 192, 0, "bf16", tuple(gi.page_lambdas(16)), 96 ** -0.5, w.s0_var, 24)
    S = gi.decode_state(w, DEV, seed=37, layer=0)
    Sref = f64(S)
    lam = torch.tensor(w.lambdas, dtype=torch.float32, device=DEV)
    for step in range(8):
        d = gi.decode_token_inputs(w, DEV, seed=37, layer=0, step=step)
        o = gla.decode_step(d["q"], d["k"], d["v"], lam, S, scale=w.scale)
        torch.cuda.synchronize()
        ro, Sref = oracle.decode(f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(lam), Sref, scale=w.scale)
        assert_close(f64(o), ro, "bf16", f"o step {step}")
        assert_close(f64(S), Sref, "bf16", f"S step {step}")

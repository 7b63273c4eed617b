"""GPU parity of the mixer epilogue (gla_mixer_epilogue and the fused
gla_decode_step_epilogue) against the fp64 oracle, through the C ABI."""
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


def _wl(dtype, dk, dv, H=16):
    lam = tuple(gi.laplace_lambdas(H))
    return gi.Workload(f"epi-{dtype}-{dk}x{dv}", 1, 1, H, dk, dv, 0, dtype, lam, dk ** -0.5)


def _rows(w, seed, lead):
    dt = gi.torch_dtype(w.dtype)
    q = gi.normal(tuple(lead) + (w.H, w.dk), 1.0 / w.dk, dt, DEV, seed, "q")
    k = gi.normal(tuple(lead) + (w.H, w.dk), 1.0 / w.dk, dt, DEV, seed, "k")
    v = gi.normal(tuple(lead) + (w.H, w.dv), 1.0, dt, DEV, seed, "v")
    o = gi.normal(tuple(lead) + (w.H, w.dv), 0.3, dt, DEV, seed, "do")
    return q, k, v, o


def _ref(q, k, v, o, e, aug=True, eps=1e-6):
    a = f64(e["aug_a"]) if aug else None
    return oracle.epilogue(f64(q), f64(k), f64(v), f64(o), f64(e["g"]), a, f64(e["norm_w"]), e["tier"], eps=eps)


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 96, 192), ("f32", 96, 192), ("bf16", 16, 32), ("f32", 16, 32)])
@pytest.mark.parametrize("aug", [True, False])
def test_epilogue_matches_oracle(dtype, dk, dv, aug):
    w = _wl(dtype, dk, dv)
    lead = (2, 37)                                   # 74 rows x 16 heads: a ragged last workgroup
    q, k, v, o = _rows(w, 21, lead)
    e = gi.epilogue_inputs(w, DEV, 21, lead)
    _say(f"epilogue {dtype} dk={dk} dv={dv} aug={aug} rows={lead}")
    y = gla.mixer_epilogue(q, k, v, o, e["g"], e["norm_w"], e["tier"], aug_a=e["aug_a"] if aug else None)
    torch.cuda.synchronize()
    assert_close(f64(y), _ref(q, k, v, o, e, aug), dtype, "y")


@pytest.mark.parametrize("tiers", ["one", "per_head", "alternate", "contiguous"])
def test_epilogue_tier_maps(tiers):
    w = _wl("bf16", 96, 192)
    lead = (3, 5)
    q, k, v, o = _rows(w, 5, lead)
    n = {"one": 1, "per_head": 16, "alternate": 3, "contiguous": 4}[tiers]
    e = gi.epilogue_inputs(w, DEV, 5, lead, n_tiers=n)
    if tiers == "alternate":
        e["tier"] = [(2 * h + 1) % 3 for h in range(w.H)]
    elif tiers == "per_head":
        e["tier"] = list(range(w.H))[::-1]
    _say(f"epilogue tiers={tiers}")
    y = gla.mixer_epilogue(q, k, v, o, e["g"], e["norm_w"], e["tier"], aug_a=e["aug_a"])
    torch.cuda.synchronize()
    assert_close(f64(y), _ref(q, k, v, o, e), "bf16", f"y tiers={tiers}")


def test_epilogue_saturated_gate_and_large_eps():
    """Gate logits of size ~30 (sigmoid saturates to 0 or 1) and eps far above the
    mean square (the norm becomes a plain 1/sqrt(eps) scale)."""
    w = _wl("f32", 96, 192)
    lead = (40,)
    q, k, v, o = _rows(w, 8, lead)
    e = gi.epilogue_inputs(w, DEV, 8, lead, aug_var=900.0 * w.dk)
    for eps in (1e-6, 1e4):
        _say(f"epilogue saturated eps={eps}")
        y = gla.mixer_epilogue(q, k, v, o, e["g"], e["norm_w"], e["tier"], aug_a=e["aug_a"], eps=eps)
        torch.cuda.synchronize()
        assert_close(f64(y), _ref(q, k, v, o, e, eps=eps), "f32", f"y eps={eps}")


def test_epilogue_in_place_and_empty():
    w = _wl("bf16", 96, 192)
    lead = (9,)
    q, k, v, o = _rows(w, 3, lead)
    e = gi.epilogue_inputs(w, DEV, 3, lead)
    ref = _ref(q, k, v, o, e)
    y = gla.mixer_epilogue(q, k, v, o, e["g"], e["norm_w"], e["tier"], aug_a=e["aug_a"], y=o)
    torch.cuda.synchronize()
    assert y.data_ptr() == o.data_ptr()
    assert_close(f64(y), ref, "bf16", "y in place")
    z = torch.empty((0, w.H, w.dk), dtype=torch.bfloat16, device=DEV)
    zv = torch.empty((0, w.H, w.dv), dtype=torch.bfloat16, device=DEV)
    out = gla.mixer_epilogue(z, z, zv, zv, zv, e["norm_w"], e["tier"], aug_a=e["aug_a"])
    assert out.shape == (0, w.H, w.dv)


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 96, 192), ("f32", 96, 192), ("bf16", 16, 32), ("f32", 16, 32)])
@pytest.mark.parametrize("rows", [1, 37, 1000])
def test_epilogue_writes_only_its_rows(dtype, dk, dv, rows):
    """y is a view at the start of a larger buffer: the guard rows after it (more than
    the workgroups' strided batches reach) keep their bits."""
    w = _wl(dtype, dk, dv)
    q, k, v, o = _rows(w, 40 + rows, (rows,))
    e = gi.epilogue_inputs(w, DEV, 40 + rows, (rows,))
    guard = 8192
    big = torch.full((rows + guard, w.H, w.dv), 7.0, dtype=q.dtype, device=DEV)
    _say(f"epilogue guard {dtype} dk={dk} dv={dv} rows={rows}")
    y = gla.mixer_epilogue(q, k, v, o, e["g"], e["norm_w"], e["tier"], aug_a=e["aug_a"], y=big[:rows])
    torch.cuda.synchronize()
    assert_close(f64(y), _ref(q, k, v, o, e), dtype, "y")
    assert bool((big[rows:] == 7.0).all()), "epilogue wrote past its rows"


@pytest.mark.parametrize("dtype,chunk", [("bf16", 128), ("bf16", 64)])
def test_forward_then_epilogue_full_layer(dtype, chunk):
    """The Laplace layer's prefill (B=1, T=2048, H=16, 96x192): the forward's output
    fed to the epilogue; every row checked against the oracle's epilogue of that o,
    and the end-to-end y against the oracle's forward followed by its epilogue."""
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, seed=31)
    e = gi.epilogue_inputs(w, DEV, 31, (1, w.T))
    _say(f"forward+epilogue {dtype} C={chunk} T={w.T}")
    o, _ = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], scale=x["scale"], chunk=chunk, S_final=False)
    y = gla.mixer_epilogue(x["q"], x["k"], x["v"], o, e["g"], e["norm_w"], e["tier"], aug_a=e["aug_a"])
    torch.cuda.synchronize()
    assert_close(f64(y), _ref(x["q"], x["k"], x["v"], o, e), dtype, "y of the GPU readout")
    ro, _ = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), scale=x["scale"])
    ry = oracle.epilogue(f64(x["q"]), f64(x["k"]), f64(x["v"]), ro, f64(e["g"]), f64(e["aug_a"]),
                         f64(e["norm_w"]), e["tier"])
    assert_close(f64(y), ry, dtype, "y end to end")


def test_epilogue_training_width_sampled():
    """The training step's width (B=8, T=2048): 262,144 (row, head) units in one launch,
    checked on a seeded sample of 512 rows."""
    w = gi.workloads()[2]
    lead = (w.B, w.T)
    q, k, v, o = _rows(w, 17, lead)
    e = gi.epilogue_inputs(w, DEV, 17, lead)
    _say("epilogue B=8 T=2048")
    y = gla.mixer_epilogue(q, k, v, o, e["g"], e["norm_w"], e["tier"], aug_a=e["aug_a"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(17)
    idx = np.sort(rng.choice(w.B * w.T, 512, replace=False))
    flat = lambda t: t.reshape(w.B * w.T, w.H, -1)[idx]
    es = dict(e, g=flat(e["g"]))
    assert_close(f64(flat(y)), _ref(flat(q), flat(k), flat(v), flat(o), es), "bf16", "y sampled")


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 96, 192), ("f32", 96, 192), ("bf16", 16, 32), ("f32", 16, 32)])
def test_decode_epilogue_matches_oracle(dtype, dk, dv):
    w = gi.workloads()[4]
    w = gi.Workload(w.name, 7, 1, 16, dk, dv, 0, dtype, w.lambdas, dk ** -0.5, w.s0_var, 24)
    lam = torch.tensor(w.lambdas, device=DEV)
    S = gi.decode_state(w, DEV, seed=6, layer=0)
    Sref = f64(S)
    e = gi.epilogue_inputs(w, DEV, 6, (w.B,))
    _say(f"decode+epilogue {dtype} dk={dk} dv={dv} N=7, 5 steps")
    for step in range(5):
        d = gi.decode_token_inputs(w, DEV, seed=6, layer=0, step=step)
        g = gi.epilogue_inputs(w, DEV, 6, (w.B,), step=step)["g"]
        y = gla.decode_step_epilogue(d["q"], d["k"], d["v"], g, lam, S, e["norm_w"], e["tier"],
                                     aug_a=e["aug_a"], scale=w.scale)
        torch.cuda.synchronize()
        ro, Sref = oracle.decode(f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(lam), Sref, scale=w.scale)
        ry = oracle.epilogue(f64(d["q"]), f64(d["k"]), f64(d["v"]), ro, f64(g), f64(e["aug_a"]),
                             f64(e["norm_w"]), e["tier"])
        assert_close(f64(y), ry, dtype, f"y step {step}")
        assert_close(f64(S), Sref, dtype, f"S step {step}")


def test_decode_epilogue_pool_padding_and_invariance():
    """Pool form: padding rows give zero y and leave every page alone; a sequence's y
    and page bits do not depend on the batch it is decoded in; a = None works."""
    w = gi.workloads()[4]
    lam = torch.tensor(w.lambdas, device=DEV)
    P = 6
    pool = gi.decode_state(w, DEV, seed=2, layer=1, N=P)
    pool2 = pool.clone()
    slots = torch.tensor([4, -1, 0, 9, 2], dtype=torch.int32, device=DEV)   # -1 and 9: padding
    d = gi.decode_token_inputs(w, DEV, seed=2, layer=1, step=0, N=5)
    e = gi.epilogue_inputs(w, DEV, 2, (5,))
    _say("decode+epilogue pool N=5 P=6")
    y = gla.decode_step_epilogue(d["q"], d["k"], d["v"], e["g"], lam, pool, e["norm_w"], e["tier"],
                                 aug_a=None, scale=w.scale, slots=slots)
    torch.cuda.synchronize()
    live = [0, 2, 4]
    page = {0: 4, 2: 0, 4: 2}
    ro, rS = oracle.decode(f64(d["q"][live]), f64(d["k"][live]), f64(d["v"][live]), f64(lam),
                           f64(pool2[[page[n] for n in live]]), scale=w.scale)
    ry = oracle.epilogue(f64(d["q"][live]), f64(d["k"][live]), f64(d["v"][live]), ro, f64(e["g"][live]), None,
                         f64(e["norm_w"]), e["tier"])
    assert_close(f64(y[live]), ry, "bf16", "y live rows")
    assert torch.count_nonzero(y[[1, 3]]) == 0
    assert_close(f64(pool[[page[n] for n in live]]), rS, "bf16", "pages")
    untouched = [p for p in range(P) if p not in page.values()]
    assert torch.equal(pool[untouched], pool2[untouched])
    # the same sequence alone, on a copy of its page
    one = pool2[4:5].clone()
    y1 = gla.decode_step_epilogue(d["q"][:1].contiguous(), d["k"][:1].contiguous(), d["v"][:1].contiguous(),
                                  e["g"][:1].contiguous(), lam, one, e["norm_w"], e["tier"], aug_a=None,
                                  scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(y1[0], y[0])
    assert torch.equal(one[0], pool[4])


def test_decode_epilogue_full_width_sampled():
    """The decode bench's launch (N=1,280, H=16, 96x192 pages) with the fused epilogue:
    2 steps, checked on a seeded sample of 64 sequences."""
    w = gi.workloads()[4]
    lam = torch.tensor(w.lambdas, device=DEV)
    S = gi.decode_state(w, DEV, seed=13, layer=3)
    e = gi.epilogue_inputs(w, DEV, 13, (w.B,))
    rng = np.random.default_rng(13)
    idx = np.sort(rng.choice(w.B, 64, replace=False))
    Sref = f64(S[idx])
    _say("decode+epilogue N=1280, 2 steps")
    for step in range(2):
        d = gi.decode_token_inputs(w, DEV, seed=13, layer=3, step=step)
        y = gla.decode_step_epilogue(d["q"], d["k"], d["v"], e["g"], lam, S, e["norm_w"], e["tier"],
                                     aug_a=e["aug_a"], scale=w.scale)
        torch.cuda.synchronize()
        ro, Sref = oracle.decode(f64(d["q"][idx]), f64(d["k"][idx]), f64(d["v"][idx]), f64(lam), Sref,
                                 scale=w.scale)
        ry = oracle.epilogue(f64(d["q"][idx]), f64(d["k"][idx]), f64(d["v"][idx]), ro, f64(e["g"][idx]),
                             f64(e["aug_a"]), f64(e["norm_w"]), e["tier"])
        assert_close(f64(y[idx]), ry, "bf16", f"y step {step}")
        assert_close(f64(S[idx]), Sref, "bf16", f"S step {step}")
    del S
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,T,chunk,chain", [(1, 2048, 128, 1), (1, 2048, 128, 0), (1, 300, 128, 1),
                                             (1, 300, 128, 0), (2, 700, 128, None), (1, 2048, 64, None),
                                             (2, 700, 256, None)])
@pytest.mark.parametrize("aug", [True, False])
def test_forward_epilogue_matches_oracle(B, T, chunk, chain, aug):
    """gla_fwd_chunked_epilogue: fused into the output kernel on tiled-chain plans
    (chain = "1"), forward then the epilogue pass otherwise; y and S_final against the
    oracle's forward followed by its epilogue."""
    plan = None if chain is None else {"chain": chain}
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, seed=51 + T, B=B, T=T, s0_var=0.01)
    e = gi.epilogue_inputs(w, DEV, 51 + T, (B, T))
    a = e["aug_a"] if aug else None
    _say(f"fwd+epilogue B={B} T={T} C={chunk} chain={chain} aug={aug}")
    y, S = gla.fwd_chunked_epilogue(x["q"], x["k"], x["v"], x["lam"], e["g"], e["norm_w"], e["tier"], aug_a=a,
                                    S0=x["S0"], scale=x["scale"], chunk=chunk, plan=plan)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), S0=f64(x["S0"]), scale=x["scale"])
    ry = oracle.epilogue(f64(x["q"]), f64(x["k"]), f64(x["v"]), ro, f64(e["g"]), None if a is None else f64(a),
                         f64(e["norm_w"]), e["tier"])
    assert_close(f64(y), ry, "bf16", "y")
    assert_close(f64(S), rS, "bf16", "S_final")


def test_forward_epilogue_fp32_tiny():
    w = gi.workloads()[0]
    x = gi.fwd_inputs(w, DEV, seed=3)
    e = gi.epilogue_inputs(w, DEV, 3, (w.B, w.T), n_tiers=2)
    y, S = gla.fwd_chunked_epilogue(x["q"], x["k"], x["v"], x["lam"], e["g"], e["norm_w"], e["tier"],
                                    aug_a=e["aug_a"], scale=x["scale"], chunk=w.chunk)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["lam"]), scale=x["scale"])
    ry = oracle.epilogue(f64(x["q"]), f64(x["k"]), f64(x["v"]), ro, f64(e["g"]), f64(e["aug_a"]), f64(e["norm_w"]),
                         e["tier"])
    assert_close(f64(y), ry, "f32", "y")
    assert_close(f64(S), rS, "f32", "S_final")

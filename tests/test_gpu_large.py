"""GPU parity with tensors larger than 2 GiB (the maximum-size end of the hot path).

Every token-major tensor of a 48-sequence, 8,192-token batch of the Laplace layer's
heads is beyond 2^31 bytes for v, o, do and dv (48 x 8192 x 16 x 192 bf16 = 2.4 GB),
and a decode pool of 2,048 sequences holds 2.4 GB of fp32 pages: batch and page offsets
must be formed in 64 bits everywhere.  The results of the first and the last sequences
(or a sample of decode rows) are compared element by element with the fp64 oracle on the
bits the kernels consumed; the oracle runs on those sequences alone.
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
B, T = 48, 8192
PICK = [0, B - 1]


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _pick(t, idx=PICK):
    return f64(t[idx])


@pytest.fixture(scope="module")
def big():
    w = gi.workloads()[1]
    x = gi.fwd_inputs(w, DEV, 9001, B=B, T=T, with_do=True, s0_var=0.01)
    assert x["v"].numel() * x["v"].element_size() > 2 ** 31
    yield w, x
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("plan", [None, {"chain": 1}])
def test_forward_beyond_2gib(big, plan):
    w, x = big
    _say(f"fwd B={B} T={T} plan={plan} (v, o: {x['v'].numel() * 2 / 2 ** 30:.2f} GiB)")
    o, S = gla.fwd_chunked(x["q"], x["k"], x["v"], x["lam"], S0=x["S0"], scale=x["scale"], chunk=128, plan=plan)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(_pick(x["q"]), _pick(x["k"]), _pick(x["v"]), f64(x["lam"]), S0=_pick(x["S0"]),
                        scale=x["scale"])
    assert_close(_pick(o), ro, "bf16", "o")
    assert_close(_pick(S), rS, "bf16", "S_final")
    del o, S


def test_training_pair_beyond_2gib(big):
    w, x = big
    _say(f"fwd+bwd with saved states B={B} T={T}")
    args = (x["q"], x["k"], x["v"], x["lam"])
    _, _, st = gla.fwd_chunked_states(*args, S0=x["S0"], scale=x["scale"], chunk=128, S_final=False)
    dq, dk, dv, dl, dS0 = gla.bwd_chunked_states(*args, x["do"], st, S0=x["S0"], scale=x["scale"], chunk=128)
    torch.cuda.synchronize()
    assert torch.isfinite(dl).all()
    r = oracle.bwd(_pick(x["q"]), _pick(x["k"]), _pick(x["v"]), f64(x["lam"]), _pick(x["do"]), S0=_pick(x["S0"]),
                   scale=x["scale"])
    for got, ref, name in zip((dq, dk, dv, dS0), (r[0], r[1], r[2], r[4]), ("dq", "dk", "dv", "dS0")):
        assert_close(_pick(got), ref, "bf16", name)
    del st, dq, dk, dv, dl, dS0


def test_epilogue_beyond_2gib(big):
    w, x = big
    e = gi.epilogue_inputs(w, DEV, 9002, (B, T))
    _say(f"epilogue pass B={B} T={T}")
    y = gla.mixer_epilogue(x["q"], x["k"], x["v"], x["v"], e["g"], e["norm_w"], e["tier"], aug_a=e["aug_a"])
    torch.cuda.synchronize()
    ry = oracle.epilogue(_pick(x["q"]), _pick(x["k"]), _pick(x["v"]), _pick(x["v"]), _pick(e["g"]), f64(e["aug_a"]),
                         f64(e["norm_w"]), e["tier"])
    assert_close(_pick(y), ry, "bf16", "y")
    del y, e


def test_conv_beyond_2gib():
    c = gi.conv_inputs(B, T, 3072, "bf16", DEV, seed=9003)
    assert c["x"].numel() * 2 > 2 ** 31
    _say(f"conv prefill B={B} T={T} D=3072")
    y, wo = gla.conv1d_silu(c["x"], c["w"], c["bias"], c["win"])
    torch.cuda.synchronize()
    ry, rw = oracle.conv1d(_pick(c["x"]), f64(c["w"]), f64(c["bias"]), _pick(c["win"]))
    assert_close(_pick(y), ry, "bf16", "y")
    assert np.array_equal(_pick(wo), rw), "window carry"
    del c, y, wo
    torch.cuda.empty_cache()


def test_decode_pages_beyond_2gib():
    """2,048 sequences of 16 pages (2.4 GB fp32), plain and through a pool of 2,100
    slots in shuffled order; rows sampled across the batch."""
    N = 2048
    w = gi.workloads()[4]
    w = gi.Workload(w.name, N, 1, 16, 96, 192, 0, "bf16", w.lambdas, w.scale, w.s0_var, 1)
    lam = torch.tensor(w.lambdas, dtype=torch.float32, device=DEV)
    S = gi.decode_state(w, DEV, seed=9004, layer=0)
    assert S.numel() * 4 > 2 ** 31
    d = gi.decode_token_inputs(w, DEV, seed=9004, layer=0, step=0)
    rows = [0, 1, 777, 1500, N - 1]
    S_rows = f64(S[rows])
    slots = torch.tensor(np.random.default_rng(9004).permutation(2100)[:N], dtype=torch.int32, device=DEV)
    pool = torch.empty(2100, 16, 96, 192, device=DEV)
    pool[slots.long()] = S
    _say(f"decode N={N} (pages {S.numel() * 4 / 2 ** 30:.2f} GiB), plain and pool")
    o = gla.decode_step(d["q"], d["k"], d["v"], lam, S, scale=w.scale)
    op = gla.decode_step_pool(d["q"], d["k"], d["v"], lam, pool, slots, scale=w.scale)
    torch.cuda.synchronize()
    ro, rS = oracle.decode(f64(d["q"][rows]), f64(d["k"][rows]), f64(d["v"][rows]), f64(lam), S_rows, scale=w.scale)
    assert_close(f64(o[rows]), ro, "bf16", "o")
    assert_close(f64(S[rows]), rS, "bf16", "S")
    assert_close(f64(op[rows]), ro, "bf16", "pool o")
    assert_close(f64(pool[slots[rows].long()]), rS, "bf16", "pool pages")
    del S, pool
    torch.cuda.empty_cache()

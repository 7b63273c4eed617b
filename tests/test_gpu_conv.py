"""GPU parity of the depth-wise causal conv + SiLU (gla_conv1d_silu and
gla_conv1d_silu_decode) against the fp64 oracle, through the C ABI."""
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


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [264, 1032, 3072])
@pytest.mark.parametrize("window,bias", [(False, True), (True, True), (True, False)])
def test_conv_prefill_matches_oracle(dtype, D, window, bias):
    B, T = 2, 77                                  # runs of 32, 32 and a ragged 13
    c = gi.conv_inputs(B, T, D, dtype, DEV, seed=D + T)
    win = c["win"] if window else None
    b = c["bias"] if bias else None
    _say(f"conv prefill {dtype} D={D} window={window} bias={bias}")
    y, wo = gla.conv1d_silu(c["x"], c["w"], b, win)
    torch.cuda.synchronize()
    ry, rw = oracle.conv1d(f64(c["x"]), f64(c["w"]), None if b is None else f64(b),
                           None if win is None else f64(win))
    assert_close(f64(y), ry, dtype, "y")
    assert np.array_equal(f64(wo), rw), "window carry"


@pytest.mark.parametrize("T", [0, 1, 3, 4, 5, 32, 33])
def test_conv_short_and_boundary_lengths(T):
    """Lengths around the width and the 32-token run; T = 0 passes the window through."""
    B, D = 3, 3072
    c = gi.conv_inputs(B, T, D, "bf16", DEV, seed=100 + T)
    _say(f"conv prefill T={T}")
    y, wo = gla.conv1d_silu(c["x"], c["w"], c["bias"], c["win"])
    torch.cuda.synchronize()
    ry, rw = oracle.conv1d(f64(c["x"]), f64(c["w"]), f64(c["bias"]), f64(c["win"]))
    if T:
        assert_close(f64(y), ry, "bf16", "y")
    assert np.array_equal(f64(wo), rw), "window carry"


def test_conv_in_place_window_and_split_resume_bitwise():
    """win_out may be win_in; prefill in two parts through the window gives the same
    bits as one prefill (the same four fmas per output either way)."""
    B, T, D = 2, 200, 1032
    c = gi.conv_inputs(B, T, D, "bf16", DEV, seed=5)
    y, wo = gla.conv1d_silu(c["x"], c["w"], c["bias"], c["win"])
    win = c["win"].clone()
    for t1 in (70, 3):
        w2 = c["win"].clone()
        ya, _ = gla.conv1d_silu(c["x"][:, :t1].contiguous(), c["w"], c["bias"], w2, win_out=w2)
        yb, _ = gla.conv1d_silu(c["x"][:, t1:].contiguous(), c["w"], c["bias"], w2, win_out=w2)
        torch.cuda.synchronize()
        assert torch.equal(torch.cat([ya, yb], 1), y), f"split at {t1}"
        assert torch.equal(w2, wo), f"window after split at {t1}"
    assert torch.equal(win, c["win"])


def test_conv_full_training_width_sampled():
    """The Laplace layer's conv at the training width (B=8, T=2048, D=3,072, bf16) in one
    launch; two whole sequences checked against the oracle."""
    B, T, D = 8, 2048, 3072
    c = gi.conv_inputs(B, T, D, "bf16", DEV, seed=9)
    _say("conv prefill B=8 T=2048 D=3072")
    y, wo = gla.conv1d_silu(c["x"], c["w"], c["bias"], c["win"])
    torch.cuda.synchronize()
    for b in (2, 7):
        ry, rw = oracle.conv1d(f64(c["x"][b:b + 1]), f64(c["w"]), f64(c["bias"]), f64(c["win"][b:b + 1]))
        assert_close(f64(y[b:b + 1]), ry, "bf16", f"y[{b}]")
        assert np.array_equal(f64(wo[b:b + 1]), rw)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv_decode_steps_match_oracle_and_prefill(dtype):
    N, D, steps = 5, 3072, 6
    c = gi.conv_inputs(N, steps, D, dtype, DEV, seed=12)
    win = c["win"].clone()
    rwin = f64(c["win"])
    ys = []
    _say(f"conv decode {dtype} N={N} {steps} steps")
    for t in range(steps):
        yt = gla.conv1d_silu_decode(c["x"][:, t].contiguous(), c["w"], c["bias"], win)
        torch.cuda.synchronize()
        ry, rwin = oracle.conv1d_decode(f64(c["x"][:, t]), f64(c["w"]), f64(c["bias"]), rwin)
        assert_close(f64(yt), ry, dtype, f"y step {t}")
        assert np.array_equal(f64(win), rwin), f"window step {t}"
        ys.append(yt)
    yp, wp = gla.conv1d_silu(c["x"], c["w"], c["bias"], c["win"])
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(ys, 1), yp), "decode steps == prefill (bits)"
    assert torch.equal(win, wp)


def test_conv_decode_pool_padding_and_invariance():
    N, D, P = 4, 3072, 6
    c = gi.conv_inputs(N, 1, D, "bf16", DEV, seed=21)
    pool = gi.conv_inputs(P, 1, D, "bf16", DEV, seed=22)["win"]
    pool0 = pool.clone()
    slots = torch.tensor([3, -1, 0, 6], dtype=torch.int32, device=DEV)
    x = c["x"][:, 0].contiguous()
    _say("conv decode pool")
    y = gla.conv1d_silu_decode(x, c["w"], c["bias"], pool, slots=slots)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y[[1, 3]]) == 0
    for n, s in ((0, 3), (2, 0)):
        ry, rw = oracle.conv1d_decode(f64(x[n:n + 1]), f64(c["w"]), f64(c["bias"]), f64(pool0[s:s + 1]))
        assert_close(f64(y[n:n + 1]), ry, "bf16", f"y row {n}")
        assert np.array_equal(f64(pool[s:s + 1]), rw)
        alone = pool0[s:s + 1].clone()
        y1 = gla.conv1d_silu_decode(x[n:n + 1].contiguous(), c["w"], c["bias"], alone)
        torch.cuda.synchronize()
        assert torch.equal(y1[0], y[n]) and torch.equal(alone[0], pool[s])
    for s in (1, 2, 4, 5):
        assert torch.equal(pool[s], pool0[s])

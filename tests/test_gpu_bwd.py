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


def _run(w, seed, B=None, T=None, chunk=None, s0_var=None, with_dS=True):
    chunk = chunk or w.chunk
    x = gi.fwd_inputs(w, DEV, seed, B=B, T=T, with_do=True, with_dS=with_dS, s0_var=s0_var)
    _say(f"bwd {w.name} dtype={w.dtype} B={x['q'].shape[0]} T={x['q'].shape[1]} C={chunk} "
         f"S0={'yes' if x['S0'] is not None else 'no'} dS_T={'yes' if with_dS else 'no'} seed={seed}")
    dq, dk, dv, dl, dS0 = gla.bwd_chunked(x["q"], x["k"], x["v"], x["lam"], x["do"], S0=x["S0"],
                                          dS_final=x.get("dS"), scale=x["scale"], chunk=chunk)
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


@pytest.mark.parametrize("chunk", [128, 64])
@pytest.mark.parametrize("T", [1, 100, 300, 1000])
def test_bf16_ragged_with_states(chunk, T):
    _run(gi.workloads()[1], seed=70 + T + chunk, B=2, T=T, chunk=chunk, s0_var=0.01)


@pytest.mark.parametrize("nseg", [1, 3, 5])
def test_bf16_segment_split(nseg, monkeypatch):
    monkeypatch.setenv("GLA_FWD_SEGMENTS", str(nseg))
    _run(gi.workloads()[1], seed=90 + nseg, B=1, T=1000, chunk=64, s0_var=0.01)


@pytest.mark.parametrize("chunk", [128, 64])
def test_train_step_config(chunk):
    """B=8, H=16, T=2048, dk=96, dv=192, bf16, do ~ N(0,1); C=128 and C=64."""
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

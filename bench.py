#!/usr/bin/env python3
"""Benchmark of the Simple GLA mixer hot path on one MI355X.

A step is one pass of the hot path on synthetic inputs already resident in HBM:
  * forward: one gla_fwd_chunked call on the Laplace-layer workload
    (B=1, H=16, T=2048, dk=96, dv=192, chunk 128, bf16, fp32 state);
  * training step: gla_fwd_chunked_states + gla_bwd_chunked_states (dq, dk, dv,
    dlambda) on the mixer-train workload (B=8, H=16, T=2048, do ~ N(0,1)), at
    chunk 128 (part of the step) and chunk 64 (timed alongside);
  * decode: one decode step of the 1,280-sequence x 24-layer serving workload
    (24 gla_decode_step launches over a 36 GB fp32 state pool).
Timed alongside (not part of the step): the 64k-token prefill (B=1, T=65,536,
S0 given), the Laplace-layer forward from a cold cache, the decode variants,
the mixer epilogue and the depth-wise conv.
Each leg is timed over K steps after W warm-up steps, bracketed by device
synchronisation; per-launch durations come from HIP events recorded on the
stream the library launches on.  The headline value is forward tokens/s; the
decode leg reports state-update GB/s and output tokens/s in the same line.
MFMA fractions use the algorithmic (causal) FLOP count of each call: the work
of the method's chunked form, not counting the blocks above the causal
diagonal; the FLOPs the kernels issue are reported beside it.

The CPU baseline leg times the fp64 oracle on a bounded sample of the same
workloads (rank 0, one GPU only).  Usage: python bench.py [--gpus 1] [--steps K]
[--warmup W] [--no-cpu-baseline] [--counters]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "GLA chunked fwd tokens/s (H16,dk96,dv192,T2048) + decode GB/s at 1280 seqs"

# Algorithmic work (per token-head for the forward, per sequence-head for decode)
FWD_BYTES_PER_TOKEN_HEAD = {"bf16": 2 * 96 + 2 * 96 + 2 * 192 + 2 * 192, "f32": 4 * (96 + 96 + 192 + 192)}


def fwd_flops_per_token_head(C, dk=96, dv=192):
    """Algorithmic (causal) work of the chunked forward: QK^T and AV over the C(C+1)/2
    (query, key) pairs at or below the diagonal, (C+1)(dk+dv) per token, plus 4 dk dv for
    the inter-chunk readout Q S and the state update K^T V."""
    return (C + 1) * (dk + dv) + 4 * dk * dv


def fwd_issued_flops_per_token_head(C, dk=96, dv=192):
    """MFMA work the forward's kernels issue: the 16x16 score blocks at or below the
    diagonal (NIB(NIB+1)/2 of them, NIB = C/16) times dk, the 32-key pairs of the output
    strips (C/32 strips, strip K spanning K+1 pairs) times dv, and Q S, K^T V in full."""
    nib = C // 16
    score = nib * (nib + 1) // 2 * 256 * dk * 2
    out = sum(32 * 32 * (K + 1) * dv * 2 for K in range(C // 32))
    return (score + out) // C + 4 * dk * dv


def train_bytes_per_token_head(C, dk=96, dv=192):
    """Forward I/O + backward I/O (q,k,v,do in; dq,dk,dv out, bf16) + the per-chunk
    state snapshots (bf16 start state written by the forward and read back, state
    gradient written and read by the backward): 1152 + 1920 + 8 dk dv / C."""
    return 1152 + 1920 + 2 * 4 * dk * dv // C


def train_flops_per_token_head(C, dk=96, dv=192):
    """Algorithmic work of the saved-state training pair: the forward's, plus the
    backward's causal intra-chunk terms (dP, the recomputed scores, dQ, dK, dV:
    (C+1)(3dk + 2dv)) and 8 dk dv for the inter-chunk terms of dQ, dK, dV and the
    reverse state-gradient chain."""
    return fwd_flops_per_token_head(C, dk, dv) + (C + 1) * (3 * dk + 2 * dv) + 8 * dk * dv


DEC_BYTES_PER_SEQ_HEAD = 2 * 96 * 192 * 4 + 2 * (96 + 96 + 192 + 192)   # state R+W + q,k,v,o bf16
DEC_FLOPS_PER_SEQ_HEAD = 4 * 96 * 192
# Mixer epilogue: q, k in (dk each), v, o, g in and y out (dv each), bf16
EPI_BYTES_PER_TOKEN_HEAD = 2 * (2 * 96 + 4 * 192)
# Decode with the epilogue fused: the decode step's bytes plus the gate g (y replaces o)
DEC_EPI_BYTES_PER_SEQ_HEAD = DEC_BYTES_PER_SEQ_HEAD + 2 * 192
# Depth-wise conv (width 4), per channel: prefill x in + y out (bf16) per token; decode
# x in + y out (bf16) + 3 fp32 window slots read + 4 written per row
CONV_BYTES_PER_TOKEN_CHANNEL = 2 + 2
CONV_DEC_BYTES_PER_ROW_CHANNEL = 2 + 2 + 4 * 3 + 4 * 4
CONV_D = 3072


# Sources whose kernels the counters of each group measure (with the shared headers and
# the C ABI, which picks the launch plan): a change elsewhere leaves them valid.
DIGEST_FILES = {
    "fwd": ["gla_fwd.hip", "gla_fwd_bf16.hip"],
    "long": ["gla_fwd.hip", "gla_fwd_bf16.hip"],
    "decode": ["gla_decode.hip"],
    "grad": ["gla_grad_bf16.hip", "gla_bwd.hip"],
}
DIGEST_SHARED = ["gla_api.hip", "gla_common.hpp", "gla_internal.hpp", "gla_tile.hpp"]


def src_digest(group=None):
    """sha256 prefix of the kernel sources a counter group depends on (all sources if None)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_linear_attention_simple_amd", "csrc")
    names = sorted(os.listdir(csrc)) if group is None else sorted(DIGEST_FILES[group] + DIGEST_SHARED)
    for fn in names:
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, bytes_per_launch_alg: float):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get("kernels", {}).get(kernel)
    if not rec or rec.get("src_digest") != src_digest(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode leg (debugging only)")
    ap.add_argument("--no-train", action="store_true", help="skip the training legs (debugging only)")
    ap.add_argument("--counters", action="store_true",
                    help="run a short fixed sequence (copy kernel + each hot kernel) for rocprofv3 --pmc")
    ap.add_argument("--chunk", type=int, default=128)
    ap.add_argument("--ingest-ktrace", metavar="STATS_CSV",
                    help="turn rocprofv3 --kernel-trace --stats kernel_stats.csv into profiles/kernel_time_by_kernel.md")
    ap.add_argument("--ingest-counters", nargs="+", metavar="CSV",
                    help="turn the rocprofv3 --pmc counter_collection.csv files of the --counters pass "
                         "(one per COUNTER_PASSES entry) into profiles/counters.json")
    return ap.parse_args()


class FwdLeg:
    """Pre-marshalled gla_fwd_chunked call on one workload (no per-call allocation)."""

    def __init__(self, gla, gi, torch, w, seed, chunk):
        self.torch = torch
        dev = torch.device("cuda:0")
        x = gi.fwd_inputs(w, dev, seed)
        self.x = x
        B, T, H, dk = x["q"].shape
        dv = x["v"].shape[3]
        self.tokens = B * T
        self.token_heads = B * T * H
        self.o = torch.empty((B, T, H, dv), dtype=x["q"].dtype, device=dev)
        self.S = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        dt = gla.GLA_BF16 if x["q"].dtype == torch.bfloat16 else gla.GLA_F32
        need = gla.fwd_workspace_bytes(dt, B, T, H, dk, dv, chunk)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream()
        p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
        self.fn = gla.load().gla_fwd_chunked
        self.head = (dt, B, T, H, dk, dv, chunk, p(x["q"]), p(x["k"]), p(x["v"]), p(x["lam"]),
                     p(x["S0"]), ctypes.c_float(x["scale"]), p(self.o), p(self.S), None, p(self.ws),
                     ctypes.c_size_t(need))
        self.gla = gla

    def __call__(self, stream=None):
        s = self.stream if stream is None else stream
        st = self.fn(*self.head, ctypes.c_void_p(s.cuda_stream))
        if st != 0:
            raise RuntimeError(f"gla_fwd_chunked: {self.gla.status_str(st)}")


class SplitLeg:
    """A single-sequence prefill as two gla_fwd_chunked calls of T/2 tokens each, the
    first one's final state the second one's initial state (the split a sequence-parallel
    prefill would make); pre-marshalled on the inputs and outputs of a FwdLeg (B = 1, so
    each half of every token-major tensor is contiguous)."""

    def __init__(self, leg, gla, torch, chunk):
        x = leg.x
        B, T, H, dk = x["q"].shape
        dv = x["v"].shape[3]
        assert B == 1 and T % 2 == 0
        half = T // 2
        dev = x["q"].device
        dt = gla.GLA_BF16 if x["q"].dtype == torch.bfloat16 else gla.GLA_F32
        es = x["q"].element_size()
        need = gla.fwd_workspace_bytes(dt, 1, half, H, dk, dv, chunk)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        self.S1 = torch.empty((1, H, dk, dv), dtype=torch.float32, device=dev)
        self.stream = leg.stream
        self.tokens = T
        p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
        off = lambda t, d: ctypes.c_void_p(t.data_ptr() + half * H * d * es)
        sc = ctypes.c_float(x["scale"])
        self.fn = gla.load().gla_fwd_chunked
        tail = (p(self.ws), ctypes.c_size_t(need))
        self.first = (dt, 1, half, H, dk, dv, chunk, p(x["q"]), p(x["k"]), p(x["v"]), p(x["lam"]), p(x["S0"]),
                      sc, p(leg.o), p(self.S1), None) + tail
        self.second = (dt, 1, half, H, dk, dv, chunk, off(x["q"], dk), off(x["k"], dk), off(x["v"], dv),
                       p(x["lam"]), p(self.S1), sc, off(leg.o, dv), p(leg.S), None) + tail
        self.gla = gla

    def __call__(self):
        for args in (self.first, self.second):
            st = self.fn(*args, ctypes.c_void_p(self.stream.cuda_stream))
            if st != 0:
                raise RuntimeError(f"gla_fwd_chunked: {self.gla.status_str(st)}")


class TrainLeg:
    """Pre-marshalled forward + backward (dq, dk, dv, dlambda) on the mixer-train workload:
    the forward saving every chunk's start state and the backward reading them
    (saved=True), or the plain pair whose backward recomputes them."""

    def __init__(self, gla, gi, torch, w, seed, chunk, saved=True):
        dev = torch.device("cuda:0")
        x = gi.fwd_inputs(w, dev, seed, with_do=True)
        self.x = x
        B, T, H, dk = x["q"].shape
        dv = x["v"].shape[3]
        self.tokens = B * T
        self.token_heads = B * T * H
        dt = gla.GLA_BF16
        self.o = torch.empty_like(x["v"])
        self.dq, self.dk, self.dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
        self.dl = torch.empty(H, dtype=torch.float32, device=dev)
        nf = gla.fwd_workspace_bytes(dt, B, T, H, dk, dv, chunk)
        nb = gla.bwd_workspace_bytes(dt, B, T, H, dk, dv, chunk, saved_states=saved)
        self.wsf = torch.empty(max(nf, 16), dtype=torch.uint8, device=dev)
        self.wsb = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream()
        p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
        st = ctypes.c_void_p(self.stream.cuda_stream)
        lib = gla.load()
        sc = ctypes.c_float(x["scale"])
        if saved:
            self.states = torch.empty(lib.gla_fwd_states_bytes(dt, B, T, H, dk, dv, chunk), dtype=torch.uint8,
                                      device=dev)
            self.f, self.b = lib.gla_fwd_chunked_states, lib.gla_bwd_chunked_states
            self.fargs = (dt, B, T, H, dk, dv, chunk, p(x["q"]), p(x["k"]), p(x["v"]), p(x["lam"]), None, sc,
                          p(self.o), None, p(self.states), None, p(self.wsf), ctypes.c_size_t(nf), st)
            self.bargs = (dt, B, T, H, dk, dv, chunk, p(x["q"]), p(x["k"]), p(x["v"]), p(x["lam"]), None, sc,
                          p(x["do"]), None, p(self.states), p(self.dq), p(self.dk), p(self.dv), p(self.dl), None,
                          None, p(self.wsb), ctypes.c_size_t(nb), st)
        else:
            self.f, self.b = lib.gla_fwd_chunked, lib.gla_bwd_chunked
            self.fargs = (dt, B, T, H, dk, dv, chunk, p(x["q"]), p(x["k"]), p(x["v"]), p(x["lam"]), None, sc,
                          p(self.o), None, None, p(self.wsf), ctypes.c_size_t(nf), st)
            self.bargs = (dt, B, T, H, dk, dv, chunk, p(x["q"]), p(x["k"]), p(x["v"]), p(x["lam"]), None, sc,
                          p(x["do"]), None, p(self.dq), p(self.dk), p(self.dv), p(self.dl), None, None, p(self.wsb),
                          ctypes.c_size_t(nb), st)
        self.gla = gla

    def __call__(self):
        for fn, args, name in ((self.f, self.fargs, "gla_fwd_chunked"), (self.b, self.bargs, "gla_bwd_chunked")):
            st = fn(*args)
            if st != 0:
                raise RuntimeError(f"{name}: {self.gla.status_str(st)}")


def epi_params(gla, e):
    """gla_epilogue_params for seeded epilogue inputs; returns (struct, tier array) to keep alive."""
    tiers = (ctypes.c_int * len(e["tier"]))(*e["tier"])
    p = gla.EpilogueParams(e["aug_a"].data_ptr(), e["norm_w"].data_ptr(),
                           ctypes.cast(tiers, ctypes.POINTER(ctypes.c_int)), e["norm_w"].shape[0], 1e-6)
    return p, tiers


class EpilogueLeg:
    """Pre-marshalled gla_mixer_epilogue over B*T token rows of the mixer shape (bf16)."""

    def __init__(self, gla, gi, torch, w, seed):
        dev = torch.device("cuda:0")
        x = gi.fwd_inputs(w, dev, seed, with_do=True)
        e = gi.epilogue_inputs(w, dev, seed, (w.B, w.T))
        self.keep = (x, e)
        self.y = torch.empty_like(x["v"])
        self.token_heads = w.B * w.T * w.H
        self.params, self.tiers = epi_params(gla, e)
        self.stream = torch.cuda.current_stream()
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        # the readout o is stood in for by another N(0, 1) tensor of its shape
        self.args = (gla.GLA_BF16, w.B * w.T, w.H, w.dk, w.dv, p(x["q"]), p(x["k"]), p(x["v"]), p(x["do"]),
                     p(e["g"]), ctypes.byref(self.params), p(self.y), ctypes.c_void_p(self.stream.cuda_stream))
        self.fn = gla.load().gla_mixer_epilogue
        self.gla = gla

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"gla_mixer_epilogue: {self.gla.status_str(st)}")


class FwdEpilogueLeg:
    """Pre-marshalled gla_fwd_chunked_epilogue on the Laplace layer (the epilogue fused into
    the forward's output kernel there)."""

    def __init__(self, gla, gi, torch, w, seed, chunk):
        dev = torch.device("cuda:0")
        x = gi.fwd_inputs(w, dev, seed)
        e = gi.epilogue_inputs(w, dev, seed, (w.B, w.T))
        self.keep = (x, e)
        B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
        self.token_heads = B * T * H
        self.y = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
        self.S = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        need = gla.fwd_workspace_bytes(gla.GLA_BF16, B, T, H, dk, dv, chunk)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        self.params, self.tiers = epi_params(gla, e)
        self.stream = torch.cuda.current_stream()
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        self.args = (gla.GLA_BF16, B, T, H, dk, dv, chunk, p(x["q"]), p(x["k"]), p(x["v"]), p(x["lam"]), None,
                     ctypes.c_float(x["scale"]), p(e["g"]), ctypes.byref(self.params), p(self.y), p(self.S), None,
                     p(self.ws), ctypes.c_size_t(need), ctypes.c_void_p(self.stream.cuda_stream))
        self.fn = gla.load().gla_fwd_chunked_epilogue
        self.gla = gla

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"gla_fwd_chunked_epilogue: {self.gla.status_str(st)}")


class ConvLeg:
    """Pre-marshalled depth-wise conv prefill (B, T, D=3,072 bf16) or decode step (N rows)."""

    def __init__(self, gla, gi, torch, B, T, seed, decode=False):
        dev = torch.device("cuda:0")
        c = gi.conv_inputs(B, T, CONV_D, "bf16", dev, seed)
        self.keep = c
        self.stream = torch.cuda.current_stream()
        st = ctypes.c_void_p(self.stream.cuda_stream)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        lib = gla.load()
        if decode:
            self.y = torch.empty((B, CONV_D), dtype=torch.bfloat16, device=dev)
            self.fn = lib.gla_conv1d_silu_decode
            self.args = (gla.GLA_BF16, B, CONV_D, 4, p(c["x"][:, 0]), p(c["w"]), p(c["bias"]), p(c["win"]), 0,
                         None, p(self.y), st)
            self.bytes = CONV_DEC_BYTES_PER_ROW_CHANNEL * B * CONV_D
        else:
            self.y = torch.empty_like(c["x"])
            self.wo = torch.empty_like(c["win"])
            self.fn = lib.gla_conv1d_silu
            self.args = (gla.GLA_BF16, B, T, CONV_D, 4, p(c["x"]), p(c["w"]), p(c["bias"]), p(c["win"]), p(self.y),
                         p(self.wo), st)
            self.bytes = CONV_BYTES_PER_TOKEN_CHANNEL * B * T * CONV_D
        self.gla = gla

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"conv: {self.gla.status_str(st)}")


class DecodeLeg:
    """The 1,280-sequence x 24-layer decode workload with its fp32 state pool on the GPU."""

    def __init__(self, gla, gi, torch, w, seed, n_inputs=4):
        dev = torch.device("cuda:0")
        self.torch = torch
        self.w = w
        L = w.decode_layers
        self.pool = torch.empty((L, w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
        for layer in range(L):
            gi.decode_state(w, dev, seed, layer, out=self.pool[layer])
        self.inputs = [[gi.decode_token_inputs(w, dev, seed, layer, s) for s in range(n_inputs)]
                       for layer in range(L)]
        self.lam = torch.tensor(w.lambdas, dtype=torch.float32, device=dev)
        self.o = torch.empty((w.B, w.H, w.dv), dtype=torch.bfloat16, device=dev)
        self.stream = torch.cuda.current_stream()
        self.fn = gla.load().gla_decode_step
        self.gla = gla
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        self.args = [[(gla.GLA_BF16, w.B, w.H, w.dk, w.dv, p(d["q"]), p(d["k"]), p(d["v"]), p(self.lam),
                       p(self.pool[layer]), ctypes.c_float(w.scale), p(self.o),
                       ctypes.c_void_p(self.stream.cuda_stream)) for d in self.inputs[layer]]
                     for layer in range(L)]
        self.layers = L
        self.n_inputs = n_inputs
        # page-pool form: the same pages addressed through a fixed shuffle of slots
        perm = torch.randperm(w.B, generator=torch.Generator().manual_seed(seed)).to(torch.int32)
        self.slots = perm.to(dev)
        self.fn_pool = gla.load().gla_decode_step_pool
        self.args_pool = [[(gla.GLA_BF16, w.B, w.H, w.dk, w.dv, p(d["q"]), p(d["k"]), p(d["v"]), p(self.lam),
                            p(self.pool[layer]), w.B, p(self.slots), ctypes.c_float(w.scale), p(self.o),
                            ctypes.c_void_p(self.stream.cuda_stream)) for d in self.inputs[layer]]
                          for layer in range(L)]
        # epilogue-fused form on the direct pages: gate g per (layer, input), shared parameters
        e = gi.epilogue_inputs(w, dev, seed, (w.B,))
        self.epi_keep = [e] + [gi.epilogue_inputs(w, dev, seed, (w.B,), layer=layer, step=s)["g"]
                               for layer in range(L) for s in range(n_inputs)]
        self.params, self.tiers = epi_params(gla, e)
        self.fn_epi = gla.load().gla_decode_step_epilogue
        self.args_epi = [[(gla.GLA_BF16, w.B, w.H, w.dk, w.dv, p(d["q"]), p(d["k"]), p(d["v"]),
                           p(self.epi_keep[1 + layer * n_inputs + s]), p(self.lam), p(self.pool[layer]), 0, None,
                           ctypes.c_float(w.scale), ctypes.byref(self.params), p(self.o),
                           ctypes.c_void_p(self.stream.cuda_stream)) for s, d in enumerate(self.inputs[layer])]
                         for layer in range(L)]
        self.use_pool = False
        self.use_epi = False

    def launch(self, layer, step):
        if self.use_epi:
            st = self.fn_epi(*self.args_epi[layer][step % self.n_inputs])
        elif self.use_pool:
            st = self.fn_pool(*self.args_pool[layer][step % self.n_inputs])
        else:
            st = self.fn(*self.args[layer][step % self.n_inputs])
        if st != 0:
            raise RuntimeError(f"gla_decode_step: {self.gla.status_str(st)}")


def time_region(torch, stream, fn, K, W):
    """W untimed calls, then K calls bracketed by synchronisation and by HIP events
    recorded on the stream the library launches on.  Returns (wall seconds, GPU
    seconds of the region); no per-call host work is added inside the region."""
    for _ in range(W):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(K):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, a.elapsed_time(b) * 1e-3


def time_cold(torch, stream, fn, reps, W, flush_bytes=2 << 30):
    """Each call alone, from a cold cache: before every call a fill kernel writes
    flush_bytes (far beyond the 256 MB last-level cache) outside the timed region;
    HIP events on the launch stream bracket the call only.  Returns the per-call
    seconds (sorted)."""
    for _ in range(W):
        fn()
    scratch = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda:0")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        scratch.fill_(1.0)   # on torch's current stream, the launch stream here
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    del scratch
    return sorted(a.elapsed_time(b) * 1e-3 for a, b in evs)


def time_decode(torch, leg, K, W):
    """K decode steps (each: one launch per layer) -> (wall, GPU region seconds)."""
    step = [0]

    def one_step():
        for layer in range(leg.layers):
            leg.launch(layer, step[0])
        step[0] += 1

    return time_region(torch, leg.stream, one_step, K, W)


def _read(path):
    try:
        with open(path) as f:
            return f.read().strip()
    except OSError:
        return None


def _dpm_current(text):
    """The active level of a pp_dpm_* sysfs table ('1: 2400Mhz *' -> '2400Mhz')."""
    for line in (text or "").splitlines():
        if line.rstrip().endswith("*"):
            return line.split(":", 1)[-1].replace("*", "").strip()
    return None


def machine_info(torch):
    """ROCm / HIP versions, the device, and its current engine and memory clock levels
    (from the driver's sysfs tables; null where the box does not expose them)."""
    import glob

    info = {"rocm": _read("/opt/rocm/.info/version"), "torch": torch.__version__,
            "hip_runtime": getattr(torch.version, "hip", None)}
    try:
        p = torch.cuda.get_device_properties(0)
        info.update({"device": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
                     "hbm_gib": round(p.total_memory / 2 ** 30, 1)})
    except Exception:  # noqa: BLE001  (no device: report what is known)
        pass
    sclk = mclk = None
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        if _read(os.path.join(dev, "vendor")) == "0x1002":
            sclk = sclk or _dpm_current(_read(os.path.join(dev, "pp_dpm_sclk")))
            mclk = mclk or _dpm_current(_read(os.path.join(dev, "pp_dpm_mclk")))
    info.update({"sclk": sclk, "mclk": mclk})
    return info


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _repeat(fn, budget_s, max_reps):
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= max_reps:
            return reps, el


def cpu_baseline_fwd(gi, w, seed, budget_s=4.0):
    """fp64 oracle on the Laplace layer's inputs (drawn on the CPU), repeated for ~budget_s."""
    import oracle

    x = gi.fwd_inputs(w, "cpu", seed)
    f = lambda t: t.double().numpy()
    q, k, v, lam = f(x["q"]), f(x["k"]), f(x["v"]), f(x["lam"])
    reps, el = _repeat(lambda: oracle.fwd(q, k, v, lam, scale=x["scale"]), budget_s, 200)
    return {"value": reps * w.B * w.T / el, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"fp64 per-token recurrence, the whole Laplace-layer forward (B=1, H=16, T=2048) x {reps} "
                      f"repetitions in {el:.1f} s, OpenMP over the 16 (batch, head) units"}


def cpu_baseline_train(gi, w, seed, budget_s=4.0):
    """fp64 oracle forward + reverse mode on one of the training step's 8 sequences."""
    import oracle

    x = gi.fwd_inputs(w, "cpu", seed, B=1, with_do=True)
    f = lambda t: t.double().numpy()
    q, k, v, lam, do = f(x["q"]), f(x["k"]), f(x["v"]), f(x["lam"]), f(x["do"])

    def step():
        oracle.fwd(q, k, v, lam, scale=x["scale"])
        oracle.bwd(q, k, v, lam, do, scale=x["scale"])

    reps, el = _repeat(step, budget_s, 50)
    return {"value": reps * w.T / el, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"fp64 forward + reverse mode (dq, dk, dv, dlambda) of 1 of the 8 sequences "
                      f"(H=16, T=2048) x {reps} in {el:.1f} s; tokens/s of that sample"}


def cpu_baseline_long(gi, w, seed, tokens=8192, budget_s=3.0):
    """fp64 oracle forward over the first `tokens` tokens of the 64k-token prefill."""
    import oracle

    x = gi.fwd_inputs(w, "cpu", seed, T=tokens)
    f = lambda t: t.double().numpy()
    q, k, v, lam, S0 = f(x["q"]), f(x["k"]), f(x["v"]), f(x["lam"]), f(x["S0"])
    reps, el = _repeat(lambda: oracle.fwd(q, k, v, lam, S0=S0, scale=x["scale"]), budget_s, 100)
    return {"value": reps * tokens / el, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"fp64 forward over the first {tokens} of the 65,536 tokens (B=1, H=16, S0 given) x {reps} "
                      f"in {el:.1f} s (the recurrence's cost is linear in T)"}


def cpu_baseline_epilogue(gi, w, seed, budget_s=2.0):
    """fp64 oracle mixer epilogue over the Laplace layer's 2,048 rows (inputs drawn on the CPU)."""
    import oracle

    x = gi.fwd_inputs(w, "cpu", seed)
    e = gi.epilogue_inputs(w, "cpu", seed, (w.B, w.T))
    f = lambda t: t.double().numpy()
    q, k, v, g, a, nw = f(x["q"]), f(x["k"]), f(x["v"]), f(e["g"]), f(e["aug_a"]), f(e["norm_w"])
    reps, el = _repeat(lambda: oracle.epilogue(q, k, v, v, g, a, nw, e["tier"]), budget_s, 200)
    rows = w.B * w.T
    return {"value": reps * rows / el, "unit": "rows/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"fp64 epilogue (gate, tier RMSNorm, SiLU gate) of the {rows} rows x 16 heads of the "
                      f"Laplace layer x {reps} in {el:.1f} s"}


def cpu_baseline_conv(gi, seed, budget_s=2.0):
    """fp64 oracle depth-wise conv + SiLU over one 2,048-token sequence of width 3,072."""
    import oracle

    c = gi.conv_inputs(1, 2048, 3072, "bf16", "cpu", seed=seed)
    f = lambda t: t.double().numpy()
    x, wt, b, win = f(c["x"]), f(c["w"]), f(c["bias"]), f(c["win"])
    reps, el = _repeat(lambda: oracle.conv1d(x, wt, b, win), budget_s, 200)
    return {"value": reps * 2048 / el, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"fp64 conv (width 4) + SiLU of 1 of the 8 sequences (T=2048, D=3072) x {reps} in "
                      f"{el:.1f} s; tokens/s of that sample"}


def cpu_baseline_decode(gi, w, seed, budget_s=3.0):
    import oracle

    n = 64
    x = gi.decode_token_inputs(w, "cpu", seed, 0, 0, N=n)
    S = gi.decode_state(w, "cpu", seed, 0, N=n).double().numpy()
    f = lambda t: t.double().numpy()
    q, k, v = f(x["q"]), f(x["k"]), f(x["v"])
    import torch
    lam = torch.tensor(w.lambdas, dtype=torch.float32).double().numpy()   # the fp32 values the kernel reads
    box = [S]

    def step():
        _, box[0] = oracle.decode(q, k, v, lam, box[0], scale=w.scale)

    reps, el = _repeat(step, budget_s, 10000)
    seq_heads = reps * n * w.H
    return {"value": seq_heads * DEC_BYTES_PER_SEQ_HEAD / el / 1e9, "unit": "GB/s",
            "tokens_per_s": reps * n / el / w.decode_layers, "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"fp64 decode steps of 64 sequences x 16 heads (one layer), {reps} steps in {el:.1f} s; "
                      f"GB/s counts the fp32 workload's algorithmic bytes"}


# rocprofv3 --pmc passes over the --counters sequence: HBM traffic (one counter per run),
# then SQ counters (at most 8 SQ_ and 2 GRBM_ counters per run)
COUNTER_PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "sq_mfma": ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA",
                "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"],
    "sq_wait": ["SQ_LDS_IDX_ACTIVE", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_WAIT_INST_ANY",
                "SQ_ACTIVE_INST_VMEM", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR", "SQ_ACTIVE_INST_VALU",
                "GRBM_GUI_ACTIVE"],
}
# groups of the --counters sequence, in launch order; each group is followed by a
# device copy (a marker between groups, and the traffic calibration)
COUNTER_GROUPS = ["train", "fwd", "long", "decode"]
MARKER_BYTES = 1 << 28          # each marker copy reads and writes 256 MiB


def counters_pass(torch, gla, gi, chunk):
    """Fixed launch sequence for rocprofv3 --pmc: 3 training steps (mixer-train workload,
    forward saving chunk states + backward), 3 Laplace-layer forward calls, 3 calls of the
    64k-token prefill and 3 decode launches (one layer of the serving workload), each group
    followed by a 256 MiB device copy (the marker between groups and the calibration of
    the traffic counters)."""
    dev = torch.device("cuda:0")
    ws = gi.workloads()
    src = torch.empty(MARKER_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)

    def marker():
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    t = TrainLeg(gla, gi, torch, ws[2], 2, chunk)
    for _ in range(3):
        t()
    marker()
    del t
    f = FwdLeg(gla, gi, torch, ws[1], 1, chunk)
    for _ in range(3):
        f()
    marker()
    del f
    torch.cuda.empty_cache()
    lg = FwdLeg(gla, gi, torch, ws[3], 3, chunk)
    for _ in range(3):
        lg()
    marker()
    del lg
    torch.cuda.empty_cache()
    w4 = ws[4]
    w1 = gi.Workload(w4.name, w4.B, w4.T, w4.H, w4.dk, w4.dv, 0, w4.dtype, w4.lambdas, w4.scale, w4.s0_var, 1)
    d = DecodeLeg(gla, gi, torch, w1, 4, n_inputs=1)
    for s in range(3):
        d.launch(0, s)
    marker()
    print(json.dumps({"counters_pass": "done", "marker_bytes_each": 2 * MARKER_BYTES}), flush=True)


ENGINE_GHZ = 2.4    # MI355X peak engine clock: counter cycles per ns of kernel time
N_SIMD, N_CU = 1024, 256


def _read_counter_csv(path):
    """{dispatch_id: {"kernel": name, "dur_ns": duration, counter: value}} (one row per
    dispatch and counter, already reduced over the hardware instances)."""
    import csv

    out = {}
    for r in csv.DictReader(open(path)):
        rec = out.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"]})
        rec["dur_ns"] = float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        rec[r["Counter_Name"]] = rec.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _group_dispatches(disp):
    """Split the --counters sequence into its groups at the marker copies; returns
    ({group: [dispatch ids]}, [marker dispatch ids])."""
    ids = sorted(disp)
    markers = [d for d in ids if "copy" in disp[d]["kernel"].lower() or "elementwise" in disp[d]["kernel"].lower()]
    # the markers are the copies that follow a group: the last copy-like dispatch before
    # each run of library kernels ends
    lib = lambda d: any(k in disp[d]["kernel"] for k in ("gla", "fwd_", "grad_", "chain_", "seg_scan", "decode_",
                                                          "dlambda", "rev_scan", "bwd_"))
    groups, cur, gi_ = {}, [], 0
    marks = []
    for d in ids:
        if lib(d):
            cur.append(d)
        elif cur and d in markers:
            groups[COUNTER_GROUPS[gi_]] = cur
            marks.append(d)
            cur, gi_ = [], gi_ + 1
            if gi_ == len(COUNTER_GROUPS):
                break
    return groups, marks


def _short_kernel_name(full):
    """'void gla::(anonymous namespace)::fwd_out_kernel<128, 104, 2, false>(gla::FwdArgs, ...)'
    -> 'fwd_out_kernel<128, 104, 2, false>'."""
    import re

    m = re.search(r"(\w+)(<[^()]*>)?\(", full)
    return (m.group(1) + (m.group(2) or "")) if m else full


def ingest_counters(csvs):
    """Per-dispatch counters of the --counters pass -> profiles/counters.json: HBM traffic
    per call of each group (FETCH_SIZE and WRITE_SIZE scaled by what they read for the
    256 MiB marker copies), and per-kernel SQ summaries (MFMA busy, LDS activity, bank
    conflicts, waits) for every kernel of the sequence."""
    data = {}
    for path in csvs:
        pas = os.path.basename(os.path.dirname(path))
        for d, rec in _read_counter_csv(path).items():
            dst = data.setdefault(d, {"kernel": rec["kernel"], "dur_ns": {}})
            dst["dur_ns"][pas] = rec["dur_ns"]
            dst.update({k: v for k, v in rec.items() if k not in ("kernel", "dur_ns")})
    groups, marks = _group_dispatches(data)
    out = {"src_digest": src_digest(), "groups": {}, "kernels": {}}
    fac = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        vals = [data[m][counter] for m in marks if counter in data[m]]
        if vals:   # counters in KiB; the copy reads and writes MARKER_BYTES each
            fac[counter] = MARKER_BYTES / (sorted(vals)[len(vals) // 2] * 1024.0)
    out["copy_calibration"] = {"fetch_factor": fac.get("FETCH_SIZE"), "write_factor": fac.get("WRITE_SIZE"),
                               "marker_bytes_read_and_written": MARKER_BYTES}
    digest_of = {"train": "grad", "fwd": "fwd", "long": "fwd", "decode": "decode"}
    for g, ids in groups.items():
        calls = 3.0
        rec = {"src_digest": src_digest(digest_of[g]), "dispatches": len(ids)}
        if fac:
            fb = sum(data[d].get("FETCH_SIZE", 0.0) for d in ids) / calls * 1024.0 * fac["FETCH_SIZE"]
            wb = sum(data[d].get("WRITE_SIZE", 0.0) for d in ids) / calls * 1024.0 * fac["WRITE_SIZE"]
            rec.update({"fetch_bytes_per_call": fb, "write_bytes_per_call": wb, "hbm_bytes_per_call": fb + wb})
        # per kernel inside the group
        per = {}
        for d in ids:
            per.setdefault(_short_kernel_name(data[d]["kernel"]), []).append(d)
        rec["kernels"] = {}
        for name, ds in per.items():
            kr = {"dispatches_per_call": len(ds) / calls}
            if fac:
                kr["hbm_bytes_per_dispatch"] = sum(data[d].get("FETCH_SIZE", 0.0) * fac["FETCH_SIZE"] +
                                                   data[d].get("WRITE_SIZE", 0.0) * fac["WRITE_SIZE"]
                                                   for d in ds) * 1024.0 / len(ds)
            tot = lambda c: sum(data[d].get(c, 0.0) for d in ds)
            # kernel time of the dispatches in the run that read a counter (each
            # dispatch runs alone while counters are collected)
            dur = lambda pas: sum(data[d]["dur_ns"].get(pas, 0.0) for d in ds)
            kr["avg_us"] = sum(dur(p) for p in data[ds[0]]["dur_ns"]) / len(data[ds[0]]["dur_ns"]) / len(ds) / 1e3
            if dur("sq_mfma") > 0 and "SQ_VALU_MFMA_BUSY_CYCLES" in data[ds[0]]:
                kr["mfma_busy_pct"] = 100.0 * tot("SQ_VALU_MFMA_BUSY_CYCLES") / (dur("sq_mfma") * ENGINE_GHZ * N_SIMD)
            if dur("sq_wait") > 0 and "SQ_LDS_IDX_ACTIVE" in data[ds[0]]:
                kr["lds_active_pct"] = 100.0 * tot("SQ_LDS_IDX_ACTIVE") / (dur("sq_wait") * ENGINE_GHZ * N_CU)
                kr["lds_bank_conflict_pct_of_lds_active"] = (100.0 * tot("SQ_LDS_BANK_CONFLICT") /
                                                             max(tot("SQ_LDS_IDX_ACTIVE"), 1.0))
            for c in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR",
                      "SQ_WAVES"):
                if tot(c):
                    kr[c.lower() + "_per_dispatch"] = tot(c) / len(ds)
            if tot("SQ_INSTS_MFMA"):
                kr["valu_per_mfma"] = tot("SQ_INSTS_VALU") / tot("SQ_INSTS_MFMA")
            if tot("SQ_WAVE_CYCLES"):
                for c in ("SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM",
                          "SQ_ACTIVE_INST_VALU"):
                    if tot(c):
                        kr[c.lower() + "_pct_of_wave_cycles"] = 100.0 * tot(c) / tot("SQ_WAVE_CYCLES")
            rec["kernels"][name] = kr
        out["groups"][g] = rec
    # traffic per group under the keys the bench reads
    for g, key in (("fwd", "fwd"), ("long", "long"), ("decode", "decode")):
        if g in out["groups"] and "hbm_bytes_per_call" in out["groups"][g]:
            r = out["groups"][g]
            out["kernels"][key] = {"src_digest": r["src_digest"], "hbm_bytes_per_launch": r["hbm_bytes_per_call"],
                                   "fetch_bytes_per_launch": r["fetch_bytes_per_call"],
                                   "write_bytes_per_launch": r["write_bytes_per_call"]}
    tr = out["groups"].get("train", {}).get("kernels", {})
    for name, kr in tr.items():
        if name.startswith("grad_fused") and "hbm_bytes_per_dispatch" in kr:
            out["kernels"]["grad"] = {"src_digest": src_digest("grad"),
                                      "hbm_bytes_per_launch": kr["hbm_bytes_per_dispatch"]}
    with open(os.path.join(ROOT, "profiles", "counters.json"), "w") as f:
        json.dump(out, f, indent=1)
    write_counter_summary(out)
    print(json.dumps(out, indent=1))


COUNTER_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 170 rocprofv3 --pmc {counters} -f csv "
               "-d $R/gpurun_out/pmc/{name} -o pmc -- python3 $R/bench.py --counters")
GROUP_DESC = {"train": "training step, B=8 H=16 T=2048 C=128 (saved-state pair)",
              "fwd": "Laplace-layer forward, B=1 H=16 T=2048 C=128",
              "long": "64k-token prefill, B=1 H=16 T=65536 C=128, S0 given",
              "decode": "decode, 1,280 sequences x H=16, one layer"}


def write_counter_summary(out):
    """profiles/counters_by_kernel.md: the per-kernel table of counters.json."""
    lines = ["# rocprofv3 counters per kernel (bench.py --counters sequence)", "",
             "Commands (one run per counter set, the sets of bench.COUNTER_PASSES):", ""]
    for name, cs in COUNTER_PASSES.items():
        lines.append("    " + COUNTER_CMD.format(counters=" ".join(cs), name=name))
    lines += ["", "with R the repository root; then `python bench.py --ingest-counters "
                  "gpurun_out/pmc/{fetch,write,sq_mfma,sq_wait}/"
                  "pmc_counter_collection.csv`.", "",
              "HBM bytes: FETCH_SIZE x %.3f + WRITE_SIZE x %.3f (the factors that make the 256 MiB marker "
              "copies read and write 256 MiB). Utilisations: counter / (dispatch time x %.1f GHz x units) with "
              "units = %d SIMDs (MFMA busy) or %d CUs (LDS active); waits and VMEM activity as a share of wave "
              "cycles. Source digest %s." % (out["copy_calibration"]["fetch_factor"] or 0,
                                              out["copy_calibration"]["write_factor"] or 0, ENGINE_GHZ, N_SIMD,
                                              N_CU, out["src_digest"]), ""]
    for g, r in out["groups"].items():
        lines += [f"## {GROUP_DESC.get(g, g)}", "",
                  f"HBM per call: {r.get('hbm_bytes_per_call', 0) / 1e6:.1f} MB over {r['dispatches']} dispatches "
                  f"(3 calls).", "",
                  "| kernel | us | HBM MB | MFMA busy % | LDS active % | bank conflicts % of LDS | VALU/MFMA | "
                  "wait % | MFMA insts | LDS insts |", "|---|---|---|---|---|---|---|---|---|---|"]
        for k, kr in r["kernels"].items():
            lines.append("| `%s` | %.1f | %.1f | %.1f | %.1f | %.1f | %.2f | %.1f | %.3g | %.3g |" % (
                k, kr.get("avg_us", 0), kr.get("hbm_bytes_per_dispatch", 0) / 1e6, kr.get("mfma_busy_pct", 0),
                kr.get("lds_active_pct", 0), kr.get("lds_bank_conflict_pct_of_lds_active", 0),
                kr.get("valu_per_mfma", 0), kr.get("sq_wait_inst_any_pct_of_wave_cycles", 0),
                kr.get("sq_insts_mfma_per_dispatch", 0), kr.get("sq_insts_lds_per_dispatch", 0)))
        lines.append("")
    with open(os.path.join(ROOT, "profiles", "counters_by_kernel.md"), "w") as f:
        f.write("\n".join(lines))


def ingest_ktrace(stats_csv):
    """profiles/kernel_time_by_kernel.md from rocprofv3 --kernel-trace --stats of a bench run."""
    import csv

    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["# Kernel time per kernel (rocprofv3 --kernel-trace --stats of a bench run)", "",
             "    cd /tmp && export TMPDIR=/tmp && timeout -s KILL 200 rocprofv3 --kernel-trace --stats -f csv "
             "-d $R/gpurun_out/pmc/ktrace -o kt -- python3 $R/bench.py --steps 10 --warmup 3 --no-cpu-baseline", "",
             "with R the repository root; then `python bench.py --ingest-ktrace "
             "gpurun_out/pmc/ktrace/kt_kernel_stats.csv`.", "",
             "(source digest %s; every leg of the bench, so a kernel's average mixes the workloads that "
             "launch it: fwd_bf16_kernel<128, ...> runs in the training step's forward and in the 64k prefill)"
             % src_digest(), "", "| kernel | calls | average us | min us | max us | share of GPU time % |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| `%s` | %s | %.2f | %.2f | %.2f | %s |" % (
            _short_kernel_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, r["Percentage"][:5]))
    with open(os.path.join(ROOT, "profiles", "kernel_time_by_kernel.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(args.ingest_counters)
        return
    if args.ingest_ktrace:
        ingest_ktrace(args.ingest_ktrace)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the mixer's hot path is single-GPU here); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import gated_linear_attention_simple_amd as gla
    import gla_inputs as gi

    gla.load()
    if args.counters:
        counters_pass(torch, gla, gi, args.chunk)
        return
    K, W = args.steps, args.warmup
    ws = gi.workloads()

    # ---- forward leg (Laplace layer)
    w1 = ws[1]
    fleg = FwdLeg(gla, gi, torch, w1, 1, args.chunk)
    f_wall, f_gpu = time_region(torch, fleg.stream, fleg, K, W)
    f_avg = f_gpu / K
    f_ms = f_wall / K * 1e3
    f_bytes = FWD_BYTES_PER_TOKEN_HEAD[w1.dtype] * fleg.token_heads
    f_flops = fwd_flops_per_token_head(args.chunk) * fleg.token_heads
    f_issued = fwd_issued_flops_per_token_head(args.chunk) * fleg.token_heads
    f_ach = f_bytes / f_avg / 1e9
    fwd_tokens_per_s = K * fleg.tokens / f_wall
    # the same call from a cold cache (each call alone after a 2 GiB write)
    cold = time_cold(torch, fleg.stream, fleg, max(K // 2, 10), 2)
    c_med, c_min = cold[len(cold) // 2], cold[0]

    result = {
        "metric": METRIC, "value": fwd_tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "laplace-layer-fwd B=1 H=16 T=2048 dk=96 dv=192 C=%d bf16 + "
                               "decode 1280 seqs x 24 layers x H=16 fp32 state" % args.chunk,
                   "global_batch": 1, "seq_len": 2048, "parallelism": "none (1 GPU)"},
        "roofline": None,
        "fwd": {"ms_per_call_wall": f_ms, "avg_call_us_events": f_avg * 1e6,
                "timing": "K back-to-back gla_fwd_chunked calls; HIP events on the launch stream around the region",
                "roofline": {"bound": "hbm", "achieved": f_ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": f_ach / HBM_PEAK_GBS, "traffic": stored_traffic("fwd", f_bytes),
                             "kernel": "gla_fwd_chunked (tiled state chain + per-chunk output kernel)",
                             "alg_bytes_per_launch": f_bytes, "avg_launch_us": f_avg * 1e6,
                             "alg_flops_per_launch": f_flops, "issued_flops_per_launch": f_issued,
                             "mfma_tflops": f_flops / f_avg / 1e12,
                             "mfma_frac": f_flops / f_avg / 1e12 / BF16_MFMA_PEAK_TFLOPS},
                "cold": {"timing": "each call alone after a 2 GiB write that evicts the caches; HIP events "
                                   "around the call", "calls": len(cold), "median_us": c_med * 1e6,
                         "min_us": c_min * 1e6, "tokens_per_s_median": fleg.tokens / c_med,
                         "hbm_frac_median": f_bytes / c_med / 1e9 / HBM_PEAK_GBS}},
    }
    del fleg
    torch.cuda.empty_cache()

    # ---- 64k-token prefill (B=1, T=65,536, S0 ~ N(0, 0.01)): one call per step
    w3 = ws[3]
    lleg = FwdLeg(gla, gi, torch, w3, 3, args.chunk)
    l_wall, l_gpu = time_region(torch, lleg.stream, lleg, max(K // 4, 8), W)
    l_avg = l_gpu / max(K // 4, 8)
    l_bytes = FWD_BYTES_PER_TOKEN_HEAD[w3.dtype] * lleg.token_heads
    l_flops = fwd_flops_per_token_head(args.chunk) * lleg.token_heads
    result["long_prefill"] = {
        "workload": "long-prefill-64k B=1 H=16 T=65536 dk=96 dv=192 C=%d bf16, S0 given" % args.chunk,
        "calls": max(K // 4, 8), "avg_call_us": l_avg * 1e6, "tokens_per_s": lleg.tokens / l_avg,
        "plan": gla.plan_resolve(gla.GLA_BF16, 1, w3.T, 16, 96, 192, args.chunk),
        "roofline": {"bound": "hbm", "achieved": l_bytes / l_avg / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": l_bytes / l_avg / 1e9 / HBM_PEAK_GBS, "traffic": stored_traffic("long", l_bytes),
                     "alg_bytes_per_launch": l_bytes,
                     "alg_flops_per_launch": l_flops, "mfma_tflops": l_flops / l_avg / 1e12,
                     "mfma_frac": l_flops / l_avg / 1e12 / BF16_MFMA_PEAK_TFLOPS}}
    # the same prefill split in two halves carrying the state
    sleg = SplitLeg(lleg, gla, torch, args.chunk)
    s_wall, s_gpu = time_region(torch, sleg.stream, sleg, max(K // 4, 8), W)
    s_avg = s_gpu / max(K // 4, 8)
    result["long_prefill"]["split_2x%d" % (w3.T // 2)] = {
        "calls": "two gla_fwd_chunked calls of %d tokens, the state carried between them" % (w3.T // 2),
        "avg_pair_us": s_avg * 1e6, "tokens_per_s": sleg.tokens / s_avg,
        "plan_per_half": gla.plan_resolve(gla.GLA_BF16, 1, w3.T // 2, 16, 96, 192, args.chunk),
        "hbm_frac": l_bytes / s_avg / 1e9 / HBM_PEAK_GBS}
    del sleg, lleg
    torch.cuda.empty_cache()

    # ---- the forward by chunk size (the pages' chunk-size trade-off, on MI355X): the
    # Laplace layer and the training width's forward at C = 32, 64, 128, 256 (256-token
    # chunks run in the tiled-chain form only; 32 in the segment form only)
    result["fwd_chunks"] = {}
    nk = max(K // 2, 10)
    for name, wi in (("laplace_layer", 1), ("train_width", 2)):
        wk = ws[wi]
        row = {}
        for C in (32, 64, 128, 256):
            cl = FwdLeg(gla, gi, torch, wk, wi, C)
            _, g = time_region(torch, cl.stream, cl, nk, W)
            avg = g / nk
            cb = FWD_BYTES_PER_TOKEN_HEAD[wk.dtype] * cl.token_heads
            row[str(C)] = {"avg_call_us": avg * 1e6, "tokens_per_s": cl.tokens / avg,
                           "hbm_frac": cb / avg / 1e9 / HBM_PEAK_GBS,
                           "alg_flops_per_call": fwd_flops_per_token_head(C) * cl.token_heads,
                           "plan": gla.plan_resolve(gla.GLA_BF16, wk.B, wk.T, 16, 96, 192, C)}
            del cl
            torch.cuda.empty_cache()
        result["fwd_chunks"][name] = row

    # ---- training-step legs (mixer-train workload, chunks 128, 64, 32 and 256)
    w2 = ws[2]
    t_ms = 0.0
    result["train"] = {}
    for C in (() if args.no_train else (128, 64, 32, 256)):
        tleg = TrainLeg(gla, gi, torch, w2, 2, C)
        t_wall, t_gpu = time_region(torch, tleg.stream, tleg, K, W)
        t_avg = t_gpu / K
        tb = train_bytes_per_token_head(C) * tleg.token_heads
        tf = train_flops_per_token_head(C) * tleg.token_heads
        leg = {"value": K * tleg.tokens / t_wall, "unit": "tokens/s", "ms_per_step": t_wall / K * 1e3,
               "workload": f"mixer-train B=8 H=16 T=2048 dk=96 dv=192 C={C} bf16, fwd + bwd (dq,dk,dv,dlambda)",
               "calls": "gla_fwd_chunked_states + gla_bwd_chunked_states (chunk states saved by the forward)",
               "avg_step_us": t_avg * 1e6, "alg_bytes_per_step": tb, "alg_flops_per_step": tf,
               "plan": gla.plan_resolve(gla.GLA_BF16, w2.B, w2.T, 16, 96, 192, C),
               "hbm_gbs": tb / t_avg / 1e9, "hbm_frac": tb / t_avg / 1e9 / HBM_PEAK_GBS,
               "mfma_tflops": tf / t_avg / 1e12, "mfma_frac": tf / t_avg / 1e12 / BF16_MFMA_PEAK_TFLOPS}
        if C == args.chunk:
            # the backward's gradient kernel: q, k, v, do and both chunk-state snapshots in,
            # dq, dk, dv out, against its measured HBM traffic (rocprofv3 counters)
            gb = (4 * w2.dk + 3 * w2.dv + 2 * w2.dk * w2.dv / C) * 2 * tleg.token_heads
            leg["grad_kernel"] = {"kernel": f"grad_fused_bf16<{C}> (one workgroup per chunk and unit)",
                                  "alg_bytes_per_call": gb, "traffic": stored_traffic("grad", gb)}
        del tleg
        torch.cuda.empty_cache()
        rleg = TrainLeg(gla, gi, torch, w2, 2, C, saved=False)
        r_wall, r_gpu = time_region(torch, rleg.stream, rleg, K, W)
        leg["recompute"] = {"calls": "gla_fwd_chunked + gla_bwd_chunked (the backward recomputes the states)",
                            "avg_step_us": r_gpu / K * 1e6, "value": K * rleg.tokens / r_wall}
        tleg = rleg
        result["train"][f"chunk{C}"] = leg
        if C == 128:
            t_ms = leg["ms_per_step"]
        del tleg
        torch.cuda.empty_cache()

    # ---- decode leg (1,280 sequences x 24 layers)
    d_ms = 0.0
    if not args.no_decode:
        w4 = ws[4]
        dleg = DecodeLeg(gla, gi, torch, w4, 4)
        d_wall, d_gpu = time_decode(torch, dleg, K, W)
        d_ms = d_wall / K * 1e3
        per_launch_bytes = DEC_BYTES_PER_SEQ_HEAD * w4.B * w4.H
        d_avg = d_gpu / (K * w4.decode_layers)
        d_ach = per_launch_bytes / d_avg / 1e9
        result["decode"] = {
            "value": per_launch_bytes * w4.decode_layers * K / d_wall / 1e9, "unit": "GB/s",
            "tokens_per_s": w4.B * K / d_wall, "ms_per_step": d_ms,
            "launches_per_step": w4.decode_layers,
            "roofline": {"bound": "hbm", "achieved": d_ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": d_ach / HBM_PEAK_GBS,
                         "traffic": stored_traffic("decode", per_launch_bytes),
                         "kernel": "gla_decode_step", "alg_bytes_per_launch": per_launch_bytes,
                         "avg_launch_us": d_avg * 1e6},
        }
        # the same steps through gla_decode_step_pool, pages addressed by shuffled slots
        dleg.use_pool = True
        p_wall, p_gpu = time_decode(torch, dleg, K, W)
        p_avg = p_gpu / (K * w4.decode_layers)
        result["decode"]["pool"] = {
            "kernel": "gla_decode_step_pool (1,280 rows, pages at a shuffled slot permutation)",
            "ms_per_step": p_wall / K * 1e3, "avg_launch_us": p_avg * 1e6,
            "achieved": per_launch_bytes / p_avg / 1e9, "unit": "GB/s",
            "frac": per_launch_bytes / p_avg / 1e9 / HBM_PEAK_GBS}
        # the rate depends on how far apart the pages of neighbouring rows lie, not on the
        # indirection: the same pool with the batch in slot order, and with runs of 16 rows
        # on consecutive pages (the runs themselves shuffled)
        shuffled = dleg.slots.clone()
        g = torch.Generator().manual_seed(4)
        runs = torch.randperm(w4.B // 16, generator=g)
        patterns = {"sorted": torch.arange(w4.B),
                    "runs_of_16": (runs[:, None] * 16 + torch.arange(16)[None, :]).reshape(-1)}
        result["decode"]["pool"]["slot_order"] = {}
        for name, perm in patterns.items():
            dleg.slots.copy_(perm.to(torch.int32))
            s_wall, s_gpu = time_decode(torch, dleg, K, W)
            s_avg = s_gpu / (K * w4.decode_layers)
            result["decode"]["pool"]["slot_order"][name] = {
                "avg_launch_us": s_avg * 1e6, "achieved": per_launch_bytes / s_avg / 1e9,
                "frac": per_launch_bytes / s_avg / 1e9 / HBM_PEAK_GBS}
        dleg.slots.copy_(shuffled)
        # the same steps with the mixer epilogue fused into the decode kernel
        dleg.use_pool, dleg.use_epi = False, True
        e_wall, e_gpu = time_decode(torch, dleg, K, W)
        e_avg = e_gpu / (K * w4.decode_layers)
        eb = DEC_EPI_BYTES_PER_SEQ_HEAD * w4.B * w4.H
        result["decode"]["epilogue_fused"] = {
            "kernel": "gla_decode_step_epilogue (decode + gated value copy, tier RMSNorm, SiLU gate)",
            "ms_per_step": e_wall / K * 1e3, "avg_launch_us": e_avg * 1e6, "alg_bytes_per_launch": eb,
            "achieved": eb / e_avg / 1e9, "unit": "GB/s", "frac": eb / e_avg / 1e9 / HBM_PEAK_GBS}
        del dleg
        torch.cuda.empty_cache()
    result["ms_per_step"] = f_ms + t_ms + d_ms
    # the top-level roofline is the step's dominant kernel: the decode kernel (24 launches,
    # ~95% of the step's time) when the decode leg runs, else the forward
    if "decode" in result:
        result["roofline"] = dict(result["decode"]["roofline"],
                                  dominant=f"{d_ms:.2f} of {result['ms_per_step']:.2f} ms per step")
    else:
        result["roofline"] = dict(result["fwd"]["roofline"])

    # ---- depth-wise conv (not part of the step): training-width prefill, decode rows of one layer
    result["conv"] = {}
    for name, B, T, dec in (("prefill", w2.B, w2.T, False), ("decode", ws[4].B, 1, True)):
        cleg = ConvLeg(gla, gi, torch, B, T, 11, decode=dec)
        c_wall, c_gpu = time_region(torch, cleg.stream, cleg, K, W)
        c_avg = c_gpu / K
        result["conv"][name] = {
            "kernel": "gla_conv1d_silu_decode" if dec else "gla_conv1d_silu",
            "workload": f"{'N' if dec else 'B'}={B}" + ("" if dec else f" T={T}") + f" D={CONV_D} bf16, width 4",
            "avg_launch_us": c_avg * 1e6, "alg_bytes_per_launch": cleg.bytes,
            "achieved": cleg.bytes / c_avg / 1e9, "unit": "GB/s", "frac": cleg.bytes / c_avg / 1e9 / HBM_PEAK_GBS}
        del cleg
        torch.cuda.empty_cache()

    # ---- mixer epilogue pass (not part of the step): the layer's prefill rows and the training width
    result["epilogue"] = {}
    for name, wk in (("layer", w1), ("train_width", w2)):
        eleg = EpilogueLeg(gla, gi, torch, wk, 7)
        e_wall, e_gpu = time_region(torch, eleg.stream, eleg, K, W)
        e_avg = e_gpu / K
        eb = EPI_BYTES_PER_TOKEN_HEAD * eleg.token_heads
        result["epilogue"][name] = {
            "kernel": "gla_mixer_epilogue", "rows": wk.B * wk.T, "avg_launch_us": e_avg * 1e6,
            "alg_bytes_per_launch": eb, "achieved": eb / e_avg / 1e9, "unit": "GB/s",
            "frac": eb / e_avg / 1e9 / HBM_PEAK_GBS}
        del eleg
        torch.cuda.empty_cache()
    # the forward with the epilogue in its output kernel, Laplace layer
    fe = FwdEpilogueLeg(gla, gi, torch, w1, 1, args.chunk)
    fe_wall, fe_gpu = time_region(torch, fe.stream, fe, K, W)
    fe_avg = fe_gpu / K
    fe_bytes = (FWD_BYTES_PER_TOKEN_HEAD["bf16"] + 2 * 192) * fe.token_heads   # + the gate g
    result["epilogue"]["fwd_fused_layer"] = {
        "kernel": "gla_fwd_chunked_epilogue (chain + output kernel with the epilogue in its store)",
        "avg_call_us": fe_avg * 1e6, "tokens_per_s": K * w1.B * w1.T / fe_wall,
        "alg_bytes_per_call": fe_bytes, "achieved": fe_bytes / fe_avg / 1e9, "unit": "GB/s",
        "frac": fe_bytes / fe_avg / 1e9 / HBM_PEAK_GBS}
    del fe
    torch.cuda.empty_cache()

    result["env"] = machine_info(torch)   # clocks read right after the timed legs
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_fwd(gi, w1, 1)
        result["long_prefill"]["cpu_baseline"] = cpu_baseline_long(gi, ws[3], 3)
        if result["train"]:
            result["train"]["cpu_baseline"] = cpu_baseline_train(gi, w2, 2)
        if not args.no_decode:
            result["decode"]["cpu_baseline"] = cpu_baseline_decode(gi, ws[4], 4)
        result["epilogue"]["cpu_baseline"] = cpu_baseline_epilogue(gi, w1, 7)
        if "conv" in result:
            result["conv"]["cpu_baseline"] = cpu_baseline_conv(gi, 5)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

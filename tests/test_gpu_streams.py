"""Calls on explicit streams and from several host threads at once.

The boundary launches on the stream it is given, and the binding allocates each call's
outputs and workspace on that stream (so the caching allocator cannot hand their
memory to work on another stream while the call's kernels still use it).  The library
keeps no state between calls (the allocation-free forward aside, whose shared array
is documented as racing), so calls from different threads on different streams, in
flight together, give the bits that the same calls give one after another.
"""
import sys
import threading

import pytest
import torch

import gated_linear_attention_simple_amd as gla
import gla_inputs as gi

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _jobs():
    """Four independent calls, each a function of a stream returning its outputs."""
    w1, w2, w4 = gi.workloads()[1], gi.workloads()[2], gi.workloads()[4]
    xf = gi.fwd_inputs(w1, DEV, 8101, s0_var=0.01)
    xt = gi.fwd_inputs(w2, DEV, 8102, B=2, T=1000, with_do=True, s0_var=0.01)
    wd = gi.Workload(w4.name, 64, 1, 16, 96, 192, 0, "bf16", w4.lambdas, w4.scale, w4.s0_var, 1)
    lam_d = torch.tensor(wd.lambdas, dtype=torch.float32, device=DEV)
    S_d = gi.decode_state(wd, DEV, seed=8103, layer=0)
    d = gi.decode_token_inputs(wd, DEV, seed=8103, layer=0, step=0)
    xe = gi.fwd_inputs(w1, DEV, 8104, B=2, T=700)
    ee = gi.epilogue_inputs(w1, DEV, 8104, (2, 700))

    def fwd(s):
        return gla.fwd_chunked(xf["q"], xf["k"], xf["v"], xf["lam"], S0=xf["S0"], scale=xf["scale"], stream=s)

    def train(s):
        args = (xt["q"], xt["k"], xt["v"], xt["lam"])
        _, _, st = gla.fwd_chunked_states(*args, S0=xt["S0"], scale=xt["scale"], chunk=64, stream=s)
        return gla.bwd_chunked_states(*args, xt["do"], st, S0=xt["S0"], scale=xt["scale"], chunk=64, stream=s)

    def decode(s):
        with torch.cuda.stream(s):
            S = S_d.clone()
        o = gla.decode_step(d["q"], d["k"], d["v"], lam_d, S, scale=wd.scale, stream=s)
        return o, S

    def epilogue(s):
        return (gla.mixer_epilogue(xe["q"], xe["k"], xe["v"], xe["v"], ee["g"], ee["norm_w"], ee["tier"],
                                   aug_a=ee["aug_a"], stream=s),)

    return {"fwd": fwd, "train": train, "decode": decode, "epilogue": epilogue}


def _flat(out):
    return [t for t in out if t is not None]


def test_explicit_side_stream_while_current_is_default():
    """Each call on a side stream, the current stream left as the default one; right after
    each call (no wait) the current stream allocates and overwrites fresh memory, as a
    caller's next work would.  The results equal those of the same calls on the current
    stream."""
    jobs = _jobs()
    ref = {name: [t.clone() for t in _flat(f(None))] for name, f in jobs.items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for name, f in jobs.items():
        _say(f"side stream: {name}")
        out = _flat(f(side))
        junk = [torch.full((1 << 22,), float(i), device=DEV) for i in range(8)]   # current-stream allocations
        del junk
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for a, b in zip(out, ref[name]):
            assert torch.equal(a, b), f"{name}: side-stream result differs"


def test_concurrent_threads_and_streams():
    """Four host threads, each with its own stream, run their call four times while the
    others run theirs; every result equals the sequential one bit for bit."""
    jobs = _jobs()
    ref = {name: [t.clone() for t in _flat(f(None))] for name, f in jobs.items()}
    torch.cuda.synchronize()
    _say("4 threads x 4 calls on 4 streams")
    results, errors = {}, []

    def worker(name, f):
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            outs = [_flat(f(s)) for _ in range(4)]
            s.synchronize()
            results[name] = outs
        except Exception as exc:   # reported by the main thread
            errors.append((name, repr(exc)))

    threads = [threading.Thread(target=worker, args=(n, f)) for n, f in jobs.items()]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    torch.cuda.synchronize()
    assert not errors, errors
    assert sorted(results) == sorted(jobs)
    for name, outs in results.items():
        for i, out in enumerate(outs):
            for a, b in zip(out, ref[name]):
                assert torch.equal(a, b), f"{name} call {i}: differs from the sequential result"

"""Seeded synthetic inputs for the Simple GLA mixer (shared by tests, bench, smoke).

This module holds no arithmetic of the method: it only draws seeded Gaussian
tensors of the workload shapes and lists the workload definitions.  Both the
HIP path and the fp64 oracle consume what it returns (the oracle always gets
the exact values the GPU consumed, copied back and widened to fp64).

Workloads (shapes from the Laplace 3B post, section "i14 and the Laplace 3B
architecture": H=16 heads, dk=96, dv=192, sequence 2,048 in 16 chunks of 128;
decode at 1,280 concurrent sequences over 24 layers from section "Optimizing
inference on Trainium2").  "N(0, x)" means variance x.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

_TID = {"q": 0, "k": 1, "v": 2, "do": 3, "S0": 4, "state": 5, "dS": 6, "g": 7, "aug": 8, "normw": 9,
        "cx": 10, "cw": 11, "cb": 12, "cwin": 13}


def laplace_lambdas(H: int = 16):
    """1 - lambda_h log-spaced from 0.1 down to 0.001 across the heads."""
    if H == 1:
        return [0.9]
    return [1.0 - 10.0 ** (-1.0 - 2.0 * h / (H - 1)) for h in range(H)]


def page_lambdas(H: int = 16, t_min: float = 1.0, t_max: float = 2048.0):
    """The Laplace 3B post's geometric decay schedule (section "i14 and the Laplace 3B
    architecture", paragraph *Decay schedule*) read as half-lives spaced geometrically
    from t_min to t_max tokens: lambda_h = 2^(-1 / half-life_h).  Head 0 is 0.5, so
    lambda^C underflows fp32's normal range at C = 128 (a stress input)."""
    if H == 1:
        return [2.0 ** (-1.0 / t_min)]
    return [2.0 ** (-1.0 / (t_min * (t_max / t_min) ** (h / (H - 1)))) for h in range(H)]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    chunk: int
    dtype: str                     # "f32" or "bf16"
    lambdas: tuple
    scale: float
    s0_var: float = 0.0            # 0 -> no initial state
    decode_layers: int = 0         # decode workloads only
    extra: dict = field(default_factory=dict)


def workloads():
    lam16 = tuple(laplace_lambdas(16))
    s = 96 ** -0.5
    return {
        0: Workload("tiny-fwd-f32", 1, 256, 2, 16, 32, 32, "f32", (0.9, 0.99), 1.0),
        1: Workload("laplace-layer-fwd", 1, 2048, 16, 96, 192, 128, "bf16", lam16, s),
        2: Workload("mixer-train-step", 8, 2048, 16, 96, 192, 128, "bf16", lam16, s,
                    extra={"chunks": (128, 64)}),
        3: Workload("long-prefill-64k", 1, 65536, 16, 96, 192, 128, "bf16", lam16, s,
                    s0_var=0.01),
        4: Workload("decode-1280x24", 1280, 1, 16, 96, 192, 0, "bf16", lam16, s,
                    s0_var=0.1, decode_layers=24),
    }


def _mix(*vals: int) -> int:
    """splitmix64 over the key words -> a 63-bit generator seed."""
    x = 0x9E3779B97F4A7C15
    for v in vals:
        x = (x ^ (int(v) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        x = (x + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        x = z ^ (z >> 31)
    return x & 0x7FFFFFFFFFFFFFFF


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def normal(shape, var, dtype, device, seed, tensor, layer=0, step=0, out=None):
    """Seeded N(0, var) tensor, drawn in fp32 then rounded (RNE) to `dtype`."""
    g = torch.Generator(device=device)
    g.manual_seed(_mix(seed, _TID[tensor], layer, step))
    std = math.sqrt(var)
    if out is not None:
        assert out.dtype == torch.float32
        out.normal_(0.0, std, generator=g)
        return out
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def fwd_inputs(w: Workload, device, seed: int, B=None, T=None, with_do=False,
               with_dS=False, s0_var=None):
    """q, k ~ N(0, 1/dk), v ~ N(0, 1) in the workload dtype; fp32 lambda; optional S0/do/dS_T."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    dt = torch_dtype(w.dtype)
    out = {
        "q": normal((B, T, w.H, w.dk), 1.0 / w.dk, dt, device, seed, "q"),
        "k": normal((B, T, w.H, w.dk), 1.0 / w.dk, dt, device, seed, "k"),
        "v": normal((B, T, w.H, w.dv), 1.0, dt, device, seed, "v"),
        "lam": torch.tensor(w.lambdas, dtype=torch.float32, device=device),
        "scale": float(w.scale),
        "S0": None,
    }
    var = w.s0_var if s0_var is None else s0_var
    if var > 0:
        out["S0"] = normal((B, w.H, w.dk, w.dv), var, torch.float32, device, seed, "S0")
    if with_do:
        out["do"] = normal((B, T, w.H, w.dv), 1.0, dt, device, seed, "do")
    if with_dS:
        out["dS"] = normal((B, w.H, w.dk, w.dv), 1.0, torch.float32, device, seed, "dS")
    return out


def decode_token_inputs(w: Workload, device, seed: int, layer: int, step: int, N=None):
    """One decode token per sequence for (layer, step): q, k [N,H,dk], v [N,H,dv]."""
    N = w.B if N is None else N
    dt = torch_dtype(w.dtype)
    return {
        "q": normal((N, w.H, w.dk), 1.0 / w.dk, dt, device, seed, "q", layer, step),
        "k": normal((N, w.H, w.dk), 1.0 / w.dk, dt, device, seed, "k", layer, step),
        "v": normal((N, w.H, w.dv), 1.0, dt, device, seed, "v", layer, step),
    }


def decode_state(w: Workload, device, seed: int, layer: int, N=None, out=None):
    """fp32 state pool slice [N,H,dk,dv] ~ N(0, s0_var) for one layer."""
    N = w.B if N is None else N
    return normal((N, w.H, w.dk, w.dv), w.s0_var, torch.float32, device, seed,
                  "state", layer, 0, out=out)


def contiguous_tiers(H: int, n_tiers: int):
    """Head h -> tier h * n_tiers // H: contiguous groups of heads in decay order."""
    return [h * n_tiers // H for h in range(H)]


def epilogue_inputs(w: Workload, device, seed: int, lead, n_tiers=4, aug_var=None, layer=0, step=0):
    """Epilogue parameters and gate for rows `lead` (a shape tuple): g [*lead, H, dv] ~ N(0, 1)
    in the workload dtype; fp32 aug_a [H, dk] ~ N(0, aug_var) (default dk, which makes the
    gate logit q . (a k) about N(0, 1) for q, k ~ N(0, 1/dk)); fp32 norm_w [n_tiers, dv] =
    1 + N(0, 0.1); the contiguous tier map."""
    dt = torch_dtype(w.dtype)
    av = float(w.dk) if aug_var is None else aug_var
    return {
        "g": normal(tuple(lead) + (w.H, w.dv), 1.0, dt, device, seed, "g", layer, step),
        "aug_a": normal((w.H, w.dk), av, torch.float32, device, seed, "aug"),
        "norm_w": normal((n_tiers, w.dv), 0.1, torch.float32, device, seed, "normw") + 1.0,
        "tier": contiguous_tiers(w.H, n_tiers),
    }


def conv_inputs(B: int, T: int, D: int, dtype: str, device, seed: int, K: int = 4, layer=0, step=0):
    """Depth-wise conv inputs: x [B, T, D] ~ N(0, 1) in `dtype`; fp32 taps w [D, K] ~ N(0, 1/K),
    bias [D] ~ N(0, 0.01), and a carried window [B, K, D] of earlier inputs (N(0, 1) rounded
    to `dtype`, as a window of that dtype's inputs holds)."""
    dt = torch_dtype(dtype)
    return {
        "x": normal((B, T, D), 1.0, dt, device, seed, "cx", layer, step),
        "w": normal((D, K), 1.0 / K, torch.float32, device, seed, "cw"),
        "bias": normal((D,), 0.01, torch.float32, device, seed, "cb"),
        "win": normal((B, K, D), 1.0, dt, device, seed, "cwin", layer).float(),
    }

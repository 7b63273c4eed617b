"""Pins for the fp64 oracle: results fixed by the pages and by mathematics.

Every check here is an implementation *other than* the oracle's per-token
recurrence, written from what the Laplace 3B post states:

* section "GLA mixer": the decayed rank-1 state update and the readout;
  with lambda = 1 the mixer is causal (cumulative) linear attention, with
  lambda = 0 it keeps only the current key-value pair, so o_t = (q_t.k_t) v_t;
* section "Challenge 1" (chunked GLA): inside a chunk the output is a
  decay-masked linear attention plus the running state's contribution, and the
  state advances by the decay compounded over the chunk -- the chunked form
  must equal the recurrent one for any chunk size;
* the state is a fixed dk x dv matrix per head whatever the sequence length
  (section "GLA mixer" and the closing remark of the architecture section);
* the gradient checks use central finite differences, fp64 autograd of the
  quadratic (all-pairs) form, and a scaling identity for dlambda;
* the mixer epilogue (section "GLA mixer", after the readout: a value copy
  gated by sigmoid(q . (a (.) k)), half strength at a = 0; per-tier head
  RMSNorm; SiLU(g) gate) is checked on closed forms: sigmoid(ln 3) = 3/4,
  a constant vector normalises to its sign times the tier's weight, a
  one-hot value shows the gate as a channel ratio.

Each pin takes an oracle-like object (the ``oracle`` package or a variant with
a planted mistake) and returns True when it holds.
"""
from __future__ import annotations

import numpy as np

RNG_SEED = 1234


def _rand(shape, rng, scale=1.0):
    return rng.normal(size=shape) * scale


def tiny_case(B=2, T=13, H=3, dk=4, dv=6, seed=RNG_SEED, s0=True):
    rng = np.random.default_rng(seed)
    q = _rand((B, T, H, dk), rng, 0.5)
    k = _rand((B, T, H, dk), rng, 0.5)
    v = _rand((B, T, H, dv), rng)
    lam = np.array([0.3, 0.83, 0.97, 0.6, 0.999][:H])
    S0 = _rand((B, H, dk, dv), rng, 0.3) if s0 else None
    return q, k, v, lam, S0


def decay_matrix(lam, n):
    """D[t, s] = lam^(t-s) for t >= s else 0, with lam^0 = 1 (also for lam = 0)."""
    t = np.arange(n)[:, None]
    s = np.arange(n)[None, :]
    e = np.clip(t - s, 0, None).astype(float)
    D = np.where(e == 0, 1.0, np.power(lam, e))
    return np.where(t >= s, D, 0.0)


def powers(lam, e):
    e = np.asarray(e, dtype=float)
    return np.where(e == 0, 1.0, np.power(lam, e))


def quadratic_fwd(q, k, v, lam, S0, scale):
    """All-pairs form: o = scale[(QK^T (.) D) V + diag(lam^(t+1)) Q S0],
    S_T = lam^T S0 + K^T diag(lam^(T-1-s)) V."""
    B, T, H, dk = q.shape
    dv = v.shape[3]
    o = np.zeros((B, T, H, dv))
    S = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, :, h], k[b, :, h], v[b, :, h]
            D = decay_matrix(lam[h], T)
            o[b, :, h] = scale * ((Q @ K.T) * D) @ V
            S[b, h] = K.T @ (powers(lam[h], T - 1 - np.arange(T))[:, None] * V)
            if S0 is not None:
                o[b, :, h] += scale * powers(lam[h], np.arange(T) + 1)[:, None] * (Q @ S0[b, h])
                S[b, h] += powers(lam[h], T) * S0[b, h]
    return o, S


def chunked_fwd(q, k, v, lam, S0, scale, C):
    """Chunked-parallel form with chunk C (last chunk may be partial)."""
    B, T, H, dk = q.shape
    dv = v.shape[3]
    o = np.zeros((B, T, H, dv))
    Sfin = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
            for c0 in range(0, T, C):
                L = min(C, T - c0)
                Q, K, V = q[b, c0:c0 + L, h], k[b, c0:c0 + L, h], v[b, c0:c0 + L, h]
                i = np.arange(L)
                intra = ((Q @ K.T) * decay_matrix(lam[h], L)) @ V
                inter = powers(lam[h], i + 1)[:, None] * (Q @ S)
                o[b, c0:c0 + L, h] = scale * (intra + inter)
                S = powers(lam[h], L) * S + K.T @ (powers(lam[h], L - 1 - i)[:, None] * V)
            Sfin[b, h] = S
    return o, Sfin


def rel(a, b):
    a = np.asarray(a, dtype=float)
    b = np.asarray(b, dtype=float)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# --------------------------------------------------------------------------- pins

def pin_lambda_one(orc, tol=1e-12):
    """lambda = 1: causal linear attention o = scale(tril(QK^T) V + Q S0), S = S0 + K^T V."""
    q, k, v, lam, S0 = tiny_case()
    lam = np.ones_like(lam)
    o, S = orc.fwd(q, k, v, lam, S0=S0, scale=0.7)
    B, T, H, _ = q.shape
    ok = True
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, :, h], k[b, :, h], v[b, :, h]
            ref_o = 0.7 * (np.tril(Q @ K.T) @ V + Q @ S0[b, h])
            ref_S = S0[b, h] + K.T @ V
            ok &= rel(o[b, :, h], ref_o) < tol and rel(S[b, h], ref_S) < tol
    return bool(ok)


def pin_lambda_zero(orc, tol=1e-12):
    """lambda = 0: only the current pair survives, o_t = scale (q_t.k_t) v_t."""
    q, k, v, lam, S0 = tiny_case()
    lam = np.zeros_like(lam)
    o, S = orc.fwd(q, k, v, lam, S0=S0, scale=1.3)
    ref_o = 1.3 * np.einsum("bthd,bthd->bth", q, k)[..., None] * v
    ref_S = np.einsum("bhd,bhe->bhde", k[:, -1], v[:, -1])
    return bool(rel(o, ref_o) < tol and rel(S, ref_S) < tol)


def pin_quadratic(orc, tol=1e-12):
    """General lambda: equals the decay-masked all-pairs form (with S0)."""
    q, k, v, lam, S0 = tiny_case()
    o, S = orc.fwd(q, k, v, lam, S0=S0, scale=0.9)
    ro, rS = quadratic_fwd(q, k, v, lam, S0, 0.9)
    return bool(rel(o, ro) < tol and rel(S, rS) < tol)


def pin_chunked(orc, tol=1e-12):
    """Chunked form == recurrent form for several chunk sizes, ragged tails included."""
    q, k, v, lam, S0 = tiny_case(T=23)
    o, S = orc.fwd(q, k, v, lam, S0=S0, scale=0.8)
    ok = True
    for C in (1, 3, 8, 16, 23, 32):
        co, cS = chunked_fwd(q, k, v, lam, S0, 0.8, C)
        ok &= rel(o, co) < tol and rel(S, cS) < tol
    return bool(ok)


def pin_resume(orc, tol=1e-12):
    """fwd(T1) then fwd(T2) from the carried state == fwd(T1 + T2)."""
    q, k, v, lam, S0 = tiny_case(T=17)
    o, S = orc.fwd(q, k, v, lam, S0=S0, scale=0.6)
    o1, S1 = orc.fwd(q[:, :7], k[:, :7], v[:, :7], lam, S0=S0, scale=0.6)
    o2, S2 = orc.fwd(q[:, 7:], k[:, 7:], v[:, 7:], lam, S0=S1, scale=0.6)
    return bool(rel(np.concatenate([o1, o2], 1), o) < tol and rel(S2, S) < tol)


def pin_batch_independent(orc, tol=0.0):
    """Each sequence of a batch gives exactly what it gives alone."""
    q, k, v, lam, S0 = tiny_case(B=3)
    o, S = orc.fwd(q, k, v, lam, S0=S0, scale=0.5)
    ok = True
    for b in range(3):
        ob, Sb = orc.fwd(q[b:b + 1], k[b:b + 1], v[b:b + 1], lam, S0=S0[b:b + 1], scale=0.5)
        ok &= rel(ob, o[b:b + 1]) <= tol and rel(Sb, S[b:b + 1]) <= tol
    return bool(ok)


def pin_state_size(orc):
    """The state is dk x dv per head for every T, and does not depend on scale."""
    q, k, v, lam, S0 = tiny_case(T=29)
    shapes = set()
    for T in (1, 5, 29):
        _, S = orc.fwd(q[:, :T], k[:, :T], v[:, :T], lam, S0=S0, scale=0.3)
        shapes.add(S.shape)
    _, Sa = orc.fwd(q, k, v, lam, S0=S0, scale=0.3)
    _, Sb = orc.fwd(q, k, v, lam, S0=S0, scale=2.0)
    return shapes == {(q.shape[0], q.shape[2], q.shape[3], v.shape[3])} and rel(Sa, Sb) == 0.0


def pin_decode_equals_fwd(orc, tol=1e-12):
    """T successive decode steps from S0 reproduce the forward over the same T tokens."""
    q, k, v, lam, S0 = tiny_case(T=9)
    o, S = orc.fwd(q, k, v, lam, S0=S0, scale=0.7)
    St = S0.copy()
    outs = []
    for t in range(q.shape[1]):
        ot, St = orc.decode(q[:, t], k[:, t], v[:, t], lam, St, scale=0.7)
        outs.append(ot)
    return bool(rel(np.stack(outs, 1), o) < tol and rel(St, S) < tol)


def pin_decode_closed_forms(orc, tol=1e-12):
    """Decode at lambda=0 keeps k v^T; at lambda=1 adds k v^T to the page."""
    q, k, v, lam, S0 = tiny_case(T=1)
    z = np.zeros_like(lam)
    o0, S_0 = orc.decode(q[:, 0], k[:, 0], v[:, 0], z, S0, scale=0.4)
    r_S0 = np.einsum("bhd,bhe->bhde", k[:, 0], v[:, 0])
    r_o0 = 0.4 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0])[..., None] * v[:, 0]
    o1, S_1 = orc.decode(q[:, 0], k[:, 0], v[:, 0], np.ones_like(lam), S0, scale=0.4)
    r_S1 = S0 + r_S0
    r_o1 = 0.4 * np.einsum("bhde,bhd->bhe", r_S1, q[:, 0])
    return bool(rel(S_0, r_S0) < tol and rel(o0, r_o0) < tol
                and rel(S_1, r_S1) < tol and rel(o1, r_o1) < tol)


def _loss(orc, q, k, v, lam, S0, do, dS, scale):
    o, S = orc.fwd(q, k, v, lam, S0=S0, scale=scale)
    return float(np.sum(o * do) + np.sum(S * dS))


def pin_finite_differences(orc, tol=1e-6, h=1e-6):
    """Every gradient of <do,o> + <dS_T,S_T> against central differences."""
    rng = np.random.default_rng(7)
    q, k, v, lam, S0 = tiny_case(B=1, T=9, H=2, dk=3, dv=4, seed=5)
    do = rng.normal(size=v.shape)
    dS = rng.normal(size=S0.shape)
    sc = 0.8
    dq, dk_, dv_, dlam, dS0 = orc.bwd(q, k, v, lam, do, S0=S0, dS_T=dS, scale=sc)
    ok = True
    for name, arr, grad in (("q", q, dq), ("k", k, dk_), ("v", v, dv_),
                            ("S0", S0, dS0), ("lam", lam, dlam)):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = {"q": q, "k": k, "v": v, "S0": S0, "lam": lam}
            plus = {n: a.copy() for n, a in args.items()}
            minus = {n: a.copy() for n, a in args.items()}
            plus[name][idx] += h
            minus[name][idx] -= h
            lp = _loss(orc, plus["q"], plus["k"], plus["v"], plus["lam"], plus["S0"], do, dS, sc)
            lm = _loss(orc, minus["q"], minus["k"], minus["v"], minus["lam"], minus["S0"], do, dS, sc)
            num[idx] = (lp - lm) / (2 * h)
        ok &= rel(grad, num) < tol
    return bool(ok)


def pin_autograd_quadratic(orc, tol=1e-11):
    """fp64 torch autograd of the all-pairs form gives the same gradients."""
    import torch

    rng = np.random.default_rng(11)
    q, k, v, lam, S0 = tiny_case(B=2, T=11, H=3, seed=9)
    do = rng.normal(size=v.shape)
    dS = rng.normal(size=S0.shape)
    sc = 0.9
    dq, dk_, dv_, dlam, dS0 = orc.bwd(q, k, v, lam, do, S0=S0, dS_T=dS, scale=sc)

    tq, tk, tv, tl, tS0 = (torch.tensor(a, dtype=torch.float64, requires_grad=True)
                           for a in (q, k, v, lam, S0))
    B, T, H, _ = q.shape
    t = torch.arange(T, dtype=torch.float64)
    diff = t[:, None] - t[None, :]
    mask = diff >= 0
    loss = 0.0
    for b in range(B):
        for hh in range(H):
            Q, K, V = tq[b, :, hh], tk[b, :, hh], tv[b, :, hh]
            lam_h = tl[hh]
            D = torch.where(mask, torch.pow(lam_h, diff.clamp(min=0)), torch.zeros(()))
            o = sc * ((Q @ K.T) * D) @ V + sc * torch.pow(lam_h, t + 1)[:, None] * (Q @ tS0[b, hh])
            S = K.T @ (torch.pow(lam_h, T - 1 - t)[:, None] * V) + torch.pow(lam_h, T) * tS0[b, hh]
            loss = loss + (o * torch.tensor(do[b, :, hh])).sum() + (S * torch.tensor(dS[b, hh])).sum()
    loss.backward()
    return bool(rel(dq, tq.grad.numpy()) < tol and rel(dk_, tk.grad.numpy()) < tol
                and rel(dv_, tv.grad.numpy()) < tol and rel(dlam, tl.grad.numpy()) < tol
                and rel(dS0, tS0.grad.numpy()) < tol)


def pin_dlambda_identity(orc, tol=1e-10):
    """With gamma = ln(lambda), substituting q~_t = q_t e^{gamma(t+1)}, k~_s = k_s e^{-gamma(s+1)}
    makes o depend on gamma only through q~, k~ (and S_T through e^{gamma T}); hence
    dgamma = sum_t (t+1)(q_t.dq_t - k_t.dk_t) + T <dS_T, S_T>, and dlambda = dgamma / lambda."""
    rng = np.random.default_rng(3)
    q, k, v, lam, S0 = tiny_case(B=2, T=15, H=3, seed=21)
    do = rng.normal(size=v.shape)
    dS = rng.normal(size=S0.shape)
    sc = 0.75
    dq, dk_, dv_, dlam, dS0 = orc.bwd(q, k, v, lam, do, S0=S0, dS_T=dS, scale=sc)
    _, S = orc.fwd(q, k, v, lam, S0=S0, scale=sc)
    T = q.shape[1]
    w = (np.arange(T) + 1.0)[None, :, None]
    dgamma = (w * (np.einsum("bthd,bthd->bth", q, dq) - np.einsum("bthd,bthd->bth", k, dk_))).sum(axis=(0, 1))
    dgamma = dgamma + T * np.einsum("bhde,bhde->h", dS, S)
    return bool(rel(dlam, dgamma / lam) < tol)


ALL_PINS = {
    "lambda_one": pin_lambda_one,
    "lambda_zero": pin_lambda_zero,
    "quadratic": pin_quadratic,
    "chunked": pin_chunked,
    "resume": pin_resume,
    "batch_independent": pin_batch_independent,
    "state_size": pin_state_size,
    "decode_equals_fwd": pin_decode_equals_fwd,
    "decode_closed_forms": pin_decode_closed_forms,
    "finite_differences": pin_finite_differences,
    "autograd_quadratic": pin_autograd_quadratic,
    "dlambda_identity": pin_dlambda_identity,
}


# ---------------------------------------------------------------- epilogue


def _epi_case(H=3, dk=5, dv=7):
    rng = np.random.default_rng(RNG_SEED + 7)
    w = rng.uniform(0.5, 2.0, size=(2, dv))
    tier = [h % 2 for h in range(H)]
    return rng, w, tier


def pin_epilogue_constant_vector(orc, tol=1e-12):
    """o + s v constant over the channels (v = 0, o = c): RMSNorm gives sign(c) w,
    and silu(ln 3) = (3/4) ln 3, so y = sign(c) (3/4) ln 3 w[tier(h)], eps = 0."""
    rng, w, tier = _epi_case()
    M, H, dk, dv = 4, 3, 5, 7
    c = np.array([-2.5, 0.3, 7.0, -0.01])
    o = np.broadcast_to(c[:, None, None], (M, H, dv)).copy()
    v = np.zeros((M, H, dv))
    q, k = rng.normal(size=(M, H, dk)), rng.normal(size=(M, H, dk))
    g = np.full((M, H, dv), np.log(3.0))
    y = orc.epilogue(q, k, v, o, g, rng.normal(size=(H, dk)), w, tier, eps=0.0)
    want = np.sign(c)[:, None, None] * 0.75 * np.log(3.0) * w[np.array(tier)][None]
    return bool(rel(y, want) < tol)


def pin_epilogue_gate_ratio(orc, tol=1e-12):
    """o = 1, v = e_0 and q . (a (.) k) = ln 3 give the gate 3/4, so channel 0 of x
    is 7/4 and the others 1: y_0 / y_c = 7/4 (w = 1, g constant); with a = 0 the
    gate is 1/2 and the ratio 3/2."""
    M, H, dk, dv = 2, 2, 4, 6
    o = np.ones((M, H, dv))
    v = np.zeros((M, H, dv))
    v[..., 0] = 1.0
    q = np.zeros((M, H, dk))
    k = np.zeros((M, H, dk))
    q[..., 2] = 2.0
    k[..., 2] = 0.5
    a = np.zeros((H, dk))
    a[:, 2] = np.log(3.0)               # q . (a (.) k) = 2 * ln 3 * 0.5
    g = np.full((M, H, dv), 1.3)
    w = np.ones((1, dv))
    y = orc.epilogue(q, k, v, o, g, a, w, [0] * H, eps=0.0)
    y0 = orc.epilogue(q, k, v, o, g, None, w, [0] * H, eps=0.0)
    r = y[..., 0][..., None] / y[..., 1:]
    r0 = y0[..., 0][..., None] / y0[..., 1:]
    return bool(np.abs(r - 1.75).max() < tol and np.abs(r0 - 1.5).max() < tol)


def pin_epilogue_zero_and_scale(orc, tol=1e-12):
    """A zero head vector stays zero (eps > 0, no division by zero), and with
    eps = 0 scaling o and v by any positive factor leaves y unchanged."""
    rng, w, tier = _epi_case()
    M, H, dk, dv = 3, 3, 5, 7
    q, k = rng.normal(size=(M, H, dk)), rng.normal(size=(M, H, dk))
    g = rng.normal(size=(M, H, dv))
    a = rng.normal(size=(H, dk))
    z = orc.epilogue(q, k, np.zeros((M, H, dv)), np.zeros((M, H, dv)), g, a, w, tier, eps=1e-6)
    o, v = rng.normal(size=(M, H, dv)), rng.normal(size=(M, H, dv))
    y1 = orc.epilogue(q, k, v, o, g, a, w, tier, eps=0.0)
    y2 = orc.epilogue(q, k, 37.0 * v, 37.0 * o, g, a, w, tier, eps=0.0)
    return bool(np.all(z == 0.0) and rel(y1, y2) < tol)


def pin_epilogue_eps_inside_root(orc, tol=1e-12):
    """Where eps enters the norm: with v = 0 and o = c on every channel, mean x^2 = c^2,
    so y = silu(ln 3) c / sqrt(c^2 + eps) w = (3/4) ln 3 c / sqrt(c^2 + eps) w.  With
    eps = 0.5 and |c| between 0.1 and 3 this differs from c / (|c| + eps) and from
    sign(c) (eps outside the root, or dropped) by 3% or more on every row."""
    rng, w, tier = _epi_case()
    M, H, dk, dv = 5, 3, 5, 7
    eps = 0.5
    c = np.array([-2.5, 0.3, 1.0, -0.1, 3.0])
    o = np.broadcast_to(c[:, None, None], (M, H, dv)).copy()
    v = np.zeros((M, H, dv))
    q, k = rng.normal(size=(M, H, dk)), rng.normal(size=(M, H, dk))
    g = np.full((M, H, dv), np.log(3.0))
    y = orc.epilogue(q, k, v, o, g, rng.normal(size=(H, dk)), w, tier, eps=eps)
    want = (0.75 * np.log(3.0) * c / np.sqrt(c * c + eps))[:, None, None] * w[np.array(tier)][None]
    return bool(rel(y, want) < tol)


ALL_PINS.update({
    "epilogue_eps_inside_root": pin_epilogue_eps_inside_root,
    "epilogue_constant_vector": pin_epilogue_constant_vector,
    "epilogue_gate_ratio": pin_epilogue_gate_ratio,
    "epilogue_zero_and_scale": pin_epilogue_zero_and_scale,
})


# ---------------------------------------------------------------- conv1d


def _conv_case(B=2, T=11, D=5, K=4, seed=RNG_SEED + 11):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(B, T, D)), rng.normal(size=(D, K)), rng.normal(size=D),
            rng.normal(size=(B, K, D)))


def _silu(u):
    return u / (1.0 + np.exp(-u))


def pin_conv_torch(orc, tol=1e-12):
    """fp64 torch grouped conv1d (cross-correlation; K-1 zeros of left padding for a
    fresh sequence, the window's last K-1 inputs prepended otherwise), then SiLU."""
    import torch
    x, w, b, win = _conv_case()
    B, T, D = x.shape
    K = w.shape[1]
    wt = torch.from_numpy(w).reshape(D, 1, K)
    bt = torch.from_numpy(b)
    xt = torch.from_numpy(x).transpose(1, 2)                     # [B, D, T]
    fresh = torch.nn.functional.conv1d(torch.nn.functional.pad(xt, (K - 1, 0)), wt, bt, groups=D)
    ctx = torch.cat([torch.from_numpy(win[:, 1:, :]).transpose(1, 2), xt], dim=2)
    carried = torch.nn.functional.conv1d(ctx, wt, bt, groups=D)
    y0, _ = orc.conv1d(x, w, b)
    y1, _ = orc.conv1d(x, w, b, win)
    ok0 = rel(y0, _silu(fresh.transpose(1, 2).numpy())) < tol
    ok1 = rel(y1, _silu(carried.transpose(1, 2).numpy())) < tol
    return bool(ok0 and ok1)


def pin_conv_impulse(orc, tol=1e-14):
    """A unit impulse at token t0 of channel d, no bias: u_{t0+m}[d] = w[d][K-1-m]
    for m < K and 0 elsewhere, other channels stay 0."""
    x, w, _, _ = _conv_case(B=1, T=12, D=3)
    K = w.shape[1]
    t0, d = 5, 1
    x = np.zeros_like(x)
    x[0, t0, d] = 1.0
    y, _ = orc.conv1d(x, w, None)
    want = np.zeros_like(y)
    for m in range(K):
        want[0, t0 + m, d] = _silu(w[d, K - 1 - m])
    return bool(np.abs(y - want).max() < tol)


def pin_conv_decode_equals_prefill(orc, tol=1e-12):
    """T decode steps from a window equal one prefill over the same T tokens, and
    both leave the same window."""
    x, w, b, win = _conv_case()
    y, wo = orc.conv1d(x, w, b, win)
    cur = win.copy()
    ys = []
    for t in range(x.shape[1]):
        yt, cur = orc.conv1d_decode(x[:, t], w, b, cur)
        ys.append(yt)
    return bool(rel(np.stack(ys, 1), y) < tol and rel(cur, wo) < tol)


def pin_conv_split_resume(orc, tol=0.0):
    """Prefill of tokens [0, T1) then [T1, T) through the window equals one prefill
    (exactly: the same products in the same order), for T1 below and above K."""
    x, w, b, win = _conv_case(T=13)
    y, wo = orc.conv1d(x, w, b, win)
    ok = True
    for t1 in (2, 7):
        ya, wa = orc.conv1d(x[:, :t1], w, b, win)
        yb, wb = orc.conv1d(x[:, t1:], w, b, wa)
        ok &= rel(np.concatenate([ya, yb], 1), y) <= tol and rel(wb, wo) <= tol
    return bool(ok)


def pin_conv_window_carry(orc, tol=0.0):
    """The window after a prefill is the last K inputs, oldest first; with T < K its
    head is the end of the previous window; T = 0 returns the window unchanged."""
    x, w, b, win = _conv_case(T=9)
    K = w.shape[1]
    _, wo = orc.conv1d(x, w, b, win)
    _, w2 = orc.conv1d(x[:, :2], w, b, win)
    _, w0 = orc.conv1d(x[:, :0], w, b, win)
    ok = np.array_equal(wo, x[:, -K:, :])
    ok &= np.array_equal(w2, np.concatenate([win[:, 2:, :], x[:, :2, :]], 1))
    ok &= np.array_equal(w0, win)
    return bool(ok)


ALL_PINS.update({
    "conv_torch": pin_conv_torch,
    "conv_impulse": pin_conv_impulse,
    "conv_decode_equals_prefill": pin_conv_decode_equals_prefill,
    "conv_split_resume": pin_conv_split_resume,
    "conv_window_carry": pin_conv_window_carry,
})

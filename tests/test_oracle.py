"""CPU tests of the fp64 oracle against what the pages and mathematics fix.

No GPU is used.  The oracle is checked against independent closed forms,
all-pairs and chunked reformulations, finite differences, fp64 autograd, a
dlambda identity, and the sizes the Laplace 3B post prints (tests/golden).
A second group plants plausible mistakes in a copy of the oracle's C source
and shows that at least one pin fails for each.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle_pins as P

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("name", sorted(P.ALL_PINS))
def test_pin(name):
    assert P.ALL_PINS[name](oracle), f"oracle fails pin {name}"


def test_empty_sequence_keeps_state():
    q, k, v, lam, S0 = P.tiny_case(T=0)
    o, S = oracle.fwd(q, k, v, lam, S0=S0, scale=1.0)
    assert o.shape == (2, 0, 3, 6)
    assert np.array_equal(S, S0)
    _, Sz = oracle.fwd(q, k, v, lam, S0=None, scale=1.0)
    assert not Sz.any()


def test_bwd_without_upstream_state_grad():
    """dS_T omitted == dS_T of zeros, and dS0 of a zero-S0 run is still returned."""
    rng = np.random.default_rng(0)
    q, k, v, lam, S0 = P.tiny_case(T=10)
    do = rng.normal(size=v.shape)
    a = oracle.bwd(q, k, v, lam, do, S0=None, dS_T=None, scale=0.5)
    b = oracle.bwd(q, k, v, lam, do, S0=np.zeros_like(S0), dS_T=np.zeros_like(S0), scale=0.5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ------------------------------------------------------------- page-printed sizes

def _golden():
    with open(os.path.join(HERE, "golden", "page_sizes.json")) as f:
        return json.load(f)


def test_page_sizes_state_and_projection():
    g = _golden()
    H, dk, dv = g["heads"]["value"], g["dk"]["value"], g["dv"]["value"]
    assert H * (2 * dk + 2 * dv) == g["qkvg_width"]["value"]
    # the oracle's state for one head is dk x dv whatever T (checked on a small T)
    rng = np.random.default_rng(1)
    q = rng.normal(size=(1, 3, 1, dk))
    v = rng.normal(size=(1, 3, 1, dv))
    _, S = oracle.fwd(q, q, v, [0.9], scale=1.0)
    assert S.shape[-2:] == (dk, dv)


def test_page_sizes_serving_state():
    """29.5 MB per sequence = fp32 GLA states of 24 layers x 16 heads x 96 x 192
    (28.31 MB) plus an fp32 (conv_width x hidden) convolution window per layer
    (1.18 MB); the KV cache of a comparable bf16 transformer at 8,192 tokens is
    ~82x larger.  The conv-window share is an inferred reading, not printed."""
    g = _golden()
    L, H, dk, dv = (g[k]["value"] for k in ("layers", "heads", "dk", "dv"))
    gla = L * H * dk * dv * 4
    conv = L * g["conv_width"]["value"] * g["hidden"]["value"] * 4
    assert abs((gla + conv) / 1e6 - g["state_mb_per_sequence"]["value"]) < 0.05
    kv = 2 * L * 8192 * g["hidden"]["value"] * 2
    assert round(kv / (gla + conv)) == g["kv_cache_ratio_at_8192"]["value"]


def test_page_decay_schedule_endpoints():
    """Half-life reading of the geometric schedule: head h has half-life
    T_min (T_max/T_min)^(h/(H-1)) tokens, lambda_h = 2^(-1/half-life)."""
    g = _golden()
    H, tmin, tmax = g["heads"]["value"], g["decay_t_min"]["value"], g["decay_t_max"]["value"]
    lam = [2.0 ** (-1.0 / (tmin * (tmax / tmin) ** (h / (H - 1)))) for h in range(H)]
    assert lam[0] == g["lambda_head0"]["value"]
    assert round(lam[-1], g["lambda_head15"]["digits"]) == g["lambda_head15"]["value"]
    assert g["seq_len"]["value"] // g["chunk"]["value"] == 16


# ------------------------------------------------------- planted mistakes (mutants)

MUTANTS = [
    ("no_decay", "S[(size_t)r * dv + c] = lam * S[(size_t)r * dv + c] + kt[r] * vt[c];",
     "S[(size_t)r * dv + c] = S[(size_t)r * dv + c] + kt[r] * vt[c];"),
    ("minus_update", "S[(size_t)r * dv + c] = lam * S[(size_t)r * dv + c] + kt[r] * vt[c];",
     "S[(size_t)r * dv + c] = lam * S[(size_t)r * dv + c] - kt[r] * vt[c];"),
    ("decay_squared", "S[(size_t)r * dv + c] = lam * S[(size_t)r * dv + c] + kt[r] * vt[c];",
     "S[(size_t)r * dv + c] = lam * lam * S[(size_t)r * dv + c] + kt[r] * vt[c];"),
    ("readout_wrong_index", "ot[c] += S[(size_t)r * dv + c] * qt[r];",
     "ot[c] += S[(size_t)r * dv + c] * qt[c % dk];"),
    ("no_scale", "for (int c = 0; c < dv; ++c) ot[c] *= scale;", "for (int c = 0; c < dv; ++c) ot[c] *= 1.0;"),
    ("readout_before_update",
     """            state_update(S, dk, dv, lambda[h], k + IDX_TOK(b, t, h, 0, T, H, dk),
                         v + IDX_TOK(b, t, h, 0, T, H, dv));
            readout(S, dk, dv, scale, q + IDX_TOK(b, t, h, 0, T, H, dk),
                    o + IDX_TOK(b, t, h, 0, T, H, dv));""",
     """            readout(S, dk, dv, scale, q + IDX_TOK(b, t, h, 0, T, H, dk),
                    o + IDX_TOK(b, t, h, 0, T, H, dv));
            state_update(S, dk, dv, lambda[h], k + IDX_TOK(b, t, h, 0, T, H, dk),
                         v + IDX_TOK(b, t, h, 0, T, H, dv));"""),
    ("s0_ignored", "if (S0) memcpy(S, S0 + IDX_ST(b, h, H, dk, dv), st * sizeof(double));\n        else memset(S, 0, st * sizeof(double));\n        for (int t = 0; t < T; ++t) {\n            state_update(S, dk, dv, lambda[h]",
     "memset(S, 0, st * sizeof(double));\n        for (int t = 0; t < T; ++t) {\n            state_update(S, dk, dv, lambda[h]"),
    ("bwd_G_no_scale", "G[(size_t)r * dv + c] += scale * qt[r] * dot[c];",
     "G[(size_t)r * dv + c] += qt[r] * dot[c];"),
    ("bwd_dq_previous_state", "for (int c = 0; c < dv; ++c) acc += St[(size_t)r * dv + c] * dot[c];",
     "for (int c = 0; c < dv; ++c) acc += Sp[(size_t)r * dv + c] * dot[c];"),
    ("bwd_dk_transposed", "for (int c = 0; c < dv; ++c) acc += G[(size_t)r * dv + c] * vt[c];",
     "for (int c = 0; c < dv; ++c) acc += G[(size_t)r * dv + c] * vt[(c + r) % dv];"),
    ("bwd_dv_uses_q", "for (int c = 0; c < dv; ++c) dvt[c] += G[(size_t)r * dv + c] * kt[r];",
     "for (int c = 0; c < dv; ++c) dvt[c] += G[(size_t)r * dv + c] * qt[r];"),
    ("bwd_dlambda_current_state", "for (size_t e = 0; e < st; ++e) inner += G[e] * Sp[e];",
     "for (size_t e = 0; e < st; ++e) inner += G[e] * St[e];"),
    ("bwd_no_adjoint_decay", "for (size_t e = 0; e < st; ++e) G[e] *= lam;",
     "for (size_t e = 0; e < st; ++e) G[e] *= 1.0;"),
    ("decode_readout_before_update",
     """        state_update(Sp, dk, dv, lambda[h], k + IDX_TOK(n, 0, h, 0, 1, H, dk),
                     v + IDX_TOK(n, 0, h, 0, 1, H, dv));
        readout(Sp, dk, dv, scale, q + IDX_TOK(n, 0, h, 0, 1, H, dk),
                o + IDX_TOK(n, 0, h, 0, 1, H, dv));""",
     """        readout(Sp, dk, dv, scale, q + IDX_TOK(n, 0, h, 0, 1, H, dk),
                o + IDX_TOK(n, 0, h, 0, 1, H, dv));
        state_update(Sp, dk, dv, lambda[h], k + IDX_TOK(n, 0, h, 0, 1, H, dk),
                     v + IDX_TOK(n, 0, h, 0, 1, H, dv));"""),
    ("batch_index_slip", "#define IDX_ST(b, h, H, DK, DV) (((size_t)(b) * (H) + (h)) * (size_t)(DK) * (DV))",
     "#define IDX_ST(b, h, H, DK, DV) (((size_t)(0) * (H) + (h)) * (size_t)(DK) * (DV))"),
    ("epi_gate_ignores_a", "z += qu[i] * (a ? a[(size_t)h * dk + i] : 0.0) * ku[i];", "z += qu[i] * ku[i];"),
    ("epi_norm_sum_not_mean", "const double inv = 1.0 / sqrt(ss / dv + eps);", "const double inv = 1.0 / sqrt(ss + eps);"),
    ("epi_eps_outside_root", "const double inv = 1.0 / sqrt(ss / dv + eps);",
     "const double inv = 1.0 / (sqrt(ss / dv) + eps);"),
    ("epi_eps_dropped", "const double inv = 1.0 / sqrt(ss / dv + eps);",
     "const double inv = ss > 0 ? 1.0 / sqrt(ss / dv) : 1.0 / sqrt(eps);"),
    ("epi_ungated_value", "x[c] = o[(size_t)u * dv + c] + s * v[(size_t)u * dv + c];",
     "x[c] = o[(size_t)u * dv + c] + v[(size_t)u * dv + c];"),
    ("epi_silu_is_identity", "y[(size_t)u * dv + c] = gc * sigmoid(gc) * x[c] * inv * wt[c];",
     "y[(size_t)u * dv + c] = gc * x[c] * inv * wt[c];"),
    ("epi_wrong_tier", "const double* wt = w + (size_t)tier[h] * dv;", "const double* wt = w;"),
    ("conv_taps_reversed", "u += w[(size_t)d * K + j] * x_at(x, win_in, b, t - (K - 1) + j, d, T, D, K);",
     "u += w[(size_t)d * K + j] * x_at(x, win_in, b, t - j, d, T, D, K);"),
    ("conv_excludes_current", "u += w[(size_t)d * K + j] * x_at(x, win_in, b, t - (K - 1) + j, d, T, D, K);",
     "u += w[(size_t)d * K + j] * x_at(x, win_in, b, t - K + j, d, T, D, K);"),
    ("conv_no_silu", "y[((size_t)b * T + t) * D + d] = u * sigmoid(u);", "y[((size_t)b * T + t) * D + d] = u;"),
    ("conv_bias_dropped", "            double u = bias ? bias[d] : 0.0;", "            double u = 0.0;"),
    ("conv_decode_bias_dropped", "double u = bias ? bias[d] : 0.0;\n        for (int j = 0; j < K; ++j) u += w[(size_t)d * K + j] * wn",
     "double u = 0.0;\n        for (int j = 0; j < K; ++j) u += w[(size_t)d * K + j] * wn"),
    ("conv_window_newest_first", "return win_in ? win_in[((size_t)b * K + (K + t)) * D + d] : 0.0;",
     "return win_in ? win_in[((size_t)b * K + (-1 - t)) * D + d] : 0.0;"),
    ("conv_decode_no_shift", "for (int s2 = 0; s2 + 1 < K; ++s2) wn[(size_t)s2 * D] = wn[(size_t)(s2 + 1) * D];", ""),
    ("conv_decode_channel_slip", "u += w[(size_t)d * K + j] * wn[(size_t)j * D];",
     "u += w[(size_t)((d + 1) % D) * K + j] * wn[(size_t)j * D];"),
]

CHEAP_PINS = [n for n in P.ALL_PINS if n != "autograd_quadratic"]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    variant = oracle.compile_variant(src.replace(old, new), str(tmp_path / f"mut_{name}.so"))
    failed = []
    for pin in CHEAP_PINS:
        try:
            ok = P.ALL_PINS[pin](variant)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin)
    assert failed, f"no pin catches the planted mistake {name}"


def test_dlambda_cancellation_scale():
    """Sanity of the fp64 dlambda at the Laplace shape on a short sequence:
    the recurrence value and the (t+1) identity agree to ~1e-9 relative even
    with lambda near 1, so the oracle's dlambda is usable as a reference."""
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 1, 64, 2, 96, 192
    q = rng.normal(size=(B, T, H, dk)) / math.sqrt(dk)
    k = rng.normal(size=(B, T, H, dk)) / math.sqrt(dk)
    v = rng.normal(size=(B, T, H, dv))
    do = rng.normal(size=(B, T, H, dv))
    lam = np.array([0.9, 0.999])
    dq, dk_, dv_, dlam, _ = oracle.bwd(q, k, v, lam, do, scale=dk ** -0.5)
    w = (np.arange(T) + 1.0)[None, :, None]
    dg = (w * (np.einsum("bthd,bthd->bth", q, dq) - np.einsum("bthd,bthd->bth", k, dk_))).sum(axis=(0, 1))
    assert P.rel(dlam, dg / lam) < 1e-9

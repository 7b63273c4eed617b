/*
 * gla_oracle.c -- plain fp64 CPU oracle for the Simple GLA mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code, header or table with the HIP
 * library and includes nothing from it.
 *
 * Source of the method: the AWS machine-learning blog post "Beyond the KV
 * cache: training and serving i14's Laplace 3B linear attention model on AWS
 * Trainium2 with native PyTorch" (called "the Laplace 3B post" below).
 *   - Section "i14 and the Laplace 3B architecture", paragraph "GLA mixer":
 *     each head keeps a dk x dv matrix state; per token it decays by the
 *     fixed per-head factor lambda_h and absorbs the rank-1 outer product
 *     k_t v_t^T; the readout queries the state with q_t.  The equation images
 *     are missing from the page text; the readings used here are
 *         S_t = lambda_h * S_{t-1} + k_t v_t^T,      o_t = scale * S_t^T q_t
 *     with the readout taken AFTER the update (so token t sees itself) and
 *     `scale` multiplying the readout only (S does not depend on it).
 *   - Same section, paragraph "Decay schedule": lambda_h is fixed, one per
 *     head, shared by every sequence of a batch.
 *   - Section "Optimizing inference" (decode): one fixed state page per
 *     sequence, read and written by one decode step per token.
 *   - Section "i14 and the Laplace 3B architecture", paragraph "GLA mixer",
 *     the sentences after the readout (gla_oracle_epilogue): a self-augmentation
 *     adds a copy of the value gated by the sigmoid of the query dotted with a
 *     learned per-channel rescaling a of the key (a = 0 gives a half-strength
 *     skip); each head's output then goes through the RMSNorm of its decay
 *     tier, the heads are concatenated and gated by SiLU(g).  The equation
 *     image is missing; the readings are written at the function.
 *   - Same section, paragraph "Normalization and convolution", and the
 *     parameter table row "Conv" (gla_oracle_conv1d, gla_oracle_conv1d_decode):
 *     before the mixer each channel of the residual stream goes through a
 *     depth-wise causal convolution of width 4 followed by SiLU, a summary of
 *     the last 4 tokens.  Readings at the functions.
 *
 * Everything is the plain per-token recurrence: no chunking, no blocking, no
 * reassociation.  The reverse-mode routine is the textbook adjoint of that
 * recurrence.  The only liberty taken is memory: the backward re-runs the
 * forward recurrence from stored checkpoints instead of keeping every S_t,
 * which recomputes bit-identical doubles.
 *
 * Layouts (row-major, last index fastest):
 *   q, k, dq, dk : [B][T][H][dk]      v, o, do, dv : [B][T][H][dv]
 *   S0, S_final, dS_T, dS0 : [B][H][dk][dv]      lambda, dlambda : [H]
 *   decode: q, k [N][H][dk], v, o [N][H][dv], S [N][H][dk][dv]
 *   epilogue: q, k [M][H][dk], v, o, g, y [M][H][dv] (M = rows, e.g. B*T),
 *             a [H][dk], w [n_tiers][dv], tier [H]
 *   conv: x, y [B][T][D] (decode: [N][D]), w [D][K], bias [D], window [B][K][D]
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX_TOK(b, t, h, d, T, H, D) ((((size_t)(b) * (T) + (t)) * (H) + (h)) * (D) + (d))
#define IDX_ST(b, h, H, DK, DV) (((size_t)(b) * (H) + (h)) * (size_t)(DK) * (DV))

int gla_oracle_abi(void) { return 1; }

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int gla_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One token of the recurrence on one head's state:  S <- lam*S + k v^T. */
static void state_update(double* S, int dk, int dv, double lam,
                         const double* kt, const double* vt) {
    for (int r = 0; r < dk; ++r)
        for (int c = 0; c < dv; ++c)
            S[(size_t)r * dv + c] = lam * S[(size_t)r * dv + c] + kt[r] * vt[c];
}

/* Readout  o = scale * S^T q  (o[c] = scale * sum_r S[r][c] q[r]). */
static void readout(const double* S, int dk, int dv, double scale,
                    const double* qt, double* ot) {
    for (int c = 0; c < dv; ++c) ot[c] = 0.0;
    for (int r = 0; r < dk; ++r)
        for (int c = 0; c < dv; ++c) ot[c] += S[(size_t)r * dv + c] * qt[r];
    for (int c = 0; c < dv; ++c) ot[c] *= scale;
}

/*
 * Forward: for every (b, h), S <- S0 (or 0); for t = 0..T-1:
 *   S <- lambda_h S + k_t v_t^T;  o_t = scale S^T q_t.   S_final = S.
 * S0 and S_final may be NULL.  Returns 0, or -1 on bad sizes / allocation.
 */
int gla_oracle_fwd(int B, int T, int H, int dk, int dv,
                   const double* q, const double* k, const double* v,
                   const double* lambda, const double* S0, double scale,
                   double* o, double* S_final, int nthreads) {
    if (B < 0 || T < 0 || H < 1 || dk < 1 || dv < 1) return -1;
    set_threads(nthreads);
    int failed = 0;
    const size_t st = (size_t)dk * dv;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long u = 0; u < (long)B * H; ++u) {
        const int b = (int)(u / H), h = (int)(u % H);
        double* S = (double*)malloc(st * sizeof(double));
        if (!S) { failed = 1; continue; }
        if (S0) memcpy(S, S0 + IDX_ST(b, h, H, dk, dv), st * sizeof(double));
        else memset(S, 0, st * sizeof(double));
        for (int t = 0; t < T; ++t) {
            state_update(S, dk, dv, lambda[h], k + IDX_TOK(b, t, h, 0, T, H, dk),
                         v + IDX_TOK(b, t, h, 0, T, H, dv));
            readout(S, dk, dv, scale, q + IDX_TOK(b, t, h, 0, T, H, dk),
                    o + IDX_TOK(b, t, h, 0, T, H, dv));
        }
        if (S_final) memcpy(S_final + IDX_ST(b, h, H, dk, dv), S, st * sizeof(double));
        free(S);
    }
    return failed ? -1 : 0;
}

/*
 * Reverse mode of the forward above for the scalar loss
 *     L = <do, o> + <dS_T, S_final>          (dS_T may be NULL = 0).
 * With G the adjoint of the running state, walking t = T-1 .. 0:
 *   G   += scale q_t do_t^T          (o_t reads S_t)
 *   dq_t = scale S_t do_t
 *   dk_t = G v_t ,  dv_t = G^T k_t   (S_t gained k_t v_t^T)
 *   dlambda_h += <G, S_{t-1}>        (S_t gained lambda_h S_{t-1}; S_{-1} = S0)
 *   G    = lambda_h G                (adjoint of S_{t-1})
 * and finally dS0 = G.  dlambda[h] is summed over the batch (lambda is shared),
 * in batch order, so the result is deterministic.  Any output pointer may be
 * NULL.  S_t is regenerated from checkpoints every `ck` tokens.
 */
int gla_oracle_bwd(int B, int T, int H, int dk, int dv,
                   const double* q, const double* k, const double* v,
                   const double* lambda, const double* S0, double scale,
                   const double* d_o, const double* dS_T,
                   double* dq, double* dk_out, double* dv_out,
                   double* dlambda, double* dS0, int nthreads) {
    if (B < 0 || T < 0 || H < 1 || dk < 1 || dv < 1) return -1;
    set_threads(nthreads);
    const size_t st = (size_t)dk * dv;
    int ck = 1;
    while ((long)ck * ck < (long)T) ++ck;          /* ~sqrt(T) tokens per block */
    const int nck = T > 0 ? (T + ck - 1) / ck : 0;
    double* dlam_unit = (double*)calloc((size_t)B * H + 1, sizeof(double));
    if (!dlam_unit) return -1;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long u = 0; u < (long)B * H; ++u) {
        const int b = (int)(u / H), h = (int)(u % H);
        const double lam = lambda[h];
        /* ckpt[i] = state before token i*ck;  blk[j] = state after token i*ck+j */
        double* ckpt = (double*)malloc(((size_t)nck + 1) * st * sizeof(double));
        double* blk = (double*)malloc(((size_t)ck + 1) * st * sizeof(double));
        double* G = (double*)malloc(st * sizeof(double));
        if (!ckpt || !blk || !G) { free(ckpt); free(blk); free(G); failed = 1; continue; }
        double* S = blk; /* scratch for the forward sweep */
        if (S0) memcpy(S, S0 + IDX_ST(b, h, H, dk, dv), st * sizeof(double));
        else memset(S, 0, st * sizeof(double));
        for (int t = 0; t < T; ++t) {
            if (t % ck == 0) memcpy(ckpt + (size_t)(t / ck) * st, S, st * sizeof(double));
            state_update(S, dk, dv, lam, k + IDX_TOK(b, t, h, 0, T, H, dk),
                         v + IDX_TOK(b, t, h, 0, T, H, dv));
        }
        if (dS_T) memcpy(G, dS_T + IDX_ST(b, h, H, dk, dv), st * sizeof(double));
        else memset(G, 0, st * sizeof(double));
        double dlam = 0.0;
        for (int i = nck - 1; i >= 0; --i) {
            const int t0 = i * ck;
            const int t1 = (t0 + ck < T) ? t0 + ck : T;
            /* blk[0] = S_{t0-1}; blk[j+1] = S_{t0+j} */
            memcpy(blk, ckpt + (size_t)i * st, st * sizeof(double));
            for (int t = t0; t < t1; ++t) {
                double* dst = blk + (size_t)(t - t0 + 1) * st;
                memcpy(dst, dst - st, st * sizeof(double));
                state_update(dst, dk, dv, lam, k + IDX_TOK(b, t, h, 0, T, H, dk),
                             v + IDX_TOK(b, t, h, 0, T, H, dv));
            }
            for (int t = t1 - 1; t >= t0; --t) {
                const double* St = blk + (size_t)(t - t0 + 1) * st;
                const double* Sp = St - st;
                const double* qt = q + IDX_TOK(b, t, h, 0, T, H, dk);
                const double* kt = k + IDX_TOK(b, t, h, 0, T, H, dk);
                const double* vt = v + IDX_TOK(b, t, h, 0, T, H, dv);
                const double* dot = d_o + IDX_TOK(b, t, h, 0, T, H, dv);
                for (int r = 0; r < dk; ++r)
                    for (int c = 0; c < dv; ++c)
                        G[(size_t)r * dv + c] += scale * qt[r] * dot[c];
                if (dq) {
                    double* dqt = dq + IDX_TOK(b, t, h, 0, T, H, dk);
                    for (int r = 0; r < dk; ++r) {
                        double acc = 0.0;
                        for (int c = 0; c < dv; ++c) acc += St[(size_t)r * dv + c] * dot[c];
                        dqt[r] = scale * acc;
                    }
                }
                if (dk_out) {
                    double* dkt = dk_out + IDX_TOK(b, t, h, 0, T, H, dk);
                    for (int r = 0; r < dk; ++r) {
                        double acc = 0.0;
                        for (int c = 0; c < dv; ++c) acc += G[(size_t)r * dv + c] * vt[c];
                        dkt[r] = acc;
                    }
                }
                if (dv_out) {
                    double* dvt = dv_out + IDX_TOK(b, t, h, 0, T, H, dv);
                    for (int c = 0; c < dv; ++c) dvt[c] = 0.0;
                    for (int r = 0; r < dk; ++r)
                        for (int c = 0; c < dv; ++c) dvt[c] += G[(size_t)r * dv + c] * kt[r];
                }
                double inner = 0.0;
                for (size_t e = 0; e < st; ++e) inner += G[e] * Sp[e];
                dlam += inner;
                for (size_t e = 0; e < st; ++e) G[e] *= lam;
            }
        }
        if (dS0) memcpy(dS0 + IDX_ST(b, h, H, dk, dv), G, st * sizeof(double));
        dlam_unit[u] = dlam;
        free(ckpt); free(blk); free(G);
    }
    if (!failed && dlambda) {
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int b = 0; b < B; ++b) acc += dlam_unit[(size_t)b * H + h];
            dlambda[h] = acc;
        }
    }
    free(dlam_unit);
    return failed ? -1 : 0;
}

/*
 * One decode step for N independent sequences: for every (n, h), in place,
 *   S <- lambda_h S + k v^T ;  o = scale S^T q     (the updated S is read).
 */
int gla_oracle_decode(int N, int H, int dk, int dv,
                      const double* q, const double* k, const double* v,
                      const double* lambda, double* S, double scale, double* o,
                      int nthreads) {
    if (N < 0 || H < 1 || dk < 1 || dv < 1) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (long u = 0; u < (long)N * H; ++u) {
        const int n = (int)(u / H), h = (int)(u % H);
        double* Sp = S + IDX_ST(n, h, H, dk, dv);
        state_update(Sp, dk, dv, lambda[h], k + IDX_TOK(n, 0, h, 0, 1, H, dk),
                     v + IDX_TOK(n, 0, h, 0, 1, H, dv));
        readout(Sp, dk, dv, scale, q + IDX_TOK(n, 0, h, 0, 1, H, dk),
                o + IDX_TOK(n, 0, h, 0, 1, H, dv));
    }
    return 0;
}

/*
 * Mixer epilogue, for every row m and head h (readings of the missing image):
 *   gate   s  = sigmoid( sum_i q_i a_{h,i} k_i )        raw q and k, no `scale`
 *   x_c       = o_c + s v_c                              o: the mixer readout
 *   x_hat_c   = x_c / sqrt( mean_c' x_c'^2 + eps ) * w_{tier(h), c}
 *   y_c       = silu(g_c) x_hat_c,   silu(z) = z sigmoid(z),   sigmoid(z) = 1 / (1 + e^-z)
 * a == NULL means a = 0 (s = 1/2).  Concatenating the heads is the layout itself.
 */
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

int gla_oracle_epilogue(int M, int H, int dk, int dv, const double* q, const double* k,
                        const double* v, const double* o, const double* g, const double* a,
                        const double* w, const int* tier, int n_tiers, double eps, double* y,
                        int nthreads) {
    if (M < 0 || H < 1 || dk < 1 || dv < 1 || n_tiers < 1 || eps < 0) return -1;
    for (int h = 0; h < H; ++h)
        if (tier[h] < 0 || tier[h] >= n_tiers) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (long u = 0; u < (long)M * H; ++u) {
        const int h = (int)(u % H);
        const double* qu = q + (size_t)u * dk;
        const double* ku = k + (size_t)u * dk;
        double z = 0.0;
        for (int i = 0; i < dk; ++i) z += qu[i] * (a ? a[(size_t)h * dk + i] : 0.0) * ku[i];
        const double s = sigmoid(z);
        double* x = (double*)malloc(sizeof(double) * (size_t)dv);
        double ss = 0.0;
        for (int c = 0; c < dv; ++c) {
            x[c] = o[(size_t)u * dv + c] + s * v[(size_t)u * dv + c];
            ss += x[c] * x[c];
        }
        const double inv = 1.0 / sqrt(ss / dv + eps);
        const double* wt = w + (size_t)tier[h] * dv;
        for (int c = 0; c < dv; ++c) {
            const double gc = g[(size_t)u * dv + c];
            y[(size_t)u * dv + c] = gc * sigmoid(gc) * x[c] * inv * wt[c];
        }
        free(x);
    }
    return 0;
}

/*
 * Depth-wise causal convolution of width K with SiLU, per channel d:
 *   u_t[d] = bias[d] + sum_{j=0..K-1} w[d][j] * x_{t-(K-1)+j}[d],   y_t[d] = silu(u_t[d])
 * so w[d][K-1] weighs the current token (the cross-correlation of a Conv1d with
 * K-1 zeros of left padding).  Readings of what the page leaves open:
 *   - bias == NULL means no bias;
 *   - inputs before the first token come from a window of the K most recent
 *     earlier inputs, win_in[b][s][d] = x_{s-K}[d] (oldest first); win_in ==
 *     NULL means zeros (a fresh sequence);
 *   - win_out (if not NULL) receives the window after the last token,
 *     x_{T-K..T-1}, the carry a decode step or the next prefill continues from.
 * win_out may alias win_in (every window value is read before any is written).
 */
static double x_at(const double* x, const double* win_in, int b, int t, int d, int T, int D, int K) {
    if (t >= 0) return x[((size_t)b * T + t) * D + d];
    return win_in ? win_in[((size_t)b * K + (K + t)) * D + d] : 0.0;
}

int gla_oracle_conv1d(int B, int T, int D, int K, const double* x, const double* w, const double* bias,
                      const double* win_in, double* y, double* win_out, int nthreads) {
    if (B < 0 || T < 0 || D < 1 || K < 1 || K > 64) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (long bd = 0; bd < (long)B * D; ++bd) {
        const int b = (int)(bd / D), d = (int)(bd % D);
        double carry[64];  /* the window of this channel, read before anything is written */
        for (int s2 = 0; s2 < K; ++s2) carry[s2] = x_at(x, win_in, b, T - K + s2, d, T, D, K);
        for (int t = 0; t < T; ++t) {
            double u = bias ? bias[d] : 0.0;
            for (int j = 0; j < K; ++j) u += w[(size_t)d * K + j] * x_at(x, win_in, b, t - (K - 1) + j, d, T, D, K);
            y[((size_t)b * T + t) * D + d] = u * sigmoid(u);
        }
        if (win_out)
            for (int s2 = 0; s2 < K; ++s2) win_out[((size_t)b * K + s2) * D + d] = carry[s2];
    }
    return 0;
}

/*
 * One decode token per sequence: the window [N][K][D] drops its oldest input
 * and appends x_n, then y_n = silu(bias + sum_j w[d][j] * window[j]).
 */
int gla_oracle_conv1d_decode(int N, int D, int K, const double* x, const double* w, const double* bias,
                             double* win, double* y, int nthreads) {
    if (N < 0 || D < 1 || K < 1) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (long nd = 0; nd < (long)N * D; ++nd) {
        const int n = (int)(nd / D), d = (int)(nd % D);
        double* wn = win + (size_t)n * K * D + d;
        for (int s2 = 0; s2 + 1 < K; ++s2) wn[(size_t)s2 * D] = wn[(size_t)(s2 + 1) * D];
        wn[(size_t)(K - 1) * D] = x[(size_t)n * D + d];
        double u = bias ? bias[d] : 0.0;
        for (int j = 0; j < K; ++j) u += w[(size_t)d * K + j] * wn[(size_t)j * D];
        y[(size_t)n * D + d] = u * sigmoid(u);
    }
    return 0;
}

// gla_grad_bf16.hip -- per-chunk gradient kernels of the chunked GLA backward
// for bf16 q/k/v/do (dk = 96, dv = 192, chunks of 32, 64, 128 or 256 tokens)
// on gfx950.
//
// Laplace 3B post, section "Challenge 1" (chunk form) differentiated as in the
// header of gla_bwd.hip: for chunk c with start state Sbar and end-of-chunk
// state gradient Gbar (both from the chain kernels),
//   dK = scale dP^T Q + diag(c) V Gbar^T,      dV = scale Abar^T dO + diag(c) K Gbar,
//   dQ = scale (dP K + diag(b) dO Sbar^T),
// with Abar = (Q K^T) (.) D and dP = (dO V^T) (.) D, and the lam-derivative terms
//   T2 = sum_j c'_j v_j . (Gbar^T k_j),  T3 = scale sum_i b'_i q_i . (Sbar do_i),
//   T4 = scale sum_{i>j} D'_ij (q_i . k_j)(do_i . v_j),
// and the term through the chunk decay, T1 = ceff lam^(ceff-1) <Gbar, Sbar>,
// from the two bf16 snapshots (each workgroup that stages one has the other's
// pieces at hand; dlam slot 0).
//
// One workgroup per (chunk, unit) forms dQ, dK and dV of its chunk from one set
// of operand tiles (grad_fused_bf16 below).  Decay factors lam^d and their
// derivatives d lam^(d-1) come from per-workgroup tables indexed by d + 1
// (index 0: above the diagonal, both 0).
#include "gla_common.hpp"
#include "gla_internal.hpp"
#include "gla_tile.hpp"


namespace gla {
namespace {

constexpr int kDK = 96, kDV = 192;
constexpr int kST = 64;                   // query rows per half of a chunk
constexpr int kFNW = 8, kFNT = 512;       // waves, threads of the gradient workgroup
constexpr int kFHalf = kST;
constexpr int kLDK = kDK + 8, kLDV = kDV + 8;

// pw[x + 1] = lam^x and dpw[x + 1] = x lam^(x-1) for x = 0..C; index 0 = 0 (x < 0).
template <int C>
__device__ __forceinline__ void fill_decay_tables(float* pw, float* dpw, float lam, int tid) {
    for (int i = tid; i < C + 2; i += kFNT) {
        pw[i] = i == 0 ? 0.f : pow_int(lam, i - 1);
        dpw[i] = i <= 1 ? 0.f : (float)(i - 1) * pow_int(lam, i - 2);
    }
}

__device__ __forceinline__ int decay_index(int d) { return (d < -1 ? -1 : d) + 1; }

// acc + sum of the 8 elementwise products of two 16-byte bf16 pieces, in fp32
// (bf16 -> fp32 is exact: the element's bits in the upper half of a word).
__device__ __forceinline__ float dot_piece(uint4 x, uint4 y, float acc) {
    const unsigned xv[4] = {x.x, x.y, x.z, x.w}, yv[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc = fmaf(__builtin_bit_cast(float, xv[j] << 16), __builtin_bit_cast(float, yv[j] << 16), acc);
        acc = fmaf(__builtin_bit_cast(float, xv[j] & 0xffff0000u), __builtin_bit_cast(float, yv[j] & 0xffff0000u), acc);
    }
    return acc;
}

// This thread's part of <G, S> for two dk x dv snapshots: G's pieces staged in
// registers (BufStage<kDK, kDV, NT>), S's the same pieces of a row-major LDS
// tile of row stride LD.
template <int NT, int LD, typename Stage>
__device__ __forceinline__ float snap_dot_lds(const Stage& gs, const bf16* S, int tid) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < Stage::PER; ++i) {
        const int p = tid + NT * i;
        if (Stage::NP % NT != 0 && p >= Stage::NP) continue;
        acc = dot_piece(gs.r[i], *reinterpret_cast<const uint4*>(S + (p / Stage::KC) * LD + (p % Stage::KC) * 8), acc);
    }
    return acc;
}

// All three gradients of one chunk of C = 128 or 64 tokens (one workgroup of
// 8 waves per (chunk, unit)): every operand tile and both snapshots are read
// from HBM once.  Wave w owns key
// block w (keys 16w .. 16w+15, if the chunk has them) for dK, dV and one
// 16-query block of dQ.  LDS holds K and V whole, one snapshot (Sbar, then
// Gbar) and the queries and output gradients of one 64-query half at a time:
// ~157 KB at C = 128 (~116 KB at 64), one workgroup per CU.
//   A (queries 0..63):   waves 0..3 add the intra-chunk terms of their key
//                        blocks; waves 4..7 form dQ of query blocks 0..3.
//   B (queries 64..127, C = 128 only): waves 4..7 form dQ of query blocks
//                        4..7, then every wave adds its key block's terms.
//   C (Gbar):            the waves with key blocks add the inter-chunk terms
//                        of dK, dV.
// No wave holds dQ and dK/dV accumulators at the same time (waves 4..7 start
// their key blocks, which only see queries 64..127, after their dQ blocks).
template <int C>
__global__ __launch_bounds__(kFNT, 1) void grad_fused_bf16(GradArgs a) {
    static_assert(C == 128 || C == 64 || C == 32, "one or two query halves of at most 64 rows");
    constexpr int HALF = C < kFHalf ? C : kFHalf;  // query rows per half
    constexpr int NSUB = C / HALF;                 // halves
    constexpr int NKB = C / 16;                    // key blocks (waves that own one)
    constexpr int NQB = HALF / 16;                 // query blocks per half
    __shared__ __align__(16) bf16 Ks[C * kLDK];
    __shared__ __align__(16) bf16 Vs[C * kLDV];
    __shared__ __align__(16) bf16 Xs[kDK * kLDV];            // Sbar, then Gbar
    __shared__ __align__(16) bf16 Qs[HALF * kLDK];           // one half's queries
    __shared__ __align__(16) bf16 Ds[HALF * kLDV];           // and output gradients
    __shared__ float pw[C + 2], dpw[C + 2];
    __shared__ float red[3][kFNW];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, n = lane % 16, g = lane / 16;
    const int cid = blockIdx.x, bh = blockIdx.y;
    const int H = a.H, T = a.T;
    const int hd = bh % H, b = bh / H;
    const int t0 = cid * C;
    const int ceff = min(C, T - t0);
    float* part = a.part + ((size_t)bh * a.nc + cid) * kNPart + kChainSlots;
    fill_decay_tables<C>(pw, dpw, a.lambda[hd], tid);

    const int tokQ = a.sq.t, tokK = a.sk.t, tokV = a.sv.t, tokD = a.sdo.t;
    const size_t snap = ((size_t)bh * a.nc + cid) * kDK * kDV;
    const bf16* qb = static_cast<const bf16*>(a.q) + b * a.sq.b + (size_t)t0 * tokQ + hd * kDK;
    const bf16* kb = static_cast<const bf16*>(a.k) + b * a.sk.b + (size_t)t0 * tokK + hd * kDK;
    const bf16* vb = static_cast<const bf16*>(a.v) + b * a.sv.b + (size_t)t0 * tokV + hd * kDV;
    const bf16* db_ = static_cast<const bf16*>(a.d_o) + b * a.sdo.b + (size_t)t0 * tokD + hd * kDV;
    BufStage<HALF, kDK, kFNT> tq;
    BufStage<HALF, kDV, kFNT> td;
    {
        BufStage<C, kDK, kFNT> tk;
        BufStage<C, kDV, kFNT> tv;
        BufStage<kDK, kDV, kFNT> ts;
        tk.load(kb, tokK, ceff, tid);
        tv.load(vb, tokV, ceff, tid);
        ts.load(static_cast<const bf16*>(a.sbar) + snap, kDV, kDK, tid);
        tq.load(qb, tokQ, ceff, tid);
        td.load(db_, tokD, ceff, tid);
        tk.template store<kLDK>(Ks, tid);
        tv.template store<kLDV>(Vs, tid);
        ts.template store<kLDV>(Xs, tid);
        tq.template store<kLDK>(Qs, tid);
        td.template store<kLDV>(Ds, tid);
    }
    // Gbar: at C = 64 (one query half, one workgroup per CU) requested now, to
    // arrive during the intra-chunk terms (the training step -6.5 us); at 128 at
    // the start of the second half; at 32, where two workgroups share a CU and
    // registers are short, after the intra-chunk terms (+1.7 us if requested now).
    BufStage<kDK, kDV, kFNT> tg;
    constexpr bool kGbarEarly = C == 64;
    if constexpr (kGbarEarly) tg.load(static_cast<const bf16*>(a.gbar) + snap, kDV, kDK, tid);
    // the second half's queries and output gradients, in registers meanwhile
    if (HALF < ceff) {
        tq.load(qb + (size_t)HALF * tokQ, tokQ, ceff - HALF, tid);
        td.load(db_ + (size_t)HALF * tokD, tokD, ceff - HALF, tid);
    }
    __syncthreads();

    const int jb = wave;
    const float sc = a.scale;
    f32x4 dKT[kDK / 16], dVT[kDV / 16];
#pragma unroll
    for (int d = 0; d < kDK / 16; ++d) dKT[d] = zero4();
#pragma unroll
    for (int c = 0; c < kDV / 16; ++c) dVT[c] = zero4();
    float t4 = 0.f, t3 = 0.f;

    // Intra-chunk terms of key block jb from the query pairs of the half at
    // qt0 at or below the diagonal: Abar = (Q K^T) (.) D and dP = (dO V^T) (.) D
    // blocks, then dV^T += dO-side products, dK^T += Q-side products.
    auto key_terms = [&](int qt0) {
        const int jl = jb * 16 + n;  // chunk-local key index of this lane's column
        // this key block's row operands, read once for every query pair
        bf16x8 kr[kDK / 32], vr[kDV / 32];
#pragma unroll
        for (int p = 0; p < kDK / 32; ++p) kr[p] = op_row8(Ks, kLDK, jb * 16 + n, 32 * p + 8 * g);
#pragma unroll
        for (int p = 0; p < kDV / 32; ++p) vr[p] = op_row8(Vs, kLDV, jb * 16 + n, 32 * p + 8 * g);
#pragma unroll
        for (int pr = 0; pr < HALF / 32; ++pr) {
            if (qt0 + 32 * pr + 31 < jb * 16) continue;  // pair entirely above the diagonal (uniform)
            f32x4 Ab[2], Pb[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ib = pr * 2 + u;      // block within the half
                const int il0 = qt0 + ib * 16;  // chunk-local first query of the block
                Ab[u] = zero4();
                Pb[u] = zero4();
                if (il0 + 15 < jb * 16) continue;  // block entirely above the diagonal (uniform)
#pragma unroll
                for (int p = 0; p < kDK / 32; ++p)
                    Ab[u] = mfma(op_row8(Qs, kLDK, ib * 16 + n, 32 * p + 8 * g), kr[p], Ab[u]);
#pragma unroll
                for (int p = 0; p < kDV / 32; ++p)
                    Pb[u] = mfma(op_row8(Ds, kLDV, ib * 16 + n, 32 * p + 8 * g), vr[p], Pb[u]);
                // Ab[u][r] = q_i . k_j, Pb[u][r] = do_i . v_j for i = il0 + 4g + r, j = jl
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int di = decay_index(il0 + 4 * g + r - jl);
                    const float f = sc * pw[di];
                    t4 = fmaf(dpw[di] * Ab[u][r], Pb[u][r], t4);
                    Ab[u][r] *= f;
                    Pb[u][r] *= f;
                }
            }
            const bf16x8 ab = pack_acc(Ab[0], Ab[1]);
            const bf16x8 pb = pack_acc(Pb[0], Pb[1]);
#pragma unroll
            for (int c = 0; c < kDV / 16; ++c) dVT[c] = mfma(op_col_pair(Ds, kLDV, 32 * pr, c * 16, n, g), ab, dVT[c]);
#pragma unroll
            for (int d = 0; d < kDK / 16; ++d) dKT[d] = mfma(op_col_pair(Qs, kLDK, 32 * pr, d * 16, n, g), pb, dKT[d]);
        }
    };
    // dQ of query block ib of the half at qt0, stored:
    //   dQ = scale (b_i Sbar do_i + sum_{j <= i} dP_ij k_j);
    // scale b'_i q_i . (Sbar do_i) feeds dlam.
    auto query_block = [&](int qt0, int ib) {
        const int il = qt0 + ib * 16 + n;  // chunk-local query index of this lane's column
        const float bi = pw[il + 2];       // lam^(il+1)
        const float dbi = dpw[il + 2];     // (il+1) lam^il
        // this query block's output-gradient row operands, read once
        bf16x8 dr[kDV / 32];
#pragma unroll
        for (int p = 0; p < kDV / 32; ++p) dr[p] = op_row8(Ds, kLDV, ib * 16 + n, 32 * p + 8 * g);
        f32x4 dQT[kDK / 16];
#pragma unroll
        for (int d = 0; d < kDK / 16; ++d) {
            dQT[d] = zero4();
#pragma unroll
            for (int p = 0; p < kDV / 32; ++p) dQT[d] = mfma(op_row8(Xs, kLDV, d * 16 + n, 32 * p + 8 * g), dr[p], dQT[d]);
            const f32x4 qi = load4<bf16>(Qs + (ib * 16 + n) * kLDK + d * 16 + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                t3 = fmaf(dbi * qi[r], dQT[d][r], t3);
                dQT[d][r] *= sc * bi;
            }
        }
#pragma unroll
        for (int pr = 0; pr < C / 32; ++pr) {
            if (32 * pr > qt0 + ib * 16 + 15) continue;  // pair entirely above the diagonal (uniform)
            f32x4 Pt[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int kb2 = pr * 2 + u;
                const int jl0 = kb2 * 16;  // chunk-local first key of the block
                Pt[u] = zero4();
                if (jl0 > qt0 + ib * 16 + 15) continue;  // block entirely above the diagonal (uniform)
#pragma unroll
                for (int p = 0; p < kDV / 32; ++p) Pt[u] = mfma(op_row8(Vs, kLDV, kb2 * 16 + n, 32 * p + 8 * g), dr[p], Pt[u]);
                // Pt[u][r] = v_j . do_i for j = jl0 + 4g + r, i = il
#pragma unroll
                for (int r = 0; r < 4; ++r) Pt[u][r] *= sc * pw[decay_index(il - (jl0 + 4 * g + r))];
            }
            const bf16x8 pt = pack_acc(Pt[0], Pt[1]);
#pragma unroll
            for (int d = 0; d < kDK / 16; ++d) dQT[d] = mfma(op_col_pair(Ks, kLDK, 32 * pr, d * 16, n, g), pt, dQT[d]);
        }
        if (il < ceff) {
            bf16* dqr = static_cast<bf16*>(a.dq) + b * a.sdq.b + (size_t)(t0 + il) * a.sdq.t + hd * kDK;
#pragma unroll
            for (int d = 0; d < kDK / 16; ++d) store4<bf16>(dqr + d * 16 + 4 * g, dQT[d]);
        }
    };

    // A: queries 0 .. HALF-1 (waves past the chunk's key or query blocks idle).
    // With one query half (C <= 64) this is the whole intra-chunk work, and the
    // dQ waves 4..7 get their SIMD's issue priority (the training step -2.3 us at
    // C = 64, -1.2 at 32 against the same kernel without it; no gain at 128, not
    // used there).
    if constexpr (C < 128)
        if (wave >= 4) __builtin_amdgcn_s_setprio(1);
    if (wave < 4) {
        if (wave < NKB) key_terms(0);
    } else if (wave - 4 < NQB) {
        query_block(0, wave - 4);
    }
    if constexpr (C < 128) __builtin_amdgcn_s_setprio(0);
    // B: queries 64..127 (Gbar requested for C meanwhile)
    if (C > HALF && HALF < ceff) {
        __syncthreads();  // half 0 reads are done
        tq.template store<kLDK>(Qs, tid);
        td.template store<kLDV>(Ds, tid);
        __syncthreads();
        tg.load(static_cast<const bf16*>(a.gbar) + snap, kDV, kDK, tid);
        // Waves 4..7 carry about twice the work of waves 0..3 here (a dQ block and a
        // key block each); with the issue priority of their SIMD they no longer
        // trail the lighter partner wave into the barrier (the training step at
        // C = 128: -2.2 us against the same kernel without it, timed alternately).
        if (wave >= 4) __builtin_amdgcn_s_setprio(1);
        if (wave >= 4) query_block(HALF, wave - 4);
        key_terms(HALF);
        __builtin_amdgcn_s_setprio(0);
    } else if constexpr (!kGbarEarly) {
        tg.load(static_cast<const bf16*>(a.gbar) + snap, kDV, kDK, tid);
    }
    // <Gbar, Sbar> (dlam through lam^ceff): this thread's Gbar pieces against
    // the same pieces of Sbar, still in Xs
    float gsd = snap_dot_lds<kFNT, kLDV>(tg, Xs, tid);
    // C: inter-chunk terms.  dK^T[d][j] += c_j sum_c Gbar[d][c] v_j[c];
    // dV^T[c][j] += c_j X[c][j], X = sum_d Gbar[d][c] k_j[d]; c'_j v_j . X_j feeds dlam.
    __syncthreads();  // Sbar reads are done
    tg.template store<kLDV>(Xs, tid);
    __syncthreads();
    int tid_v = threadIdx.x;
    asm volatile("" : "+v"(tid_v));
    const int lane2 = tid_v % 64, n2 = lane2 % 16, g2 = lane2 / 16;
    const int jl = jb * 16 + n2;
    const float cj = pw[decay_index(ceff - 1 - jl)];
    const float dcj = dpw[decay_index(ceff - 1 - jl)];
    float t2 = 0.f;
    if (jb < NKB) {
#pragma unroll
    for (int d = 0; d < kDK / 16; ++d) {
        f32x4 x = zero4();
#pragma unroll
        for (int p = 0; p < kDV / 32; ++p)
            x = mfma(op_row8(Xs, kLDV, d * 16 + n2, 32 * p + 8 * g2), op_row8(Vs, kLDV, jb * 16 + n2, 32 * p + 8 * g2), x);
#pragma unroll
        for (int r = 0; r < 4; ++r) dKT[d][r] = fmaf(cj, x[r], dKT[d][r]);
    }
#pragma unroll
    for (int c = 0; c < kDV / 16; ++c) {
        f32x4 x = zero4();
#pragma unroll
        for (int p = 0; p < kDK / 32; ++p)
            x = mfma(op_col8(Xs, kLDV, 32 * p, c * 16, n2, g2), op_row8(Ks, kLDK, jb * 16 + n2, 32 * p + 8 * g2), x);
        const f32x4 vj = load4<bf16>(Vs + (jb * 16 + n2) * kLDV + c * 16 + 4 * g2);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            t2 = fmaf(dcj * vj[r], x[r], t2);
            dVT[c][r] = fmaf(cj, x[r], dVT[c][r]);
        }
    }
    }

    if (jl < ceff) {
        bf16* dkr = static_cast<bf16*>(a.dk) + b * a.sdk.b + (size_t)(t0 + jl) * a.sdk.t + hd * kDK;
        bf16* dvr = static_cast<bf16*>(a.dv) + b * a.sdv.b + (size_t)(t0 + jl) * a.sdv.t + hd * kDV;
#pragma unroll
        for (int d = 0; d < kDK / 16; ++d) store4<bf16>(dkr + d * 16 + 4 * g2, dKT[d]);
#pragma unroll
        for (int c = 0; c < kDV / 16; ++c) store4<bf16>(dvr + c * 16 + 4 * g2, dVT[c]);
    }
    // dlam partials: the key-side terms (t2 + scale t4) and the query-side term
    // (scale t3), each summed over the waves in a fixed order
    t2 = wave_sum(t2 + sc * t4);
    t3 = wave_sum(sc * t3);
    gsd = wave_sum(gsd);
    if (lane2 == 0) {
        red[0][wave] = t2;
        red[1][wave] = t3;
        red[2][wave] = gsd;
    }
    __syncthreads();
    // slots kChainSlots + [0, NSUB): key side (all in the first), + [NSUB, 2 NSUB):
    // query side (all in the first); the reduction sums every slot
    if (tid_v < 2 * NSUB) {
        float s = 0.f;
        if (tid_v % NSUB == 0)
#pragma unroll
            for (int w = 0; w < kFNW; ++w) s += red[tid_v / NSUB][w];
        part[tid_v] = s;
    } else if (tid_v == 2 * NSUB) {
        // the chunk's term through lam^ceff, ceff lam^(ceff-1) <Gbar, Sbar>, in slot 0
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kFNW; ++w) s += red[2][w];
        a.part[((size_t)bh * a.nc + cid) * kNPart] = dpw[ceff + 1] * s;
    }
}


// ------------------------------------------------------------ 256-token chunks
//
// The gradients of a 256-token chunk from four workgroups of 8 waves: K and V
// of the whole chunk (~155 KB with padding) do not fit LDS beside anything
// else, so the work is split by side and half, each workgroup holding at most
// ~78 KB:
//   role 0, 1 (key side):   wave w owns key block 8 role + w: dK and dV of
//                           those keys.  Its key and value rows stay in
//                           registers (row operands); the queries at or after
//                           the half's first key and their output gradients
//                           pass through LDS in 64-row quarters, then Gbar takes
//                           their place for the inter terms c (.) V Gbar^T and
//                           c (.) K Gbar.
//   role 2, 3 (query side): wave w owns query block 8 (role - 2) + w: dQ.  The
//                           key halves at or before its queries pass through
//                           LDS (K and V of 128 keys at a time) for the intra
//                           term dP K, then Sbar takes their place for b Sbar do.
// The four workgroups of a (chunk, unit) are dispatched back to back on one
// XCD (workgroup i runs on XCD i mod 8), so the tiles that several of them
// read come from that XCD's L2.  dlam partials: key side t2 + scale t4 (slots
// kChainSlots + role), query side scale t3 (slots kChainSlots + role), the
// chunk-decay term ceff lam^(ceff-1) <Gbar, Sbar> from role 0 (slot 0), which
// also clears the remaining gradient slots.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const bf16* base, int tok_stride, int valid) {
    const unsigned rows = valid <= 0 ? 0u : (unsigned)valid;
    const int range = __builtin_amdgcn_readfirstlane((int)(rows * (unsigned)tok_stride * 2u));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), 0, range, kBufWord3);
}
// 8 / 4 bf16 at element offset `off` of a row resource (zeros outside its rows)
__device__ __forceinline__ bf16x8 ld_row8(__amdgpu_buffer_rsrc_t rs, unsigned off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off * 2u), 0, 0));
}
__device__ __forceinline__ f32x4 ld_row4(__amdgpu_buffer_rsrc_t rs, unsigned off) {
    const bf16x4 x = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(off * 2u), 0, 0));
    return f32x4{to_f32(x[0]), to_f32(x[1]), to_f32(x[2]), to_f32(x[3])};
}

__global__ __launch_bounds__(kFNT, 1) void grad_c256_bf16(GradArgs a) {
    constexpr int C = 256, R = 128, QR = 64;   // chunk, half, quarter (rows)
    // key side: Q quarter | dO quarter, then Gbar; query side: K half | V half, then Sbar
    __shared__ __align__(16) bf16 buf[R * kLDK + R * kLDV];
    __shared__ float pw[C + 2], dpw[C + 2];
    __shared__ float red[2][kFNW];

    // (chunk, unit) and role from the dispatch order: the four roles of one
    // (chunk, unit) are workgroups 8 (4 s + role) + x, all on XCD x
    const int lin = blockIdx.x;
    const int slot = lin / 8;
    const int role = slot % 4;
    const int cu = (slot / 4) * 8 + lin % 8;
    if (cu >= a.nc * a.units) return;   // (whole workgroup, before any barrier)
    const int cid = cu % a.nc, bh = cu / a.nc;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, n = lane % 16, g = lane / 16;
    const int H = a.H, T = a.T;
    const int hd = bh % H, b = bh / H;
    const int t0 = cid * C;
    const int ceff = min(C, T - t0);
    const float sc = a.scale;
    fill_decay_tables<C>(pw, dpw, a.lambda[hd], tid);

    const int tokQ = a.sq.t, tokK = a.sk.t, tokV = a.sv.t, tokD = a.sdo.t;
    const size_t snap = ((size_t)bh * a.nc + cid) * kDK * kDV;
    const bf16* qb = static_cast<const bf16*>(a.q) + b * a.sq.b + (size_t)t0 * tokQ + hd * kDK;
    const bf16* kb = static_cast<const bf16*>(a.k) + b * a.sk.b + (size_t)t0 * tokK + hd * kDK;
    const bf16* vb = static_cast<const bf16*>(a.v) + b * a.sv.b + (size_t)t0 * tokV + hd * kDV;
    const bf16* db_ = static_cast<const bf16*>(a.d_o) + b * a.sdo.b + (size_t)t0 * tokD + hd * kDV;
    float* part = a.part + ((size_t)bh * a.nc + cid) * kNPart;

    if (role < 2) {
        // ------------------------------------------------------ key side
        const int jb = 8 * role + wave;  // chunk-local key block
        const int jl = jb * 16 + n;      // chunk-local key of this lane's accumulator column
        bf16* Qs = buf;
        bf16* Ds = buf + QR * kLDK;
        bf16* Xs = buf;  // Gbar, once the quarters are done
        const int q_first = 2 * role;              // first quarter holding queries at or after the keys
        const int q_end = (ceff + QR - 1) / QR;    // quarters holding tokens
        BufStage<QR, kDK, kFNT> tq;
        BufStage<QR, kDV, kFNT> td;
        if (q_first < q_end) {
            tq.load(qb + (size_t)(q_first * QR) * tokQ, tokQ, ceff - q_first * QR, tid);
            td.load(db_ + (size_t)(q_first * QR) * tokD, tokD, ceff - q_first * QR, tid);
        }
        // this wave's key and value rows (row operands), zeros past the chunk end
        const auto rk = rows_rsrc(kb, tokK, ceff);
        const auto rv = rows_rsrc(vb, tokV, ceff);
        bf16x8 kr[kDK / 32], vr[kDV / 32];
#pragma unroll
        for (int p = 0; p < kDK / 32; ++p) kr[p] = ld_row8(rk, (unsigned)(jl * tokK + 32 * p + 8 * g));
#pragma unroll
        for (int p = 0; p < kDV / 32; ++p) vr[p] = ld_row8(rv, (unsigned)(jl * tokV + 32 * p + 8 * g));

        f32x4 dKT[kDK / 16], dVT[kDV / 16];
#pragma unroll
        for (int d = 0; d < kDK / 16; ++d) dKT[d] = zero4();
#pragma unroll
        for (int c = 0; c < kDV / 16; ++c) dVT[c] = zero4();
        float t4 = 0.f;
        // Intra-chunk terms of key block jb from the query pairs of the quarter
        // at qt0 at or below the diagonal (as in the fused kernel's key terms)
        auto key_terms = [&](int qt0) {
#pragma unroll
            for (int pr = 0; pr < QR / 32; ++pr) {
                if (qt0 + 32 * pr + 31 < jb * 16) continue;  // pair above the diagonal (uniform)
                f32x4 Ab[2], Pb[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int ibl = pr * 2 + u;       // block within the quarter
                    const int il0 = qt0 + ibl * 16;   // chunk-local first query of the block
                    Ab[u] = zero4();
                    Pb[u] = zero4();
                    if (il0 + 15 < jb * 16) continue;  // block above the diagonal (uniform)
#pragma unroll
                    for (int p = 0; p < kDK / 32; ++p)
                        Ab[u] = mfma(op_row8(Qs, kLDK, ibl * 16 + n, 32 * p + 8 * g), kr[p], Ab[u]);
#pragma unroll
                    for (int p = 0; p < kDV / 32; ++p)
                        Pb[u] = mfma(op_row8(Ds, kLDV, ibl * 16 + n, 32 * p + 8 * g), vr[p], Pb[u]);
                    // Ab[u][r] = q_i . k_j, Pb[u][r] = do_i . v_j for i = il0 + 4g + r, j = jl
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int di = decay_index(il0 + 4 * g + r - jl);
                        const float f = sc * pw[di];
                        t4 = fmaf(dpw[di] * Ab[u][r], Pb[u][r], t4);
                        Ab[u][r] *= f;
                        Pb[u][r] *= f;
                    }
                }
                const bf16x8 ab = pack_acc(Ab[0], Ab[1]);
                const bf16x8 pb = pack_acc(Pb[0], Pb[1]);
#pragma unroll
                for (int c = 0; c < kDV / 16; ++c) dVT[c] = mfma(op_col_pair(Ds, kLDV, 32 * pr, c * 16, n, g), ab, dVT[c]);
#pragma unroll
                for (int d = 0; d < kDK / 16; ++d) dKT[d] = mfma(op_col_pair(Qs, kLDK, 32 * pr, d * 16, n, g), pb, dKT[d]);
            }
        };
        for (int q = q_first; q < q_end; ++q) {
            __syncthreads();  // the previous quarter's reads are done
            tq.template store<kLDK>(Qs, tid);
            td.template store<kLDV>(Ds, tid);
            __syncthreads();
            if (q + 1 < q_end) {  // the next quarter, in registers meanwhile
                tq.load(qb + (size_t)((q + 1) * QR) * tokQ, tokQ, ceff - (q + 1) * QR, tid);
                td.load(db_ + (size_t)((q + 1) * QR) * tokD, tokD, ceff - (q + 1) * QR, tid);
            }
            if (jb * 16 <= q * QR + QR - 1) key_terms(q * QR);  // some query at or after the keys (uniform)
        }
        BufStage<kDK, kDV, kFNT> tg;
        tg.load(static_cast<const bf16*>(a.gbar) + snap, kDV, kDK, tid);
        __syncthreads();  // Q, dO reads are done
        tg.template store<kLDV>(Xs, tid);
        // (role 0) Sbar pieces for <Gbar, Sbar>, dotted with Gbar once it is in LDS
        BufStage<kDK, kDV, kFNT> ts;
        if (role == 0) ts.load(static_cast<const bf16*>(a.sbar) + snap, kDV, kDK, tid);
        // this lane's value row in the accumulator layout (4 features per block) for t2
        f32x4 vj[kDV / 16];
#pragma unroll
        for (int c = 0; c < kDV / 16; ++c) vj[c] = ld_row4(rv, (unsigned)(jl * tokV + c * 16 + 4 * g));
        __syncthreads();
        // inter-chunk terms: dK^T[d][j] += c_j sum_c Gbar[d][c] v_j[c];
        // dV^T[c][j] += c_j X[c][j], X = sum_d Gbar[d][c] k_j[d]; c'_j v_j . X_j feeds dlam
        const float cj = pw[decay_index(ceff - 1 - jl)];
        const float dcj = dpw[decay_index(ceff - 1 - jl)];
        float t2 = 0.f;
#pragma unroll
        for (int d = 0; d < kDK / 16; ++d) {
            f32x4 x = zero4();
#pragma unroll
            for (int p = 0; p < kDV / 32; ++p) x = mfma(op_row8(Xs, kLDV, d * 16 + n, 32 * p + 8 * g), vr[p], x);
#pragma unroll
            for (int r = 0; r < 4; ++r) dKT[d][r] = fmaf(cj, x[r], dKT[d][r]);
        }
#pragma unroll
        for (int c = 0; c < kDV / 16; ++c) {
            f32x4 x = zero4();
#pragma unroll
            for (int p = 0; p < kDK / 32; ++p) x = mfma(op_col8(Xs, kLDV, 32 * p, c * 16, n, g), kr[p], x);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                t2 = fmaf(dcj * vj[c][r], x[r], t2);
                dVT[c][r] = fmaf(cj, x[r], dVT[c][r]);
            }
        }
        float gsd = 0.f;
        if (role == 0) gsd = snap_dot_lds<kFNT, kLDV>(ts, Xs, tid);
        if (jl < ceff) {
            bf16* dkr = static_cast<bf16*>(a.dk) + b * a.sdk.b + (size_t)(t0 + jl) * a.sdk.t + hd * kDK;
            bf16* dvr = static_cast<bf16*>(a.dv) + b * a.sdv.b + (size_t)(t0 + jl) * a.sdv.t + hd * kDV;
#pragma unroll
            for (int d = 0; d < kDK / 16; ++d) store4<bf16>(dkr + d * 16 + 4 * g, dKT[d]);
#pragma unroll
            for (int c = 0; c < kDV / 16; ++c) store4<bf16>(dvr + c * 16 + 4 * g, dVT[c]);
        }
        t2 = wave_sum(t2 + sc * t4);
        gsd = wave_sum(gsd);
        if (lane == 0) {
            red[0][wave] = t2;
            red[1][wave] = gsd;
        }
        __syncthreads();
        if (tid == 0) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < kFNW; ++w) s += red[0][w];
            part[kChainSlots + role] = s;
        } else if (tid == 1 && role == 0) {
            // the chunk's term through lam^ceff, ceff lam^(ceff-1) <Gbar, Sbar>
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < kFNW; ++w) s += red[1][w];
            part[0] = dpw[ceff + 1] * s;
        } else if (role == 0 && tid >= 2 && tid < 2 + (kNPart - kChainSlots - 4)) {
            part[kChainSlots + 4 + (tid - 2)] = 0.f;   // slots no role writes
        }
    } else {
        // ---------------------------------------------------- query side
        //   dQ = scale (sum_{j <= i} dP_ij k_j + b_i Sbar do_i);
        //   scale b'_i q_i . (Sbar do_i) feeds dlam
        const int half = role - 2;
        const int ib = 8 * half + wave;  // chunk-local query block
        const int il = ib * 16 + n;      // chunk-local query of this lane's accumulator column
        bf16* Ks = buf;
        bf16* Vs = buf + R * kLDK;
        bf16* Xs = buf;  // Sbar, once the intra terms are done
        BufStage<R, kDK, kFNT> tk;
        BufStage<R, kDV, kFNT> tv;
        tk.load(kb, tokK, ceff, tid);
        tv.load(vb, tokV, ceff, tid);
        // this wave's output-gradient rows (row operands) and query pieces,
        // zeros past the chunk end
        const auto rd = rows_rsrc(db_, tokD, ceff);
        const auto rq = rows_rsrc(qb, tokQ, ceff);
        bf16x8 dr[kDV / 32];
#pragma unroll
        for (int p = 0; p < kDV / 32; ++p) dr[p] = ld_row8(rd, (unsigned)(il * tokD + 32 * p + 8 * g));
        f32x4 qi[kDK / 16];
#pragma unroll
        for (int d = 0; d < kDK / 16; ++d) qi[d] = ld_row4(rq, (unsigned)(il * tokQ + d * 16 + 4 * g));

        f32x4 dQT[kDK / 16];
#pragma unroll
        for (int d = 0; d < kDK / 16; ++d) dQT[d] = zero4();
        for (int kh = 0; kh <= half; ++kh) {
            if (kh > 0) {
                __syncthreads();  // key half 0's reads are done
                tk.load(kb + (size_t)R * tokK, tokK, ceff - R, tid);
                tv.load(vb + (size_t)R * tokV, tokV, ceff - R, tid);
            }
            tk.template store<kLDK>(Ks, tid);
            tv.template store<kLDV>(Vs, tid);
            __syncthreads();
#pragma unroll
            for (int pr = 0; pr < R / 32; ++pr) {
                if (R * kh + 32 * pr > ib * 16 + 15) continue;  // pair entirely above the diagonal (uniform)
                f32x4 Pt[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int kb2 = pr * 2 + u;         // block within the key half
                    const int jl0 = R * kh + kb2 * 16;  // chunk-local first key of the block
                    Pt[u] = zero4();
                    if (jl0 > ib * 16 + 15) continue;   // block entirely above the diagonal (uniform)
#pragma unroll
                    for (int p = 0; p < kDV / 32; ++p)
                        Pt[u] = mfma(op_row8(Vs, kLDV, kb2 * 16 + n, 32 * p + 8 * g), dr[p], Pt[u]);
                    // Pt[u][r] = v_j . do_i for j = jl0 + 4g + r, i = il
#pragma unroll
                    for (int r = 0; r < 4; ++r) Pt[u][r] *= sc * pw[decay_index(il - (jl0 + 4 * g + r))];
                }
                const bf16x8 pt = pack_acc(Pt[0], Pt[1]);
#pragma unroll
                for (int d = 0; d < kDK / 16; ++d) dQT[d] = mfma(op_col_pair(Ks, kLDK, 32 * pr, d * 16, n, g), pt, dQT[d]);
            }
        }
        BufStage<kDK, kDV, kFNT> ts;
        ts.load(static_cast<const bf16*>(a.sbar) + snap, kDV, kDK, tid);
        __syncthreads();  // K, V reads are done
        ts.template store<kLDV>(Xs, tid);
        __syncthreads();
        const float bi = pw[il + 2];    // lam^(il+1)
        const float dbi = dpw[il + 2];  // (il+1) lam^il
        float t3 = 0.f;
#pragma unroll
        for (int d = 0; d < kDK / 16; ++d) {
            f32x4 x = zero4();
#pragma unroll
            for (int p = 0; p < kDV / 32; ++p) x = mfma(op_row8(Xs, kLDV, d * 16 + n, 32 * p + 8 * g), dr[p], x);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                t3 = fmaf(dbi * qi[d][r], x[r], t3);
                dQT[d][r] = fmaf(sc * bi, x[r], dQT[d][r]);
            }
        }
        if (il < ceff) {
            bf16* dqr = static_cast<bf16*>(a.dq) + b * a.sdq.b + (size_t)(t0 + il) * a.sdq.t + hd * kDK;
#pragma unroll
            for (int d = 0; d < kDK / 16; ++d) store4<bf16>(dqr + d * 16 + 4 * g, dQT[d]);
        }
        t3 = wave_sum(sc * t3);
        if (lane == 0) red[0][wave] = t3;
        __syncthreads();
        if (tid == 0) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < kFNW; ++w) s += red[0][w];
            part[kChainSlots + role] = s;
        }
    }
}

}  // namespace

hipError_t launch_grad_bf16(int chunk, const GradArgs& ga, unsigned units, hipStream_t stream) {
    if (chunk == 128)
        hipLaunchKernelGGL(grad_fused_bf16<128>, dim3((unsigned)ga.nc, units), dim3(kFNT), 0, stream, ga);
    else if (chunk == 64)
        hipLaunchKernelGGL(grad_fused_bf16<64>, dim3((unsigned)ga.nc, units), dim3(kFNT), 0, stream, ga);
    else if (chunk == 32)
        hipLaunchKernelGGL(grad_fused_bf16<32>, dim3((unsigned)ga.nc, units), dim3(kFNT), 0, stream, ga);
    else if (chunk == 256) {
        // four workgroups per (chunk, unit), in groups of 8 (chunk, unit)s: one per XCD
        const unsigned groups = (unsigned)(((long)ga.nc * units + 7) / 8);
        hipLaunchKernelGGL(grad_c256_bf16, dim3(groups * 32), dim3(kFNT), 0, stream, ga);
    } else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gla

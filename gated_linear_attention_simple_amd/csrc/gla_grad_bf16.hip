// gla_grad_bf16.hip -- per-chunk gradient kernels of the chunked GLA backward
// for bf16 q/k/v/do (dk = 96, dv = 192, chunks of 64 or 128 tokens) on gfx950.
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
// Two forms.  grad_fused_bf16 (the default, below the other two) forms dQ, dK
// and dV of a chunk in one workgroup from one set of operand tiles.  The
// two-kernel form, grad_dkdv_bf16 then grad_dq_bf16, kept for comparison
// (GLA_GRAD_SPLIT=1), runs one workgroup of 4 waves per (chunk, 64-token tile);
// wave w owns token block w of the tile.  There the chunk-state snapshot (Gbar
// or Sbar) is staged in LDS for the inter-chunk terms and its space is then
// reused for the other operand tiles of the intra-chunk terms, so a workgroup
// needs ~78 KB of LDS and two run per CU; the first intra tile is loaded into
// registers during the inter-chunk MFMAs, later ones during the previous
// tile's.  Decay factors lam^d and their derivatives d lam^(d-1) come from
// per-workgroup tables indexed by d + 1 (index 0: above the diagonal, both 0).
#include "gla_common.hpp"
#include "gla_internal.hpp"
#include "gla_tile.hpp"

#include <stdlib.h>

namespace gla {
namespace {

constexpr int kDK = 96, kDV = 192;
constexpr int kST = 64;                   // token tile
constexpr int kNW = 4, kNT = 256;         // one 16-token block per wave
constexpr int kLDK = kDK + 8, kLDV = kDV + 8;
constexpr int kSnapElems = kDK * kLDV;                  // Gbar or Sbar tile
constexpr int kPairElems = kST * kLDK + kST * kLDV;     // a (dk-wide, dv-wide) tile pair
constexpr int kUnionElems = kSnapElems > kPairElems ? kSnapElems : kPairElems;

// pw[x + 1] = lam^x and dpw[x + 1] = x lam^(x-1) for x = 0..C; index 0 = 0 (x < 0).
template <int C>
__device__ __forceinline__ void fill_decay_tables(float* pw, float* dpw, float lam, int tid) {
    for (int i = tid; i < C + 2; i += kNT) {
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

// dK, dV of one 64-key tile (jt) of one chunk.
template <int C>
__global__ __launch_bounds__(kNT, 2) void grad_dkdv_bf16(GradArgs a) {
    constexpr int NSUB = C / kST;
    __shared__ __align__(16) bf16 Ks[kST * kLDK];
    __shared__ __align__(16) bf16 Vs[kST * kLDV];
    __shared__ __align__(16) bf16 Un[kUnionElems];  // Gbar, then the query tile's q and do
    __shared__ float pw[C + 2], dpw[C + 2];
    __shared__ float red[kNW];
    bf16* const Gs = Un;
    bf16* const Qs = Un;
    bf16* const Ds = Un + kST * kLDK;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, n = lane % 16, g = lane / 16;
    const int cid = blockIdx.x / NSUB, jt = blockIdx.x % NSUB, bh = blockIdx.y;
    const int H = a.H, T = a.T;
    const int hd = bh % H, b = bh / H;
    const int t0 = cid * C;
    const int ceff = min(C, T - t0);
    const int kt0 = jt * kST;  // chunk-local first key of the tile
    float* part = a.part + ((size_t)bh * a.nc + cid) * kNPart + kChainSlots + jt;
    if (kt0 >= ceff) {
        if (tid == 0) *part = 0.f;
        return;
    }
    fill_decay_tables<C>(pw, dpw, a.lambda[hd], tid);

    const int tokK = H * kDK, tokV = H * kDV;
    const size_t tok0 = (size_t)b * T * H + hd;
    const bf16* qb = static_cast<const bf16*>(a.q) + tok0 * kDK;
    const bf16* kb = static_cast<const bf16*>(a.k) + tok0 * kDK;
    const bf16* vb = static_cast<const bf16*>(a.v) + tok0 * kDV;
    const bf16* db_ = static_cast<const bf16*>(a.d_o) + tok0 * kDV;
    {
        BufStage<kST, kDK, kNT> tk;
        BufStage<kST, kDV, kNT> tv;
        BufStage<kDK, kDV, kNT> tg;
        tk.load(kb + (size_t)(t0 + kt0) * tokK, tokK, ceff - kt0, tid);
        tv.load(vb + (size_t)(t0 + kt0) * tokV, tokV, ceff - kt0, tid);
        tg.load(static_cast<const bf16*>(a.gbar) + ((size_t)bh * a.nc + cid) * kDK * kDV, kDV, kDK, tid);
        tk.template store<kLDK>(Ks, tid);
        tv.template store<kLDV>(Vs, tid);
        tg.template store<kLDV>(Gs, tid);
    }
    // first query tile (it = jt), in registers while the inter-chunk terms run
    BufStage<kST, kDK, kNT> tq;
    BufStage<kST, kDV, kNT> td;
    tq.load(qb + (size_t)(t0 + kt0) * tokK, tokK, ceff - kt0, tid);
    td.load(db_ + (size_t)(t0 + kt0) * tokV, tokV, ceff - kt0, tid);
    __syncthreads();

    const int jb = wave;
    const int jl = kt0 + jb * 16 + n;  // chunk-local key index of this lane's column
    const float cj = pw[decay_index(ceff - 1 - jl)];
    const float dcj = dpw[decay_index(ceff - 1 - jl)];

    // Inter-chunk terms.  dK^T[d][j] = c_j sum_c Gbar[d][c] v_j[c];
    // dV^T[c][j] = c_j X[c][j], X = sum_d Gbar[d][c] k_j[d]; c'_j v_j . X_j feeds dlam.
    f32x4 dKT[kDK / 16], dVT[kDV / 16];
#pragma unroll
    for (int d = 0; d < kDK / 16; ++d) {
        dKT[d] = zero4();
#pragma unroll
        for (int p = 0; p < kDV / 32; ++p)
            dKT[d] = mfma(op_row8(Gs, kLDV, d * 16 + n, 32 * p + 8 * g), op_row8(Vs, kLDV, jb * 16 + n, 32 * p + 8 * g),
                          dKT[d]);
#pragma unroll
        for (int r = 0; r < 4; ++r) dKT[d][r] *= cj;
    }
    float t2 = 0.f;
#pragma unroll
    for (int c = 0; c < kDV / 16; ++c) {
        dVT[c] = zero4();
#pragma unroll
        for (int p = 0; p < kDK / 32; ++p)
            dVT[c] = mfma(op_col8(Gs, kLDV, 32 * p, c * 16, n, g), op_row8(Ks, kLDK, jb * 16 + n, 32 * p + 8 * g),
                          dVT[c]);
        const f32x4 vj = load4<bf16>(Vs + (jb * 16 + n) * kLDV + c * 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            t2 = fmaf(dcj * vj[r], dVT[c][r], t2);
            dVT[c][r] *= cj;
        }
    }

    // Intra-chunk terms over the query tiles at or after this key tile.
    float t4 = 0.f;
    const float sc = a.scale;
    for (int it = jt; it < NSUB; ++it) {
        const int qt0 = it * kST;
        if (qt0 >= ceff) break;
        // lane-derived addresses recomputed per tile
        int tid_v = threadIdx.x;
        asm volatile("" : "+v"(tid_v));
        const int tid = tid_v, lane = tid % 64, n = lane % 16, g = lane / 16;
        const int jl = kt0 + jb * 16 + n;
        __syncthreads();  // Gbar / previous tile reads are done
        tq.template store<kLDK>(Qs, tid);
        td.template store<kLDV>(Ds, tid);
        __syncthreads();
        if (it + 1 < NSUB && qt0 + kST < ceff) {
            tq.load(qb + (size_t)(t0 + qt0 + kST) * tokK, tokK, ceff - qt0 - kST, tid);
            td.load(db_ + (size_t)(t0 + qt0 + kST) * tokV, tokV, ceff - qt0 - kST, tid);
        }
#pragma unroll
        for (int pr = 0; pr < kST / 32; ++pr) {
            f32x4 Ab[2], Pb[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ib = pr * 2 + u;
                const int il0 = qt0 + ib * 16;  // chunk-local first query of the block
                Ab[u] = zero4();
                Pb[u] = zero4();
                if (il0 + 15 < kt0 + jb * 16) continue;  // block entirely above the diagonal (uniform)
#pragma unroll
                for (int p = 0; p < kDK / 32; ++p)
                    Ab[u] = mfma(op_row8(Qs, kLDK, ib * 16 + n, 32 * p + 8 * g),
                                 op_row8(Ks, kLDK, jb * 16 + n, 32 * p + 8 * g), Ab[u]);
#pragma unroll
                for (int p = 0; p < kDV / 32; ++p)
                    Pb[u] = mfma(op_row8(Ds, kLDV, ib * 16 + n, 32 * p + 8 * g),
                                 op_row8(Vs, kLDV, jb * 16 + n, 32 * p + 8 * g), Pb[u]);
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
    }

    if (jl < ceff) {
        bf16* dkr = static_cast<bf16*>(a.dk) + tok0 * kDK + (size_t)(t0 + jl) * tokK;
        bf16* dvr = static_cast<bf16*>(a.dv) + tok0 * kDV + (size_t)(t0 + jl) * tokV;
#pragma unroll
        for (int d = 0; d < kDK / 16; ++d) store4<bf16>(dkr + d * 16 + 4 * g, dKT[d]);
#pragma unroll
        for (int c = 0; c < kDV / 16; ++c) store4<bf16>(dvr + c * 16 + 4 * g, dVT[c]);
    }
    t2 = wave_sum(t2 + sc * t4);
    if (lane == 0) red[wave] = t2;
    __syncthreads();
    if (tid == 0) *part = (red[0] + red[1]) + (red[2] + red[3]);
}

// dQ of one 64-query tile (it) of one chunk.
template <int C>
__global__ __launch_bounds__(kNT, 2) void grad_dq_bf16(GradArgs a) {
    constexpr int NSUB = C / kST;
    __shared__ __align__(16) bf16 Qs[kST * kLDK];
    __shared__ __align__(16) bf16 Ds[kST * kLDV];
    __shared__ __align__(16) bf16 Un[kUnionElems];  // Sbar, then the key tile's k and v
    __shared__ float pw[C + 2], dpw[C + 2];
    __shared__ float red[kNW], redg[kNW];
    bf16* const Ss = Un;
    bf16* const Ks = Un;
    bf16* const Vs = Un + kST * kLDK;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, n = lane % 16, g = lane / 16;
    const int cid = blockIdx.x / NSUB, it = blockIdx.x % NSUB, bh = blockIdx.y;
    const int H = a.H, T = a.T;
    const int hd = bh % H, b = bh / H;
    const int t0 = cid * C;
    const int ceff = min(C, T - t0);
    const int qt0 = it * kST;
    float* part = a.part + ((size_t)bh * a.nc + cid) * kNPart + kChainSlots + NSUB + it;
    if (qt0 >= ceff) {
        if (tid == 0) *part = 0.f;
        return;
    }
    fill_decay_tables<C>(pw, dpw, a.lambda[hd], tid);

    const int tokK = H * kDK, tokV = H * kDV;
    const size_t tok0 = (size_t)b * T * H + hd;
    const bf16* qb = static_cast<const bf16*>(a.q) + tok0 * kDK;
    const bf16* kb = static_cast<const bf16*>(a.k) + tok0 * kDK;
    const bf16* vb = static_cast<const bf16*>(a.v) + tok0 * kDV;
    const bf16* db_ = static_cast<const bf16*>(a.d_o) + tok0 * kDV;
    {
        BufStage<kST, kDK, kNT> tq;
        BufStage<kST, kDV, kNT> td;
        BufStage<kDK, kDV, kNT> ts;
        tq.load(qb + (size_t)(t0 + qt0) * tokK, tokK, ceff - qt0, tid);
        td.load(db_ + (size_t)(t0 + qt0) * tokV, tokV, ceff - qt0, tid);
        ts.load(static_cast<const bf16*>(a.sbar) + ((size_t)bh * a.nc + cid) * kDK * kDV, kDV, kDK, tid);
        tq.template store<kLDK>(Qs, tid);
        td.template store<kLDV>(Ds, tid);
        ts.template store<kLDV>(Ss, tid);
    }
    float gsd = 0.f;  // first query tile: this thread's part of <Gbar, Sbar>
    if (it == 0) {    // (against the Sbar pieces this thread has just put in LDS)
        BufStage<kDK, kDV, kNT> tg;
        tg.load(static_cast<const bf16*>(a.gbar) + ((size_t)bh * a.nc + cid) * kDK * kDV, kDV, kDK, tid);
        gsd = snap_dot_lds<kNT, kLDV>(tg, Ss, tid);
    }
    // first key tile (jt = 0), in registers while the inter-chunk term runs
    BufStage<kST, kDK, kNT> tk;
    BufStage<kST, kDV, kNT> tv;
    tk.load(kb + (size_t)t0 * tokK, tokK, ceff, tid);
    tv.load(vb + (size_t)t0 * tokV, tokV, ceff, tid);
    __syncthreads();

    const int ib = wave;
    const int il = qt0 + ib * 16 + n;  // chunk-local query index of this lane's column
    const float bi = pw[il + 2];       // lam^(il+1)
    const float dbi = dpw[il + 2];     // (il+1) lam^il
    const float sc = a.scale;

    // Inter-chunk term: Y^T[d][i] = sum_c Sbar[d][c] do_i[c]; dQ += scale b_i Y; scale b'_i q_i . Y_i feeds dlam.
    f32x4 dQT[kDK / 16];
    float t3 = 0.f;
#pragma unroll
    for (int d = 0; d < kDK / 16; ++d) {
        dQT[d] = zero4();
#pragma unroll
        for (int p = 0; p < kDV / 32; ++p)
            dQT[d] = mfma(op_row8(Ss, kLDV, d * 16 + n, 32 * p + 8 * g), op_row8(Ds, kLDV, ib * 16 + n, 32 * p + 8 * g),
                          dQT[d]);
        const f32x4 qi = load4<bf16>(Qs + (ib * 16 + n) * kLDK + d * 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            t3 = fmaf(dbi * qi[r], dQT[d][r], t3);
            dQT[d][r] *= sc * bi;
        }
    }

    // Intra-chunk term over the key tiles at or before this query tile.
    for (int jt = 0; jt <= it; ++jt) {
        const int kt0 = jt * kST;
        int tid_v = threadIdx.x;
        asm volatile("" : "+v"(tid_v));
        const int tid = tid_v, lane = tid % 64, n = lane % 16, g = lane / 16;
        const int il = qt0 + ib * 16 + n;
        __syncthreads();  // Sbar / previous tile reads are done
        tk.template store<kLDK>(Ks, tid);
        tv.template store<kLDV>(Vs, tid);
        __syncthreads();
        if (jt + 1 <= it) {
            tk.load(kb + (size_t)(t0 + kt0 + kST) * tokK, tokK, ceff - kt0 - kST, tid);
            tv.load(vb + (size_t)(t0 + kt0 + kST) * tokV, tokV, ceff - kt0 - kST, tid);
        }
#pragma unroll
        for (int pr = 0; pr < kST / 32; ++pr) {
            f32x4 Pt[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int jb = pr * 2 + u;
                const int jl0 = kt0 + jb * 16;  // chunk-local first key of the block
                Pt[u] = zero4();
                if (jl0 > qt0 + ib * 16 + 15) continue;  // block entirely above the diagonal (uniform)
#pragma unroll
                for (int p = 0; p < kDV / 32; ++p)
                    Pt[u] = mfma(op_row8(Vs, kLDV, jb * 16 + n, 32 * p + 8 * g),
                                 op_row8(Ds, kLDV, ib * 16 + n, 32 * p + 8 * g), Pt[u]);
                // Pt[u][r] = v_j . do_i for j = jl0 + 4g + r, i = il
#pragma unroll
                for (int r = 0; r < 4; ++r) Pt[u][r] *= sc * pw[decay_index(il - (jl0 + 4 * g + r))];
            }
            const bf16x8 pt = pack_acc(Pt[0], Pt[1]);
#pragma unroll
            for (int d = 0; d < kDK / 16; ++d) dQT[d] = mfma(op_col_pair(Ks, kLDK, 32 * pr, d * 16, n, g), pt, dQT[d]);
        }
    }

    if (il < ceff) {
        bf16* dqr = static_cast<bf16*>(a.dq) + tok0 * kDK + (size_t)(t0 + il) * tokK;
#pragma unroll
        for (int d = 0; d < kDK / 16; ++d) store4<bf16>(dqr + d * 16 + 4 * g, dQT[d]);
    }
    t3 = wave_sum(sc * t3);
    gsd = wave_sum(gsd);
    if (lane == 0) {
        red[wave] = t3;
        redg[wave] = gsd;
    }
    __syncthreads();
    if (tid == 0) {
        *part = (red[0] + red[1]) + (red[2] + red[3]);
        // the chunk's term through lam^ceff, ceff lam^(ceff-1) <Gbar, Sbar>, in slot 0
        if (it == 0)
            a.part[((size_t)bh * a.nc + cid) * kNPart] = dpw[ceff + 1] * ((redg[0] + redg[1]) + (redg[2] + redg[3]));
    }
}


// All three gradients of one chunk of C = 128 or 64 tokens (one workgroup of
// 8 waves per (chunk, unit)): every operand tile is read once, where the
// two-kernel form reads the tiles and both snapshots twice.  Wave w owns key
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
constexpr int kFNW = 8, kFNT = 512;
constexpr int kFHalf = 64;  // query rows per half

template <int C>
__global__ __launch_bounds__(kFNT, 1) void grad_fused_bf16(GradArgs a) {
    static_assert(C == 128 || C == 64, "one or two 64-query halves");
    constexpr int NSUB = C / kST;
    constexpr int NKB = C / 16;  // key blocks (waves that own one)
    __shared__ __align__(16) bf16 Ks[C * kLDK];
    __shared__ __align__(16) bf16 Vs[C * kLDV];
    __shared__ __align__(16) bf16 Xs[kDK * kLDV];            // Sbar, then Gbar
    __shared__ __align__(16) bf16 Qs[kFHalf * kLDK];         // one half's queries
    __shared__ __align__(16) bf16 Ds[kFHalf * kLDV];         // and output gradients
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

    const int tokK = H * kDK, tokV = H * kDV;
    const size_t tok0 = (size_t)b * T * H + hd;
    const size_t snap = ((size_t)bh * a.nc + cid) * kDK * kDV;
    const bf16* qb = static_cast<const bf16*>(a.q) + tok0 * kDK + (size_t)t0 * tokK;
    const bf16* kb = static_cast<const bf16*>(a.k) + tok0 * kDK + (size_t)t0 * tokK;
    const bf16* vb = static_cast<const bf16*>(a.v) + tok0 * kDV + (size_t)t0 * tokV;
    const bf16* db_ = static_cast<const bf16*>(a.d_o) + tok0 * kDV + (size_t)t0 * tokV;
    BufStage<kFHalf, kDK, kFNT> tq;
    BufStage<kFHalf, kDV, kFNT> td;
    {
        BufStage<C, kDK, kFNT> tk;
        BufStage<C, kDV, kFNT> tv;
        BufStage<kDK, kDV, kFNT> ts;
        tk.load(kb, tokK, ceff, tid);
        tv.load(vb, tokV, ceff, tid);
        ts.load(static_cast<const bf16*>(a.sbar) + snap, kDV, kDK, tid);
        tq.load(qb, tokK, ceff, tid);
        td.load(db_, tokV, ceff, tid);
        tk.template store<kLDK>(Ks, tid);
        tv.template store<kLDV>(Vs, tid);
        ts.template store<kLDV>(Xs, tid);
        tq.template store<kLDK>(Qs, tid);
        td.template store<kLDV>(Ds, tid);
    }
    // the second half's queries and output gradients, in registers meanwhile
    if (kFHalf < ceff) {
        tq.load(qb + (size_t)kFHalf * tokK, tokK, ceff - kFHalf, tid);
        td.load(db_ + (size_t)kFHalf * tokV, tokV, ceff - kFHalf, tid);
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
        for (int pr = 0; pr < kFHalf / 32; ++pr) {
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
            bf16* dqr = static_cast<bf16*>(a.dq) + tok0 * kDK + (size_t)(t0 + il) * tokK;
#pragma unroll
            for (int d = 0; d < kDK / 16; ++d) store4<bf16>(dqr + d * 16 + 4 * g, dQT[d]);
        }
    };

    // A: queries 0..63
    if (wave < 4) key_terms(0);
    else query_block(0, wave - 4);
    // B: queries 64..127 (Gbar requested for C meanwhile)
    BufStage<kDK, kDV, kFNT> tg;
    if (C > kFHalf && kFHalf < ceff) {
        __syncthreads();  // half 0 reads are done
        tq.template store<kLDK>(Qs, tid);
        td.template store<kLDV>(Ds, tid);
        __syncthreads();
        tg.load(static_cast<const bf16*>(a.gbar) + snap, kDV, kDK, tid);
        if (wave >= 4) query_block(kFHalf, wave - 4);
        key_terms(kFHalf);
    } else {
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
        bf16* dkr = static_cast<bf16*>(a.dk) + tok0 * kDK + (size_t)(t0 + jl) * tokK;
        bf16* dvr = static_cast<bf16*>(a.dv) + tok0 * kDV + (size_t)(t0 + jl) * tokV;
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
    // slots kChainSlots + [0, NSUB): key side (here all in the first),
    // + [NSUB, 2 NSUB): query side, as the two-kernel form lays them out
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

}  // namespace

hipError_t launch_grad_bf16(int chunk, const GradArgs& ga, unsigned units, hipStream_t stream) {
    if (chunk != 128 && chunk != 64) return hipErrorInvalidValue;
    const unsigned tiles = (unsigned)ga.nc * (unsigned)(chunk / kST);
    if (chunk == 128) {
        // one kernel for all three gradients (the two-kernel form moves about
        // twice the bytes); GLA_GRAD_SPLIT=1 selects the two kernels (tests, sweeps)
        const char* e = getenv("GLA_GRAD_SPLIT");
        if (!(e && atoi(e) == 1)) {
            hipLaunchKernelGGL(grad_fused_bf16<128>, dim3((unsigned)ga.nc, units), dim3(kFNT), 0, stream, ga);
            return hipGetLastError();
        }
        hipLaunchKernelGGL(grad_dkdv_bf16<128>, dim3(tiles, units), dim3(kNT), 0, stream, ga);
        if (hipError_t err = hipGetLastError(); err != hipSuccess) return err;
        hipLaunchKernelGGL(grad_dq_bf16<128>, dim3(tiles, units), dim3(kNT), 0, stream, ga);
    } else {
        const char* e = getenv("GLA_GRAD_SPLIT");
        if (!(e && atoi(e) == 1)) {
            hipLaunchKernelGGL(grad_fused_bf16<64>, dim3((unsigned)ga.nc, units), dim3(kFNT), 0, stream, ga);
            return hipGetLastError();
        }
        hipLaunchKernelGGL(grad_dkdv_bf16<64>, dim3(tiles, units), dim3(kNT), 0, stream, ga);
        if (hipError_t err = hipGetLastError(); err != hipSuccess) return err;
        hipLaunchKernelGGL(grad_dq_bf16<64>, dim3(tiles, units), dim3(kNT), 0, stream, ga);
    }
    return hipGetLastError();
}

}  // namespace gla

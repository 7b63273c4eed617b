// gla_fwd.hip -- chunked-parallel GLA forward for fp32 q/k/v, plus the launch
// plan, segment scan and dispatch shared with the bf16 kernel (gla_fwd_bf16.hip).
//
// Method: Laplace 3B post, section "Challenge 1" (chunked GLA).  For chunk c
// of C tokens with start state S (positions i, j in [0, C) inside the chunk,
// decay factors b_i = lam^(i+1), c_j = lam^(C-1-j), D_ij = lam^(i-j) for
// i >= j else 0):
//     O_c   = scale * ( (Q K^T (.) D) V  +  diag(b) Q S )
//     S_new = lam^C S + (diag(c) K)^T V
// which is the per-token recurrence S_t = lam S_{t-1} + k_t v_t^T,
// o_t = scale S_t^T q_t regrouped exactly (only rounding differs).  A partial
// last chunk uses its own length in place of C.
//
// fp32 kernel (16x16x4 fp32 MFMA; one workgroup of NW waves per (batch, head,
// segment)): the fp32 state lives in accumulator registers across the chunk
// loop, wave w owning state/output columns [w*DV/NW, (w+1)*DV/NW); q, k, a
// c_j-scaled copy of k and v are staged row-major in LDS; decay-masked score
// blocks are computed once per workgroup and shared through LDS; O^T = S^T Q^T
// takes S straight from its accumulators.
//
// Long sequences are cut into segments run by separate workgroups: a prologue
// launch (STATE_ONLY) computes each segment's local end state U_s from zero, a
// scan launch turns them into segment start states
// S_in(s+1) = lam^L S_in(s) + U_s (L tokens per segment), and the main launch
// runs every segment from its start state -- the same recurrence regrouped.
#include "gla_common.hpp"
#include "gla_internal.hpp"
#include "gla_tile.hpp"


namespace gla {


// Row of block t of a lower triangle of 16x16 blocks numbered row by row
// (block (ib, jb) is t = ib(ib+1)/2 + jb), for t < 136 (up to 16 block rows).
__device__ __forceinline__ int tri_row(int t) {
    int ib = static_cast<int>((sqrtf(8.f * t + 1.f) - 1.f) * 0.5f);
    ib -= (ib * (ib + 1) / 2 > t);        // guard against sqrt rounding either way
    ib += ((ib + 1) * (ib + 2) / 2 <= t);
    return ib;
}

// LDS layout of one fp32 workgroup:
//   Qs, Ks, Kc  [C][DK + 4]   queries, keys, keys scaled by c_j   (main only: Qs, Ks)
//   Vs          [C][DV + 4]   values
//   As          lower-triangular 16x16 blocks of the decay-masked scores
//               A[i][j] = (q_i . k_j) lam^(i-j), block (ib, jb) at
//               (ib(ib+1)/2 + jb) * 16 * ALD, row i - 16 ib, column j - 16 jb
//   pw          [C + 1] powers lam^n
template <int DK, int DV, int C, bool STATE_ONLY>
struct FwdLds {
    static constexpr int LDK = DK + 4;
    static constexpr int LDV = DV + 4;
    static constexpr int ALD = 20;  // padded 16-wide score block rows
    static constexpr int NIB = C / 16;
    static constexpr int NTRI = NIB * (NIB + 1) / 2;
    static constexpr int QK = STATE_ONLY ? 8 : C * LDK;
    static constexpr int AS = STATE_ONLY ? 8 : NTRI * 16 * ALD;
};

template <int DK, int DV, int C, int NW, bool STATE_ONLY>
__global__ __launch_bounds__(NW * 64, 1) void fwd_f32_kernel(FwdArgs a) {
    using L = FwdLds<DK, DV, C, STATE_ONLY>;
    using E = float;
    constexpr int NT = NW * 64;
    constexpr int NCW = DV / NW;   // state / output columns per wave
    constexpr int NCB = NCW / 16;
    constexpr int NDB = DK / 16;
    constexpr int NIB = C / 16;
    constexpr int LDK = L::LDK, LDV = L::LDV, ALD = L::ALD;
    static_assert(NCW % 16 == 0 && DK % 16 == 0 && C % 16 == 0, "16x16 tiles");

    __shared__ __align__(16) E Qs[L::QK];
    __shared__ __align__(16) E Ks[L::QK];
    __shared__ __align__(16) E Kc[C * LDK];  // keys scaled by c_j = lam^(ceff-1-j)
    __shared__ __align__(16) E Vs[C * LDV];
    __shared__ __align__(16) E As[L::AS];
    __shared__ float pw[C + 1];              // lam^n, n = 0..C

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64, n = lane % 16, g = lane / 16;
    const int seg = blockIdx.x, bh = blockIdx.y;
    const int H = a.H, T = a.T;
    const int h = bh % H, b = bh / H;
    const int c_begin = seg * a.seg_chunks;
    const int c_end = min(a.nc, c_begin + a.seg_chunks);
    const int colbase = wave * NCW;
    const float lam = a.lambda[h];

    for (int i = tid; i <= C; i += NT) pw[i] = pow_int(lam, i);
    DecayLane dl;
    float hlane = 1.f;   // lam^(n+1): b_i = lam^(16 ib) * lam^(n+1) for query i = 16 ib + n
    if constexpr (!STATE_ONLY) {
        dl.init(lam, n, g);
        hlane = pow_int(lam, n + 1);
    }

    const int tokQ = a.sq.t, tokK = a.sk.t, tokV = a.sv.t, tokO = a.so.t;
    const E* qb = static_cast<const E*>(a.q) + b * a.sq.b + h * DK;
    const E* kb = static_cast<const E*>(a.k) + b * a.sk.b + h * DK;
    const E* vb = static_cast<const E*>(a.v) + b * a.sv.b + h * DV;
    E* ob = static_cast<E*>(a.o) + b * a.so.b + h * DV;

    // State registers: Sacc[db][cb][r] = S[db*16 + 4g + r][colbase + cb*16 + n].
    f32x4 Sacc[NDB][NCB];
    auto sidx = [&](int db, int cb, int r) -> size_t {
        return (size_t)(db * 16 + 4 * g + r) * DV + colbase + cb * 16 + n;
    };
    const float* Sin = nullptr;  // segment start state (nullptr = zero)
    if constexpr (!STATE_ONLY) {
        if (seg == 0) Sin = a.S0 ? a.S0 + (size_t)bh * DK * DV : nullptr;
        else Sin = a.U + ((size_t)bh * (a.nseg - 1) + (seg - 1)) * DK * DV;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) Sacc[db][cb][r] = Sin ? Sin[sidx(db, cb, r)] : 0.f;

    TileStage<E, C, DK, NT> tq, tk;
    TileStage<E, C, DV, NT> tv;
    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * C;
        const int ceff = min(C, T - t0);
        if constexpr (!STATE_ONLY) {
            if (a.sbar) {  // the chunk's start state, for the backward
                E* sb = static_cast<E*>(a.sbar) + ((size_t)bh * a.nc + c) * DK * DV;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) sb[sidx(db, cb, r)] = Sacc[db][cb][r];
            }
        }
        if (!STATE_ONLY) tq.load(qb + (size_t)t0 * tokQ, tokQ, T - t0, tid);
        tk.load(kb + (size_t)t0 * tokK, tokK, T - t0, tid);
        tv.load(vb + (size_t)t0 * tokV, tokV, T - t0, tid);
        __syncthreads();  // previous chunk's LDS reads are done (and pw is visible)
        if (!STATE_ONLY) {
            tq.template store<LDK>(Qs, tid);
            tk.template store<LDK>(Ks, tid);
        }
        tk.template store_scaled<LDK>(Kc, tid, [&](int row) { return row < ceff ? pw[ceff - 1 - row] : 0.f; });
        tv.template store<LDV>(Vs, tid);
        __syncthreads();

        if constexpr (!STATE_ONLY) {
            // Decay-masked score blocks, each computed by one wave and shared:
            // A[i][j] = (q_i . k_j) lam^(i-j) for j <= i (block (ib, jb), jb <= ib).
            // Block t = NW*k + wave of the triangle; the blocks of a wave are
            // independent, so their MFMA chains are interleaved k-step by k-step.
            constexpr int NBW = (L::NTRI + NW - 1) / NW;  // blocks per wave
            constexpr int GRP = NBW < 3 ? NBW : 3;           // blocks interleaved at a time
            const int nib = (ceff + 15) / 16;
            const int ntri = nib * (nib + 1) / 2;
#pragma unroll
            for (int k0 = 0; k0 < NBW; k0 += GRP) {
                if (wave + NW * k0 >= ntri) break;
                f32x4 AT[GRP];
                int bib[GRP], bjb[GRP];
#pragma unroll
                for (int k = 0; k < GRP; ++k) {
                    const int t = wave + NW * (k0 + k);  // slots past the triangle point at block 0 (unused)
                    bib[k] = t < L::NTRI ? tri_row(t) : 0;
                    bjb[k] = t < L::NTRI ? t - bib[k] * (bib[k] + 1) / 2 : 0;
                    AT[k] = zero4();
                }
#pragma unroll
                for (int p = 0; p < DK / 4; ++p)
#pragma unroll
                    for (int k = 0; k < GRP; ++k)
                        if (k0 + k < NBW && wave + NW * (k0 + k) < ntri)
                            AT[k] = mfma(Ks[(bjb[k] * 16 + n) * LDK + 4 * p + g],
                                         Qs[(bib[k] * 16 + n) * LDK + 4 * p + g], AT[k]);
#pragma unroll
                for (int k = 0; k < GRP; ++k) {
                    const int t = wave + NW * (k0 + k);
                    if (k0 + k >= NBW || t >= ntri) break;
                    const int ib = bib[k], jb = bjb[k];
                    const float blk = jb == ib ? 1.f : pw[16 * (ib - jb - 1)];  // lam^(16(ib-jb-1))
#pragma unroll
                    for (int r = 0; r < 4; ++r) AT[k][r] *= (jb == ib) ? dl.diag[r] : blk * dl.off[r];
                    store4<E>(As + t * 16 * ALD + n * ALD + 4 * g, AT[k]);
                }
            }
            __syncthreads();  // score blocks complete
#pragma unroll 1
            for (int ib = 0; ib < NIB; ++ib) {
                if (ib * 16 >= ceff) break;
                const int irow = ib * 16 + n;  // this lane's query row in the chunk
                const float bi = pw[16 * ib] * hlane;
                // O^T = b_i S^T Q^T (inter-chunk, S^T from its accumulators)
                //      + V^T A^T     (intra-chunk, A from the shared score blocks)
                f32x4 OT[NCB];
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) OT[cb] = zero4();
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            OT[cb] = mfma(Sacc[db][cb][r], Qs[irow * LDK + db * 16 + 4 * g + r], OT[cb]);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) OT[cb][r] *= bi;
                for (int jb = 0; jb <= ib; ++jb) {
                    const E* blk = As + (ib * (ib + 1) / 2 + jb) * 16 * ALD + n * ALD + 4 * g;
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            OT[cb] = mfma(Vs[(jb * 16 + 4 * g + r) * LDV + colbase + cb * 16 + n], blk[r], OT[cb]);
                }
                if (irow < ceff) {
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) OT[cb][r] *= a.scale;
                        store4<E>(ob + (size_t)(t0 + irow) * tokO + colbase + cb * 16 + 4 * g, OT[cb]);
                    }
                }
            }
        }

        // State advance: S <- lam^ceff S + (diag(c) K)^T V
        const float Lam = pw[ceff];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) Sacc[db][cb][r] *= Lam;
#pragma unroll 2
        for (int p = 0; p < C / 4; ++p)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    Sacc[db][cb] = mfma(Kc[(4 * p + g) * LDK + db * 16 + n],
                                        Vs[(4 * p + g) * LDV + colbase + cb * 16 + n], Sacc[db][cb]);
    }

    float* dst = nullptr;
    if (STATE_ONLY) dst = a.U + ((size_t)bh * (a.nseg - 1) + seg) * DK * DV;
    else if (seg == a.nseg - 1 && a.S_final) dst = a.S_final + (size_t)bh * DK * DV;
    if (dst) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[sidx(db, cb, r)] = Sacc[db][cb][r];
    }
}

// Segment start states: turns the segment-local end states U_0..U_{nseg-2} (from
// zero) into the start states of segments 1..nseg-1, in place:
//   S_in(s+1) = lam^L S_in(s) + U_s,   S_in(0) = S0 (or 0),   L = tokens per segment.
// One thread per 4 consecutive state elements; all loads are issued before the
// (short, sequential) multiply-add chain.
__global__ __launch_bounds__(256) void seg_scan_kernel(const float* __restrict__ S0, float* __restrict__ U,
                                                       const float* __restrict__ lambda, int H, int nseg,
                                                       int seg_tokens, int dkdv) {
    const int bh = blockIdx.y;
    const int e4 = blockIdx.x * blockDim.x + threadIdx.x;
    if (e4 * 4 >= dkdv) return;
    const float lamL = pow_int(lambda[bh % H], seg_tokens);
    f32x4 run = S0 ? *reinterpret_cast<const f32x4*>(S0 + (size_t)bh * dkdv + 4 * e4) : zero4();
    f32x4* u = reinterpret_cast<f32x4*>(U + (size_t)bh * (nseg - 1) * dkdv) + e4;
    const size_t step = (size_t)dkdv / 4;
    f32x4 x[kMaxSegments - 1];
#pragma unroll
    for (int s = 0; s < kMaxSegments - 1; ++s)
        if (s < nseg - 1) x[s] = u[s * step];
#pragma unroll
    for (int s = 0; s < kMaxSegments - 1; ++s) {
        if (s < nseg - 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) run[e] = fmaf(lamL, run[e], x[s][e]);
            u[s * step] = run;
        }
    }
}

hipError_t launch_seg_scan(const float* S0, float* U, const float* lambda, int H, int nseg, int seg_tokens,
                           int dkdv, unsigned units, hipStream_t stream) {
    hipLaunchKernelGGL(seg_scan_kernel, dim3((dkdv / 4 + 255) / 256, units), dim3(256), 0, stream, S0, U, lambda, H,
                       nseg, seg_tokens, dkdv);
    return hipGetLastError();
}

// T == 0: the final state is the initial one (or zeros).
__global__ void copy_state_kernel(const float* __restrict__ S0, float* __restrict__ S, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        S[i] = S0 ? S0[i] : 0.f;
}

bool fwd_supported(bool bf16_io, int dk, int dv, int chunk) {
    // fp32 tiles of 128 tokens would need ~250 KB of LDS, so fp32 stops at 64;
    // bf16 MFMA steps contract 32 values, so the dk = 16 shape is fp32 only.
    return (dk == 96 && dv == 192 && (chunk == 64 || (bf16_io && (chunk == 128 || chunk == 32 || chunk == 256)))) ||
           (dk == 16 && dv == 32 && chunk == 32 && !bf16_io);
}

FwdPlan fwd_plan(bool bf16_io, int B, int T, int H, int dk, int dv, int chunk, int num_cu, const PlanHint* hint) {
    FwdPlan p{};
    p.nc = T > 0 ? (T + chunk - 1) / chunk : 0;
    const long units = (long)B * H;
    int nseg = 1;
    // Split the sequence until the grid covers every compute unit (segments of
    // at least one chunk, at most kMaxSegments of them).
    while (units * nseg < num_cu && nseg * 2 <= p.nc && nseg < kMaxSegments) nseg *= 2;
    if (hint && hint->nseg >= 1) nseg = hint->nseg < kMaxSegments ? hint->nseg : kMaxSegments;
    if (p.nc == 0) nseg = 1;
    nseg = nseg > p.nc && p.nc > 0 ? p.nc : nseg;
    p.seg_chunks = p.nc > 0 ? (p.nc + nseg - 1) / nseg : 0;
    p.nseg = p.nc > 0 ? (p.nc + p.seg_chunks - 1) / p.seg_chunks : 1;
    // bf16: when the state-only prologue (one workgroup per unit and segment before
    // the last) would occupy at most half the compute units, it runs over
    // half-length sub-segments instead, the scan combining their states (B = 8,
    // H = 16, T = 2,048: 256 workgroups of 4 chunks instead of 128 of 8).
    p.psub = 1;
    // (the scan holds at most kMaxSegments - 1 states per unit)
    if (bf16_io && p.nseg > 1 && p.seg_chunks % 2 == 0 && units * (p.nseg - 1) * 2 <= num_cu &&
        (p.nseg - 1) * 2 <= kMaxSegments - 1)
        p.psub = 2;
    if (hint && hint->psub == 1) p.psub = 1;
    // fp32 segment states (psub per segment boundary); the bf16 path adds a bf16
    // copy of each start state
    p.ws_bytes = (size_t)units * (p.nseg - 1) * p.psub * dk * dv * (sizeof(float) + (bf16_io ? 2 : 0));
    // bf16, short sequence: a tiled state chain can emit every chunk's start
    // state for one output workgroup per chunk.  Measured on gfx950 it beats the
    // segment split only for 128-token chunks, at most 16 (batch, head) units
    // and at most 16 chunks (16 units: 21.1 vs 23.7 us at 512 tokens, 21.5 vs
    // 24.8 at 1,024, 30.9 vs 31.6 at 2,048; 8 units x 4,096 tokens: 38.4 vs
    // 32.2, its 32 passes being sequential at ~0.7 us each, bound by LDS
    // transposed reads).
    p.chain = bf16_io && chunk == 128 && units <= 16 && p.nseg > 1 && p.nc <= 16;
    if (hint && hint->chain == 0) p.chain = 0;
    // (the tiled chain and its output kernel are built for 64- and 128-token chunks)
    if (hint && hint->chain == 1 && bf16_io && chunk >= 64 && p.nc > 1 && p.nc <= kChainMaxChunks) p.chain = 1;
    // 256-token chunks run in the chain form only: their q, k, v tiles alone
    // exceed a compute unit's LDS, so the segment kernels do not take them
    if (bf16_io && chunk == 256 && p.nc > 0) p.chain = 1;
    if (p.chain) p.ws_bytes = (size_t)units * p.nc * dk * dv * 2;  // every chunk's start state, bf16
    // bf16 segments with at most kFuseMaxStates local states before the last segment
    // (e.g. two segments with the sub-segment prologue): no scan launch, each segment
    // folds them into its start state in the scan's order (same bits)
    p.fuse_scan = bf16_io && !p.chain && p.nseg > 1 && (p.nseg - 1) * p.psub <= kFuseMaxStates;
    if (hint && hint->scan == 0) p.fuse_scan = 0;
    return p;
}

template <int DK, int DV, int C, int NW>
static hipError_t launch_fwd_f32(const FwdPlan& plan, int B, int T, int H, const FwdIO& io, const float* lambda,
                                 const float* S0, float scale, float* S_final, void* sbar, void* ws,
                                 hipStream_t stream) {
    FwdArgs a{};
    a.T = T;
    a.H = H;
    a.q = io.q;
    a.k = io.k;
    a.v = io.v;
    a.sq = io.sq;
    a.sk = io.sk;
    a.sv = io.sv;
    a.so = io.so;
    a.lambda = lambda;
    a.S0 = S0;
    a.scale = scale;
    a.o = io.o;
    a.S_final = S_final;
    a.U = static_cast<float*>(ws);
    a.sbar = sbar;
    a.nseg = plan.nseg;
    a.seg_chunks = plan.seg_chunks;
    a.nc = plan.nc;
    const unsigned units = (unsigned)B * H;
    if (plan.nseg > 1) {
        hipLaunchKernelGGL((fwd_f32_kernel<DK, DV, C, NW, true>), dim3(plan.nseg - 1, units), dim3(NW * 64), 0,
                           stream, a);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        err = launch_seg_scan(S0, a.U, lambda, H, plan.nseg, plan.seg_chunks * C, DK * DV, units, stream);
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL((fwd_f32_kernel<DK, DV, C, NW, false>), dim3(plan.nseg, units), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fwd(bool bf16_io, const FwdPlan& plan, int B, int T, int H, int dk, int dv, int chunk,
                      const FwdIO& io, const float* lambda, const float* S0, float scale, float* S_final, void* sbar,
                      void* ws, hipStream_t stream) {
    if (B == 0 || H == 0) return hipSuccess;
    if (T == 0) {
        if (!S_final) return hipSuccess;
        const size_t n = (size_t)B * H * dk * dv;
        hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)),
                           dim3(256), 0, stream, S0, S_final, n);
        return hipGetLastError();
    }
    if (bf16_io) {
        if (dk == 96 && dv == 192)
            return launch_fwd_bf16(plan, B, T, H, chunk, io, lambda, S0, scale, S_final, sbar, ws, stream);
        return hipErrorInvalidValue;
    }
#define GLA_FWD_CASE(DK_, DV_, C_, NW_)                                                                    \
    if (dk == DK_ && dv == DV_ && chunk == C_)                                                              \
        return launch_fwd_f32<DK_, DV_, C_, NW_>(plan, B, T, H, io, lambda, S0, scale, S_final, sbar, ws, stream);
    GLA_FWD_CASE(96, 192, 64, 4)
    GLA_FWD_CASE(16, 32, 32, 2)
#undef GLA_FWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace gla

// gla_fwd.hip -- chunked-parallel GLA forward on gfx950 MFMA.
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
// Work decomposition (one workgroup of NW waves per (batch, head, segment)):
//  * the fp32 state lives in MFMA accumulator registers for the whole chunk
//    loop; wave w owns state columns [w*DV/NW, (w+1)*DV/NW) and the output
//    columns with them, so the state is never written to LDS or HBM;
//  * per chunk the q, k, v tiles are staged global -> registers (prefetched one
//    chunk ahead) -> LDS, as row-major Q and K plus transposed copies K'^T
//    (pre-scaled by c_j) and V^T, so every MFMA operand is a contiguous LDS
//    read along its contraction dimension;
//  * A^T = K Q^T is computed per 16-row output block with its decay mask in
//    fp32, rounded to bf16 and fed straight back from the accumulator
//    registers as the B operand of O^T += V^T A^T (the accumulator's row index
//    is the contraction index, so no LDS round trip is needed);
//  * O^T = S^T Q^T (the inter-chunk term) likewise takes S from its
//    accumulators; outputs leave as 4 consecutive columns per lane.
//  * Long sequences are cut into segments run by separate workgroups: a
//    prologue launch (STATE_ONLY) computes each segment's local end state U_s
//    from zero; the main launch starts segment s from
//    lam^(sL) S0 + sum_{s'<s} lam^((s-1-s')L) U_s' (Horner, L tokens per
//    segment), which is the same recurrence regrouped by segments.
#include "gla_common.hpp"
#include "gla_internal.hpp"

#include <stdlib.h>

namespace gla {

struct FwdArgs {
    int T, H;
    const void* q;
    const void* k;
    const void* v;
    const float* lambda;
    const float* S0;
    float scale;
    void* o;
    float* S_final;
    float* U;          // [B*H][nseg-1][DK][DV] segment-local end states
    int nseg, seg_chunks, nc;
};

// Loads one chunk tile (C rows of D elements, token stride `tok_stride`) into
// registers as 16-byte pieces.  Piece p covers RP consecutive rows (2 for bf16
// so a transposed LDS store writes one dword = two tokens) and one 16-byte
// column group; rows at or past T read as zeros.
template <typename E, int D, int C, int NT>
struct TileLoader {
    static constexpr int VEC = 16 / sizeof(E);
    static constexpr int RP = 4 / sizeof(E);
    static constexpr int KC = D / VEC;
    static constexpr int NRG = C / RP;
    static constexpr int NP = NRG * KC;
    static constexpr int PER = (NP + NT - 1) / NT;
    uint4 r[PER][RP];

    __device__ __forceinline__ void load(const E* base, size_t tok_stride, int t0, int T, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = tid + NT * i;
            const int rgp = p % NRG, kc = p / NRG;
#pragma unroll
            for (int j = 0; j < RP; ++j) {
                const int t = t0 + rgp * RP + j;
                if ((NP % NT == 0 || p < NP) && t < T)
                    r[i][j] = *reinterpret_cast<const uint4*>(base + (size_t)t * tok_stride + kc * VEC);
                else
                    r[i][j] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    }

    // Row-major copy dst[row * LD + col].
    template <int LD>
    __device__ __forceinline__ void store_rows(E* dst, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = tid + NT * i;
            if (NP % NT != 0 && p >= NP) continue;
            const int rgp = p % NRG, kc = p / NRG;
#pragma unroll
            for (int j = 0; j < RP; ++j)
                *reinterpret_cast<uint4*>(dst + (rgp * RP + j) * LD + kc * VEC) = r[i][j];
        }
    }

    // Transposed copy dst[col * LDT + row]; with SCALED, row j is multiplied by
    // lam^(ceff-1-j) (0 past the chunk end) before rounding to E.
    template <int LDT, bool SCALED>
    __device__ __forceinline__ void store_cols(E* dst, int tid, const float* pw, int ceff) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = tid + NT * i;
            if (NP % NT != 0 && p >= NP) continue;
            const int rgp = p % NRG, kc = p / NRG;
            const int row0 = rgp * RP;
            if constexpr (sizeof(E) == 2) {
                const bf16* x0 = reinterpret_cast<const bf16*>(&r[i][0]);
                const bf16* x1 = reinterpret_cast<const bf16*>(&r[i][1]);
                float c0 = 1.f, c1 = 1.f;
                if constexpr (SCALED) {
                    c0 = row0 < ceff ? pw[ceff - 1 - row0] : 0.f;
                    c1 = row0 + 1 < ceff ? pw[ceff - 2 - row0] : 0.f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    bf16 a0 = x0[e], a1 = x1[e];
                    if constexpr (SCALED) {
                        a0 = to_bf16(to_f32(a0) * c0);
                        a1 = to_bf16(to_f32(a1) * c1);
                    }
                    const uint32_t w = (uint32_t)__builtin_bit_cast(uint16_t, a0) |
                                       ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
                    *reinterpret_cast<uint32_t*>(dst + (kc * 8 + e) * LDT + row0) = w;
                }
            } else {
                const float* x = reinterpret_cast<const float*>(&r[i][0]);
                float c0 = 1.f;
                if constexpr (SCALED) c0 = row0 < ceff ? pw[ceff - 1 - row0] : 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(kc * 4 + e) * LDT + row0] = x[e] * c0;
            }
        }
    }
};

__device__ __forceinline__ bf16x8 lds_k8(const bf16* base, int ld, int row, int k0) {
    return *reinterpret_cast<const bf16x8*>(base + row * ld + k0);
}
// k0..k0+3 and k0+16..k0+19: the k-set of two stacked accumulator blocks.
__device__ __forceinline__ bf16x8 lds_k4x2(const bf16* base, int ld, int row, int k0) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(base + row * ld + k0);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(base + row * ld + k0 + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 pack_acc(f32x4 a, f32x4 b) {
    return bf16x8{to_bf16(a[0]), to_bf16(a[1]), to_bf16(a[2]), to_bf16(a[3]),
                  to_bf16(b[0]), to_bf16(b[1]), to_bf16(b[2]), to_bf16(b[3])};
}

template <typename E>
__device__ __forceinline__ void store4(E* dst, f32x4 x);
template <>
__device__ __forceinline__ void store4<float>(float* dst, f32x4 x) {
    *reinterpret_cast<f32x4*>(dst) = x;
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* dst, f32x4 x) {
    *reinterpret_cast<bf16x4*>(dst) = bf16x4{to_bf16(x[0]), to_bf16(x[1]), to_bf16(x[2]), to_bf16(x[3])};
}

template <typename E, int DK, int DV, int C, int NW, bool STATE_ONLY>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(FwdArgs a) {
    constexpr bool BF = sizeof(E) == 2;
    constexpr int NT = NW * 64;
    constexpr int NCW = DV / NW;   // state / output columns per wave
    constexpr int NCB = NCW / 16;
    constexpr int NDB = DK / 16;
    constexpr int NIB = C / 16;
    constexpr int PAD = BF ? 8 : 4;
    constexpr int LDK = DK + PAD;  // row stride of Qs, Ks
    constexpr int LDC = C + PAD;   // row stride of KTs, VTs
    static_assert(NCW % 16 == 0 && DK % 16 == 0 && C % 16 == 0, "16x16 tiles");
    static_assert(!BF || (DK % 32 == 0 && C % 32 == 0), "bf16 k-steps of 32");

    __shared__ __align__(16) E KTs[DK * LDC];
    __shared__ __align__(16) E VTs[DV * LDC];
    __shared__ __align__(16) E Qs[STATE_ONLY ? 8 : C * LDK];
    __shared__ __align__(16) E Ks[STATE_ONLY ? 8 : C * LDK];
    __shared__ float pw[C + 1];

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

    const size_t tokK = (size_t)H * DK, tokV = (size_t)H * DV;
    const size_t tok0 = (size_t)b * T * H + h;
    const E* qb = static_cast<const E*>(a.q) + tok0 * DK;
    const E* kb = static_cast<const E*>(a.k) + tok0 * DK;
    const E* vb = static_cast<const E*>(a.v) + tok0 * DV;
    E* ob = static_cast<E*>(a.o) + tok0 * DV;

    // State registers: Sacc[db][cb][r] = S[db*16 + 4g + r][colbase + cb*16 + n].
    f32x4 Sacc[NDB][NCB];
    auto sidx = [&](int db, int cb, int r) -> size_t {
        return (size_t)(db * 16 + 4 * g + r) * DV + colbase + cb * 16 + n;
    };
    const float* S0 = STATE_ONLY ? nullptr : a.S0;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Sacc[db][cb][r] = S0 ? S0[(size_t)bh * DK * DV + sidx(db, cb, r)] : 0.f;
    if (!STATE_ONLY && seg > 0) {
        const float lamL = pow_int(lam, a.seg_chunks * C);
        const float* U = a.U + (size_t)bh * (a.nseg - 1) * DK * DV;
        for (int s = 0; s < seg; ++s) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Sacc[db][cb][r] = fmaf(lamL, Sacc[db][cb][r], U[(size_t)s * DK * DV + sidx(db, cb, r)]);
        }
    }

    TileLoader<E, DK, C, NT> lq, lk;
    TileLoader<E, DV, C, NT> lv;
    if (c_begin < c_end) {
        if (!STATE_ONLY) lq.load(qb, tokK, c_begin * C, T, tid);
        lk.load(kb, tokK, c_begin * C, T, tid);
        lv.load(vb, tokV, c_begin * C, T, tid);
    }

    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * C;
        const int ceff = min(C, T - t0);
        __syncthreads();  // previous chunk's LDS reads are done (and pw is visible)
        if (!STATE_ONLY) {
            lq.template store_rows<LDK>(Qs, tid);
            lk.template store_rows<LDK>(Ks, tid);
        }
        lk.template store_cols<LDC, true>(KTs, tid, pw, ceff);
        lv.template store_cols<LDC, false>(VTs, tid, pw, ceff);
        __syncthreads();
        if (c + 1 < c_end) {
            if (!STATE_ONLY) lq.load(qb, tokK, t0 + C, T, tid);
            lk.load(kb, tokK, t0 + C, T, tid);
            lv.load(vb, tokV, t0 + C, T, tid);
        }

        if constexpr (!STATE_ONLY) {
#pragma unroll
            for (int ib = 0; ib < NIB; ++ib) {
                if (ib * 16 >= ceff) break;
                const int irow = ib * 16 + n;  // this lane's output row (token) in the chunk
                // A^T blocks (jb, ib): AT[jb][r] = (k_j . q_i) * lam^(i-j), j = jb*16+4g+r.
                f32x4 AT[NIB];
#pragma unroll
                for (int jb = 0; jb <= ib; ++jb) {
                    AT[jb] = zero4();
                    if constexpr (BF) {
#pragma unroll
                        for (int p = 0; p < DK / 32; ++p)
                            AT[jb] = mfma(lds_k8(Ks, LDK, jb * 16 + n, 32 * p + 8 * g),
                                          lds_k8(Qs, LDK, irow, 32 * p + 8 * g), AT[jb]);
                    } else {
#pragma unroll
                        for (int p = 0; p < DK / 4; ++p)
                            AT[jb] = mfma(Ks[(jb * 16 + n) * LDK + 4 * p + g], Qs[irow * LDK + 4 * p + g], AT[jb]);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int d = irow - (jb * 16 + 4 * g + r);
                        AT[jb][r] *= d >= 0 ? pw[d] : 0.f;
                    }
                }
                const float bi = pw[irow + 1];
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const int vrow = colbase + cb * 16 + n;  // this lane's column as a V^T row
                    f32x4 OT = zero4();
                    // inter-chunk: O^T += S^T Q^T
                    if constexpr (BF) {
#pragma unroll
                        for (int p = 0; p < DK / 32; ++p)  // S^T from its accumulators, pairs of dk blocks
                            OT = mfma(pack_acc(Sacc[2 * p][cb], Sacc[2 * p + 1][cb]),
                                      lds_k4x2(Qs, LDK, irow, 32 * p + 4 * g), OT);
                    } else {
#pragma unroll
                        for (int db = 0; db < NDB; ++db)
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                OT = mfma(Sacc[db][cb][r], Qs[irow * LDK + db * 16 + 4 * g + r], OT);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) OT[r] *= bi;
                    // intra-chunk: O^T += V^T A^T
                    if constexpr (BF) {
#pragma unroll
                        for (int p = 0; 2 * p <= ib; ++p) {
                            const f32x4 hi = (2 * p + 1 <= ib) ? AT[2 * p + 1] : zero4();
                            OT = mfma(lds_k4x2(VTs, LDC, vrow, 32 * p + 4 * g), pack_acc(AT[2 * p], hi), OT);
                        }
                    } else {
#pragma unroll
                        for (int jb = 0; jb <= ib; ++jb)
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                OT = mfma(VTs[vrow * LDC + jb * 16 + 4 * g + r], AT[jb][r], OT);
                    }
                    if (irow < ceff) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) OT[r] *= a.scale;
                        store4<E>(ob + (size_t)(t0 + irow) * tokV + colbase + cb * 16 + 4 * g, OT);
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
        if constexpr (BF) {
#pragma unroll
            for (int p = 0; p < C / 32; ++p)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8 ka = lds_k8(KTs, LDC, db * 16 + n, 32 * p + 8 * g);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        Sacc[db][cb] = mfma(ka, lds_k8(VTs, LDC, colbase + cb * 16 + n, 32 * p + 8 * g), Sacc[db][cb]);
                }
        } else {
#pragma unroll
            for (int p = 0; p < C / 4; ++p)
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        Sacc[db][cb] = mfma(KTs[(db * 16 + n) * LDC + 4 * p + g],
                                            VTs[(colbase + cb * 16 + n) * LDC + 4 * p + g], Sacc[db][cb]);
        }
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

// T == 0: the final state is the initial one (or zeros).
__global__ void copy_state_kernel(const float* __restrict__ S0, float* __restrict__ S, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        S[i] = S0 ? S0[i] : 0.f;
}

bool fwd_supported(bool bf16_io, int dk, int dv, int chunk) {
    // fp32 tiles of 128 tokens would need ~250 KB of LDS, so fp32 stops at 64;
    // bf16 MFMA steps contract 32 values, so the dk = 16 shape is fp32 only.
    return (dk == 96 && dv == 192 && (chunk == 64 || (chunk == 128 && bf16_io))) ||
           (dk == 16 && dv == 32 && chunk == 32 && !bf16_io);
}

FwdPlan fwd_plan(int B, int T, int H, int dk, int dv, int chunk, int num_cu) {
    FwdPlan p{};
    p.nc = T > 0 ? (T + chunk - 1) / chunk : 0;
    const long units = (long)B * H;
    int nseg = 1;
    // Split the sequence until the grid covers every compute unit, keeping at
    // least two chunks per segment for the Horner start-up of later segments.
    while (units * nseg < num_cu && nseg * 4 <= p.nc && nseg < 16) nseg *= 2;
    if (const char* e = getenv("GLA_FWD_SEGMENTS")) {
        const int forced = atoi(e);
        if (forced >= 1) nseg = forced;
    }
    if (p.nc == 0) nseg = 1;
    nseg = nseg > p.nc && p.nc > 0 ? p.nc : nseg;
    p.seg_chunks = p.nc > 0 ? (p.nc + nseg - 1) / nseg : 0;
    p.nseg = p.nc > 0 ? (p.nc + p.seg_chunks - 1) / p.seg_chunks : 1;
    p.ws_bytes = (size_t)units * (p.nseg - 1) * dk * dv * sizeof(float);
    return p;
}

template <typename E, int DK, int DV, int C, int NW>
static hipError_t launch_fwd_t(const FwdPlan& plan, int B, int T, int H, const void* q, const void* k,
                               const void* v, const float* lambda, const float* S0, float scale, void* o,
                               float* S_final, void* ws, hipStream_t stream) {
    FwdArgs a{};
    a.T = T;
    a.H = H;
    a.q = q;
    a.k = k;
    a.v = v;
    a.lambda = lambda;
    a.S0 = S0;
    a.scale = scale;
    a.o = o;
    a.S_final = S_final;
    a.U = static_cast<float*>(ws);
    a.nseg = plan.nseg;
    a.seg_chunks = plan.seg_chunks;
    a.nc = plan.nc;
    const unsigned units = (unsigned)B * H;
    if (plan.nseg > 1) {
        hipLaunchKernelGGL((fwd_kernel<E, DK, DV, C, NW, true>), dim3(plan.nseg - 1, units), dim3(NW * 64), 0,
                           stream, a);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL((fwd_kernel<E, DK, DV, C, NW, false>), dim3(plan.nseg, units), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fwd(bool bf16_io, const FwdPlan& plan, int B, int T, int H, int dk, int dv, int chunk,
                      const void* q, const void* k, const void* v, const float* lambda, const float* S0,
                      float scale, void* o, float* S_final, void* ws, hipStream_t stream) {
    if (B == 0 || H == 0) return hipSuccess;
    if (T == 0) {
        if (!S_final) return hipSuccess;
        const size_t n = (size_t)B * H * dk * dv;
        hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)),
                           dim3(256), 0, stream, S0, S_final, n);
        return hipGetLastError();
    }
#define GLA_FWD_CASE(E_, DK_, DV_, C_, NW_)                                                            \
    if ((sizeof(E_) == 2) == bf16_io && dk == DK_ && dv == DV_ && chunk == C_)                          \
        return launch_fwd_t<E_, DK_, DV_, C_, NW_>(plan, B, T, H, q, k, v, lambda, S0, scale, o, S_final, \
                                                    ws, stream);
    GLA_FWD_CASE(bf16, 96, 192, 128, 4)
    GLA_FWD_CASE(bf16, 96, 192, 64, 4)
    GLA_FWD_CASE(float, 96, 192, 64, 4)
    GLA_FWD_CASE(float, 16, 32, 32, 2)
#undef GLA_FWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace gla

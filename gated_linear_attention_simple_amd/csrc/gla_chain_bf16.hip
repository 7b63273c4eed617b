// gla_chain_bf16.hip -- the backward's chunk-state chains for bf16 q/k/v/do
// (dk = 96, dv = 192, chunks of 32, 64, 128 or 256 tokens) on gfx950.
//
// Laplace 3B post, sections "Challenge 1" and "Challenge 3": the chunked
// backward needs, for every chunk c, the state entering it (Sbar_c) and the
// gradient of the loss with respect to the state leaving it (Gbar_c):
//   forward:  S <- lam^ceff S + K^T diag(c) V,                   c_j = lam^(ceff-1-j)
//   reverse:  G <- lam^ceff G + Q^T diag(scale b) dO,            b_i = lam^(i+1)
// (the chunk's term of dlam through lam^ceff, ceff lam^(ceff-1) <Gbar_c, Sbar_c>,
// is taken by the gradient kernel, which holds both snapshots).
// LOCAL passes start from zero and write each segment's local result; EMIT
// passes start from the scanned segment state and write, before each chunk's
// update, the state as that chunk's bf16 snapshot.
//
// Work decomposition: one workgroup of 12 waves per (batch*head, segment), as
// in the bf16 forward -- wave w keeps the state rows 16 (2i + h) .. +16
// (h = w / 6, i = 0..2) of the 32 columns [32 (w % 6), +32) in fp32 accumulator
// registers; x (k or q, pre-scaled per row) and y (v or do) tiles are staged
// row-major in LDS with buffer loads prefetched one pass ahead; both MFMA
// operands are token-contracted and come from the LDS transpose read.  A
// snapshot goes through a bf16 LDS staging tile so it leaves as coalesced
// 16-byte row pieces.  A pass covers at most 128 tokens: a 256-token chunk is
// two passes, the state decayed once, in its first.
#include "gla_common.hpp"
#include "gla_internal.hpp"
#include "gla_tile.hpp"

namespace gla {
namespace {

constexpr int kDK = 96, kDV = 192;
constexpr int kNCB = 2, kNCG = 6, kNW = 12, kNT = 768;

template <int C, bool REV, bool EMIT>
__global__ __launch_bounds__(kNT, 1) void chain_bf16_kernel(StateArgs a) {
    constexpr int R = C < 128 ? C : 128, NS = C / R;   // tokens per pass, passes per chunk
    constexpr int NP = R / 32;
    constexpr int LDK = kDK + 8, LDV = kDV + 8;
    __shared__ __align__(16) bf16 Xs[R * LDK];
    __shared__ __align__(16) bf16 Ys[R * LDV];
    __shared__ __align__(16) bf16 Sb[EMIT ? kDK * LDV : 8];
    __shared__ __align__(16) float xc[2][C];  // row factors of x: full chunk, partial last chunk

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, n = lane % 16, g = lane / 16;
    const int h = wave / kNCG, colbase = 32 * (wave % kNCG);
    const int seg = blockIdx.x + ((!EMIT && REV) ? 1 : 0);
    const int bh = blockIdx.y;
    const int H = a.H, T = a.T;
    const int hd = bh % H, b = bh / H;
    const int c_begin = seg * a.seg_chunks;
    const int c_end = min(a.nc, c_begin + a.seg_chunks);

    // The first pass's tiles are requested before anything else (decay tables,
    // start state, folded local states), which is then set up while they fly.
    const int tokX = a.sx.t, tokY = a.sy.t;
    const bf16* xb = static_cast<const bf16*>(a.x) + b * a.sx.b + hd * kDK;
    const bf16* yb = static_cast<const bf16*>(a.y) + b * a.sy.b + hd * kDV;
    RowStage<R, kDK, kNT> tx;
    RowStage<R, kDV, kNT> ty;
    const int nchunks = c_end - c_begin;
    auto chunk_of = [&](int ci) { return REV ? c_end - 1 - ci : c_begin + ci; };
    // pass (ci, sp): tokens c C + sp R .. of chunk c = chunk_of(ci)
    auto load_pass = [&](int c, int sp, int tid) {
        const int t = c * C + sp * R;
        tx.load(xb + (size_t)t * tokX, tokX, T - t, tid);
        ty.load(yb + (size_t)t * tokY, tokY, T - t, tid);
    };
    if (nchunks > 0) load_pass(chunk_of(0), 0, tid);

    const float lam = a.lambda[hd];
    const int ctail = T % C;  // length of a partial last chunk (0: none)
    for (int j = tid; j < C; j += kNT) {
        if constexpr (REV) {
            const float bi = a.xscale * pow_int(lam, j + 1);
            xc[0][j] = bi;
            xc[1][j] = j < ctail ? bi : 0.f;
        } else {
            xc[0][j] = pow_int(lam, C - 1 - j);
            xc[1][j] = j < ctail ? pow_int(lam, ctail - 1 - j) : 0.f;
        }
    }
    const float lamC = uniform_f32(pow_int(lam, C));
    const float lamTail = uniform_f32(pow_int(lam, ctail));

    // Sacc[i][cb][r] = S[16 (2i + h) + 4g + r][colbase + 16 cb + n]
    f32x4 Sacc[3][kNCB];
    auto sidx = [&](int i, int cb, int r) -> int {
        return (16 * (2 * i + h) + 4 * g + r) * kDV + colbase + cb * 16 + n;
    };
    const float* Sin = nullptr;
    if constexpr (EMIT) {
        if (a.fuse_scan) Sin = a.S_edge;  // the local states are folded in below
        else if (!REV) Sin = seg == 0 ? a.S_edge : a.U + ((size_t)bh * (a.nseg - 1) + seg - 1) * kDK * kDV;
        else Sin = seg == a.nseg - 1 ? a.S_edge : a.U + ((size_t)bh * (a.nseg - 1) + seg) * kDK * kDV;
        if (Sin && Sin == a.S_edge) Sin += (size_t)bh * kDK * kDV;
    }
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int cb = 0; cb < kNCB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) Sacc[i][cb][r] = Sin ? Sin[sidx(i, cb, r)] : 0.f;
    if constexpr (EMIT) {
        if (a.fuse_scan) {
            // Fold the local passes' states of the segments this one continues, in the
            // scan kernels' order (the same bits): forward from S0 over segments
            // 0 .. seg-1, reverse from dS_T over segments nseg-1 down to seg+1.
            const float* u = a.U + (size_t)bh * (a.nseg - 1) * kDK * kDV;
            const int seg_tokens = a.seg_chunks * C;
            for (int k = 0; k < (REV ? a.nseg - 1 - seg : seg); ++k) {
                const int s = REV ? a.nseg - 1 - k : k;   // segment folded in
                const float f = REV ? pow_int(lam, min(seg_tokens, T - s * seg_tokens)) : pow_int(lam, seg_tokens);
                const float* x = u + (size_t)(REV ? s - 1 : s) * kDK * kDV;
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int cb = 0; cb < kNCB; ++cb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) Sacc[i][cb][r] = fmaf(f, Sacc[i][cb][r], x[sidx(i, cb, r)]);
            }
        }
    }

    constexpr int NSP = kDK * (kDV / 8) / kNT;   // snapshot pieces per thread
    static_assert(kDK * (kDV / 8) % kNT == 0, "snapshot pieces per thread");

    if constexpr (NS == 1) {
    // one pass per chunk (kept apart: the two-pass loop below costs this case
    // registers and time)
    for (int ci = 0; ci < nchunks; ++ci) {
        // lane-derived addresses are recomputed per chunk, not held across the loop
        int tid_v = threadIdx.x;
        asm volatile("" : "+v"(tid_v));
        const int tid = tid_v, lane = tid % 64, n = lane % 16, g = lane / 16;
        const int c = chunk_of(ci);
        const int t0 = c * C;
        const int ceff = min(C, T - t0);
        const float* xcc = xc[ceff == C ? 0 : 1];
        __syncthreads();  // the previous chunk's LDS reads are done
        tx.template store_scaled<LDK>(Xs, tid, [&](int row) { return xcc[row]; });
        ty.template store<LDV>(Ys, tid);
        if constexpr (EMIT) {
            // this chunk's snapshot: the state before its update
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
                for (int cb = 0; cb < kNCB; ++cb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 16 * (2 * i + h) + 4 * g + r, col = colbase + 16 * cb + n;
                        Sb[row * LDV + col] = to_bf16(Sacc[i][cb][r]);
                    }
        }
        __syncthreads();
        if (ci + 1 < nchunks) load_pass(chunk_of(ci + 1), 0, tid);

        if constexpr (EMIT) {
            // Copy the snapshot out as 16-byte row pieces (96 rows x 24 pieces).
            // (non-temporal buffer stores: the training step 369.5 -> 368.2 us at C = 128,
            // 431.0 -> 427.6 at 64, the same bits)
            const auto rs = __builtin_amdgcn_make_buffer_rsrc(
                static_cast<bf16*>(a.snap) + ((size_t)bh * a.nc + c) * kDK * kDV, 0, kDK * kDV * 2, kBufWord3);
#pragma unroll
            for (int k = 0; k < NSP; ++k) {
                const int pc = tid + k * kNT, row = pc / (kDV / 8), col = (pc % (kDV / 8)) * 8;
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, *reinterpret_cast<const bf16x8*>(Sb + row * LDV + col)), rs,
                    (row * kDV + col) * 2, 0, kCpolNT);
            }
        }

        // S <- lam^ceff S + X^T Y over the chunk's tokens (X rows pre-scaled)
        const float Lam = ceff == C ? lamC : lamTail;
        bf16x8 yf[kNCB][NP];
#pragma unroll
        for (int cb = 0; cb < kNCB; ++cb)
#pragma unroll
            for (int p = 0; p < NP; ++p) yf[cb][p] = op_col8(Ys, LDV, 32 * p, colbase + 16 * cb, n, g);
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int cb = 0; cb < kNCB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) Sacc[i][cb][r] *= Lam;
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                const bf16x8 xop = op_col8(Xs, LDK, 32 * p, 16 * (2 * i + h), n, g);
#pragma unroll
                for (int cb = 0; cb < kNCB; ++cb) Sacc[i][cb] = mfma(xop, yf[cb][p], Sacc[i][cb]);
            }
    }
    } else {
    for (int ci = 0; ci < nchunks; ++ci) {
        const int c = chunk_of(ci);
        const int t0 = c * C;
        const int ceff = min(C, T - t0);
        const int npass = (ceff + R - 1) / R;   // passes holding tokens of this chunk
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) {
            if (sp >= npass) break;   // (uniform)
            // lane-derived addresses are recomputed per pass, not held across the loop
            int tid_v = threadIdx.x;
            asm volatile("" : "+v"(tid_v));
            const int tid = tid_v, lane = tid % 64, n = lane % 16, g = lane / 16;
            const float* xcc = xc[ceff == C ? 0 : 1] + sp * R;
            __syncthreads();  // the previous pass's LDS reads are done
            tx.template store_scaled<LDK>(Xs, tid, [&](int row) { return xcc[row]; });
            ty.template store<LDV>(Ys, tid);
            if constexpr (EMIT) {
                if (sp == 0) {
                    // this chunk's snapshot: the state before its update
#pragma unroll
                    for (int i = 0; i < 3; ++i)
#pragma unroll
                        for (int cb = 0; cb < kNCB; ++cb)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int row = 16 * (2 * i + h) + 4 * g + r, col = colbase + 16 * cb + n;
                                Sb[row * LDV + col] = to_bf16(Sacc[i][cb][r]);
                            }
                }
            }
            __syncthreads();
            // the next pass: this chunk's second (if it has tokens), else the next chunk's first
            if (sp + 1 < npass) load_pass(c, sp + 1, tid);
            else if (ci + 1 < nchunks) load_pass(chunk_of(ci + 1), 0, tid);

            if constexpr (EMIT) {
                if (sp == 0) {
                    // Copy the snapshot out as 16-byte row pieces (96 rows x 24 pieces).
                    const auto rs = __builtin_amdgcn_make_buffer_rsrc(
                        static_cast<bf16*>(a.snap) + ((size_t)bh * a.nc + c) * kDK * kDV, 0, kDK * kDV * 2, kBufWord3);
#pragma unroll
                    for (int k = 0; k < NSP; ++k) {
                        const int pc = tid + k * kNT, row = pc / (kDV / 8), col = (pc % (kDV / 8)) * 8;
                        __builtin_amdgcn_raw_buffer_store_b128(
                            __builtin_bit_cast(u32x4, *reinterpret_cast<const bf16x8*>(Sb + row * LDV + col)), rs,
                            (row * kDV + col) * 2, 0, kCpolNT);
                    }
                }
            }

            // S <- lam^ceff S + X^T Y over the chunk's tokens (X rows pre-scaled),
            // the decay in the chunk's first pass
            bf16x8 yf[kNCB][NP];
#pragma unroll
            for (int cb = 0; cb < kNCB; ++cb)
#pragma unroll
                for (int p = 0; p < NP; ++p) yf[cb][p] = op_col8(Ys, LDV, 32 * p, colbase + 16 * cb, n, g);
            if (sp == 0) {
                const float Lam = ceff == C ? lamC : lamTail;
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int cb = 0; cb < kNCB; ++cb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) Sacc[i][cb][r] *= Lam;
            }
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    const bf16x8 xop = op_col8(Xs, LDK, 32 * p, 16 * (2 * i + h), n, g);
#pragma unroll
                    for (int cb = 0; cb < kNCB; ++cb) Sacc[i][cb] = mfma(xop, yf[cb][p], Sacc[i][cb]);
                }
        }
    }

    }

    float* dst = nullptr;
    if (!EMIT) dst = a.U + ((size_t)bh * (a.nseg - 1) + (REV ? seg - 1 : seg)) * kDK * kDV;
    else if (REV && seg == 0 && a.S_out) dst = a.S_out + (size_t)bh * kDK * kDV;
    if (dst) {
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int cb = 0; cb < kNCB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[sidx(i, cb, r)] = Sacc[i][cb][r];
    }
}

template <int C, bool REV, bool EMIT>
hipError_t launch_chain_c(const StateArgs& s, unsigned grid_x, unsigned units, hipStream_t stream) {
    hipLaunchKernelGGL((chain_bf16_kernel<C, REV, EMIT>), dim3(grid_x, units), dim3(kNT), 0, stream, s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chain_bf16(int chunk, bool rev, bool emit, const StateArgs& s, unsigned grid_x, unsigned units,
                             hipStream_t stream) {
#define GLA_CHAIN(C_)                                                                    \
    if (chunk == C_) {                                                                   \
        if (!rev && !emit) return launch_chain_c<C_, false, false>(s, grid_x, units, stream); \
        if (!rev && emit) return launch_chain_c<C_, false, true>(s, grid_x, units, stream);   \
        if (rev && !emit) return launch_chain_c<C_, true, false>(s, grid_x, units, stream);   \
        return launch_chain_c<C_, true, true>(s, grid_x, units, stream);                      \
    }
    GLA_CHAIN(256)
    GLA_CHAIN(128)
    GLA_CHAIN(64)
    GLA_CHAIN(32)
#undef GLA_CHAIN
    return hipErrorInvalidValue;
}

}  // namespace gla

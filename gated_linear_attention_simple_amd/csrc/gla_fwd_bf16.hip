// gla_fwd_bf16.hip -- chunked-parallel GLA forward for bf16 q/k/v on gfx950
// (dk = 96, dv = 192, chunks of 32, 64 or 128 tokens; 256-token chunks in the
// tiled-chain form only, see fwd_out256_kernel).
//
// Method: Laplace 3B post, section "Challenge 1" (chunked GLA).  For chunk c
// of C tokens with start state S (positions i, j in [0, C); b_i = lam^(i+1),
// c_j = lam^(C-1-j), D_ij = lam^(i-j) for i >= j else 0):
//     O_c   = scale * ( (Q K^T (.) D) V  +  diag(b) Q S )
//     S_new = lam^C S + K^T diag(c) V
// -- the per-token recurrence S_t = lam S_{t-1} + k_t v_t^T, o_t = scale S_t^T q_t
// regrouped exactly.  A partial last chunk uses its own length in place of C.
//
// One workgroup per (batch, head, segment) of NW = 2 * NCG = 12 waves (three per
// SIMD), NCG = 6 column groups of 16 * NCB = 32 state/output columns.  (NCB, the
// 16-column blocks per wave, is a template parameter; an 8-wave layout with
// NCB = 3 measured slower and is not built.)  Waves w and w + NCG form a pair owning
// columns [16 NCB (w % NCG), +16 NCB); inside a pair, wave h = w / NCG keeps the
// 16-row state blocks db = 2i + h (i = 0..2) in fp32 accumulator registers for
// the whole chunk loop.  Per chunk:
//  * q, k, v tiles (prefetched into registers during the previous chunk) go to
//    LDS row-major, as they sit in HBM;
//  * the decay-masked score blocks A = (Q K^T) (.) D (16x16, lower triangle)
//    are dealt to the waves in sets that share query fragments, masked in fp32
//    and shared through LDS in bf16;
//  * each wave publishes a bf16 copy of its state half and reads its partner's,
//    so both hold S^T for their 16 NCB columns as MFMA operands (the
//    accumulator's row index is the contraction index) for the inter-chunk term
//    b (.) S^T Q^T;
//  * the pair splits the query strips for the output (h = 0 takes strip pairs
//    whose intra-chunk work sums to the same as h = 1's) and writes O^T blocks,
//    one strip at a time, as 4 consecutive columns per lane;
//  * the value fragments each wave loaded for O^T += V^T A^T are reused for the
//    state update S += (diag(c) K)^T V, with the keys scaled by c_j in place
//    once the score blocks are done.
// Long sequences with few (batch, head) units are cut into segments as in the
// fp32 kernel: a state-only prologue, a segment scan, then this kernel.  Here
// the segment states sit in the workspace in register order (16-byte pieces),
// and a one-chunk segment reads its start state as the bf16 copy the scan
// leaves (the only form it uses, so the result is unchanged).
#include "gla_common.hpp"
#include "gla_internal.hpp"
#include "gla_tile.hpp"

#include <type_traits>
#include <utility>

namespace gla {
namespace {

constexpr int kDK = 96, kDV = 192;

template <int C, int LDK_, int NCB_>
struct F8 {
    static constexpr int NCB = NCB_;              // 16-column blocks per wave
    static constexpr int NCG = kDV / (16 * NCB);  // column groups (wave pairs)
    static constexpr int NW = 2 * NCG, NT = 64 * NW;
    static constexpr int NIB = C / 16, NP = C / 32, NTRI = NIB * (NIB + 1) / 2;
    static constexpr int NDW = 3;                 // 16-row state blocks per wave
    static constexpr int LDK = LDK_, LDV = kDV + 8;
    static constexpr int Q_BYTES = C * LDK * 2, V_BYTES = C * LDV * 2;
    static constexpr int XS_BYTES = NW * NDW * NCB * 64 * 8;   // bf16 state halves
    static constexpr int AS_BYTES = NTRI * 16 * 16 * 2;        // score blocks, unpadded (swizzled)
    static constexpr int TAIL_BYTES = (C + 2) * 4 + 2 * C * 4 + 8;
    static constexpr int XA_BYTES = XS_BYTES + AS_BYTES;   // exchange area, then score blocks
    static constexpr int AS_OFF = XS_BYTES;
    static_assert(2 * Q_BYTES + V_BYTES + XA_BYTES + TAIL_BYTES <= 160 * 1024, "LDS budget");
    static constexpr int NSLOT = (NTRI + NW - 1) / NW;   // score blocks per wave
    static_assert(kDV % (16 * NCB) == 0, "column groups");
};

// Score blocks of wave w (slot k), packed 16 * ib + jb, or -1 for an empty slot.
// Each wave's blocks lie in at most two query strips, so per k-step it reads
// at most two query fragments; the sets balance the 36 (C = 128), 10 (C = 64)
// or 3 (C = 32) blocks of the lower triangle over the NW waves.  The first
// score_lead<C, NW>() slots of every wave lie in its first strip.
template <int C, int NW>
__host__ __device__ constexpr int score_block(int w, int k) {
    if constexpr (C == 128 && NW == 12) {
        constexpr signed char t[12][3] = {{0x70, 0x71, 0x72}, {0x73, 0x74, 0x75}, {0x76, 0x77, 0x00},
                                          {0x60, 0x61, 0x62}, {0x63, 0x64, 0x65}, {0x10, 0x11, 0x66},
                                          {0x50, 0x51, 0x52}, {0x53, 0x54, 0x55}, {0x40, 0x41, 0x42},
                                          {0x43, 0x44, 0x20}, {0x21, 0x22, 0x30}, {0x31, 0x32, 0x33}};
        return t[w][k];
    } else if constexpr (C == 64 && NW == 12) {
        constexpr signed char t[12] = {0x30, 0x31, 0x32, 0x33, 0x20, 0x21, 0x22, 0x10, 0x11, 0x00, -1, -1};
        return k == 0 ? t[w] : -1;
    } else {
        static_assert(C == 32 && NW == 12, "score block table");
        constexpr signed char t[12] = {0x10, 0x11, 0x00, -1, -1, -1, -1, -1, -1, -1, -1, -1};
        return k == 0 ? t[w] : -1;
    }
}

// The same table for a wave-uniform w without a memory load: each slot's entries
// packed as bytes into two 64-bit constants (waves 0..7, 8..15), so the lookup
// is a scalar select and shift.  (A table read would be a vector load, and its
// wait would also wait for every tile load issued before it.)
template <int C, int NW>
__host__ __device__ constexpr unsigned long long score_word(int k, int half) {
    unsigned long long r = 0;
    for (int j = 0; j < 8; ++j) {
        const int w = 8 * half + j;
        const int v = w < NW ? score_block<C, NW>(w, k) : -1;
        r |= (unsigned long long)(unsigned char)(signed char)v << (8 * j);
    }
    return r;
}

template <int C, int NW, int K>
struct ScoreWords {
    static constexpr unsigned long long lo = score_word<C, NW>(K, 0), hi = score_word<C, NW>(K, 1);
};

template <int C, int NW, int... K>
__device__ __forceinline__ void score_blocks_uniform(int w, int* blk, std::integer_sequence<int, K...>) {
    ((blk[K] = (int)(signed char)(unsigned char)((w < 8 ? ScoreWords<C, NW, K>::lo : ScoreWords<C, NW, K>::hi) >>
                                                 (8 * (w & 7)))),
     ...);
}

template <int C, int NW>
constexpr int score_lead() {
    return C == 128 ? 2 : 1;
}

// Element offset of row `row`, 16-byte unit `u` (0 or 1) of a 16x16 bf16 score
// block: the unit index is flipped on rows 8..15 so the 16 rows read by one
// lane group spread over all banks.
__device__ __forceinline__ int as_off(int row, int u) { return row * 16 + 8 * (u ^ ((row >> 3) & 1)); }

// This wave's decay-masked score blocks (slot k: block 16 ib + jb of the
// lower triangle, or -1), A = scale * (Q K^T) (.) D, written to As as bf16.
// AT[k][4g + r][n] = q_(16 ib + n) . k_(16 jb + 4g + r); query fragments of
// strips sa (the first NA slots) and sb are read once per k-step.
template <int C, int LDK, int NW, int NS>
__device__ __forceinline__ void score_blocks_to_lds(const bf16* Qs, const bf16* Ks, bf16* As, const float* pws,
                                                    const int (&blk)[NS], int sa, int sb, const bool (&use_b)[NS],
                                                    int n, int g) {
    constexpr int NA = score_lead<C, NW>();
    f32x4 AT[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) AT[k] = zero4();
#pragma unroll
    for (int p = 0; p < kDK / 32; ++p) {
        const bf16x8 qa = op_row8(Qs, LDK, 16 * sa + n, 32 * p + 8 * g);
        const bf16x8 qc = op_row8(Qs, LDK, 16 * sb + n, 32 * p + 8 * g);
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int jb = blk[k] >= 0 ? blk[k] & 15 : 0;
            const bf16x8 q = (k < NA || !use_b[k]) ? qa : qc;
            AT[k] = mfma(op_row8(Ks, LDK, 16 * jb + n, 32 * p + 8 * g), q, AT[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        if (blk[k] < 0) continue;
        const int ib = blk[k] >> 4, jb = blk[k] & 15;
        // scale * D_ij = scale * lam^(i-j) for i >= j, else 0, with
        // i - j = 16 (ib - jb) + n - 4g - r: one table read per element.
        const int d1 = 16 * (ib - jb) + n - 4 * g + 1;
        f32x4 x = AT[k];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] *= pws[max(d1 - r, 0)];
        *reinterpret_cast<bf16x4*>(As + (ib * (ib + 1) / 2 + jb) * 256 + as_off(n, g >> 1) + 4 * (g & 1)) =
            bf16x4{to_bf16(x[0]), to_bf16(x[1]), to_bf16(x[2]), to_bf16(x[3])};
    }
}

// Output of query strips 2K and 2K+1 for this wave's 16 NCB columns:
//   O^T = b (.) S^T Q^T  +  V^T A^T, scaled and stored as bf16.
//
// sop(p, cb) is the S^T operand of k-step p (features 32p .. 32p+31) for
// column block cb: this wave's state block (16 rows) paired with the partner's,
// rows 32p + 4g + r from the h = 0 wave, rows 32p + 16 + 4g + r from h = 1.
// `pws[x + 1]` = scale * lam^x and the score blocks already carry `scale`.
template <int C, int LDK, int NCB, int K, typename SopF, typename EmitF>
__device__ __forceinline__ void out_strip(const bf16* Qs, const bf16* As, SopF sop, const bf16x8 (&vf)[NCB][C / 32],
                                          const float* pws, int n, int g, EmitF emit) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        f32x4 OT[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) OT[cb] = zero4();
#pragma unroll
        for (int p = 0; p < kDK / 32; ++p) {
            const bf16x8 q0 = op_row_pair(Qs, LDK, 32 * K + 16 * u + n, 32 * p + 4 * g);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) OT[cb] = mfma(sop(p, cb), q0, OT[cb]);
        }
        const float bi = pws[32 * K + 16 * u + n + 2];  // scale * lam^(i+1), i = 16 (2K + u) + n
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) OT[cb][r] *= bi;
        const int ib = 2 * K + u;
#pragma unroll
        for (int p = 0; p <= K; ++p) {
            const int jb = 2 * p + (g >> 1);
            bf16x8 aop = bf16x8{};
            if (p < K || u == 1 || jb <= ib)
                aop = *reinterpret_cast<const bf16x8*>(As + (ib * (ib + 1) / 2 + jb) * 256 + as_off(n, g & 1));
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) OT[cb] = mfma(vf[cb][p], aop, OT[cb]);
        }
        emit(u, 32 * K + 16 * u + n, OT);
    }
}

// Output strip K stored as bf16: row irow, columns colbase + 16 cb + 4 g + r.
template <int C, int LDK, int NCB, int K, typename SopF>
__device__ __forceinline__ void out_pair(const bf16* Qs, const bf16* As, SopF sop, const bf16x8 (&vf)[NCB][C / 32],
                                         const float* pws, bf16* ob, size_t tokO, int t0, int ceff, int colbase,
                                         int n, int g) {
    out_strip<C, LDK, NCB, K>(Qs, As, sop, vf, pws, n, g, [&](int, int irow, const f32x4(&OT)[NCB]) {
        if (irow < ceff) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                store4<bf16>(ob + (size_t)(t0 + irow) * tokO + colbase + cb * 16 + 4 * g, OT[cb]);
        }
    });
}

template <int C, int LDK, int NCB, bool SO>
__global__ __launch_bounds__((F8<C, LDK, NCB>::NT), 1) void fwd_bf16_kernel(FwdArgs a) {
    using L = F8<C, LDK, NCB>;
    constexpr int NT = L::NT, NP = L::NP, NIB = L::NIB, LDV = L::LDV, NCG = L::NCG;

    __shared__ __align__(16) bf16 Qs[SO ? 8 : C * LDK];
    __shared__ __align__(16) bf16 Ks[C * LDK];
    __shared__ __align__(16) bf16 Vs[C * LDV];
    __shared__ __align__(16) unsigned char XA[SO ? 16 : L::XA_BYTES];
    __shared__ __align__(16) float cj[2][C];  // c_j = lam^(C-1-j); for the partial last chunk lam^(ceff-1-j) or 0
    __shared__ float pws[C + 2];              // pws[0] = 0, pws[x + 1] = scale * lam^x (x = 0..C)
    __shared__ float lamv[2];                 // lam^C, lam^(length of a partial last chunk)

    const int tid = threadIdx.x;
    // The wave index is wave-uniform: kept in scalar registers, so everything
    // derived from it (column base, score-block slots) is scalar too.
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, n = lane % 16, g = lane / 16;
    const int h = wave / NCG, colbase = 16 * NCB * (wave % NCG);
    const int partner = h == 0 ? wave + NCG : wave - NCG;
    const int seg = blockIdx.x, bh = blockIdx.y;
    const int H = a.H, T = a.T;
    const int hd = bh % H, b = bh / H;
    const int c_begin = seg * a.seg_chunks;
    const int c_end = min(a.nc, c_begin + a.seg_chunks);

    const int tokQ = a.sq.t, tokK = a.sk.t, tokV = a.sv.t, tokO = a.so.t;
    const bf16* qb = static_cast<const bf16*>(a.q) + b * a.sq.b + hd * kDK;
    const bf16* kb = static_cast<const bf16*>(a.k) + b * a.sk.b + hd * kDK;
    const bf16* vb = static_cast<const bf16*>(a.v) + b * a.sv.b + hd * kDV;
    bf16* ob = static_cast<bf16*>(a.o) + b * a.so.b + hd * kDV;

    // This wave's score blocks (scalar): query strips sa (slot 0) and sb (last slot).
    constexpr int NS = L::NSLOT;
    int blk[NS];
    score_blocks_uniform<C, L::NW>(wave, blk, std::make_integer_sequence<int, NS>{});
    const int sa = blk[0] >= 0 ? blk[0] >> 4 : 0;
    int sb = sa;
#pragma unroll
    for (int k = 0; k < NS; ++k)
        if (blk[k] >= 0) sb = blk[k] >> 4;
    constexpr int NA = score_lead<C, L::NW>();
    bool use_b[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) use_b[k] = k >= NA && blk[k] >= 0 && (blk[k] >> 4) != sa;

    // Sacc[i][cb][r] = S[16 (2i + h) + 4g + r][colbase + 16 cb + n].  Segment
    // states in the workspace are kept in this register order ("fragment
    // order": float4 ((wave * 3 + i) * NCB + cb) * 64 + lane holds Sacc[i][cb]),
    // so they move as 16-byte (fp32) or 8-byte (bf16) pieces.
    f32x4 Sacc[3][NCB];
    auto sidx = [&](int i, int cb, int r) -> int {
        return (16 * (2 * i + h) + 4 * g + r) * kDV + colbase + cb * 16 + n;
    };
    auto fidx = [&](int i, int cb) -> int { return ((wave * 3 + i) * NCB + cb) * 64 + lane; };
    // The start state is consumed only in the chunk loop (its bf16 copy for the
    // partner wave): its loads stay in flight until then (no conversion here, no
    // select on the loaded values; it is requested before the tiles, so a wait
    // for it never waits for a tile).  Packed bf16 start states are unpacked there.
    bool sin_packed = false;
    if constexpr (!SO) {
        if (seg == 0) {
            // S0 through a buffer descriptor whose range is empty without S0:
            // the loads then return zeros.
            const float* s0 = a.S0 ? a.S0 + (size_t)bh * kDK * kDV : a.lambda;
            const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(s0), 0,
                                                              a.S0 ? kDK * kDV * 4 : 0, kBufWord3);
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Sacc[i][cb][r] = __builtin_bit_cast(
                            float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * sidx(i, cb, r), 0, 0));
        } else if (a.fuse_scan) {
            // Fold the prologue's local states of sub-segments 0 .. seg*psub-1 into the
            // start state from S0 (or 0), in the scan kernel's order: the same bits.
            const float* s0 = a.S0 ? a.S0 + (size_t)bh * kDK * kDV : a.lambda;
            const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(s0), 0,
                                                              a.S0 ? kDK * kDV * 4 : 0, kBufWord3);
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Sacc[i][cb][r] = __builtin_bit_cast(
                            float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * sidx(i, cb, r), 0, 0));
            const float lamL = pow_int(a.lambda[hd], a.seg_chunks / a.psub * C);
            const f32x4* u = reinterpret_cast<const f32x4*>(a.U + (size_t)bh * (a.nseg - 1) * a.psub * kDK * kDV);
            for (int j = 0; j < seg * a.psub; ++j) {
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        const f32x4 x = u[(size_t)j * (kDK * kDV / 4) + fidx(i, cb)];
#pragma unroll
                        for (int e = 0; e < 4; ++e) Sacc[i][cb][e] = fmaf(lamL, Sacc[i][cb][e], x[e]);
                    }
            }
        } else {
            // (the scanned state at the segment's start: sub-segment boundary seg * psub)
            const size_t st = ((size_t)bh * (a.nseg - 1) * a.psub + (seg * a.psub - 1)) * kDK * kDV;
            // A one-chunk segment only reads its start state as a bf16 MFMA
            // operand, unless it must also produce the final state.  The four
            // bf16 values stay packed in the first two registers for now.
            if (a.seg_chunks == 1 && !(seg == a.nseg - 1 && a.S_final)) {
                const uint2* ub = reinterpret_cast<const uint2*>(static_cast<const bf16*>(a.Ub) + st);
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        const uint2 x = ub[fidx(i, cb)];
                        Sacc[i][cb] = f32x4{__builtin_bit_cast(float, x.x), __builtin_bit_cast(float, x.y), 0.f, 0.f};
                    }
                sin_packed = true;
            } else {
                const f32x4* u = reinterpret_cast<const f32x4*>(a.U + st);
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) Sacc[i][cb] = u[fidx(i, cb)];
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) Sacc[i][cb] = zero4();
    }

    // The first chunk's tiles, right after the start state.
    using StageK = std::conditional_t<NT % (kDK / 8) == 0, RowStage<C, kDK, NT>, BufStage<C, kDK, NT>>;
    using StageV = std::conditional_t<NT % (kDV / 8) == 0, RowStage<C, kDV, NT>, BufStage<C, kDV, NT>>;
    StageK tq, tk;
    StageV tv;
    // Tiles of the chunk at token t, rows [0, valid) read.
    auto load_chunk = [&](int t, int valid, int tid) {
        if constexpr (!SO) tq.load(qb + (size_t)t * tokQ, tokQ, valid, tid);
        tk.load(kb + (size_t)t * tokK, tokK, valid, tid);
        tv.load(vb + (size_t)t * tokV, tokV, valid, tid);
    };
    if (c_begin < c_end) load_chunk(c_begin * C, T - c_begin * C, tid);

    const float lam = a.lambda[hd];
    if (tid < C + 2) pws[tid] = tid == 0 ? 0.f : a.scale * pow_int(lam, tid - 1);
    const int ctail = T % C;  // length of a partial last chunk (0: none)
    if (tid < C) {
        cj[0][tid] = pow_int(lam, C - 1 - tid);
        cj[1][tid] = tid < ctail ? pow_int(lam, ctail - 1 - tid) : 0.f;
    }
    // Chunk decay read from LDS at its use (a register copy held across the loop
    // gets spilled, and its reload would wait behind the in-flight tile loads).
    if (tid < 2) lamv[tid] = pow_int(lam, tid == 0 ? C : ctail);

    bf16x4* XS = reinterpret_cast<bf16x4*>(XA);
    bf16* As = reinterpret_cast<bf16*>(XA + L::AS_OFF);

    for (int c = c_begin; c < c_end; ++c) {
        // Lane-derived addresses are recomputed every chunk from an opaque copy
        // of the thread index instead of being kept live across the loop.
        int tid_v = threadIdx.x;
        asm volatile("" : "+v"(tid_v));
        const int tid = tid_v, lane = tid % 64, n = lane % 16, g = lane / 16;
        auto xs_at = [&](int w, int i, int cb) { return XS + ((w * 3 + i) * NCB + cb) * 64 + lane; };
        const int t0 = c * C;
        const int ceff = min(C, T - t0);
        const float* cjc = cj[ceff == C ? 0 : 1];
        const bool need_state = SO || c + 1 < c_end || (seg == a.nseg - 1 && a.S_final != nullptr);
        __syncthreads();  // the previous chunk's LDS reads are done
        if constexpr (!SO) {
            tq.template store<LDK>(Qs, tid);
            tk.template store<LDK>(Ks, tid);
            tv.template store<LDV>(Vs, tid);
            if (sin_packed) {  // first chunk only: bf16 start state -> fp32 (exact)
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        // (element values taken first: a bit cast applied to a vector
                        // element itself reads element 0 with this compiler)
                        const float fx = Sacc[i][cb][0], fy = Sacc[i][cb][1];
                        const unsigned x = __builtin_bit_cast(unsigned, fx);
                        const unsigned y = __builtin_bit_cast(unsigned, fy);
                        Sacc[i][cb] = f32x4{__builtin_bit_cast(float, x << 16), __builtin_bit_cast(float, x & 0xffff0000u),
                                            __builtin_bit_cast(float, y << 16), __builtin_bit_cast(float, y & 0xffff0000u)};
                    }
                sin_packed = false;
            }
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    *xs_at(wave, i, cb) = bf16x4{to_bf16(Sacc[i][cb][0]), to_bf16(Sacc[i][cb][1]),
                                                 to_bf16(Sacc[i][cb][2]), to_bf16(Sacc[i][cb][3])};
            if (a.sbar) {  // the chunk's start state, for the backward (row-major, bf16)
                bf16* sb = static_cast<bf16*>(a.sbar) + ((size_t)bh * a.nc + c) * kDK * kDV;
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                        for (int r = 0; r < 4; ++r)   // (this chunk's lane-derived n, g)
                            sb[(16 * (2 * i + h) + 4 * g + r) * kDV + colbase + 16 * cb + n] = to_bf16(Sacc[i][cb][r]);
            }
        } else {
            // state only: keys are needed only scaled, K^T diag(c)
            tk.template store_scaled<LDK>(Ks, tid, [&](int row) { return cjc[row]; });
            tv.template store<LDV>(Vs, tid);
        }
        __syncthreads();
        if (c + 1 < c_end) load_chunk(t0 + C, T - (t0 + C), tid);  // next chunk's tiles, consumed at its start

        // This wave's value fragments: vf[cb][p] = V[32p + 8g + e][colbase + 16cb + n]
        // (loaded after the score blocks, which do not need them).
        bf16x8 vf[NCB][NP];
        auto load_vf = [&]() {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int p = 0; p < NP; ++p) vf[cb][p] = op_col8(Vs, LDV, 32 * p, colbase + 16 * cb, n, g);
        };
        if constexpr (SO) load_vf();

        if constexpr (!SO) {
            score_blocks_to_lds<C, LDK, L::NW, NS>(Qs, Ks, As, pws, blk, sa, sb, use_b, n, g);
            load_vf();
            __syncthreads();  // score blocks complete

            // The keys are only needed scaled now, K^T diag(c) for the state
            // update: scaled in place (complete at the barrier before the update).
            for (int pc = tid; need_state && pc < C * (kDK / 8); pc += NT) {
                const int row = pc / (kDK / 8), col = (pc % (kDK / 8)) * 8;
                uint4* kp = reinterpret_cast<uint4*>(Ks + row * LDK + col);
                *kp = scale_bf16x8(*kp, cjc[row]);
            }

            // S^T operands: own half from the accumulators, the partner's from its
            // published copy
            const bf16x4* xo = xs_at(partner, 0, 0);
            auto sop = [&](int p, int cb) -> bf16x8 {
                const bf16x4 own = bf16x4{to_bf16(Sacc[p][cb][0]), to_bf16(Sacc[p][cb][1]), to_bf16(Sacc[p][cb][2]),
                                          to_bf16(Sacc[p][cb][3])};
                const bf16x4 oth = xo[(p * NCB + cb) * 64];
                return h == 0 ? __builtin_shufflevector(own, oth, 0, 1, 2, 3, 4, 5, 6, 7)
                              : __builtin_shufflevector(oth, own, 0, 1, 2, 3, 4, 5, 6, 7);
            };
            if constexpr (C == 128) {
                if (h == 0) {
                    out_pair<C, LDK, NCB, 0>(Qs, As, sop, vf, pws, ob, tokO, t0, ceff, colbase, n, g);
                    out_pair<C, LDK, NCB, 3>(Qs, As, sop, vf, pws, ob, tokO, t0, ceff, colbase, n, g);
                } else {
                    out_pair<C, LDK, NCB, 1>(Qs, As, sop, vf, pws, ob, tokO, t0, ceff, colbase, n, g);
                    out_pair<C, LDK, NCB, 2>(Qs, As, sop, vf, pws, ob, tokO, t0, ceff, colbase, n, g);
                }
            } else if constexpr (C == 64) {
                if (h == 0) out_pair<C, LDK, NCB, 0>(Qs, As, sop, vf, pws, ob, tokO, t0, ceff, colbase, n, g);
                else out_pair<C, LDK, NCB, 1>(Qs, As, sop, vf, pws, ob, tokO, t0, ceff, colbase, n, g);
            } else {
                // one 32-row strip: the h = 0 wave of each pair writes it
                if (h == 0) out_pair<C, LDK, NCB, 0>(Qs, As, sop, vf, pws, ob, tokO, t0, ceff, colbase, n, g);
            }
        }

        // State advance: S <- lam^ceff S + (diag(c) K)^T V, with the scaled keys
        // in the key tile.
        // The state after a segment's last chunk is needed only by the sequence's
        // last segment (S_final); other segments hand over through the scan.
        if (!need_state) continue;
        if constexpr (!SO) __syncthreads();  // scaled keys complete
        const bf16* Ksc = Ks;
        const float Lam = lamv[ceff == C ? 0 : 1];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) Sacc[i][cb][r] *= Lam;
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                const bf16x8 kop = op_col8(Ksc, LDK, 32 * p, 16 * (2 * i + h), n, g);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) Sacc[i][cb] = mfma(kop, vf[cb][p], Sacc[i][cb]);
            }
    }

    if (SO) {
        // segment-local end state, fragment order
        f32x4* u = reinterpret_cast<f32x4*>(a.U + ((size_t)bh * (a.nseg - 1) + seg) * kDK * kDV);
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) u[fidx(i, cb)] = Sacc[i][cb];
    } else if (seg == a.nseg - 1 && a.S_final) {
        float* dst = a.S_final + (size_t)bh * kDK * kDV;
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[sidx(i, cb, r)] = Sacc[i][cb][r];
    }
}

// Segment scan over fragment-ordered states:  U[s] <- lam^L U[s-1] + U[s]
// (U[-1] = S0), i.e. the start state of segment s + 1, as in the fp32 path's
// scan.  One thread per float4 of the state.  One-chunk segments need their
// start state only as bf16 (written to Ub); fp32 is kept where a segment runs
// a state chain (several chunks) or produces the final state (the last one).
template <int NCB>
__global__ __launch_bounds__(256) void seg_scan_frag_kernel(const float* __restrict__ S0, float* __restrict__ U,
                                                            bf16* __restrict__ Ub, const float* __restrict__ lambda,
                                                            int H, int nseg, int seg_chunks, int seg_tokens,
                                                            int last_f32) {
    constexpr int NCG = kDV / (16 * NCB), NF = kDK * kDV / 4;
    const int bh = blockIdx.y;
    const int f = blockIdx.x * blockDim.x + threadIdx.x;
    if (f >= NF) return;
    const float lamL = pow_int(lambda[bh % H], seg_tokens);
    f32x4 run = zero4();
    if (S0) {
        const int lane = f % 64, rest = f / 64;
        const int cb = rest % NCB, i = (rest / NCB) % 3, wave = rest / (3 * NCB);
        const int h = wave / NCG, col = 16 * NCB * (wave % NCG) + 16 * cb + lane % 16;
        const float* s0 = S0 + (size_t)bh * kDK * kDV + (16 * (2 * i + h) + 4 * (lane / 16)) * kDV + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) run[r] = s0[r * kDV];
    }
    f32x4* u = reinterpret_cast<f32x4*>(U + (size_t)bh * (nseg - 1) * kDK * kDV) + f;
    bf16x4* ub = reinterpret_cast<bf16x4*>(Ub + (size_t)bh * (nseg - 1) * kDK * kDV) + f;
    f32x4 x[kMaxSegments - 1];
#pragma unroll
    for (int s = 0; s < kMaxSegments - 1; ++s)
        if (s < nseg - 1) x[s] = u[s * NF];
#pragma unroll
    for (int s = 0; s < kMaxSegments - 1; ++s) {
        if (s < nseg - 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) run[e] = fmaf(lamL, run[e], x[s][e]);
            if (seg_chunks > 1 || (last_f32 && s == nseg - 2)) u[s * NF] = run;
            if (seg_chunks == 1) ub[s * NF] = bf16x4{to_bf16(run[0]), to_bf16(run[1]), to_bf16(run[2]), to_bf16(run[3])};
        }
    }
}


// Output of one chunk from its start state, a bf16 snapshot in register order
// written by the tiled chain (snapshot bh * nc + c of a.Ub):
//     O_c = scale * ( (Q K^T (.) D) V  +  diag(b) Q S ).
// One workgroup per (chunk, unit), laid out like the main kernel, without the
// state update and without the pair exchange: both halves of a wave pair's
// S^T operand come straight from the snapshot.  q and k are staged first, so
// the score blocks overlap the arrival of the values and the start state.
template <int C, int LDK, int NCB, bool EPI>
__global__ __launch_bounds__((F8<C, LDK, NCB>::NT), 1) void fwd_out_kernel(FwdArgs a, EpilogueArgs ep) {
    using L = F8<C, LDK, NCB>;
    constexpr int NT = L::NT, NP = L::NP, LDV = L::LDV, NCG = L::NCG;
    __shared__ __align__(16) bf16 Qs[C * LDK];
    __shared__ __align__(16) bf16 Ks[C * LDK];
    __shared__ __align__(16) bf16 Vs[C * LDV];
    __shared__ __align__(16) bf16 As[L::AS_BYTES / 2];
    __shared__ float pws[C + 2];  // pws[0] = 0, pws[x + 1] = scale * lam^x (x = 0..C)
    // epilogue: the head's self-augmentation vector, each row's gate, and each
    // row's partial sums of squares from the NCG column groups
    __shared__ float augs[EPI ? kDK : 1];
    __shared__ float sg[EPI ? C : 1];
    __shared__ float red[EPI ? C * NCG : 1];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, n = lane % 16, g = lane / 16;
    const int h = wave / NCG, colbase = 16 * NCB * (wave % NCG);
    const int partner = h == 0 ? wave + NCG : wave - NCG;
    // (chunk, unit) from the dispatch order (workgroup i runs on XCD i mod 8).
    // With out_xcd, every chunk of unit u runs on XCD u mod 8, where the tiled
    // chain walked that unit, so its k, v and chunk start states come from that
    // XCD's L2 (the launcher sets it when those fit there); else chunk-major.
    int c, bh;
    if (a.out_xcd) {
        const int jx = blockIdx.x / 8;
        bh = (jx / a.nc) * 8 + blockIdx.x % 8;
        c = jx % a.nc;
    } else {
        c = blockIdx.x % a.nc;
        bh = blockIdx.x / a.nc;
    }
    if (bh >= a.units) return;  // (whole workgroup, before any barrier)
    const int H = a.H, T = a.T;
    const int hd = bh % H, b = bh / H;
    const int t0 = c * C, ceff = min(C, T - t0);
    const int tokQ = a.sq.t, tokK = a.sk.t, tokV = a.sv.t, tokO = a.so.t;
    const bf16* qb = static_cast<const bf16*>(a.q) + b * a.sq.b + (size_t)t0 * tokQ + hd * kDK;
    const bf16* kb = static_cast<const bf16*>(a.k) + b * a.sk.b + (size_t)t0 * tokK + hd * kDK;
    const bf16* vb = static_cast<const bf16*>(a.v) + b * a.sv.b + (size_t)t0 * tokV + hd * kDV;
    bf16* ob = static_cast<bf16*>(a.o) + b * a.so.b + hd * kDV;

    constexpr int NS = L::NSLOT;
    int blk[NS];
    score_blocks_uniform<C, L::NW>(wave, blk, std::make_integer_sequence<int, NS>{});
    const int sa = blk[0] >= 0 ? blk[0] >> 4 : 0;
    int sb = sa;
#pragma unroll
    for (int k = 0; k < NS; ++k)
        if (blk[k] >= 0) sb = blk[k] >> 4;
    constexpr int NA = score_lead<C, L::NW>();
    bool use_b[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) use_b[k] = k >= NA && blk[k] >= 0 && (blk[k] >> 4) != sa;

    using StageK = std::conditional_t<NT % (kDK / 8) == 0, RowStage<C, kDK, NT>, BufStage<C, kDK, NT>>;
    using StageV = std::conditional_t<NT % (kDV / 8) == 0, RowStage<C, kDV, NT>, BufStage<C, kDV, NT>>;
    // (epilogue) the augmentation vector is requested before the tiles, so
    // that waiting for it waits for no tile
    float augv = 0.f;
    if constexpr (EPI)
        if (ep.aug_a && tid < kDK) augv = ep.aug_a[(size_t)hd * kDK + tid];
    StageK tq, tk;
    StageV tv;
    tq.load(qb, tokQ, ceff, tid);
    tk.load(kb, tokK, ceff, tid);
    tv.load(vb, tokV, ceff, tid);
    // start state: this wave's half and the partner's, 4 bf16 per block and lane
    const uint2* sn = reinterpret_cast<const uint2*>(static_cast<const bf16*>(a.Ub) + ((size_t)bh * a.nc + c) * kDK * kDV);
    uint2 so[3][NCB], sp[3][NCB];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            so[i][cb] = sn[((wave * 3 + i) * NCB + cb) * 64 + lane];
            sp[i][cb] = sn[((partner * 3 + i) * NCB + cb) * 64 + lane];
        }
    // (epilogue) the output gate of this lane's rows and the tier's norm
    // weights of its columns, requested last: they are used last
    constexpr int NSTRIP = C == 128 ? 2 : 1;
    uint2 gq[NSTRIP][2][NCB];
    f32x4 wn[NCB];
    if constexpr (EPI) {
        const int tokG = ep.sg.t;
        const bf16* gb = static_cast<const bf16*>(ep.g) + b * ep.sg.b + (size_t)t0 * tokG + hd * kDV;  // row t0
        const auto rg = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(gb), 0,
                                                          __builtin_amdgcn_readfirstlane(ceff * tokG * 2), kBufWord3);
#pragma unroll
        for (int j = 0; j < NSTRIP; ++j)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const int K = C == 128 ? (h == 0 ? 3 * j : 1 + j) : h;
                    const int irow = 32 * K + 16 * u + n;
                    gq[j][u][cb] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                                 rg, (irow * tokG + colbase + 16 * cb + 4 * g) * 2, 0, 0));
                }
        const float* wt = ep.norm_w + (size_t)ep.tier[hd] * kDV + colbase + 4 * g;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) wn[cb] = *reinterpret_cast<const f32x4*>(wt + 16 * cb);
    }

    const float lam = a.lambda[hd];
    if (tid < C + 2) pws[tid] = tid == 0 ? 0.f : a.scale * pow_int(lam, tid - 1);
    if constexpr (EPI)
        if (tid < kDK) augs[tid] = augv;

    tq.template store<LDK>(Qs, tid);
    tk.template store<LDK>(Ks, tid);
    __syncthreads();  // q, k, decay table
    if constexpr (EPI) {
        // gate of row tid: sigmoid(q . (a (.) k)) with the raw q and k
        if (tid < C) {
            float z = 0.f;
#pragma unroll
            for (int i8 = 0; i8 < kDK; i8 += 8) {
                const bf16x8 qv = *reinterpret_cast<const bf16x8*>(Qs + tid * LDK + i8);
                const bf16x8 kv = *reinterpret_cast<const bf16x8*>(Ks + tid * LDK + i8);
#pragma unroll
                for (int e = 0; e < 8; ++e) z += to_f32(qv[e]) * augs[i8 + e] * to_f32(kv[e]);
            }
            sg[tid] = fast_sigmoid(z);
        }
    }
    score_blocks_to_lds<C, LDK, L::NW, NS>(Qs, Ks, As, pws, blk, sa, sb, use_b, n, g);
    tv.template store<LDV>(Vs, tid);
    __syncthreads();  // score blocks, values (and the gates)

    bf16x8 vf[NCB][NP];  // vf[cb][p] = V[32p + 8g + e][colbase + 16cb + n]
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int p = 0; p < NP; ++p) vf[cb][p] = op_col8(Vs, LDV, 32 * p, colbase + 16 * cb, n, g);
    auto sop = [&](int p, int cb) -> bf16x8 {
        const bf16x4 own = __builtin_bit_cast(bf16x4, so[p][cb]);
        const bf16x4 oth = __builtin_bit_cast(bf16x4, sp[p][cb]);
        return h == 0 ? __builtin_shufflevector(own, oth, 0, 1, 2, 3, 4, 5, 6, 7)
                      : __builtin_shufflevector(oth, own, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    if constexpr (!EPI) {
        if constexpr (C == 128) {
            // o staged row-major in the value tile (free once every wave holds its
            // value fragments), then written as whole 384-byte rows with non-temporal
            // stores (23.39 against 24.94 us per Laplace-layer call with each lane's
            // 8-byte pieces stored directly; the same bits)
            __syncthreads();   // every wave's value fragments are read
            bf16* Os = Vs;
            auto stage = [&](int, int irow, const f32x4(&OT)[NCB]) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    *reinterpret_cast<bf16x4*>(Os + irow * LDV + colbase + 16 * cb + 4 * g) =
                        bf16x4{to_bf16(OT[cb][0]), to_bf16(OT[cb][1]), to_bf16(OT[cb][2]), to_bf16(OT[cb][3])};
            };
            if (h == 0) {
                out_strip<C, LDK, NCB, 0>(Qs, As, sop, vf, pws, n, g, stage);
                out_strip<C, LDK, NCB, 3>(Qs, As, sop, vf, pws, n, g, stage);
            } else {
                out_strip<C, LDK, NCB, 1>(Qs, As, sop, vf, pws, n, g, stage);
                out_strip<C, LDK, NCB, 2>(Qs, As, sop, vf, pws, n, g, stage);
            }
            __syncthreads();   // o complete in LDS
            const auto ro = __builtin_amdgcn_make_buffer_rsrc(ob + (size_t)t0 * tokO, 0,
                                                              __builtin_amdgcn_readfirstlane(ceff * (int)tokO * 2), kBufWord3);
            constexpr int KCO = kDV / 8;   // 16-byte pieces per row
#pragma unroll
            for (int k = 0; k < (C * KCO + NT - 1) / NT; ++k) {
                const int pc = tid + k * NT;
                if ((C * KCO) % NT != 0 && pc >= C * KCO) break;
                const int row = pc / KCO, col = (pc % KCO) * 8;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, *reinterpret_cast<const bf16x8*>(Os + row * LDV + col)),
                                                       ro, (row * (int)tokO + col) * 2, 0, kCpolNT);
            }
        } else {
            if (h == 0) out_pair<C, LDK, NCB, 0>(Qs, As, sop, vf, pws, ob, tokO, t0, ceff, colbase, n, g);
            else out_pair<C, LDK, NCB, 1>(Qs, As, sop, vf, pws, ob, tokO, t0, ceff, colbase, n, g);
        }
        if (a.sbar) {
            // the chunk's start state for the backward, row-major: this wave's
            // half (16-row blocks 2i + h), columns colbase + 16 cb + n
            bf16* sb = static_cast<bf16*>(a.sbar) + ((size_t)bh * a.nc + c) * kDK * kDV;
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const bf16x4 s4 = __builtin_bit_cast(bf16x4, so[i][cb]);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sb[(size_t)(16 * (2 * i + h) + 4 * g + r) * kDV + colbase + 16 * cb + n] = s4[r];
                }
        }
    } else {
        // Epilogue: x = o + s v per row; each row's sum of squares is spread
        // over the NCG column groups of the waves that own the row's strip, so
        // it goes through LDS; then y = silu(g) x / sqrt(mean x^2 + eps) w.
        const int cgp = wave % NCG;
        f32x4 X[NSTRIP][2][NCB];
        auto collect = [&](int j) {
            return [&, j](int u, int irow, const f32x4(&OT)[NCB]) {
                const float sv = sg[irow];
                float ss = 0.f;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const bf16x4 v4 = *reinterpret_cast<const bf16x4*>(Vs + irow * LDV + colbase + 16 * cb + 4 * g);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        X[j][u][cb][r] = fmaf(sv, to_f32(v4[r]), OT[cb][r]);
                        ss = fmaf(X[j][u][cb][r], X[j][u][cb][r], ss);
                    }
                }
                ss += __shfl_xor(ss, 16, 64);   // the four lanes of row irow
                ss += __shfl_xor(ss, 32, 64);
                if (g == 0) red[irow * NCG + cgp] = ss;
            };
        };
        if constexpr (C == 128) {
            if (h == 0) {
                out_strip<C, LDK, NCB, 0>(Qs, As, sop, vf, pws, n, g, collect(0));
                out_strip<C, LDK, NCB, 3>(Qs, As, sop, vf, pws, n, g, collect(1));
            } else {
                out_strip<C, LDK, NCB, 1>(Qs, As, sop, vf, pws, n, g, collect(0));
                out_strip<C, LDK, NCB, 2>(Qs, As, sop, vf, pws, n, g, collect(1));
            }
        } else {
            if (h == 0) out_strip<C, LDK, NCB, 0>(Qs, As, sop, vf, pws, n, g, collect(0));
            else out_strip<C, LDK, NCB, 1>(Qs, As, sop, vf, pws, n, g, collect(0));
        }
        __syncthreads();  // every row's partial sums of squares
#pragma unroll
        for (int j = 0; j < NSTRIP; ++j)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int K = C == 128 ? (h == 0 ? 3 * j : 1 + j) : h;
                const int irow = 32 * K + 16 * u + n;
                float tot = 0.f;
#pragma unroll
                for (int q = 0; q < NCG; ++q) tot += red[irow * NCG + q];
                const float inv = __builtin_amdgcn_rsqf(tot * (1.f / kDV) + ep.eps);
                if (irow < ceff) {
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        const bf16x4 g4 = __builtin_bit_cast(bf16x4, gq[j][u][cb]);
                        f32x4 y;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float gc = to_f32(g4[r]);
                            y[r] = gc * fast_sigmoid(gc) * X[j][u][cb][r] * inv * wn[cb][r];
                        }
                        store4<bf16>(ob + (size_t)(t0 + irow) * tokO + colbase + cb * 16 + 4 * g, y);
                    }
                }
            }
    }
}

// Output of one 256-token chunk from its start state (the tiled chain's bf16
// snapshot), as two workgroups per (chunk, unit): the chunk's 256 x 256
// decay-masked score matrix does not fit LDS (the q, k, v tiles alone would
// take ~208 KB), so each workgroup takes 128 query rows.
//   half 0 (rows 0..127): exactly the 128-token output kernel's work on the
//            chunk's first 128 tokens (same b_i, D_ij and start state);
//   half 1 (rows 128..255): b (.) Q1 S plus the intra-chunk term over all 256
//            keys: the cross block (Q1 K0^T) (.) D, a full 8 x 8 grid of 16x16
//            score blocks with D_ij = lam^(i-j) for i - j in [1, 255], and
//            the lower triangle (Q1 K1^T) (.) D as in the 128-token kernel.
//            The 100 score blocks go to LDS in bf16; then V0 and V1 pass in
//            turn through the space the keys took, each wave keeping its value
//            fragments of both halves in registers for the output strips.
// With a.sbar, the half-0 workgroup also stores the chunk's start state
// (row-major, bf16) for the backward.
// Grid (2 nc, units): blockIdx.x = half * nc + chunk.
template <int LDK, int NCB>
__global__ __launch_bounds__((F8<128, LDK, NCB>::NT), 1) void fwd_out256_kernel(FwdArgs a) {
    constexpr int C = 256, R = 128;
    using L = F8<R, LDK, NCB>;
    constexpr int NT = L::NT, NP = L::NP, LDV = L::LDV, NCG = L::NCG;
    constexpr int NCROSS = 64, NDIAG = L::NTRI, NBLK = NCROSS + NDIAG;  // half 1's score blocks
    // half 0: Q | K | V | 36 score blocks;  half 1: Q1 | K0 K1 (then V0, then V1) | 100 score blocks
    constexpr int SM = R * LDK + 2 * R * LDK + NBLK * 256;
    static_assert(2 * R * LDK + R * LDV + NDIAG * 256 <= SM && R * LDV <= 2 * R * LDK, "LDS carve-up");
    __shared__ __align__(16) bf16 sm[SM];
    __shared__ float pws[C + 2];  // pws[0] = 0, pws[x + 1] = scale * lam^x (x = 0..C)

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, n = lane % 16, g = lane / 16;
    const int h = wave / NCG, colbase = 16 * NCB * (wave % NCG);
    const int partner = h == 0 ? wave + NCG : wave - NCG;
    const int half = blockIdx.x / a.nc, c = blockIdx.x % a.nc, bh = blockIdx.y;
    const int H = a.H, T = a.T;
    const int hd = bh % H, b = bh / H;
    const int t0 = c * C + half * R;            // first token of this workgroup's rows
    const int ceff = min(R, T - t0);            // its rows (<= 0: none)
    if (ceff <= 0) return;                      // (whole workgroup)
    const int tokQ = a.sq.t, tokK = a.sk.t, tokV = a.sv.t, tokO = a.so.t;
    const bf16* qb = static_cast<const bf16*>(a.q) + b * a.sq.b + (size_t)t0 * tokQ + hd * kDK;
    const bf16* kb = static_cast<const bf16*>(a.k) + b * a.sk.b + (size_t)(c * C) * tokK + hd * kDK;  // chunk row 0
    const bf16* vb = static_cast<const bf16*>(a.v) + b * a.sv.b + (size_t)(c * C) * tokV + hd * kDV;
    bf16* ob = static_cast<bf16*>(a.o) + b * a.so.b + hd * kDV;

    using StageK = RowStage<R, kDK, NT>;
    using StageV = RowStage<R, kDV, NT>;
    static_assert(NT % (kDK / 8) == 0 && NT % (kDV / 8) == 0, "row staging");
    // start state: this wave's half and the partner's, 4 bf16 per block and lane
    const uint2* sn = reinterpret_cast<const uint2*>(static_cast<const bf16*>(a.Ub) + ((size_t)bh * a.nc + c) * kDK * kDV);
    uint2 so[3][NCB], sp[3][NCB];
    auto sop = [&](int p, int cb) -> bf16x8 {
        const bf16x4 own = __builtin_bit_cast(bf16x4, so[p][cb]);
        const bf16x4 oth = __builtin_bit_cast(bf16x4, sp[p][cb]);
        return h == 0 ? __builtin_shufflevector(own, oth, 0, 1, 2, 3, 4, 5, 6, 7)
                      : __builtin_shufflevector(oth, own, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    const float lam = a.lambda[hd];

    if (half == 0) {
        // --------------------------------- rows 0..127: the 128-token kernel's work
        bf16* Qs = sm;
        bf16* Ks = sm + R * LDK;
        bf16* Vs = sm + 2 * R * LDK;
        bf16* As = Vs + R * LDV;
        constexpr int NS = L::NSLOT;
        int blk[NS];
        score_blocks_uniform<R, L::NW>(wave, blk, std::make_integer_sequence<int, NS>{});
        const int sa = blk[0] >= 0 ? blk[0] >> 4 : 0;
        int sb = sa;
#pragma unroll
        for (int k = 0; k < NS; ++k)
            if (blk[k] >= 0) sb = blk[k] >> 4;
        constexpr int NA = score_lead<R, L::NW>();
        bool use_b[NS];
#pragma unroll
        for (int k = 0; k < NS; ++k) use_b[k] = k >= NA && blk[k] >= 0 && (blk[k] >> 4) != sa;
        StageK tq, tk;
        StageV tv;
        tq.load(qb, tokQ, ceff, tid);
        tk.load(kb, tokK, ceff, tid);
        tv.load(vb, tokV, ceff, tid);
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                so[i][cb] = sn[((wave * 3 + i) * NCB + cb) * 64 + lane];
                sp[i][cb] = sn[((partner * 3 + i) * NCB + cb) * 64 + lane];
            }
        if (tid < R + 2) pws[tid] = tid == 0 ? 0.f : a.scale * pow_int(lam, tid - 1);
        tq.template store<LDK>(Qs, tid);
        tk.template store<LDK>(Ks, tid);
        __syncthreads();  // q, k, decay table
        score_blocks_to_lds<R, LDK, L::NW, NS>(Qs, Ks, As, pws, blk, sa, sb, use_b, n, g);
        tv.template store<LDV>(Vs, tid);
        __syncthreads();  // score blocks, values
        bf16x8 vf[NCB][NP];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int p = 0; p < NP; ++p) vf[cb][p] = op_col8(Vs, LDV, 32 * p, colbase + 16 * cb, n, g);
        if (h == 0) {
            out_pair<R, LDK, NCB, 0>(Qs, As, sop, vf, pws, ob, tokO, t0, ceff, colbase, n, g);
            out_pair<R, LDK, NCB, 3>(Qs, As, sop, vf, pws, ob, tokO, t0, ceff, colbase, n, g);
        } else {
            out_pair<R, LDK, NCB, 1>(Qs, As, sop, vf, pws, ob, tokO, t0, ceff, colbase, n, g);
            out_pair<R, LDK, NCB, 2>(Qs, As, sop, vf, pws, ob, tokO, t0, ceff, colbase, n, g);
        }
        if (a.sbar) {
            // the chunk's start state for the backward, row-major: this wave's
            // half (16-row blocks 2i + h), columns colbase + 16 cb + n
            bf16* sbo = static_cast<bf16*>(a.sbar) + ((size_t)bh * a.nc + c) * kDK * kDV;
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const bf16x4 s4 = __builtin_bit_cast(bf16x4, so[i][cb]);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sbo[(size_t)(16 * (2 * i + h) + 4 * g + r) * kDV + colbase + 16 * cb + n] = s4[r];
                }
        }
        return;
    }

    // ------------------------------------------------------- rows 128..255
    bf16* Qs = sm;                  // Q1
    bf16* Kc = sm + R * LDK;        // K0 (rows 0..127), K1 (rows 128..255); then V0, then V1
    bf16* As = sm + 3 * R * LDK;    // cross blocks 0..63 (8 ib + jb), then the triangle of K1
    StageK tq, tk0, tk1;
    StageV tv;
    tq.load(qb, tokQ, ceff, tid);
    tk0.load(kb, tokK, R, tid);
    tk1.load(kb + (size_t)R * tokK, tokK, ceff, tid);
    tv.load(vb, tokV, R, tid);  // V0
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            so[i][cb] = sn[((wave * 3 + i) * NCB + cb) * 64 + lane];
            sp[i][cb] = sn[((partner * 3 + i) * NCB + cb) * 64 + lane];
        }
    for (int i = tid; i < C + 2; i += NT) pws[i] = i == 0 ? 0.f : a.scale * pow_int(lam, i - 1);
    tq.template store<LDK>(Qs, tid);
    tk0.template store<LDK>(Kc, tid);
    tk1.template store<LDK>(Kc + R * LDK, tid);
    __syncthreads();  // q, k, decay table
    // Score blocks: block e < 64 is cross block (ib, jb) = (e / 8, e % 8) of Q1
    // against K0, i - j = 128 + 16 (ib - jb) + ...; block 64 + t is the
    // triangle's block t = ib (ib + 1) / 2 + jb of Q1 against K1.  Wave w takes
    // blocks w, w + NW, ...; AT[4g + r][n] = q_(16 ib + n) . k_(16 jb + 4g + r).
    for (int e = wave; e < NBLK; e += L::NW) {
        int ib, jb, krow, off;
        if (e < NCROSS) {
            ib = e / 8;
            jb = e % 8;
            krow = 16 * jb;
            off = R;
        } else {
            const int t = e - NCROSS;
            ib = 0;
            while ((ib + 1) * (ib + 2) / 2 <= t) ++ib;
            jb = t - ib * (ib + 1) / 2;
            krow = R + 16 * jb;
            off = 0;
        }
        f32x4 at = zero4();
#pragma unroll
        for (int p = 0; p < kDK / 32; ++p)
            at = mfma(op_row8(Kc, LDK, krow + n, 32 * p + 8 * g), op_row8(Qs, LDK, 16 * ib + n, 32 * p + 8 * g), at);
        const int d1 = off + 16 * (ib - jb) + n - 4 * g + 1;
#pragma unroll
        for (int r = 0; r < 4; ++r) at[r] *= pws[max(d1 - r, 0)];
        *reinterpret_cast<bf16x4*>(As + e * 256 + as_off(n, g >> 1) + 4 * (g & 1)) =
            bf16x4{to_bf16(at[0]), to_bf16(at[1]), to_bf16(at[2]), to_bf16(at[3])};
    }
    StageV tv1;
    tv1.load(vb + (size_t)R * tokV, tokV, ceff, tid);
    __syncthreads();  // score blocks done, keys no longer read
    tv.template store<LDV>(Kc, tid);
    __syncthreads();
    bf16x8 vf0[NCB][NP], vf1[NCB][NP];  // vf[cb][p] = V[32p + 8g + e][colbase + 16cb + n]
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int p = 0; p < NP; ++p) vf0[cb][p] = op_col8(Kc, LDV, 32 * p, colbase + 16 * cb, n, g);
    __syncthreads();  // V0 fragments read
    tv1.template store<LDV>(Kc, tid);
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int p = 0; p < NP; ++p) vf1[cb][p] = op_col8(Kc, LDV, 32 * p, colbase + 16 * cb, n, g);

    // Output strips (the 128-token kernel's split: h = 0 takes strips 0 and 3,
    // h = 1 strips 1 and 2), O^T = b (.) S^T Q1^T + V0^T A10^T + V1^T A11^T.
    auto strip = [&](int K) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ib = 2 * K + u;
            f32x4 OT[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) OT[cb] = zero4();
#pragma unroll
            for (int p = 0; p < kDK / 32; ++p) {
                const bf16x8 q0 = op_row_pair(Qs, LDK, 16 * ib + n, 32 * p + 4 * g);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) OT[cb] = mfma(sop(p, cb), q0, OT[cb]);
            }
            const float bi = pws[R + 16 * ib + n + 2];  // scale * lam^(i+1), i = 128 + 16 ib + n
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) OT[cb][r] *= bi;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int jb = 2 * p + (g >> 1);
                const bf16x8 aop = *reinterpret_cast<const bf16x8*>(As + (8 * ib + jb) * 256 + as_off(n, g & 1));
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) OT[cb] = mfma(vf0[cb][p], aop, OT[cb]);
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                if (2 * p > ib) break;  // pair entirely above the diagonal (uniform)
                const int jb = 2 * p + (g >> 1);
                bf16x8 aop = bf16x8{};
                if (jb <= ib)
                    aop = *reinterpret_cast<const bf16x8*>(As + (NCROSS + ib * (ib + 1) / 2 + jb) * 256 + as_off(n, g & 1));
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) OT[cb] = mfma(vf1[cb][p], aop, OT[cb]);
            }
            const int irow = 16 * ib + n;
            if (irow < ceff) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    store4<bf16>(ob + (size_t)(t0 + irow) * tokO + colbase + cb * 16 + 4 * g, OT[cb]);
            }
        }
    };
    if (h == 0) {
        strip(0);
        strip(3);
    } else {
        strip(1);
        strip(2);
    }
}

// ---------------------------------------------------------------- tiled chain
//
// Chunk start states for the per-chunk output kernel, by running the state
// recurrence of the chunked form (same section: S <- lam^C S + K^T diag(c) V
// per chunk) over tiles of the state.  The recurrence is independent per state
// element, so a workgroup owns a 32-row x 16 NVB-column tile of one (batch,
// head) unit and walks all its chunks; each wave keeps NJ 16x16 blocks of it
// in fp32 registers.
// Each chunk's contribution L = K^T diag(c) V is formed on its own (MFMA from
// zero, c_j-scaled bf16 keys) and folded in as S <- fma(lam^C, S, L): exactly
// the local states and the fma scan of the segment split with one chunk per
// segment, so the start states, and the outputs, equal that path's bit for
// bit (the final state rounds like the scan too).  Chunk tiles come through a
// ring of D register sets (loads issued D chunks ahead) and three LDS buffers.
//
// Start state of chunk c goes to snap[bh * nc + c] as bf16 in the output
// kernel's register order for NCBO column blocks per wave; the state after the
// last chunk to S_final (fp32, [dk][dv]) when requested.
struct ChainArgs {
    int T, H, nc, units, ncbo;
    const bf16* k;
    const bf16* v;
    Tok sk, sv;
    const float* lambda;
    const float* S0;
    bf16* snap;
    float* S_final;
};

template <int C, int NVB, int NJ>
struct ChainShape {
    static constexpr int NW = NVB * (2 / NJ), NT = 64 * NW;  // waves: NJ 16-row blocks x one 16-column block each
    static constexpr int TK = 32, TV = 16 * NVB;
    static constexpr int NTK = kDK / TK, NTV = kDV / TV, NTILE = NTK * NTV;
    static constexpr int LKT = TK + 16, LVT = TV + 16;      // LDS row strides (elements)
    static constexpr int R = C < 128 ? C : 128, NS = C / R;  // tokens per pass, passes per chunk
    static constexpr int NPK = R * (TK / 8), NPV = R * (TV / 8);   // 16-byte pieces per pass tile
    static constexpr int PK = (NPK + NT - 1) / NT, PV = (NPV + NT - 1) / NT;
    static_assert(kDV % TV == 0 && (NJ == 1 || NJ == 2), "tile shape");
};

template <int C, int NVB, int NJ, int D>
__global__ __launch_bounds__((ChainShape<C, NVB, NJ>::NT)) void fwd_chain_kernel(ChainArgs a) {
    using L = ChainShape<C, NVB, NJ>;
    constexpr int NT = L::NT, TK = L::TK, TV = L::TV, LKT = L::LKT, LVT = L::LVT, PK = L::PK, PV = L::PV;
    constexpr int NPK = L::NPK, NPV = L::NPV, R = L::R, NS = L::NS;
    static_assert(D % (2 * NS) == 0, "pass and chunk parities");
    __shared__ __align__(16) bf16 Kt[3][R * LKT];   // pass tiles, three buffers
    __shared__ __align__(16) bf16 Vt[3][R * LVT];

    // Workgroups of one unit share an XCD (dispatch goes round-robin over 8):
    // linear id = 8 * NTILE * (unit / 8) + 8 * tile + unit % 8.
    const int lin = blockIdx.x;
    const int grp = lin / (8 * L::NTILE), rem = lin % (8 * L::NTILE);
    const int tile = rem / 8, bh = 8 * grp + rem % 8;
    if (bh >= a.units) return;
    const int tk = tile / L::NTV, tv = tile % L::NTV;
    const int dk0 = TK * tk, dv0 = TV * tv;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, n = lane % 16, g = lane / 16;
    const int vb = wave % NVB, jlo = NJ == 2 ? 0 : wave / NVB;  // this wave's blocks: rows 16 (jlo + j), columns 16 vb
    const int H = a.H, T = a.T, nc = a.nc;
    const int nx = (T + R - 1) / R;   // passes
    const int hd = bh % H, b = bh / H;
    const int tokK = a.sk.t, tokV = a.sv.t;
    const bf16* kb = a.k + b * a.sk.b + hd * kDK + dk0;
    const bf16* vb_ = a.v + b * a.sv.b + hd * kDV + dv0;

    // Start state of the tile (fp32 [dk][dv] -> this wave's blocks), requested
    // before the tiles so that waiting for it waits for no tile.
    f32x4 S[NJ];
    const float* s0 = a.S0 ? a.S0 + (size_t)bh * kDK * kDV : nullptr;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[j][r] = s0 ? s0[(dk0 + 16 * (jlo + j) + 4 * g + r) * kDV + dv0 + 16 * vb + n] : 0.f;

    // Ring of register tiles: piece p = tid + NT i is row p / (W / 8), 16-byte
    // column group p % (W / 8) of the chunk's W-wide tile.  Every pass issues
    // the same loads (chunks past the end with an empty range: nothing is
    // read), so each wait for a tile is exact and never waits for the tiles
    // requested after it.
    uint4 rk[D][PK], rv[D][PV];
    auto load = [&](uint4 (&xk)[PK], uint4 (&xv)[PV], int t) {
        const int valid = t < T ? min(R, T - t) : 0;
        const auto rsk = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(kb + (size_t)t * tokK), 0,
                                                           __builtin_amdgcn_readfirstlane(valid * tokK * 2), kBufWord3);
        const auto rsv = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(vb_ + (size_t)t * tokV), 0,
                                                           __builtin_amdgcn_readfirstlane(valid * tokV * 2), kBufWord3);
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int p = tid + NT * i, row = p / (TK / 8), kc = p % (TK / 8);
            if (NPK % NT == 0 || p < NPK)
                xk[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsk, (row * tokK + 8 * kc) * 2, 0, 0));
        }
#pragma unroll
        for (int i = 0; i < PV; ++i) {
            const int p = tid + NT * i, row = p / (TV / 8), kc = p % (TV / 8);
            if (NPV % NT == 0 || p < NPV)
                xv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsv, (row * tokV + 8 * kc) * 2, 0, 0));
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) load(rk[d], rv[d], d * R);

    // Decay factors: c_j of the key rows this thread stages, for each pass of a
    // chunk (chunk row R s + row), in a full chunk and in a partial last chunk,
    // and the chunk decays lam^C, lam^(partial length).
    const float lam = a.lambda[hd];
    const int ctail = T % C;
    float ck[PK][2][NS];
#pragma unroll
    for (int i = 0; i < PK; ++i) {
        const int row = (tid + NT * i) / (TK / 8);
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) {
            const int jj = R * sp + row;
            ck[i][0][sp] = pow_int(lam, C - 1 - jj);
            ck[i][1][sp] = jj < ctail ? pow_int(lam, ctail - 1 - jj) : 0.f;
        }
    }
    const float lamC = uniform_f32(pow_int(lam, C)), lamT = uniform_f32(pow_int(lam, ctail));

    // Snapshot positions (bf16x4 units) of this wave's blocks in the output
    // kernel's register order.
    int spos[NJ];
    {
        const int ncgo = kDV / (16 * a.ncbo), vblk = dv0 / 16 + vb;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int db = dk0 / 16 + jlo + j, h = db & 1, i = db >> 1;
            const int wo = h * ncgo + vblk / a.ncbo, cb = vblk % a.ncbo;
            spos[j] = ((wo * 3 + i) * a.ncbo + cb) * 64 + lane;
        }
    }
    // (written with non-temporal buffer stores, one resource per chunk's snapshot: 24.97
    // against 25.59 us per Laplace-layer call with plain stores, the same bits)
    bf16* const snap = a.snap + (size_t)bh * nc * kDK * kDV;

    // Pass x (chunk x / NS, its rows R (x % NS) ..) sits in ring slot x % D;
    // staging writes it to LDS buffer x % 3 (keys scaled by c_j), then the slot
    // is refilled with pass x + D.
    auto stage = [&](uint4 (&xk)[PK], uint4 (&xv)[PV], int x) {
        const bool full = T - (x / NS) * C >= C;
        const int sp = x % NS;
        bf16* kt = Kt[x % 3];
        bf16* vt = Vt[x % 3];
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int p = tid + NT * i, row = p / (TK / 8), kc = p % (TK / 8);
            float cf = full ? ck[i][0][0] : ck[i][1][0];
#pragma unroll
            for (int q = 1; q < NS; ++q)
                if (sp == q) cf = full ? ck[i][0][q] : ck[i][1][q];
            if (NPK % NT == 0 || p < NPK)
                *reinterpret_cast<uint4*>(kt + row * LKT + 8 * kc) = scale_bf16x8(xk[i], cf);
        }
#pragma unroll
        for (int i = 0; i < PV; ++i) {
            const int p = tid + NT * i, row = p / (TV / 8), kc = p % (TV / 8);
            if (NPV % NT == 0 || p < NPV) *reinterpret_cast<uint4*>(vt + row * LVT + 8 * kc) = xv[i];
        }
    };
    // Operands of pass x (LDS buffer x % 3): this wave's value and key columns.
    bf16x8 vop[2][R / 32], kop[2][R / 32][NJ];  // [pass parity]
    auto operands = [&](int par, int x) {
        const bf16* kt = Kt[x % 3];
        const bf16* vt = Vt[x % 3];
#pragma unroll
        for (int p = 0; p < R / 32; ++p) {
            vop[par][p] = op_col8(vt, LVT, 32 * p, 16 * vb, n, g);
#pragma unroll
            for (int j = 0; j < NJ; ++j) kop[par][p][j] = op_col8(kt, LKT, 32 * p, 16 * (jlo + j), n, g);
        }
    };
    stage(rk[0], rv[0], 0);
    load(rk[0], rv[0], D * R);
    stage(rk[1], rv[1], 1);
    load(rk[1], rv[1], (D + 1) * R);
    __syncthreads();
    operands(0, 0);

    // Pass x: its operands are in registers (read a pass earlier), pass x + 1
    // is complete in LDS, pass x + 2 is staged into the third buffer (last read
    // two passes ago).  Chunk c's own contribution Lc = (diag(c) K)^T V is
    // multiplied in its NS passes; the chain itself, S <- lam^C S + L(c-1), one
    // fma per element, runs in chunk c's first pass, so the chunk's MFMAs never
    // wait for the chain, and LDS reads, LDS writes and MFMAs of neighbouring
    // passes overlap.  One barrier per pass.  (With NS = 1 a pass is a chunk.)
    f32x4 Lc[2][NJ];  // [chunk parity][block]
    for (int x0 = 0; x0 < nx; x0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int x = x0 + d;
            if (x >= nx) break;
            const int po = d & 1, pn = po ^ 1;                   // pass parity (compile time)
            const int sp = d % NS;                               // pass within the chunk
            const int cur = (d / NS) & 1, prv = cur ^ 1;         // chunk parity (x0 is a multiple of 2 NS)
            const int c = x / NS;
            if (sp == 0) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) Lc[cur][j] = zero4();
            }
            // The pass's LDS traffic is issued first: the next pass's operands
            // (a pass is bound by these transposed reads), then pass x + 2 staged
            // and its ring slot refilled (issued on every pass, past the end:
            // zeros, no reads, so the waits for the ring stay exact).  The MFMAs
            // below only need registers read a pass ago.  (Left to itself the
            // scheduler puts the MFMAs first: ~0.7 us more per Laplace-layer call.)
            operands(pn, x + 1);
            const int d2 = (d + 2) % D;  // compile-time once unrolled
            stage(rk[d2], rv[d2], x + 2);
            load(rk[d2], rv[d2], (x + 2 + D) * R);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = 0; p < R / 32; ++p)
#pragma unroll
                for (int j = 0; j < NJ; ++j) Lc[cur][j] = mfma(kop[po][p][j], vop[po][p], Lc[cur][j]);
            if (sp == 0) {
                // chain step of the previous chunk: S = start state of chunk c
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if (c >= 1) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) S[j][r] = fmaf(lamC, S[j][r], Lc[prv][j][r]);  // a full chunk
                    }
                    __builtin_amdgcn_raw_buffer_store_b64(
                        __builtin_bit_cast(u32x2, bf16x4{to_bf16(S[j][0]), to_bf16(S[j][1]), to_bf16(S[j][2]),
                                                         to_bf16(S[j][3])}),
                        __builtin_amdgcn_make_buffer_rsrc(snap + (size_t)c * kDK * kDV, 0, kDK * kDV * 2, kBufWord3),
                        spos[j] * 8, 0, kCpolNT);
                }
            }
            __syncthreads();  // pass x + 2 staged; pass x + 1's operands read
        }
    }
    {
        // the last chunk (possibly partial): S_final = lam^ceff S + L(nc-1)
        const float Lam = T - (nc - 1) * C >= C ? lamC : lamT;
        const int last = (nc - 1) & 1;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[j][r] = fmaf(Lam, S[j][r], last ? Lc[1][j][r] : Lc[0][j][r]);
    }
    if (a.S_final) {
        float* dst = a.S_final + (size_t)bh * kDK * kDV;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[(dk0 + 16 * (jlo + j) + 4 * g + r) * kDV + dv0 + 16 * vb + n] = S[j][r];
    }
}

template <int C>
hipError_t launch_chain(const FwdPlan& plan, int B, int T, int H, int ncbo, const FwdIO& io, const float* lambda,
                        const float* S0, float* S_final, void* ws, hipStream_t stream) {
    // 8 waves, one 16x16 block each, over a 32 x 64 tile: the fastest of the
    // shapes measured on gfx950 (Laplace layer 29.8 us against 30.6 for 4 waves
    // of two blocks, 31.6 for 4 waves over 32 x 32 tiles; a deeper ring of 10 or
    // 12 chunks was slower).  A pass costs ~0.7 us at 128 tokens and its time
    // follows the tokens.  Chunks in flight: at most what the wave's memory
    // counter can follow exactly (at most 63 outstanding operations; a chunk
    // costs PK + PV loads and NJ snapshot stores); even, so the pass parity is
    // known at compile time in the unrolled loop.
    constexpr int NVB = 4, NJ = 1;
    using L = ChainShape<C, NVB, NJ>;
    constexpr int D = C == 256 ? 8 : C == 128 ? 6 : 12;  // (256: 128-token passes, two per chunk)
    static_assert(D * (L::PK + L::PV + NJ) <= 63, "memory counter");
    ChainArgs c{};
    c.T = T;
    c.H = H;
    c.nc = plan.nc;
    c.units = B * H;
    c.ncbo = ncbo;
    c.k = static_cast<const bf16*>(io.k);
    c.v = static_cast<const bf16*>(io.v);
    c.sk = io.sk;
    c.sv = io.sv;
    c.lambda = lambda;
    c.S0 = S0;
    c.snap = static_cast<bf16*>(ws);
    c.S_final = S_final;
    const unsigned groups = (unsigned)((c.units + 7) / 8);
    hipLaunchKernelGGL((fwd_chain_kernel<C, NVB, NJ, D>), dim3(groups * 8 * L::NTILE), dim3(L::NT), 0, stream, c);
    return hipGetLastError();
}

template <int C, int LDK, int NCB>
hipError_t launch_c(const FwdPlan& plan, int B, int T, int H, const FwdIO& io, const float* lambda, const float* S0,
                    float scale, float* S_final, void* sbar, void* ws, const EpilogueArgs* ep, hipStream_t stream) {
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
    a.Ub = static_cast<char*>(ws) +
           (size_t)B * H * (plan.nseg > 1 ? plan.nseg - 1 : 0) * plan.psub * kDK * kDV * sizeof(float);
    a.psub = plan.psub;
    a.fuse_scan = plan.fuse_scan;
    a.sbar = sbar;
    a.nseg = plan.nseg;
    a.seg_chunks = plan.seg_chunks;
    a.nc = plan.nc;
    const unsigned units = (unsigned)B * H;
    if constexpr (C >= 64) {
      if (plan.chain) {
        // every chunk's start state from the tiled chain, then one output
        // workgroup per chunk
        hipError_t err = launch_chain<C>(plan, B, T, H, NCB, io, lambda, S0, S_final, ws, stream);
        if (err != hipSuccess) return err;
        a.U = nullptr;
        a.Ub = ws;
        a.S_final = nullptr;
        // one workgroup per (chunk, unit); units in groups of 8 (one per XCD)
        // when an XCD's units' k and v (T (dk + dv) bf16 each) fit its 4 MB L2
        // with room to spare
        a.units = (int)units;
        a.out_xcd = (size_t)((units + 7) / 8) * T * (kDK + kDV) * 2 <= (size_t)3 << 20;
        const unsigned ogrid = (unsigned)plan.nc * (a.out_xcd ? (units + 7) / 8 * 8 : units);
        if (ep)
            hipLaunchKernelGGL((fwd_out_kernel<C, LDK, NCB, true>), dim3(ogrid), dim3(F8<C, LDK, NCB>::NT), 0, stream,
                               a, *ep);
        else
            hipLaunchKernelGGL((fwd_out_kernel<C, LDK, NCB, false>), dim3(ogrid), dim3(F8<C, LDK, NCB>::NT), 0,
                               stream, a, EpilogueArgs{});
        return hipGetLastError();
      }
    }
    if (ep) return hipErrorNotSupported;   // the epilogue is fused into the chain form only
    if (plan.nseg > 1) {
        // state-only prologue over the psub (nseg - 1) sub-segments before the last
        // segment, then the scan turns their local states into the states at every
        // sub-segment boundary (fp32 whenever a segment has several chunks)
        FwdArgs pa = a;
        pa.nseg = (plan.nseg - 1) * plan.psub + 1;
        pa.seg_chunks = plan.seg_chunks / plan.psub;
        hipLaunchKernelGGL((fwd_bf16_kernel<C, LDK, NCB, true>), dim3(pa.nseg - 1, units), dim3(F8<C, LDK, NCB>::NT),
                           0, stream, pa);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        if (!plan.fuse_scan) {
            hipLaunchKernelGGL(seg_scan_frag_kernel<NCB>, dim3((kDK * kDV / 4 + 255) / 256, units), dim3(256), 0,
                               stream, S0, a.U, static_cast<bf16*>(a.Ub), lambda, H, pa.nseg, plan.seg_chunks,
                               pa.seg_chunks * C, S_final != nullptr ? 1 : 0);
            err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
    }
    hipLaunchKernelGGL((fwd_bf16_kernel<C, LDK, NCB, false>), dim3(plan.nseg, units), dim3(F8<C, LDK, NCB>::NT), 0,
                       stream, a);
    return hipGetLastError();
}

// 256-token chunks: the tiled chain (two 128-token passes per chunk), then two
// output workgroups per (chunk, unit).
hipError_t launch_c256(const FwdPlan& plan, int B, int T, int H, const FwdIO& io, const float* lambda,
                       const float* S0, float scale, float* S_final, void* sbar, void* ws, hipStream_t stream) {
    constexpr int LDK = 104, NCB = 2;
    hipError_t err = launch_chain<256>(plan, B, T, H, NCB, io, lambda, S0, S_final, ws, stream);
    if (err != hipSuccess) return err;
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
    a.scale = scale;
    a.o = io.o;
    a.Ub = ws;
    a.sbar = sbar;
    a.nc = plan.nc;
    hipLaunchKernelGGL((fwd_out256_kernel<LDK, NCB>), dim3(2 * plan.nc, (unsigned)B * H), dim3(F8<128, LDK, NCB>::NT),
                       0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdPlan& plan, int B, int T, int H, int chunk, const FwdIO& io, const float* lambda,
                           const float* S0, float scale, float* S_final, void* sbar, void* ws, hipStream_t stream) {
    // 12 waves per workgroup, two 16-column blocks each
    if (chunk == 128)
        return launch_c<128, 104, 2>(plan, B, T, H, io, lambda, S0, scale, S_final, sbar, ws, nullptr, stream);
    if (chunk == 64)
        return launch_c<64, 104, 2>(plan, B, T, H, io, lambda, S0, scale, S_final, sbar, ws, nullptr, stream);
    if (chunk == 32 && !plan.chain)
        return launch_c<32, 104, 2>(plan, B, T, H, io, lambda, S0, scale, S_final, sbar, ws, nullptr, stream);
    if (chunk == 256 && plan.chain)
        return launch_c256(plan, B, T, H, io, lambda, S0, scale, S_final, sbar, ws, stream);
    return hipErrorInvalidValue;
}

// The forward with the mixer epilogue applied in the output kernel's store
// (the tiled-chain form only; hipErrorNotSupported otherwise, the caller then
// runs the forward and the epilogue pass).
hipError_t launch_fwd_bf16_epilogue(const FwdPlan& plan, int B, int T, int H, int chunk, const FwdIO& io,
                                    const float* lambda, const float* S0, float scale, float* S_final, void* ws,
                                    const EpilogueArgs& ep, hipStream_t stream) {
    if (!plan.chain || chunk != 128) return hipErrorNotSupported;
    return launch_c<128, 104, 2>(plan, B, T, H, io, lambda, S0, scale, S_final, nullptr, ws, &ep, stream);
}

}  // namespace gla

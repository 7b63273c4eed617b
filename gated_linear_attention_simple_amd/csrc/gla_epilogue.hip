// gla_epilogue.hip -- the mixer epilogue after the readout (Laplace 3B post,
// section "i14 and the Laplace 3B architecture", paragraph "GLA mixer", the
// sentences after the readout), as a bandwidth-bound pass over the mixer
// output.  For every row m (token) and head h:
//     s    = sigmoid( q . (a_h (.) k) )                   self-augmentation gate
//     x    = o + s v                                      (a = 0: half-strength skip)
//     y    = silu(g) (.) x / sqrt(mean(x^2) + eps) (.) w_tier(h)
// i.e. the value copy, the head RMSNorm of the head's decay tier, and the SiLU
// gate; concatenating the heads is the [M][H][dv] layout itself.
//
// A group of LPU lanes per (row, head) (a power of two, 4..64): lane l holds the
// 16-byte pieces l of the row's q, k (dk) and v, o, g, y (dv).  Rows of each
// tensor lie a row stride apart (H * d when packed), heads packed inside a row.
// Every tensor moves in 16-byte buffer loads and stores whose range ends after
// the batch's last (row, head), so lanes past a row's end and units past the
// last read zeros without a branch, and all loads of a lane (the two parameter
// rows included) are issued back to back before any arithmetic.  The two sums (gate logit, sum of
// squares) are butterfly reductions inside the group, in a fixed order.
// 2 dk + 4 dv elements move per (row, head) for ~10 dv flops: bound by HBM.
#include "gla_common.hpp"
#include "gla_internal.hpp"
#include "gla_tile.hpp"

namespace gla {
namespace {

// Sum over aligned groups of LPU lanes, every lane of a group receiving the
// group's sum; a fixed pairing order, so the result is deterministic.  Inside
// a 16-lane row the pairs come from DPP lane permutations (quad swaps, then
// the half-row and row mirrors); rows pair up through a 32-lane swizzle, and
// the two halves of a wave through lane reads.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
template <int LPU>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(LPU == 4 || LPU == 8 || LPU == 16 || LPU == 32 || LPU == 64, "power-of-two group");
    x += dpp<0xB1>(x);                                  // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);                                  // quad_perm [2,3,0,1]
    if constexpr (LPU >= 8) x += dpp<0x141>(x);         // row_half_mirror
    if constexpr (LPU >= 16) x += dpp<0x140>(x);        // row_mirror
    if constexpr (LPU >= 32)                            // swap the two rows of each 32-lane half
        x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
    if constexpr (LPU == 64)
        x = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    return x;
}

constexpr int lanes_for(int n) { return n <= 4 ? 4 : n <= 8 ? 8 : n <= 16 ? 16 : n <= 32 ? 32 : 64; }
constexpr int kEpiThreads = 256;

// 16-byte piece <-> VEC floats
template <typename E> struct Piece;
template <> struct Piece<bf16> {
    static constexpr int N = 8;
    __device__ static void unpack(uint4 u, float* f) {
        const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
        }
    }
    __device__ static uint4 pack(const float* f) {
        unsigned w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const unsigned lo = __builtin_bit_cast(unsigned short, to_bf16(f[2 * i]));
            const unsigned hi = __builtin_bit_cast(unsigned short, to_bf16(f[2 * i + 1]));
            w[i] = lo | (hi << 16);
        }
        return uint4{w[0], w[1], w[2], w[3]};
    }
};
template <> struct Piece<float> {
    static constexpr int N = 4;
    __device__ static void unpack(uint4 u, float* f) {
        f[0] = __builtin_bit_cast(float, u.x);
        f[1] = __builtin_bit_cast(float, u.y);
        f[2] = __builtin_bit_cast(float, u.z);
        f[3] = __builtin_bit_cast(float, u.w);
    }
    __device__ static uint4 pack(const float* f) {
        return uint4{__builtin_bit_cast(unsigned, f[0]), __builtin_bit_cast(unsigned, f[1]),
                     __builtin_bit_cast(unsigned, f[2]), __builtin_bit_cast(unsigned, f[3])};
    }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int range) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, __builtin_amdgcn_readfirstlane(range),
                                             kBufWord3);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <typename E, int DK, int DV>
struct EpiShape {
    static constexpr int VEC = Piece<E>::N;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int NVL = DV / VEC;        // lanes holding a piece of a dv row
    static constexpr int NKL = DK / VEC;        // lanes holding a piece of a dk row
    static constexpr int LPU = lanes_for(NVL);  // lanes per (row, head)
    static constexpr int UPB = kEpiThreads / LPU;  // (row, head) units per batch
    static_assert(DV % VEC == 0 && DK % VEC == 0 && NVL <= 64 && NKL <= LPU, "row pieces must fit the group");
};

// Workgroup w takes the batches w, w + G, w + 2G, ... of UPB consecutive units
// (G = gridDim.x, a multiple of H, so a thread keeps one head throughout and
// loads its parameter rows once).  The next batch's five row loads are issued
// before the current batch's arithmetic, into the other of two register sets;
// a batch past the end has an empty range: it reads zeros and stores nothing.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(kEpiThreads) void epilogue_kernel(EpilogueArgs a) {
    using Sh = EpiShape<E, DK, DV>;
    constexpr int VEC = Sh::VEC, ES = Sh::ES, NVL = Sh::NVL, NKL = Sh::NKL, LPU = Sh::LPU, UPB = Sh::UPB;
    const int lane = threadIdx.x % LPU;
    const int lu = threadIdx.x / LPU;                       // unit within a batch
    const long nb = (a.units + UPB - 1) / UPB;              // batches
    const long G = gridDim.x;
    const int h = (int)(((long)blockIdx.x * UPB % a.H + lu) % a.H);

    // tier of head h: the map sits in the kernel arguments, so select, never index
    int tier = 0;
#pragma unroll
    for (int i = 0; i < kEpiMaxHeads; ++i) tier = (h == i) ? a.tier[i] : tier;

    // parameter rows: aug_a [H][DK] (absent -> empty range -> zeros), norm_w [tiers][DV]
    const __amdgpu_buffer_rsrc_t ra = rsrc(a.aug_a, a.aug_a ? a.H * DK * 4 : 0);
    const __amdgpu_buffer_rsrc_t rw = rsrc(a.norm_w, a.n_tiers * DV * 4);
    const int oa = lane < NKL ? (h * DK + lane * VEC) * 4 : a.H * DK * 4;
    const int ow = (tier * DV + (lane < NVL ? lane : 0) * VEC) * 4;
    float av[VEC], w[VEC];
#pragma unroll
    for (int j = 0; j < VEC / 4; ++j) {
        Piece<float>::unpack(ld16(ra, oa + 16 * j), av + 4 * j);
        Piece<float>::unpack(ld16(rw, ow + 16 * j), w + 4 * j);
    }

    // units of batch b: UPB, fewer in the last batch, 0 past the end
    auto batch_units = [&](long b) -> int {
        const long left = a.units - b * UPB;
        return left <= 0 ? 0 : left < UPB ? (int)left : UPB;
    };
    // Where the units of batch b lie: the batch's first row r0; this lane's unit
    // at row r0 + dr, head hu; the last unit at row r0 + drl, head hl.  A tensor
    // of row stride R and width D is read from ptr + r0 R with the range
    // (drl R + (hl + 1) D) elements, which ends after the batch's last unit (0
    // for a batch past the end), and this lane's piece at (dr R + hu D) + lane VEC.
    // G UPB is a multiple of H, so every batch of this workgroup starts at the
    // same head m: dr and hu are fixed per thread, and batch b = blockIdx.x + k G
    // starts at row r0 = rfirst + k (G UPB / H) (no division per batch).
    struct Pos {
        long r0;
        int dr, hu, drl, hl, nu;
    };
    const int m = (int)(((long)blockIdx.x * UPB) % a.H);
    const long rfirst = (long)blockIdx.x * UPB / a.H, rstep = G * UPB / a.H;
    const int dr_lane = (m + lu) / a.H, hu_lane = (m + lu) % a.H;
    auto where = [&](long kb) {
        Pos p;
        p.nu = batch_units(blockIdx.x + kb * G);
        p.r0 = rfirst + kb * rstep;
        p.dr = dr_lane;
        p.hu = hu_lane;
        const int dl = m + (p.nu > 0 ? p.nu - 1 : 0);
        p.drl = dl / a.H;
        p.hl = dl - p.drl * a.H;
        return p;
    };
    auto range_of = [&](const Pos& p, int R, int D) { return p.nu > 0 ? (p.drl * R + (p.hl + 1) * D) * ES : 0; };
    auto off_of = [&](const Pos& p, int R, int D, int nl, int range) {
        return lane < nl ? (p.dr * R + p.hu * D + lane * VEC) * ES : range;
    };
    auto row_load = [&](const Pos& p, const void* base, int R, int D, int nl) {
        const int rg = range_of(p, R, D);
        return ld16(rsrc(static_cast<const E*>(base) + p.r0 * R, rg), off_of(p, R, D, nl, rg));
    };
    // row loads of this workgroup's batch kb: q, k, v, o, g pieces (zeros past the rows' ends)
    auto load = [&](long kb, uint4* r) {
        const Pos p = where(kb);
        r[0] = row_load(p, a.q, a.rq, DK, NKL);
        r[1] = row_load(p, a.k, a.rk, DK, NKL);
        r[2] = row_load(p, a.v, a.rv, DV, NVL);
        r[3] = row_load(p, a.o, a.ro, DV, NVL);
        r[4] = row_load(p, a.g, a.rg, DV, NVL);
    };
    // one batch: issue the loads of batch kb + 1 into `nxt`, then finish batch kb from `cur`
    auto step = [&](long kb, const uint4* cur, uint4* nxt) {
        load(kb + 1, nxt);
        __builtin_amdgcn_sched_barrier(0);   // next batch's loads ahead of this batch's arithmetic
        float q[VEC], k[VEC], v[VEC], o[VEC], g[VEC];
        Piece<E>::unpack(cur[0], q);
        Piece<E>::unpack(cur[1], k);
        Piece<E>::unpack(cur[2], v);
        Piece<E>::unpack(cur[3], o);
        Piece<E>::unpack(cur[4], g);

        float z = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) z += q[e] * av[e] * k[e];
        const float s = fast_sigmoid(group_sum<LPU>(z));

        float x[VEC];
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            x[e] = o[e] + s * v[e];
            ss += x[e] * x[e];
        }
        const float inv = __builtin_amdgcn_rsqf(group_sum<LPU>(ss) * (1.f / DV) + a.eps);
        float y[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) y[e] = g[e] * fast_sigmoid(g[e]) * x[e] * inv * w[e];
        const Pos p = where(kb);                              // (past the end: range 0, store dropped)
        const int ry = range_of(p, a.ry, DV);
        // (y leaves with non-temporal stores: 97.8 -> 93.6 us at the training width)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, Piece<E>::pack(y)),
                                               rsrc(static_cast<E*>(a.y) + p.r0 * a.ry, ry),
                                               off_of(p, a.ry, DV, NVL, ry), 0, kCpolNT);
    };

    // two register sets in turn (no copies between them); the loop body is two
    // whole steps, the second of which may be a past-the-end batch
    uint4 ra0[5], ra1[5];
    load(0, ra0);
    for (long kb = 0; blockIdx.x + kb * G < nb; kb += 2) {
        step(kb, ra0, ra1);
        step(kb + 1, ra1, ra0);
    }
}

}  // namespace

bool epilogue_supported(int dk, int dv) { return (dk == 96 && dv == 192) || (dk == 16 && dv == 32); }

// Workgroups: about kEpiBatchesPerWg batches each (enough to amortise a
// workgroup's set-up and first exposed load), rounded up to a multiple of H.
constexpr long kEpiBatchesPerWg = 4;
static unsigned epi_grid(long nb, int H) {
    const long want = (nb + kEpiBatchesPerWg - 1) / kEpiBatchesPerWg;
    return (unsigned)((want + H - 1) / H * H);
}

hipError_t launch_epilogue(bool bf16_io, int dk, int dv, const EpilogueArgs& a, hipStream_t stream) {
#define GLA_EPI(E_, DK_, DV_)                                                                            \
    do {                                                                                                 \
        const long nb = (a.units + EpiShape<E_, DK_, DV_>::UPB - 1) / EpiShape<E_, DK_, DV_>::UPB;     \
        hipLaunchKernelGGL((epilogue_kernel<E_, DK_, DV_>), dim3(epi_grid(nb, a.H)), dim3(kEpiThreads), 0, \
                           stream, a);                                                                   \
    } while (0)
    if (dk == 96 && dv == 192) {
        if (bf16_io) GLA_EPI(bf16, 96, 192);
        else GLA_EPI(float, 96, 192);
    } else {
        if (bf16_io) GLA_EPI(bf16, 16, 32);
        else GLA_EPI(float, 16, 32);
    }
#undef GLA_EPI
    return hipGetLastError();
}

}  // namespace gla

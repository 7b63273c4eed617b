// gla_tile.hpp -- LDS tile staging and MFMA operand fetch for gfx950.
//
// Tiles of chunk data live in LDS row-major, one token per row, exactly as
// they sit in HBM.  MFMA operands are fetched in the two orientations the
// mixer needs:
//   * "row" operands (contraction along the contiguous feature dimension):
//     plain 8- or 16-byte LDS reads;
//   * "column" operands (contraction along tokens, i.e. down the rows): the
//     gfx950 transpose read ds_read_b64_tr_b16.  In each 16-lane group, lane j
//     supplies the address of a 4-element piece; pieces of lanes 4e..4e+3 form
//     row e of a 4x16 block and lane j receives column j of that block.
// fp32 tiles use the 16x16x4 fp32 MFMA, whose operands are single elements, so
// both orientations are plain 4-byte reads.
#pragma once

#include "gla_common.hpp"

namespace gla {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

__device__ __forceinline__ bf16x4 ds_tr4(const bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

// Row operand, natural 8-k set: M[row][k0 .. k0+7] (16-byte read).
__device__ __forceinline__ bf16x8 op_row8(const bf16* M, int ld, int row, int k0) {
    return *reinterpret_cast<const bf16x8*>(M + row * ld + k0);
}
// Row operand, paired k set {k0..k0+3} U {k0+16..k0+19}: the k set of two stacked
// accumulator blocks (lane group g passes k0 = base + 4g).
__device__ __forceinline__ bf16x8 op_row_pair(const bf16* M, int ld, int row, int k0) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(M + row * ld + k0);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(M + row * ld + k0 + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Column operand, natural 8-k set: lane (n, g) receives M[kb + 8g + e][nb + n],
// e = 0..7, read from row-major M[k][n] with transpose reads.
__device__ __forceinline__ bf16x8 op_col8(const bf16* M, int ld, int kb, int nb, int n, int g) {
    const bf16* p = M + (kb + 8 * g + (n >> 2)) * ld + nb + 4 * (n & 3);
    const bf16x4 lo = ds_tr4(p);
    const bf16x4 hi = ds_tr4(p + 4 * ld);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Column operand, paired k set: lane (n, g) receives M[kb + 4g + e][nb + n] and
// M[kb + 16 + 4g + e][nb + n], e = 0..3.
__device__ __forceinline__ bf16x8 op_col_pair(const bf16* M, int ld, int kb, int nb, int n, int g) {
    const bf16* p = M + (kb + 4 * g + (n >> 2)) * ld + nb + 4 * (n & 3);
    const bf16x4 lo = ds_tr4(p);
    const bf16x4 hi = ds_tr4(p + 16 * ld);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 pack_acc(f32x4 a, f32x4 b) {
    return bf16x8{to_bf16(a[0]), to_bf16(a[1]), to_bf16(a[2]), to_bf16(a[3]),
                  to_bf16(b[0]), to_bf16(b[1]), to_bf16(b[2]), to_bf16(b[3])};
}

// Four consecutive elements <-> fp32x4 (8-byte bf16 / 16-byte fp32 accesses).
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
template <typename E>
__device__ __forceinline__ f32x4 load4(const E* src);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* src) {
    return *reinterpret_cast<const f32x4*>(src);
}
template <>
__device__ __forceinline__ f32x4 load4<bf16>(const bf16* src) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(src);
    return f32x4{to_f32(x[0]), to_f32(x[1]), to_f32(x[2]), to_f32(x[3])};
}

// Sum over the 64 lanes of a wave in a fixed butterfly order (deterministic);
// every lane receives the total.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// Stages a ROWS x D row-major tile (token stride `tok_stride` elements in HBM)
// through registers into LDS.  Piece p = tid + NT*i is the 16-byte group
// kc = p % KC of row p / KC, so a wave reads whole rows contiguously.  Rows at
// or past `valid` read as zeros.
template <typename E, int ROWS, int D, int NT>
struct TileStage {
    static constexpr int VEC = 16 / sizeof(E);
    static constexpr int KC = D / VEC;
    static constexpr int NP = ROWS * KC;
    static constexpr int PER = (NP + NT - 1) / NT;
    static_assert(D % VEC == 0, "rows are whole 16-byte pieces");
    uint4 r[PER];

    // Offsets inside one tile stay in 32 bits (rows * tok_stride < 2^31 for every
    // supported shape), so no 64-bit address per piece stays live.
    __device__ __forceinline__ void load(const E* base, int tok_stride, int valid, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = tid + NT * i;
            const int row = p / KC, kc = p % KC;
            if ((NP % NT == 0 || p < NP) && row < valid)
                r[i] = *reinterpret_cast<const uint4*>(base + (row * tok_stride + kc * VEC));
            else
                r[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    template <int LD>
    __device__ __forceinline__ void store(E* dst, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = tid + NT * i;
            if (NP % NT != 0 && p >= NP) continue;
            *reinterpret_cast<uint4*>(dst + (p / KC) * LD + (p % KC) * VEC) = r[i];
        }
    }
    // Row-scaled copy: dst[row] = coef(row) * tile[row], rounded to E.
    template <int LD, typename F>
    __device__ __forceinline__ void store_scaled(E* dst, int tid, F coef) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = tid + NT * i;
            if (NP % NT != 0 && p >= NP) continue;
            const int row = p / KC;
            const float c = coef(row);
            uint4 w;
            if constexpr (sizeof(E) == 2) {
                const bf16x8 x = __builtin_bit_cast(bf16x8, r[i]);
                bf16x8 y;
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = to_bf16(to_f32(x[e]) * c);
                w = __builtin_bit_cast(uint4, y);
            } else {
                const f32x4 x = __builtin_bit_cast(f32x4, r[i]);
                w = __builtin_bit_cast(uint4, f32x4{x[0] * c, x[1] * c, x[2] * c, x[3] * c});
            }
            *reinterpret_cast<uint4*>(dst + row * LD + (p % KC) * VEC) = w;
        }
    }
};

// bf16x8 scaled by one fp32 factor, rounded back to bf16.
__device__ __forceinline__ uint4 scale_bf16x8(uint4 raw, float c) {
    bf16x8 x = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = to_bf16(to_f32(x[e]) * c);
    return __builtin_bit_cast(uint4, x);
}

// Buffer resource word 3 for raw (untyped, unswizzled) buffers on gfx9-family parts.
constexpr int kBufWord3 = 0x00020000;
// Cache-policy operand of the buffer intrinsics on gfx950: non-temporal (nt).
constexpr int kCpolNT = 2;

// Stages a ROWS x D bf16 tile like TileStage, with buffer loads: the tile base
// and its byte range live in one scalar resource and each piece needs only a
// 32-bit offset.  Rows at or past `valid` lie outside the range and read as
// zeros (the hardware returns 0 for out-of-range buffer loads); with valid <= 0
// the range is empty and nothing is read at all.
template <int ROWS, int D, int NT>
struct BufStage {
    static constexpr int KC = D / 8;
    static constexpr int NP = ROWS * KC;
    static constexpr int PER = (NP + NT - 1) / NT;
    static_assert(D % 8 == 0, "rows are whole 16-byte pieces");
    uint4 r[PER];

    __device__ __forceinline__ void load(const bf16* base, int tok_stride, int valid, int tid) {
        const unsigned rows = (unsigned)(valid <= 0 ? 0 : valid < ROWS ? valid : ROWS);
        // (the range is wave-uniform; readfirstlane keeps it in a scalar register)
        const int range = __builtin_amdgcn_readfirstlane((int)(rows * (unsigned)tok_stride * 2u));
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), 0, range, kBufWord3);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = tid + NT * i;
            if (NP % NT == 0 || p < NP) {
                const int row = p / KC, kc = p % KC;
                r[i] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((unsigned)(row * tok_stride + kc * 8) * 2u), 0, 0));
            } else {
                r[i] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    }
    template <int LD>
    __device__ __forceinline__ void store(bf16* dst, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = tid + NT * i;
            if (NP % NT != 0 && p >= NP) continue;
            *reinterpret_cast<uint4*>(dst + (p / KC) * LD + (p % KC) * 8) = r[i];
        }
    }
    // Row-scaled copy: dst[row] = coef(row) * tile[row], rounded to bf16.
    template <int LD, typename F>
    __device__ __forceinline__ void store_scaled(bf16* dst, int tid, F coef) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = tid + NT * i;
            if (NP % NT != 0 && p >= NP) continue;
            *reinterpret_cast<uint4*>(dst + (p / KC) * LD + (p % KC) * 8) = scale_bf16x8(r[i], coef(p / KC));
        }
    }
};

// BufStage for thread counts that are a multiple of the 16-byte pieces per row:
// thread t always stages column piece t % KC of rows t / KC + i * (NT / KC), so
// one 32-bit offset per thread serves every load (the row step rides in the
// scalar offset) and the LDS stores differ by compile-time constants.
template <int ROWS, int D, int NT>
struct RowStage {
    static constexpr int KC = D / 8;
    static constexpr int RSTEP = NT / KC;
    static constexpr int PER = (ROWS + RSTEP - 1) / RSTEP;
    static_assert(D % 8 == 0 && NT % KC == 0, "whole rows per round");
    uint4 r[PER];

    __device__ __forceinline__ void load(const bf16* base, int tok_stride, int valid, int tid) {
        const unsigned rows = (unsigned)(valid <= 0 ? 0 : valid < ROWS ? valid : ROWS);
        // (the range is wave-uniform; readfirstlane keeps it in a scalar register)
        const int range = __builtin_amdgcn_readfirstlane((int)(rows * (unsigned)tok_stride * 2u));
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), 0, range, kBufWord3);
        const int row0 = tid / KC;
        const int vo = (int)((unsigned)(row0 * tok_stride + (tid % KC) * 8) * 2u);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (ROWS % RSTEP == 0 || row0 + i * RSTEP < ROWS)
                r[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rs, vo, (int)((unsigned)(i * RSTEP * tok_stride) * 2u), 0));
            else
                r[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    template <int LD>
    __device__ __forceinline__ void store(bf16* dst, int tid) const {
        const int row0 = tid / KC;
        bf16* d = dst + row0 * LD + (tid % KC) * 8;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (ROWS % RSTEP == 0 || row0 + i * RSTEP < ROWS) *reinterpret_cast<uint4*>(d + i * RSTEP * LD) = r[i];
    }
    template <int LD, typename F>
    __device__ __forceinline__ void store_scaled(bf16* dst, int tid, F coef) const {
        const int row0 = tid / KC;
        bf16* d = dst + row0 * LD + (tid % KC) * 8;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (ROWS % RSTEP == 0 || row0 + i * RSTEP < ROWS)
                *reinterpret_cast<uint4*>(d + i * RSTEP * LD) = scale_bf16x8(r[i], coef(row0 + i * RSTEP));
    }
};

// Per-lane decay factors of a 16x16 block of a C x C decay mask, for an
// accumulator laid out as D[4g + r][n] holding rows j (keys) and columns i
// (queries), i.e. element (j = jb*16 + 4g + r, i = ib*16 + n):
//   diagonal block (ib == jb): lam^(n - 4g - r) if n >= 4g + r, else 0
//   below (ib > jb):           lam^(16(ib - jb - 1)) * lam^(16 + n - 4g - r)
// Every factor is a product of at most two powers with non-negative exponents
// (no ratio of powers is formed).
struct DecayLane {
    float diag[4];
    float off[4];
    __device__ __forceinline__ void init(float lam, int n, int g) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = n - 4 * g - r;
            diag[r] = m >= 0 ? pow_int(lam, m) : 0.f;
            off[r] = pow_int(lam, 16 + m);
        }
    }
};

}  // namespace gla

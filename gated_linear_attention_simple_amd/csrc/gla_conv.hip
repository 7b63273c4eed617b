// gla_conv.hip -- depth-wise causal convolution of width 4 with SiLU, the step
// before the mixer (Laplace 3B post, section "i14 and the Laplace 3B
// architecture", paragraph "Normalization and convolution" and the "Conv" row
// of the parameter table).  Per channel d:
//     u_t[d] = bias[d] + sum_j w[d][j] x_{t-3+j}[d],      y_t[d] = silu(u_t[d])
// with inputs before the first token taken from a per-sequence window of the
// four most recent earlier inputs (fp32 [K][D], oldest first); the window after
// the last token is the carry a decode step continues from.
//
// Both kernels are bound by HBM (8 flops per element moved): every thread owns
// one 16-byte piece of channels and walks tokens, so each input element is read
// once (plus a 3-token halo per run of tokens), the four taps stay in
// registers, and loads and stores are whole 16-byte buffer accesses whose
// range ends at the sequence end (no branches for ragged runs).
#include "gla_common.hpp"
#include "gla_internal.hpp"
#include "gla_tile.hpp"

namespace gla {
namespace {

constexpr int kConvK = 4;
constexpr int kConvThreads = 128;
constexpr int kConvRun = 32;     // tokens per thread in the prefill
constexpr int kConvGroup = 16;   // tokens whose loads are issued together

template <typename E> struct CPiece;
template <> struct CPiece<bf16> {
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
template <> struct CPiece<float> {
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

typedef unsigned cu32x4 __attribute__((ext_vector_type(4)));

// A buffer range must be the same for the whole wave (it sits in scalar
// registers); lanes with nothing to do use an offset past every range instead,
// so their loads read zeros and their stores are dropped.
constexpr int kDead = 0x7fffff00;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t crsrc(const void* base, int range) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, __builtin_amdgcn_readfirstlane(range),
                                             kBufWord3);
}
__device__ __forceinline__ uint4 cld16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void cst16(__amdgpu_buffer_rsrc_t r, int off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(cu32x4, v), r, off, 0, 0);
}
// silu on the hardware exp2 and reciprocal (about 1 ulp each)
__device__ __forceinline__ float csilu(float u) {
    return u * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * u));
}

// VEC floats of an fp32 row at element offset e (16-byte pieces)
template <int VEC>
__device__ __forceinline__ void ld_f32(__amdgpu_buffer_rsrc_t r, int e, float* f) {
#pragma unroll
    for (int i = 0; i < VEC / 4; ++i) CPiece<float>::unpack(cld16(r, (e + 4 * i) * 4), f + 4 * i);
}
template <int VEC, int CPOL = 0>
__device__ __forceinline__ void st_f32(__amdgpu_buffer_rsrc_t r, int e, const float* f) {
#pragma unroll
    for (int i = 0; i < VEC / 4; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(cu32x4, CPiece<float>::pack(f + 4 * i)), r,
                                               (e + 4 * i) * 4, 0, CPOL);
}

// Per-thread filter: taps w[c][j] and bias of the thread's VEC channels.
template <int VEC>
struct Taps {
    float w[VEC][kConvK];
    float b[VEC];
    __device__ void load(const ConvArgs& a, int c0, bool live) {
        const __amdgpu_buffer_rsrc_t rw = crsrc(a.w, a.D * kConvK * 4);
        const int ow = live ? c0 * kConvK * 4 : kDead;
        float f[VEC * kConvK];
#pragma unroll
        for (int i = 0; i < VEC * kConvK / 4; ++i) CPiece<float>::unpack(cld16(rw, ow + 16 * i), f + 4 * i);
#pragma unroll
        for (int c = 0; c < VEC; ++c)
#pragma unroll
            for (int j = 0; j < kConvK; ++j) w[c][j] = f[c * kConvK + j];
        const __amdgpu_buffer_rsrc_t rb = crsrc(a.bias, a.bias ? a.D * 4 : 0);
        const int ob = live ? c0 * 4 : kDead;
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) CPiece<float>::unpack(cld16(rb, ob + 16 * i), b + 4 * i);
    }
    // u = bias + w0 x_{t-3} + w1 x_{t-2} + w2 x_{t-1} + w3 x_t, in that order
    __device__ float out(int c, float x3, float x2, float x1, float x0) const {
        float u = b[c];
        u = fmaf(w[c][0], x3, u);
        u = fmaf(w[c][1], x2, u);
        u = fmaf(w[c][2], x1, u);
        u = fmaf(w[c][3], x0, u);
        return csilu(u);
    }
};

// Prefill: thread (piece p, run r, sequence b) produces tokens [32 r, 32 r + 32).
template <typename E>
__global__ __launch_bounds__(kConvThreads) void conv_prefill_kernel(ConvArgs a) {
    constexpr int VEC = CPiece<E>::N, ES = (int)sizeof(E);
    const int P = a.D / VEC;
    const int p = blockIdx.x * kConvThreads + threadIdx.x;
    const bool live = p < P;
    const int c0 = live ? p * VEC : 0;
    const int b = blockIdx.z;
    const int t0 = blockIdx.y * kConvRun;
    const long T = a.T, D = a.D;

    Taps<VEC> tp;
    tp.load(a, c0, live);

    // inputs of this sequence from token t0 - 3: rows past the end read zero
    const E* xs = static_cast<const E*>(a.x) + ((long)b * T) * D;
    const int lo = t0 >= kConvK - 1 ? t0 - (kConvK - 1) : 0;          // first row read from x
    const long rows = T - lo < kConvRun + kConvK - 1 ? T - lo : kConvRun + kConvK - 1;
    const __amdgpu_buffer_rsrc_t rx = crsrc(xs + (long)lo * D, rows > 0 ? (int)(rows * D * ES) : 0);
    auto xoff = [&](int t) { return live ? (int)(((long)(t - lo) * D + c0) * ES) : kDead; };

    // the three inputs before t0: from x, or (first run) from the window
    float h[kConvK - 1][VEC];   // h[0] = x_{t0-3}, h[2] = x_{t0-1}
    const __amdgpu_buffer_rsrc_t rwin =
        crsrc(a.win_in ? a.win_in + (long)b * kConvK * D : nullptr, a.win_in ? (int)(kConvK * D * 4) : 0);
    auto woff = [&](long t) { return live ? (int)(((kConvK + t) * D + c0) * 4) : kDead; };   // t < 0
#pragma unroll
    for (int i = 0; i < kConvK - 1; ++i) {
        const int t = t0 - (kConvK - 1) + i;
        if (t >= 0) CPiece<E>::unpack(cld16(rx, xoff(t)), h[i]);
        else                                                        // zeros without a window
#pragma unroll
            for (int j = 0; j < VEC / 4; ++j) CPiece<float>::unpack(cld16(rwin, woff(t) + 16 * j), h[i] + 4 * j);
    }

    const __amdgpu_buffer_rsrc_t ry =
        crsrc(static_cast<E*>(a.y) + ((long)b * T + t0) * D, t0 < T ? (int)((T - t0 < kConvRun ? T - t0 : kConvRun) * D * ES) : 0);
#pragma unroll
    for (int g0 = 0; g0 < kConvRun; g0 += kConvGroup) {
        uint4 raw[kConvGroup];
#pragma unroll
        for (int i = 0; i < kConvGroup; ++i) raw[i] = cld16(rx, xoff(t0 + g0 + i));
#pragma unroll
        for (int i = 0; i < kConvGroup; ++i) {
            float xt[VEC], yv[VEC];
            CPiece<E>::unpack(raw[i], xt);
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                yv[c] = tp.out(c, h[0][c], h[1][c], h[2][c], xt[c]);
                h[0][c] = h[1][c];
                h[1][c] = h[2][c];
                h[2][c] = xt[c];
            }
            cst16(ry, live ? (int)(((long)(g0 + i) * D + c0) * ES) : kDead, CPiece<E>::pack(yv));
        }
    }

    // window after the last token, written by the first run's threads (which
    // alone read win_in, so the window may be updated in place)
    if (a.win_out && blockIdx.y == 0 && live) {
        float wv[kConvK][VEC];
        const int tl = (int)(T >= kConvK ? T - kConvK : 0);
        const long rl = T - tl;
        const __amdgpu_buffer_rsrc_t rt = crsrc(xs + (long)tl * D, (int)(rl * D * ES));
#pragma unroll
        for (int s = 0; s < kConvK; ++s) {
            const long t = T - kConvK + s;
            if (t >= 0) CPiece<E>::unpack(cld16(rt, (int)(((t - tl) * D + c0) * ES)), wv[s]);
            else
#pragma unroll
                for (int j = 0; j < VEC / 4; ++j) CPiece<float>::unpack(cld16(rwin, woff(t) + 16 * j), wv[s] + 4 * j);
        }
        const __amdgpu_buffer_rsrc_t ro = crsrc(a.win_out + (long)b * kConvK * D, (int)(kConvK * D * 4));
#pragma unroll
        for (int s = 0; s < kConvK; ++s) st_f32<VEC>(ro, s * a.D + c0, wv[s]);
    }
}

// Decode: thread (piece p, row n): shift the window, append x_n, one output.
template <typename E, bool POOL>
__global__ __launch_bounds__(kConvThreads) void conv_decode_kernel(ConvArgs a) {
    constexpr int VEC = CPiece<E>::N, ES = (int)sizeof(E);
    const int P = a.D / VEC;
    const int p = blockIdx.x * kConvThreads + threadIdx.x;
    if (p >= P) return;
    const int c0 = p * VEC;
    const int n = blockIdx.y;
    const long D = a.D;
    long page = n;
    bool pad = false;
    if constexpr (POOL) {
        const int slot = a.slots[n];
        pad = slot < 0 || slot >= a.P;
        page = pad ? 0 : slot;
    }
    const __amdgpu_buffer_rsrc_t ry = crsrc(static_cast<E*>(a.y) + (long)n * D, (int)(D * ES));
    if (pad) {   // padding row: zero output, no window access
        cst16(ry, c0 * ES, uint4{0u, 0u, 0u, 0u});
        return;
    }
    Taps<VEC> tp;
    tp.load(a, c0, true);
    const __amdgpu_buffer_rsrc_t rwin = crsrc(a.win_out + page * kConvK * D, (int)(kConvK * D * 4));
    float h[kConvK - 1][VEC];
#pragma unroll
    for (int s = 1; s < kConvK; ++s) ld_f32<VEC>(rwin, (int)(s * D + c0), h[s - 1]);
    float xt[VEC], yv[VEC];
    const __amdgpu_buffer_rsrc_t rx = crsrc(static_cast<const E*>(a.x) + (long)n * D, (int)(D * ES));
    CPiece<E>::unpack(cld16(rx, c0 * ES), xt);
#pragma unroll
    for (int c = 0; c < VEC; ++c) yv[c] = tp.out(c, h[0][c], h[1][c], h[2][c], xt[c]);
    cst16(ry, c0 * ES, CPiece<E>::pack(yv));
    // the window drops its oldest input: slots 0..K-2 <- old slots 1..K-1, slot K-1 <- x_n
    // (non-temporal stores: 25.2 -> 24.7 us for 1,280 rows; non-temporal loads were slower)
#pragma unroll
    for (int s = 0; s < kConvK - 1; ++s) st_f32<VEC, kCpolNT>(rwin, (int)(s * D + c0), h[s]);
    st_f32<VEC, kCpolNT>(rwin, (int)((kConvK - 1) * D + c0), xt);
}

}  // namespace

bool conv_supported(int D, int K) { return K == kConvK && D % 8 == 0 && D <= (1 << 20); }

hipError_t launch_conv_prefill(bool bf16_io, const ConvArgs& a, hipStream_t stream) {
    const int vec = bf16_io ? 8 : 4;
    // T == 0 still runs the first run's threads: they pass the window through
    const long runs = a.T > 0 ? (a.T + kConvRun - 1) / kConvRun : 1;
    const dim3 grid((unsigned)((a.D / vec + kConvThreads - 1) / kConvThreads), (unsigned)runs, (unsigned)a.B);
    if (bf16_io) hipLaunchKernelGGL(conv_prefill_kernel<bf16>, grid, dim3(kConvThreads), 0, stream, a);
    else hipLaunchKernelGGL(conv_prefill_kernel<float>, grid, dim3(kConvThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_conv_decode(bool bf16_io, const ConvArgs& a, hipStream_t stream) {
    const int vec = bf16_io ? 8 : 4;
    const dim3 grid((unsigned)((a.D / vec + kConvThreads - 1) / kConvThreads), (unsigned)a.B);
#define GLA_CD(E_, POOL_) hipLaunchKernelGGL((conv_decode_kernel<E_, POOL_>), grid, dim3(kConvThreads), 0, stream, a)
    if (bf16_io) {
        if (a.slots) GLA_CD(bf16, true);
        else GLA_CD(bf16, false);
    } else {
        if (a.slots) GLA_CD(float, true);
        else GLA_CD(float, false);
    }
#undef GLA_CD
    return hipGetLastError();
}

}  // namespace gla

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
// One wave per (row, head): lanes stride the dk and dv features, the two sums
// (gate logit and sum of squares) are butterfly reductions in a fixed order.
// 2 * dk + 4 * dv elements move per (row, head) for 7 dv + 2 dk flops-ish, so
// the pass is bound by HBM.
#include "gla_common.hpp"
#include "gla_internal.hpp"
#include "gla_tile.hpp"

namespace gla {
namespace {

template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void epilogue_kernel(EpilogueArgs a) {
    const int lane = threadIdx.x % 64;
    const long unit = (long)blockIdx.x * 4 + threadIdx.x / 64;  // m * H + h
    if (unit >= a.units) return;                                  // whole wave
    const int h = (int)(unit % a.H);
    const E* q = static_cast<const E*>(a.q) + unit * DK;
    const E* k = static_cast<const E*>(a.k) + unit * DK;
    const E* v = static_cast<const E*>(a.v) + unit * DV;
    const E* o = static_cast<const E*>(a.o) + unit * DV;
    const E* g = static_cast<const E*>(a.g) + unit * DV;
    E* y = static_cast<E*>(a.y) + unit * DV;

    float z = 0.f;
    if (a.aug_a) {
        const float* ah = a.aug_a + (size_t)h * DK;
#pragma unroll
        for (int i = lane; i < DK; i += 64) z += to_f32(q[i]) * ah[i] * to_f32(k[i]);
    }
    z = wave_sum(z);
    const float s = 1.f / (1.f + expf(-z));

    constexpr int NC = (DV + 63) / 64;
    float x[NC];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = lane + 64 * j;
        x[j] = c < DV ? to_f32(o[c]) + s * to_f32(v[c]) : 0.f;
        ss += x[j] * x[j];
    }
    ss = wave_sum(ss);
    const float inv = 1.f / sqrtf(ss / DV + a.eps);
    const float* w = a.norm_w + (size_t)a.tier[h] * DV;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = lane + 64 * j;
        if (c < DV) {
            const float gc = to_f32(g[c]);
            y[c] = from_f32<E>(gc / (1.f + expf(-gc)) * x[j] * inv * w[c]);
        }
    }
}

}  // namespace

bool epilogue_supported(int dk, int dv) { return (dk == 96 && dv == 192) || (dk == 16 && dv == 32); }

hipError_t launch_epilogue(bool bf16_io, int dk, int dv, const EpilogueArgs& a, hipStream_t stream) {
    const unsigned blocks = (unsigned)((a.units + 3) / 4);
#define GLA_EPI(E_, DK_, DV_) \
    hipLaunchKernelGGL((epilogue_kernel<E_, DK_, DV_>), dim3(blocks), dim3(256), 0, stream, a)
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

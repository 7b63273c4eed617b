// gla_decode.hip -- batched single-token decode step (one fused launch).
//
// Laplace 3B post, section "Optimizing inference on Trainium2": every sequence
// owns one fixed state page that each decode step reads and writes; section
// "GLA mixer": S <- lambda_h S + k v^T, then o = scale S^T q on the new state.
//
// The step moves 2 * dk * dv * 4 bytes of fp32 state per (sequence, head) and
// does 4 * dk * dv flops on it (0.5 flop/byte), so it is bound by HBM: no
// MFMA, just wide coalesced non-temporal loads/stores, fp32 FMAs, and an LDS
// reduction of the per-thread column partial sums.
//
// One workgroup per (sequence, head).  Thread t owns float4 column group
// cg = t % (DV/4) and rows r = rg, rg + RG, ... with rg = t / (DV/4); its
// loads of one row sweep are contiguous across the workgroup.
//
// Pool form (same section: one fixed page per sequence, serving batches padded
// to fixed widths): row n of the batch uses page slots[n] of a pool of P pages
// [P][H][dk][dv]; a slot outside [0, P) (-1 marks a padding row) touches no
// page and yields a zero output.  Every (row, head) is computed alone, so a
// sequence's results do not depend on the batch it is in.
//
// Epilogue form (section "GLA mixer", the sentences after the readout): the
// workgroup holds a head's whole output row, so the value copy gated by
// sigmoid(q . (a (.) k)), the head RMSNorm of the head's tier and the SiLU(g)
// gate are applied before the store (as in gla_epilogue.hip).
#include "gla_common.hpp"
#include "gla_internal.hpp"
#include "gla_tile.hpp"

namespace gla {

template <typename E, int DK, int DV, int RG, bool POOL, bool EPI>
__global__ __launch_bounds__((DV / 4) * RG) void decode_kernel(
    int H, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ lambda, float* __restrict__ S, const int* __restrict__ slots, int P, float scale,
    E* __restrict__ o, EpilogueArgs ep) {
    constexpr int NCG = DV / 4;          // float4 column groups per row
    constexpr int NT = NCG * RG;         // threads
    constexpr int RPT = DK / RG;         // rows per thread
    static_assert(DK % RG == 0, "rows must split evenly");

    __shared__ float qs[DK + 1];   // (slot DK: written by the threads past DK, never read)
    __shared__ float ks[DK + 1];
    __shared__ f32x4 part[RG][NCG];
    __shared__ float red[NT / 64 + 1];    // epilogue: gate logit, per-wave sums of squares

    const int unit = blockIdx.x;         // n * H + h
    const int h = unit % H;
    const int t = threadIdx.x;
    const int cg = t % NCG;
    const int rg = t / NCG;
    size_t page = unit;                  // state page of this (row, head)
    if constexpr (POOL) {
        const int slot = slots[unit / H];
        if (slot < 0 || slot >= P) {     // padding row: no state access, zero output
            for (int c = t; c < DV; c += NT) o[(size_t)unit * DV + c] = from_f32<E>(0.f);
            return;
        }
        page = (size_t)slot * H + h;
    }

    // q, k and v are requested first, then the state; q and k are staged once they
    // arrive while the state loads are still in flight (the memory counter is in
    // order, so the staging waits only for the loads issued ahead of the state).
    // (Every thread loads an element and stores it, threads past DK the first one
    // into a spare slot, so no branch holds the loads back behind the state's.)
    static_assert(DK <= NT, "one q, k element per thread");
    const int tq = t < DK ? t : 0;
    const E qv = q[(size_t)unit * DK + tq];
    const E kv = k[(size_t)unit * DK + tq];
    E vr[4];   // (converted after the state loads are issued: a conversion here would wait)
#pragma unroll
    for (int e = 0; e < 4; ++e) vr[e] = v[(size_t)unit * DV + cg * 4 + e];
    __builtin_amdgcn_sched_barrier(0);   // q, k, v issued ahead of the state loads
    f32x4* Sp = reinterpret_cast<f32x4*>(S + page * DK * DV);
    f32x4 st[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) st[i] = __builtin_nontemporal_load(Sp + (size_t)(rg + i * RG) * NCG + cg);
    __builtin_amdgcn_sched_barrier(0);   // every load above is issued before the staging waits
    qs[t < DK ? t : DK] = to_f32(qv);
    ks[t < DK ? t : DK] = to_f32(kv);
    float vc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) vc[e] = to_f32(vr[e]);
    const float lam = lambda[h];
    __syncthreads();

    f32x4 acc = zero4();
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + i * RG;
        const float kr = ks[r], qr = qs[r];
        f32x4 s = st[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s[e] = fmaf(lam, s[e], kr * vc[e]);
            acc[e] = fmaf(s[e], qr, acc[e]);
        }
        __builtin_nontemporal_store(s, Sp + (size_t)r * NCG + cg);
    }
    part[rg][cg] = acc;
    if constexpr (EPI) {
        // gate logit q . (a_h (.) k) by the first wave (a = 0 without aug_a)
        if (t < 64) {
            float zp = 0.f;
            if (ep.aug_a)
                for (int i = t; i < DK; i += 64) zp += qs[i] * ep.aug_a[(size_t)h * DK + i] * ks[i];
            zp = wave_sum(zp);
            if (t == 0) red[NT / 64] = zp;
        }
    }
    __syncthreads();
    if constexpr (!EPI) {
        for (int c = t; c < DV; c += NT) {
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < RG; ++j) sum += part[j][c / 4][c % 4];
            o[(size_t)unit * DV + c] = from_f32<E>(scale * sum);
        }
    } else {
        static_assert(DV <= NT, "one output column per thread");
        const float s = 1.f / (1.f + expf(-red[NT / 64]));
        float x = 0.f;
        if (t < DV) {
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < RG; ++j) sum += part[j][t / 4][t % 4];
            x = scale * sum + s * to_f32(v[(size_t)unit * DV + t]);
        }
        const float ssw = wave_sum(x * x);
        __syncthreads();  // the gate logit has been read
        if (t % 64 == 0) red[t / 64] = ssw;
        __syncthreads();
        float ss = 0.f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) ss += red[w];
        if (t < DV) {
            const float inv = 1.f / sqrtf(ss / DV + ep.eps);
            const float gc = to_f32(static_cast<const E*>(ep.g)[(size_t)unit * DV + t]);
            o[(size_t)unit * DV + t] =
                from_f32<E>(gc / (1.f + expf(-gc)) * x * inv * ep.norm_w[(size_t)ep.tier[h] * DV + t]);
        }
    }
}

template <typename E, int DK, int DV, int RG>
static hipError_t launch_decode_t(int N, int H, const void* q, const void* k, const void* v,
                                  const float* lambda, float* S, const int* slots, int P, float scale, void* o,
                                  const EpilogueArgs* epi, hipStream_t stream) {
    const int units = N * H;
    const EpilogueArgs ep = epi ? *epi : EpilogueArgs{};
#define GLA_DEC(POOL_, EPI_)                                                                                     \
    hipLaunchKernelGGL((decode_kernel<E, DK, DV, RG, POOL_, EPI_>), dim3(units), dim3((DV / 4) * RG), 0, stream, \
                       H, static_cast<const E*>(q), static_cast<const E*>(k), static_cast<const E*>(v), lambda,  \
                       S, slots, P, scale, static_cast<E*>(o), ep)
    if (slots) {
        if (epi) GLA_DEC(true, true);
        else GLA_DEC(true, false);
    } else {
        if (epi) GLA_DEC(false, true);
        else GLA_DEC(false, false);
    }
#undef GLA_DEC
    return hipGetLastError();
}

bool decode_supported(int dk, int dv) {
    return (dk == 96 && dv == 192) || (dk == 16 && dv == 32);
}

hipError_t launch_decode(bool bf16_io, int N, int H, int dk, int dv, const void* q, const void* k,
                         const void* v, const float* lambda, float* S, const int* slots, int P, float scale,
                         void* o, const EpilogueArgs* epi, hipStream_t stream) {
    if (dk == 96 && dv == 192) {
        return bf16_io
                   ? launch_decode_t<bf16, 96, 192, 4>(N, H, q, k, v, lambda, S, slots, P, scale, o, epi, stream)
                   : launch_decode_t<float, 96, 192, 4>(N, H, q, k, v, lambda, S, slots, P, scale, o, epi, stream);
    }
    return bf16_io ? launch_decode_t<bf16, 16, 32, 16>(N, H, q, k, v, lambda, S, slots, P, scale, o, epi, stream)
                   : launch_decode_t<float, 16, 32, 16>(N, H, q, k, v, lambda, S, slots, P, scale, o, epi, stream);
}

}  // namespace gla

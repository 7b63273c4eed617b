// gla_api.hip -- the extern "C" boundary of libgla (declared in include/gla.h).
//
// Host-side validation runs to completion before any HIP call, so an error
// return enqueues nothing.  The library allocates nothing and keeps no state.
#include "gla.h"
#include "gla_internal.hpp"

#include <stdint.h>

#include <cmath>

namespace {

// gfx950 parts (MI350X / MI355X) have 256 compute units; the launch plan is
// sized for that fixed count so workspace sizes never depend on a device query.
constexpr int kPlanCUs = 256;
constexpr long kMaxGridY = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }
bool ok_dtype(int dt) { return dt == GLA_F32 || dt == GLA_BF16; }

// Element counts must stay addressable; 2^40 elements is far above any HBM size.
bool sane_count(long a, long b, long c, long d) {
    const double n = (double)a * (double)b * (double)c * (double)d;
    return n < 1.0e12;
}

int fwd_check_shape(int dtype, int B, int T, int H, int dk, int dv, int chunk) {
    if (!ok_dtype(dtype) || B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1 || chunk < 1) return GLA_ERR_INVALID_ARG;
    if (!sane_count(B, T, H, dk > dv ? dk : dv)) return GLA_ERR_INVALID_ARG;
    if (!gla::fwd_supported(dtype == GLA_BF16, dk, dv, chunk)) return GLA_ERR_UNSUPPORTED;
    if ((long)B * H > kMaxGridY) return GLA_ERR_UNSUPPORTED;
    return GLA_OK;
}

int bwd_check_shape(int dtype, int B, int T, int H, int dk, int dv, int chunk) {
    if (!ok_dtype(dtype) || B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1 || chunk < 1) return GLA_ERR_INVALID_ARG;
    if (!sane_count(B, T, H, dk > dv ? dk : dv)) return GLA_ERR_INVALID_ARG;
    if (!gla::bwd_supported(dtype == GLA_BF16, dk, dv, chunk)) return GLA_ERR_UNSUPPORTED;
    if ((long)B * H > kMaxGridY) return GLA_ERR_UNSUPPORTED;
    return GLA_OK;
}

// Checks the epilogue parameters and fills the device-side argument block
// (tier map by value).  Tensor pointers are checked by the callers.
int epi_fill(const gla_epilogue_params* ep, int H, int dk, int dv, gla::EpilogueArgs* a) {
    if (ep == nullptr || !ok_ptr(ep->norm_w) || !ok_opt(ep->aug_a) || ep->head_tier == nullptr ||
        ep->n_tiers < 1 || ep->n_tiers > GLA_EPI_MAX_HEADS || !(ep->eps >= 0.f) || !std::isfinite(ep->eps))
        return GLA_ERR_INVALID_ARG;
    if (H > GLA_EPI_MAX_HEADS || !gla::epilogue_supported(dk, dv)) return GLA_ERR_UNSUPPORTED;
    *a = gla::EpilogueArgs{};
    for (int h = 0; h < H; ++h) {
        const int t = ep->head_tier[h];
        if (t < 0 || t >= ep->n_tiers) return GLA_ERR_INVALID_ARG;
        a->tier[h] = t;
    }
    a->H = H;
    a->aug_a = ep->aug_a;
    a->norm_w = ep->norm_w;
    a->n_tiers = ep->n_tiers;
    a->eps = ep->eps;
    return GLA_OK;
}

static_assert(GLA_EPI_MAX_HEADS == gla::kEpiMaxHeads, "tier map capacity");

}  // namespace

extern "C" {

int gla_abi_version(void) { return 3; }

const char* gla_status_str(int status) {
    switch (status) {
        case GLA_OK: return "GLA_OK";
        case GLA_ERR_INVALID_ARG: return "GLA_ERR_INVALID_ARG: null/misaligned pointer or invalid size";
        case GLA_ERR_UNSUPPORTED: return "GLA_ERR_UNSUPPORTED: no kernel for this dtype/dk/dv/chunk";
        case GLA_ERR_WORKSPACE: return "GLA_ERR_WORKSPACE: workspace missing or too small";
        case GLA_ERR_DEVICE: return "GLA_ERR_DEVICE: HIP launch failed";
        default: return "GLA_ERR_UNKNOWN";
    }
}

size_t gla_fwd_workspace_bytes(int dtype, int B, int T, int H, int dk, int dv, int chunk) {
    if (fwd_check_shape(dtype, B, T, H, dk, dv, chunk) != GLA_OK) return 0;
    return gla::fwd_plan(dtype == GLA_BF16, B, T, H, dk, dv, chunk, kPlanCUs).ws_bytes;
}

int gla_fwd_chunked(int dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q, const void* k,
                    const void* v, const float* lambda, const float* S0, float scale, void* o, float* S_final,
                    void* ws, size_t ws_bytes, void* stream) {
    int st = fwd_check_shape(dtype, B, T, H, dk, dv, chunk);
    if (st != GLA_OK) return st;
    if (T > 0 && (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(lambda)))
        return GLA_ERR_INVALID_ARG;
    if (!ok_opt(S0) || !ok_opt(S_final)) return GLA_ERR_INVALID_ARG;
    const gla::FwdPlan plan = gla::fwd_plan(dtype == GLA_BF16, B, T, H, dk, dv, chunk, kPlanCUs);
    if (plan.ws_bytes > 0 && (!ok_ptr(ws) || ws_bytes < plan.ws_bytes)) return GLA_ERR_WORKSPACE;
    const hipError_t err = gla::launch_fwd(dtype == GLA_BF16, plan, B, T, H, dk, dv, chunk, q, k, v, lambda, S0,
                                           scale, o, S_final, nullptr, ws, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GLA_OK : GLA_ERR_DEVICE;
}

size_t gla_bwd_workspace_bytes(int dtype, int B, int T, int H, int dk, int dv, int chunk) {
    if (bwd_check_shape(dtype, B, T, H, dk, dv, chunk) != GLA_OK) return 0;
    return gla::bwd_plan(dtype == GLA_BF16, B, T, H, dk, dv, chunk, kPlanCUs).ws_bytes;
}

int gla_bwd_chunked(int dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q, const void* k,
                    const void* v, const float* lambda, const float* S0, float scale, const void* d_o,
                    const float* dS_final, void* dq, void* dk_out, void* dv_out, float* dlambda, float* dS0,
                    void* ws, size_t ws_bytes, void* stream) {
    int st = bwd_check_shape(dtype, B, T, H, dk, dv, chunk);
    if (st != GLA_OK) return st;
    if (T > 0 && (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(lambda) || !ok_ptr(d_o) || !ok_ptr(dq) ||
                  !ok_ptr(dk_out) || !ok_ptr(dv_out)))
        return GLA_ERR_INVALID_ARG;
    if (!ok_opt(S0) || !ok_opt(dS_final) || !ok_opt(dlambda) || !ok_opt(dS0)) return GLA_ERR_INVALID_ARG;
    const gla::BwdPlan plan = gla::bwd_plan(dtype == GLA_BF16, B, T, H, dk, dv, chunk, kPlanCUs);
    if (T > 0 && (!ok_ptr(ws) || ws_bytes < plan.ws_bytes)) return GLA_ERR_WORKSPACE;
    const hipError_t err =
        gla::launch_bwd(dtype == GLA_BF16, plan, B, T, H, dk, dv, chunk, q, k, v, lambda, S0, scale, d_o, dS_final,
                        dq, dk_out, dv_out, dlambda, dS0, nullptr, ws, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GLA_OK : GLA_ERR_DEVICE;
}

size_t gla_fwd_states_bytes(int dtype, int B, int T, int H, int dk, int dv, int chunk) {
    if (fwd_check_shape(dtype, B, T, H, dk, dv, chunk) != GLA_OK) return 0;
    const size_t nc = ((size_t)T + chunk - 1) / chunk;
    return (size_t)B * H * nc * dk * dv * (dtype == GLA_BF16 ? 2 : 4);
}

int gla_fwd_chunked_states(int dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q, const void* k,
                           const void* v, const float* lambda, const float* S0, float scale, void* o, float* S_final,
                           void* states, void* ws, size_t ws_bytes, void* stream) {
    int st = fwd_check_shape(dtype, B, T, H, dk, dv, chunk);
    if (st != GLA_OK) return st;
    if (!gla::bwd_supported(dtype == GLA_BF16, dk, dv, chunk)) return GLA_ERR_UNSUPPORTED;
    if (T > 0 && (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(lambda) || !ok_ptr(states)))
        return GLA_ERR_INVALID_ARG;
    if (!ok_opt(S0) || !ok_opt(S_final)) return GLA_ERR_INVALID_ARG;
    const gla::FwdPlan plan = gla::fwd_plan(dtype == GLA_BF16, B, T, H, dk, dv, chunk, kPlanCUs);
    if (plan.ws_bytes > 0 && (!ok_ptr(ws) || ws_bytes < plan.ws_bytes)) return GLA_ERR_WORKSPACE;
    const hipError_t err = gla::launch_fwd(dtype == GLA_BF16, plan, B, T, H, dk, dv, chunk, q, k, v, lambda, S0,
                                           scale, o, S_final, T > 0 ? states : nullptr, ws,
                                           static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GLA_OK : GLA_ERR_DEVICE;
}

int gla_bwd_chunked_states(int dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q, const void* k,
                           const void* v, const float* lambda, const float* S0, float scale, const void* d_o,
                           const float* dS_final, const void* states, void* dq, void* dk_out, void* dv_out,
                           float* dlambda, float* dS0, void* ws, size_t ws_bytes, void* stream) {
    int st = bwd_check_shape(dtype, B, T, H, dk, dv, chunk);
    if (st != GLA_OK) return st;
    if (T > 0 && (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(lambda) || !ok_ptr(d_o) || !ok_ptr(dq) ||
                  !ok_ptr(dk_out) || !ok_ptr(dv_out) || !ok_ptr(states)))
        return GLA_ERR_INVALID_ARG;
    if (!ok_opt(S0) || !ok_opt(dS_final) || !ok_opt(dlambda) || !ok_opt(dS0)) return GLA_ERR_INVALID_ARG;
    const gla::BwdPlan plan = gla::bwd_plan(dtype == GLA_BF16, B, T, H, dk, dv, chunk, kPlanCUs);
    if (T > 0 && (!ok_ptr(ws) || ws_bytes < plan.ws_bytes)) return GLA_ERR_WORKSPACE;
    const hipError_t err =
        gla::launch_bwd(dtype == GLA_BF16, plan, B, T, H, dk, dv, chunk, q, k, v, lambda, S0, scale, d_o, dS_final,
                        dq, dk_out, dv_out, dlambda, dS0, T > 0 ? states : nullptr, ws,
                        static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GLA_OK : GLA_ERR_DEVICE;
}

int gla_decode_step(int dtype, int N, int H, int dk, int dv, const void* q, const void* k, const void* v,
                    const float* lambda, float* S, float scale, void* o, void* stream) {
    if (!ok_dtype(dtype) || N < 0 || H < 1 || dk < 1 || dv < 1) return GLA_ERR_INVALID_ARG;
    if (!sane_count(N, H, dk, dv)) return GLA_ERR_INVALID_ARG;
    if (!gla::decode_supported(dk, dv)) return GLA_ERR_UNSUPPORTED;
    if ((long)N * H > 2147483647L) return GLA_ERR_UNSUPPORTED;
    if (N == 0) return GLA_OK;
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(lambda) || !ok_ptr(S) || !ok_ptr(o))
        return GLA_ERR_INVALID_ARG;
    const hipError_t err = gla::launch_decode(dtype == GLA_BF16, N, H, dk, dv, q, k, v, lambda, S, nullptr, 0,
                                              scale, o, nullptr, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GLA_OK : GLA_ERR_DEVICE;
}

int gla_decode_step_pool(int dtype, int N, int H, int dk, int dv, const void* q, const void* k, const void* v,
                         const float* lambda, float* pool, int P, const int* slots, float scale, void* o,
                         void* stream) {
    if (!ok_dtype(dtype) || N < 0 || H < 1 || dk < 1 || dv < 1 || P < 0) return GLA_ERR_INVALID_ARG;
    if (!sane_count(N, H, dk, dv) || !sane_count(P, H, dk, dv)) return GLA_ERR_INVALID_ARG;
    if (!gla::decode_supported(dk, dv)) return GLA_ERR_UNSUPPORTED;
    if ((long)N * H > 2147483647L) return GLA_ERR_UNSUPPORTED;
    if (N == 0) return GLA_OK;
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(lambda) || !ok_ptr(o) || !ok_ptr(slots))
        return GLA_ERR_INVALID_ARG;
    if (P > 0 && !ok_ptr(pool)) return GLA_ERR_INVALID_ARG;
    const hipError_t err = gla::launch_decode(dtype == GLA_BF16, N, H, dk, dv, q, k, v, lambda, pool, slots, P,
                                              scale, o, nullptr, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GLA_OK : GLA_ERR_DEVICE;
}

int gla_mixer_epilogue(int dtype, int M, int H, int dk, int dv, const void* q, const void* k, const void* v,
                       const void* o, const void* g, const gla_epilogue_params* ep, void* y, void* stream) {
    if (!ok_dtype(dtype) || M < 0 || H < 1 || dk < 1 || dv < 1) return GLA_ERR_INVALID_ARG;
    if (!sane_count(M, H, dk, dv)) return GLA_ERR_INVALID_ARG;
    gla::EpilogueArgs a;
    const int st = epi_fill(ep, H, dk, dv, &a);
    if (st != GLA_OK) return st;
    if (M == 0) return GLA_OK;
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(g) || !ok_ptr(y))
        return GLA_ERR_INVALID_ARG;
    a.units = (long)M * H;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.g = g;
    a.y = y;
    const hipError_t err = gla::launch_epilogue(dtype == GLA_BF16, dk, dv, a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GLA_OK : GLA_ERR_DEVICE;
}

int gla_fwd_chunked_epilogue(int dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q, const void* k,
                             const void* v, const float* lambda, const float* S0, float scale, const void* g,
                             const gla_epilogue_params* ep, void* y, float* S_final, void* ws, size_t ws_bytes,
                             void* stream) {
    int st = fwd_check_shape(dtype, B, T, H, dk, dv, chunk);
    if (st != GLA_OK) return st;
    gla::EpilogueArgs a;
    st = epi_fill(ep, H, dk, dv, &a);
    if (st != GLA_OK) return st;
    if (T > 0 && (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(y) || !ok_ptr(g) || !ok_ptr(lambda)))
        return GLA_ERR_INVALID_ARG;
    if (!ok_opt(S0) || !ok_opt(S_final)) return GLA_ERR_INVALID_ARG;
    const gla::FwdPlan plan = gla::fwd_plan(dtype == GLA_BF16, B, T, H, dk, dv, chunk, kPlanCUs);
    if (plan.ws_bytes > 0 && (!ok_ptr(ws) || ws_bytes < plan.ws_bytes)) return GLA_ERR_WORKSPACE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    a.units = (long)B * T * H;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = y;
    a.g = g;
    a.y = y;
    if (dtype == GLA_BF16 && T > 0) {
        const hipError_t err = gla::launch_fwd_bf16_epilogue(plan, B, T, H, chunk, q, k, v, lambda, S0, scale, y,
                                                             S_final, ws, a, s);
        if (err == hipSuccess) return GLA_OK;
        if (err != hipErrorNotSupported) return GLA_ERR_DEVICE;
    }
    // other plans: the readout into y, then the epilogue pass over y in place
    hipError_t err = gla::launch_fwd(dtype == GLA_BF16, plan, B, T, H, dk, dv, chunk, q, k, v, lambda, S0, scale, y,
                                     S_final, nullptr, ws, s);
    if (err == hipSuccess && a.units > 0) err = gla::launch_epilogue(dtype == GLA_BF16, dk, dv, a, s);
    return err == hipSuccess ? GLA_OK : GLA_ERR_DEVICE;
}

int gla_decode_step_epilogue(int dtype, int N, int H, int dk, int dv, const void* q, const void* k, const void* v,
                             const void* g, const float* lambda, float* S, int P, const int* slots, float scale,
                             const gla_epilogue_params* ep, void* y, void* stream) {
    if (!ok_dtype(dtype) || N < 0 || H < 1 || dk < 1 || dv < 1) return GLA_ERR_INVALID_ARG;
    if (slots != nullptr && P < 0) return GLA_ERR_INVALID_ARG;
    if (!sane_count(N, H, dk, dv) || (slots != nullptr && !sane_count(P, H, dk, dv))) return GLA_ERR_INVALID_ARG;
    if (!gla::decode_supported(dk, dv)) return GLA_ERR_UNSUPPORTED;
    if ((long)N * H > 2147483647L) return GLA_ERR_UNSUPPORTED;
    gla::EpilogueArgs a;
    const int st = epi_fill(ep, H, dk, dv, &a);
    if (st != GLA_OK) return st;
    if (N == 0) return GLA_OK;
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(g) || !ok_ptr(lambda) || !ok_ptr(y) || !ok_opt(slots))
        return GLA_ERR_INVALID_ARG;
    if ((slots == nullptr || P > 0) && !ok_ptr(S)) return GLA_ERR_INVALID_ARG;
    a.units = (long)N * H;
    a.g = g;
    const hipError_t err = gla::launch_decode(dtype == GLA_BF16, N, H, dk, dv, q, k, v, lambda, S, slots,
                                              slots ? P : 0, scale, y, &a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GLA_OK : GLA_ERR_DEVICE;
}

int gla_conv1d_silu(int dtype, int B, int T, int D, int K, const void* x, const float* w, const float* bias,
                    const float* win_in, void* y, float* win_out, void* stream) {
    if (!ok_dtype(dtype) || B < 0 || T < 0 || D < 1 || K < 1) return GLA_ERR_INVALID_ARG;
    if (!sane_count(B, T, D, 1) || !sane_count(B, K, D, 1)) return GLA_ERR_INVALID_ARG;
    if (!gla::conv_supported(D, K)) return GLA_ERR_UNSUPPORTED;
    if (T > 65535L * 32 || B > 65535) return GLA_ERR_UNSUPPORTED;
    if (B == 0 || (T == 0 && win_out == nullptr)) return GLA_OK;
    if (!ok_ptr(w) || !ok_opt(bias) || !ok_opt(win_in) || !ok_opt(win_out)) return GLA_ERR_INVALID_ARG;
    if (T > 0 && (!ok_ptr(x) || !ok_ptr(y))) return GLA_ERR_INVALID_ARG;
    gla::ConvArgs a{};
    a.B = B;
    a.T = T;
    a.D = D;
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.win_in = win_in;
    a.y = y;
    a.win_out = win_out;
    const hipError_t err = gla::launch_conv_prefill(dtype == GLA_BF16, a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GLA_OK : GLA_ERR_DEVICE;
}

int gla_conv1d_silu_decode(int dtype, int N, int D, int K, const void* x, const float* w, const float* bias,
                           float* win, int P, const int* slots, void* y, void* stream) {
    if (!ok_dtype(dtype) || N < 0 || D < 1 || K < 1) return GLA_ERR_INVALID_ARG;
    if (slots != nullptr && P < 0) return GLA_ERR_INVALID_ARG;
    if (!sane_count(N, K, D, 1) || (slots != nullptr && !sane_count(P, K, D, 1))) return GLA_ERR_INVALID_ARG;
    if (!gla::conv_supported(D, K)) return GLA_ERR_UNSUPPORTED;
    if (N > 65535) return GLA_ERR_UNSUPPORTED;
    if (N == 0) return GLA_OK;
    if (!ok_ptr(x) || !ok_ptr(y) || !ok_ptr(w) || !ok_opt(bias) || !ok_opt(slots)) return GLA_ERR_INVALID_ARG;
    if ((slots == nullptr || P > 0) && !ok_ptr(win)) return GLA_ERR_INVALID_ARG;
    gla::ConvArgs a{};
    a.B = N;
    a.T = 1;
    a.D = D;
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.y = y;
    a.win_out = win;
    a.slots = slots;
    a.P = slots ? P : 0;
    const hipError_t err = gla::launch_conv_decode(dtype == GLA_BF16, a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GLA_OK : GLA_ERR_DEVICE;
}

}  // extern "C"

// gla_api.hip -- the extern "C" boundary of libgla (declared in include/gla.h
// and, for the launch-plan controls, include/gla_plan.h).
//
// Host-side validation runs to completion before any HIP call, so an error
// return enqueues nothing.  The library allocates nothing and keeps no state.
// Every chunked forward and backward entry point goes through fwd_entry /
// bwd_entry below with the optional features it exposes.
#include "gla.h"
#include "gla_internal.hpp"
#include "gla_plan.h"

#include <stdint.h>

#include <cmath>
#include <mutex>

namespace {

// gfx950 parts (MI350X / MI355X) have 256 compute units; the launch plan is
// sized for that fixed count so workspace sizes never depend on a device query.
constexpr int kPlanCUs = 256;
constexpr long kMaxGridY = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }
bool ok_dtype(int dt) { return dt == GLA_F32 || dt == GLA_BF16; }
int esize(gla_dtype dt) { return dt == GLA_BF16 ? 2 : 4; }

// Element counts must stay addressable; 2^40 elements is far above any HBM size.
bool sane_count(long a, long b, long c, long d) {
    const double n = (double)a * (double)b * (double)c * (double)d;
    return n < 1.0e12;
}

gla_status fwd_check_shape(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk) {
    if (!ok_dtype(dtype) || B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1 || chunk < 1) return GLA_ERR_INVALID_ARG;
    if (!sane_count(B, T, H, dk > dv ? dk : dv)) return GLA_ERR_INVALID_ARG;
    if (!gla::fwd_supported(dtype == GLA_BF16, dk, dv, chunk)) return GLA_ERR_UNSUPPORTED;
    if ((long)B * H > kMaxGridY) return GLA_ERR_UNSUPPORTED;
    return GLA_OK;
}

gla_status bwd_check_shape(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk) {
    if (!ok_dtype(dtype) || B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1 || chunk < 1) return GLA_ERR_INVALID_ARG;
    if (!sane_count(B, T, H, dk > dv ? dk : dv)) return GLA_ERR_INVALID_ARG;
    if (!gla::bwd_supported(dtype == GLA_BF16, dk, dv, chunk)) return GLA_ERR_UNSUPPORTED;
    if ((long)B * H > kMaxGridY) return GLA_ERR_UNSUPPORTED;
    return GLA_OK;
}

// Plan hint from the caller's gla_plan (NULL: all library choices).
bool hint_of(const gla_plan* p, gla::PlanHint* h) {
    *h = gla::PlanHint{0, -1, 0, -1};
    if (p == nullptr) return true;
    if (p->segments < 0 || p->segments > gla::kMaxSegments || p->chain < -1 || p->chain > 1 || p->psub < 0 ||
        p->psub > 1 || p->scan < -1 || p->scan > 1)
        return false;
    *h = gla::PlanHint{p->segments, p->chain, p->psub, p->scan};
    return true;
}

// One tensor's element strides; a zero field takes its packed value (token:
// H * d, batch: T * token).  Token strides are multiples of 16 bytes, at least
// a token's H * d elements and below 2^22; batch strides are multiples of 16
// bytes.  An output's sequences must not overlap each other.
bool resolve_stride(const gla_stride* s, int B, int T, int H, int D, int esz, bool output, gla::Tok* r) {
    const long long row = (long long)H * D;
    long long t = s ? s->token : 0, b = s ? s->batch : 0;
    if (t < 0 || b < 0) return false;
    if (t == 0) t = row;
    if (b == 0) b = (long long)T * t;
    const long long align = 16 / esz;
    if (t < row || t % align != 0 || t >= gla::kMaxTokStride || b % align != 0) return false;
    if (output && B > 1 && T > 0 && b < (long long)(T - 1) * t + row) return false;
    r->t = (int)t;
    r->b = b;
    return true;
}

// Checks the epilogue parameters and fills the device-side argument block
// (tier map by value).  Tensor pointers are checked by the callers.
gla_status epi_fill(const gla_epilogue_params* ep, int H, int dk, int dv, gla::EpilogueArgs* a) {
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
    a->rq = a->rk = H * dk;
    a->rv = a->ro = a->rg = a->ry = H * dv;
    return GLA_OK;
}

static_assert(GLA_EPI_MAX_HEADS == gla::kEpiMaxHeads, "tier map capacity");

gla_status device_status(hipError_t err) { return err == hipSuccess ? GLA_OK : GLA_ERR_DEVICE; }

// A validated chunked forward, ready to launch: every chunk's start state saved
// to `states` for the backward (with_states), and the fused epilogue (ep != NULL:
// o receives y).
struct FwdCall {
    bool bf;
    int B, T, H, dk, dv, chunk;
    gla::FwdIO io;
    const float* lambda;
    const float* S0;
    float scale;
    float* S_final;
    void* states;       // null unless saved
    bool epi;
    gla::EpilogueArgs ea;
    gla::FwdPlan plan;
};

// All host-side checks of a forward; fills `c` on success.  Makes no HIP call.
gla_status fwd_prepare(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q, const void* k,
                       const void* v, const float* lambda, const float* S0, float scale, void* o, float* S_final,
                       bool with_states, void* states, const void* g, const gla_epilogue_params* ep,
                       const gla_strides* st, const gla_plan* plan_in, FwdCall* c) {
    gla_status s = fwd_check_shape(dtype, B, T, H, dk, dv, chunk);
    if (s != GLA_OK) return s;
    const bool bf = dtype == GLA_BF16;
    if (with_states && !gla::bwd_supported(bf, dk, dv, chunk)) return GLA_ERR_UNSUPPORTED;
    if (with_states && ep) return GLA_ERR_UNSUPPORTED;
    gla::PlanHint hint;
    if (!hint_of(plan_in, &hint)) return GLA_ERR_INVALID_ARG;
    *c = FwdCall{};
    if (ep && (s = epi_fill(ep, H, dk, dv, &c->ea)) != GLA_OK) return s;
    if (T > 0 && (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o) || !ok_ptr(lambda))) return GLA_ERR_INVALID_ARG;
    if (T > 0 && with_states && !ok_ptr(states)) return GLA_ERR_INVALID_ARG;
    if (T > 0 && ep && !ok_ptr(g)) return GLA_ERR_INVALID_ARG;
    if (!ok_opt(S0) || !ok_opt(S_final)) return GLA_ERR_INVALID_ARG;
    const int es = esize(dtype);
    c->io = gla::FwdIO{q, k, v, o, {}, {}, {}, {}};
    gla::Tok sg{};
    if (!resolve_stride(st ? &st->q : nullptr, B, T, H, dk, es, false, &c->io.sq) ||
        !resolve_stride(st ? &st->k : nullptr, B, T, H, dk, es, false, &c->io.sk) ||
        !resolve_stride(st ? &st->v : nullptr, B, T, H, dv, es, false, &c->io.sv) ||
        !resolve_stride(st ? &st->o : nullptr, B, T, H, dv, es, true, &c->io.so) ||
        (ep && !resolve_stride(st ? &st->g : nullptr, B, T, H, dv, es, false, &sg)))
        return GLA_ERR_INVALID_ARG;
    c->bf = bf;
    c->B = B;
    c->T = T;
    c->H = H;
    c->dk = dk;
    c->dv = dv;
    c->chunk = chunk;
    c->lambda = lambda;
    c->S0 = S0;
    c->scale = scale;
    c->S_final = S_final;
    c->states = T > 0 && with_states ? states : nullptr;
    c->epi = ep != nullptr;
    c->ea.sg = sg;
    c->ea.g = g;
    c->plan = gla::fwd_plan(bf, B, T, H, dk, dv, chunk, kPlanCUs, &hint);
    return GLA_OK;
}

// Launches a prepared forward with its workspace.
gla_status fwd_run(const FwdCall& c, void* ws, size_t ws_bytes, hipStream_t stream) {
    const int B = c.B, T = c.T, H = c.H, dk = c.dk, dv = c.dv, chunk = c.chunk;
    if (c.plan.ws_bytes > 0 && T > 0 && (!ok_ptr(ws) || ws_bytes < c.plan.ws_bytes)) return GLA_ERR_WORKSPACE;
    if (!c.epi)
        return device_status(gla::launch_fwd(c.bf, c.plan, B, T, H, dk, dv, chunk, c.io, c.lambda, c.S0, c.scale,
                                             c.S_final, c.states, ws, stream));
    gla::EpilogueArgs ea = c.ea;
    if (c.bf && T > 0) {
        const hipError_t err = gla::launch_fwd_bf16_epilogue(c.plan, B, T, H, chunk, c.io, c.lambda, c.S0, c.scale,
                                                             c.S_final, ws, ea, stream);
        if (err == hipSuccess) return GLA_OK;
        if (err != hipErrorNotSupported) return GLA_ERR_DEVICE;
    }
    // other plans: the readout into y, then the epilogue pass over y in place
    hipError_t err = gla::launch_fwd(c.bf, c.plan, B, T, H, dk, dv, chunk, c.io, c.lambda, c.S0, c.scale, c.S_final,
                                     nullptr, ws, stream);
    if (err != hipSuccess || T == 0) return device_status(err);
    const gla::FwdIO& io = c.io;
    const gla::Tok sg = ea.sg;
    ea.rq = io.sq.t;
    ea.rk = io.sk.t;
    ea.rv = io.sv.t;
    ea.ro = ea.ry = io.so.t;
    ea.rg = sg.t;
    // rows equally spaced across the batch as well: one pass over all B * T rows
    const bool uniform = io.sq.b == (long long)T * io.sq.t && io.sk.b == (long long)T * io.sk.t &&
                         io.sv.b == (long long)T * io.sv.t && io.so.b == (long long)T * io.so.t &&
                         sg.b == (long long)T * sg.t;
    const int passes = uniform ? 1 : B;
    const int es = c.bf ? 2 : 4;
    ea.units = (long)(uniform ? B : 1) * T * H;
    for (int b = 0; b < passes && err == hipSuccess; ++b) {
        gla::EpilogueArgs eb = ea;
        eb.q = static_cast<const char*>(io.q) + b * io.sq.b * es;
        eb.k = static_cast<const char*>(io.k) + b * io.sk.b * es;
        eb.v = static_cast<const char*>(io.v) + b * io.sv.b * es;
        eb.o = static_cast<const char*>(io.o) + b * io.so.b * es;
        eb.y = static_cast<char*>(io.o) + b * io.so.b * es;
        eb.g = static_cast<const char*>(ea.g) + b * sg.b * es;
        err = gla::launch_epilogue(c.bf, dk, dv, eb, stream);
    }
    return device_status(err);
}

gla_status fwd_entry(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q, const void* k,
                     const void* v, const float* lambda, const float* S0, float scale, void* o, float* S_final,
                     bool with_states, void* states, const void* g, const gla_epilogue_params* ep,
                     const gla_strides* st, const gla_plan* plan_in, void* ws, size_t ws_bytes, hipStream_t stream) {
    FwdCall c;
    const gla_status s = fwd_prepare(dtype, B, T, H, dk, dv, chunk, q, k, v, lambda, S0, scale, o, S_final,
                                     with_states, states, g, ep, st, plan_in, &c);
    return s != GLA_OK ? s : fwd_run(c, ws, ws_bytes, stream);
}

size_t fwd_ws_bytes(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, const gla_plan* plan_in) {
    gla::PlanHint hint;
    if (fwd_check_shape(dtype, B, T, H, dk, dv, chunk) != GLA_OK || !hint_of(plan_in, &hint)) return 0;
    return gla::fwd_plan(dtype == GLA_BF16, B, T, H, dk, dv, chunk, kPlanCUs, &hint).ws_bytes;
}

// The chunked backward; `states` (nullable) are the chunk start states saved
// by the forward.
gla_status bwd_entry(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q, const void* k,
                     const void* v, const float* lambda, const float* S0, float scale, const void* d_o,
                     const float* dS_final, const void* states, void* dq, void* dk_out, void* dv_out, float* dlambda,
                     float* dS0, const gla_strides* st, const gla_plan* plan_in, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
    gla_status s = bwd_check_shape(dtype, B, T, H, dk, dv, chunk);
    if (s != GLA_OK) return s;
    gla::PlanHint hint;
    if (!hint_of(plan_in, &hint)) return GLA_ERR_INVALID_ARG;
    if (T > 0 && (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(lambda) || !ok_ptr(d_o) || !ok_ptr(dq) ||
                  !ok_ptr(dk_out) || !ok_ptr(dv_out)))
        return GLA_ERR_INVALID_ARG;
    if (!ok_opt(S0) || !ok_opt(dS_final) || !ok_opt(dlambda) || !ok_opt(dS0) || !ok_opt(states))
        return GLA_ERR_INVALID_ARG;
    const int es = esize(dtype);
    gla::BwdIO io{q, k, v, d_o, dq, dk_out, dv_out, {}, {}, {}, {}, {}, {}, {}};
    if (!resolve_stride(st ? &st->q : nullptr, B, T, H, dk, es, false, &io.sq) ||
        !resolve_stride(st ? &st->k : nullptr, B, T, H, dk, es, false, &io.sk) ||
        !resolve_stride(st ? &st->v : nullptr, B, T, H, dv, es, false, &io.sv) ||
        !resolve_stride(st ? &st->d_o : nullptr, B, T, H, dv, es, false, &io.sdo) ||
        !resolve_stride(st ? &st->dq : nullptr, B, T, H, dk, es, true, &io.sdq) ||
        !resolve_stride(st ? &st->dk : nullptr, B, T, H, dk, es, true, &io.sdk) ||
        !resolve_stride(st ? &st->dv : nullptr, B, T, H, dv, es, true, &io.sdv))
        return GLA_ERR_INVALID_ARG;
    const bool saved = states != nullptr && T > 0;
    const gla::BwdPlan plan = gla::bwd_plan(dtype == GLA_BF16, B, T, H, dk, dv, chunk, kPlanCUs, saved, &hint);
    if (T > 0 && (!ok_ptr(ws) || ws_bytes < plan.ws_bytes)) return GLA_ERR_WORKSPACE;
    return device_status(gla::launch_bwd(dtype == GLA_BF16, plan, B, T, H, dk, dv, chunk, io, lambda, S0, scale,
                                         dS_final, dlambda, dS0, saved ? states : nullptr, ws, stream));
}

size_t bwd_ws_bytes(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, bool saved,
                    const gla_plan* plan_in) {
    gla::PlanHint hint;
    if (bwd_check_shape(dtype, B, T, H, dk, dv, chunk) != GLA_OK || !hint_of(plan_in, &hint)) return 0;
    return gla::bwd_plan(dtype == GLA_BF16, B, T, H, dk, dv, chunk, kPlanCUs, saved && T > 0, &hint).ws_bytes;
}

}  // namespace

// ---------------------------------------------------------------- allocation-free forward
//
// gla_fwd_chunked_noalloc keeps the forward's workspace in this fixed device
// array instead of caller memory.  Every device the library runs on holds its
// own copy for the life of the process; host code never uses the array's name
// as an address (it is a host-side stand-in): it asks the runtime for each
// device's address once and passes that to the kernels.
constexpr size_t kScratchBytes = (size_t)GLA_NOALLOC_WORKSPACE_MAX;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // per device: the address of `scratch` there

// The scratch array's address on the current device (looked up on the first
// call on that device, with it current).
gla_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GLA_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GLA_ERR_DEVICE;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GLA_OK;
}

}  // namespace

extern "C" {

gla_status gla_fwd_chunked_noalloc(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q,
                                   const void* k, const void* v, const float* lambda, const float* S0, float scale,
                                   void* o, float* S_final, const gla_strides* st, void* stream) {
    FwdCall c;
    gla_status s = fwd_prepare(dtype, B, T, H, dk, dv, chunk, q, k, v, lambda, S0, scale, o, S_final, false, nullptr,
                               nullptr, nullptr, st, nullptr, &c);
    if (s != GLA_OK) return s;
    if (c.plan.ws_bytes > kScratchBytes) return GLA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (c.plan.ws_bytes > 0 && T > 0 && (s = scratch_on_current_device(&ws)) != GLA_OK) return s;
    // (the forward writes every workspace byte it reads before reading it: no clearing)
    return fwd_run(c, ws, kScratchBytes, static_cast<hipStream_t>(stream));
}

int gla_abi_version(void) { return 4; }

const char* gla_status_str(gla_status status) {
    switch (status) {
        case GLA_OK: return "GLA_OK";
        case GLA_ERR_INVALID_ARG: return "GLA_ERR_INVALID_ARG: null/misaligned pointer, invalid size or stride";
        case GLA_ERR_UNSUPPORTED: return "GLA_ERR_UNSUPPORTED: no kernel for this dtype/dk/dv/chunk";
        case GLA_ERR_WORKSPACE: return "GLA_ERR_WORKSPACE: workspace missing or too small";
        case GLA_ERR_DEVICE: return "GLA_ERR_DEVICE: HIP launch failed";
        default: return "GLA_ERR_UNKNOWN";
    }
}

size_t gla_fwd_workspace_bytes(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk) {
    return fwd_ws_bytes(dtype, B, T, H, dk, dv, chunk, nullptr);
}

gla_status gla_fwd_chunked(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q,
                           const void* k, const void* v, const float* lambda, const float* S0, float scale, void* o,
                           float* S_final, const gla_strides* st, void* ws, size_t ws_bytes, void* stream) {
    return fwd_entry(dtype, B, T, H, dk, dv, chunk, q, k, v, lambda, S0, scale, o, S_final, false, nullptr, nullptr,
                     nullptr, st, nullptr, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

size_t gla_bwd_workspace_bytes(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk) {
    return bwd_ws_bytes(dtype, B, T, H, dk, dv, chunk, false, nullptr);
}

gla_status gla_bwd_chunked(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q,
                           const void* k, const void* v, const float* lambda, const float* S0, float scale,
                           const void* d_o, const float* dS_final, void* dq, void* dk_out, void* dv_out,
                           float* dlambda, float* dS0, const gla_strides* st, void* ws, size_t ws_bytes,
                           void* stream) {
    return bwd_entry(dtype, B, T, H, dk, dv, chunk, q, k, v, lambda, S0, scale, d_o, dS_final, nullptr, dq, dk_out,
                     dv_out, dlambda, dS0, st, nullptr, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

size_t gla_fwd_states_bytes(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk) {
    if (fwd_check_shape(dtype, B, T, H, dk, dv, chunk) != GLA_OK) return 0;
    const size_t nc = ((size_t)T + chunk - 1) / chunk;
    return (size_t)B * H * nc * dk * dv * esize(dtype);
}

gla_status gla_fwd_chunked_states(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q,
                                  const void* k, const void* v, const float* lambda, const float* S0, float scale,
                                  void* o, float* S_final, void* states, const gla_strides* st, void* ws,
                                  size_t ws_bytes, void* stream) {
    return fwd_entry(dtype, B, T, H, dk, dv, chunk, q, k, v, lambda, S0, scale, o, S_final, true, states, nullptr,
                     nullptr, st, nullptr, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

size_t gla_bwd_states_workspace_bytes(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk) {
    return bwd_ws_bytes(dtype, B, T, H, dk, dv, chunk, true, nullptr);
}

gla_status gla_bwd_chunked_states(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q,
                                  const void* k, const void* v, const float* lambda, const float* S0, float scale,
                                  const void* d_o, const float* dS_final, const void* states, void* dq, void* dk_out,
                                  void* dv_out, float* dlambda, float* dS0, const gla_strides* st, void* ws,
                                  size_t ws_bytes, void* stream) {
    if (T > 0 && !ok_ptr(states)) {
        const gla_status s = bwd_check_shape(dtype, B, T, H, dk, dv, chunk);
        return s != GLA_OK ? s : GLA_ERR_INVALID_ARG;
    }
    return bwd_entry(dtype, B, T, H, dk, dv, chunk, q, k, v, lambda, S0, scale, d_o, dS_final, states, dq, dk_out,
                     dv_out, dlambda, dS0, st, nullptr, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

gla_status gla_fwd_chunked_epilogue(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q,
                                    const void* k, const void* v, const float* lambda, const float* S0, float scale,
                                    const void* g, const gla_epilogue_params* ep, void* y, float* S_final,
                                    const gla_strides* st, void* ws, size_t ws_bytes, void* stream) {
    if (ep == nullptr) {
        const gla_status s = fwd_check_shape(dtype, B, T, H, dk, dv, chunk);
        return s != GLA_OK ? s : GLA_ERR_INVALID_ARG;
    }
    return fwd_entry(dtype, B, T, H, dk, dv, chunk, q, k, v, lambda, S0, scale, y, S_final, false, nullptr, g, ep, st,
                     nullptr, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- launch-plan controls (gla_plan.h)

gla_status gla_plan_resolve(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, const gla_plan* hint_in,
                            gla_plan* out) {
    const gla_status s = fwd_check_shape(dtype, B, T, H, dk, dv, chunk);
    if (s != GLA_OK) return s;
    gla::PlanHint hint;
    if (!hint_of(hint_in, &hint) || out == nullptr) return GLA_ERR_INVALID_ARG;
    const gla::FwdPlan p = gla::fwd_plan(dtype == GLA_BF16, B, T, H, dk, dv, chunk, kPlanCUs, &hint);
    out->segments = p.nseg;
    out->chain = p.chain;
    out->psub = p.psub;
    out->scan = p.fuse_scan;
    return GLA_OK;
}

size_t gla_fwd_workspace_bytes_planned(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                                       const gla_plan* plan) {
    return fwd_ws_bytes(dtype, B, T, H, dk, dv, chunk, plan);
}

size_t gla_bwd_workspace_bytes_planned(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                                       int saved_states, const gla_plan* plan) {
    return bwd_ws_bytes(dtype, B, T, H, dk, dv, chunk, saved_states != 0, plan);
}

gla_status gla_fwd_chunked_planned(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q,
                                   const void* k, const void* v, const float* lambda, const float* S0, float scale,
                                   void* o, float* S_final, void* states, const void* g,
                                   const gla_epilogue_params* ep, const gla_strides* st, const gla_plan* plan,
                                   void* ws, size_t ws_bytes, void* stream) {
    return fwd_entry(dtype, B, T, H, dk, dv, chunk, q, k, v, lambda, S0, scale, o, S_final, states != nullptr, states,
                     g, ep, st, plan, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

gla_status gla_bwd_chunked_planned(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, const void* q,
                                   const void* k, const void* v, const float* lambda, const float* S0, float scale,
                                   const void* d_o, const float* dS_final, const void* states, void* dq, void* dk_out,
                                   void* dv_out, float* dlambda, float* dS0, const gla_strides* st,
                                   const gla_plan* plan, void* ws, size_t ws_bytes, void* stream) {
    return bwd_entry(dtype, B, T, H, dk, dv, chunk, q, k, v, lambda, S0, scale, d_o, dS_final, states, dq, dk_out,
                     dv_out, dlambda, dS0, st, plan, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- decode, epilogue, conv

gla_status gla_decode_step(gla_dtype dtype, int N, int H, int dk, int dv, const void* q, const void* k, const void* v,
                           const float* lambda, float* S, float scale, void* o, void* stream) {
    if (!ok_dtype(dtype) || N < 0 || H < 1 || dk < 1 || dv < 1) return GLA_ERR_INVALID_ARG;
    if (!sane_count(N, H, dk, dv)) return GLA_ERR_INVALID_ARG;
    if (!gla::decode_supported(dk, dv)) return GLA_ERR_UNSUPPORTED;
    if ((long)N * H > 2147483647L) return GLA_ERR_UNSUPPORTED;
    if (N == 0) return GLA_OK;
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(lambda) || !ok_ptr(S) || !ok_ptr(o))
        return GLA_ERR_INVALID_ARG;
    return device_status(gla::launch_decode(dtype == GLA_BF16, N, H, dk, dv, q, k, v, lambda, S, nullptr, 0, scale, o,
                                            nullptr, static_cast<hipStream_t>(stream)));
}

gla_status gla_decode_step_pool(gla_dtype dtype, int N, int H, int dk, int dv, const void* q, const void* k,
                                const void* v, const float* lambda, float* pool, int P, const int* slots, float scale,
                                void* o, void* stream) {
    if (!ok_dtype(dtype) || N < 0 || H < 1 || dk < 1 || dv < 1 || P < 0) return GLA_ERR_INVALID_ARG;
    if (!sane_count(N, H, dk, dv) || !sane_count(P, H, dk, dv)) return GLA_ERR_INVALID_ARG;
    if (!gla::decode_supported(dk, dv)) return GLA_ERR_UNSUPPORTED;
    if ((long)N * H > 2147483647L) return GLA_ERR_UNSUPPORTED;
    if (N == 0) return GLA_OK;
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(lambda) || !ok_ptr(o) || !ok_ptr(slots))
        return GLA_ERR_INVALID_ARG;
    if (P > 0 && !ok_ptr(pool)) return GLA_ERR_INVALID_ARG;
    return device_status(gla::launch_decode(dtype == GLA_BF16, N, H, dk, dv, q, k, v, lambda, pool, slots, P, scale, o,
                                            nullptr, static_cast<hipStream_t>(stream)));
}

gla_status gla_mixer_epilogue(gla_dtype dtype, int M, int H, int dk, int dv, const void* q, const void* k,
                              const void* v, const void* o, const void* g, const gla_epilogue_params* ep, void* y,
                              void* stream) {
    if (!ok_dtype(dtype) || M < 0 || H < 1 || dk < 1 || dv < 1) return GLA_ERR_INVALID_ARG;
    if (!sane_count(M, H, dk, dv)) return GLA_ERR_INVALID_ARG;
    gla::EpilogueArgs a;
    const gla_status st = epi_fill(ep, H, dk, dv, &a);
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
    return device_status(gla::launch_epilogue(dtype == GLA_BF16, dk, dv, a, static_cast<hipStream_t>(stream)));
}

gla_status gla_decode_step_epilogue(gla_dtype dtype, int N, int H, int dk, int dv, const void* q, const void* k,
                                    const void* v, const void* g, const float* lambda, float* S, int P,
                                    const int* slots, float scale, const gla_epilogue_params* ep, void* y,
                                    void* stream) {
    if (!ok_dtype(dtype) || N < 0 || H < 1 || dk < 1 || dv < 1) return GLA_ERR_INVALID_ARG;
    if (slots != nullptr && P < 0) return GLA_ERR_INVALID_ARG;
    if (!sane_count(N, H, dk, dv) || (slots != nullptr && !sane_count(P, H, dk, dv))) return GLA_ERR_INVALID_ARG;
    if (!gla::decode_supported(dk, dv)) return GLA_ERR_UNSUPPORTED;
    if ((long)N * H > 2147483647L) return GLA_ERR_UNSUPPORTED;
    gla::EpilogueArgs a;
    const gla_status st = epi_fill(ep, H, dk, dv, &a);
    if (st != GLA_OK) return st;
    if (N == 0) return GLA_OK;
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(g) || !ok_ptr(lambda) || !ok_ptr(y) || !ok_opt(slots))
        return GLA_ERR_INVALID_ARG;
    if ((slots == nullptr || P > 0) && !ok_ptr(S)) return GLA_ERR_INVALID_ARG;
    a.units = (long)N * H;
    a.g = g;
    return device_status(gla::launch_decode(dtype == GLA_BF16, N, H, dk, dv, q, k, v, lambda, S, slots,
                                            slots ? P : 0, scale, y, &a, static_cast<hipStream_t>(stream)));
}

gla_status gla_conv1d_silu(gla_dtype dtype, int B, int T, int D, int K, const void* x, const float* w,
                           const float* bias, const float* win_in, void* y, float* win_out, void* stream) {
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
    return device_status(gla::launch_conv_prefill(dtype == GLA_BF16, a, static_cast<hipStream_t>(stream)));
}

gla_status gla_conv1d_silu_decode(gla_dtype dtype, int N, int D, int K, const void* x, const float* w,
                                  const float* bias, float* win, int P, const int* slots, void* y, void* stream) {
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
    return device_status(gla::launch_conv_decode(dtype == GLA_BF16, a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// gla_internal.hpp -- launchers shared between the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gla {

// Element strides of a token-major tensor [B][T][H][D] whose head and feature
// dimensions are packed: element (b, t, h, d) sits at b * b_ + t * t_ + h * D + d.
// Token strides stay below 2^22 elements, so a tile's offsets fit 32 bits.
struct Tok {
    long long b;
    int t;
};
constexpr long long kMaxTokStride = 1LL << 22;

__host__ __device__ inline Tok packed_tok(int T, int H, int D) {
    return Tok{(long long)T * H * D, H * D};
}

struct FwdArgs {
    int T, H;
    const void* q;
    const void* k;
    const void* v;
    Tok sq, sk, sv, so;   // element strides of q, k, v and o
    const float* lambda;
    const float* S0;
    float scale;
    void* o;
    float* S_final;
    float* U;          // [B*H][nseg-1][DK*DV]: segment-local end states, then segment start states
    void* Ub;          // bf16 copies of the start states (bf16 path, one-chunk segments), or null
    void* sbar;        // optional: every chunk's start state, [B*H][nc][DK][DV] in the input dtype
    int nseg, seg_chunks, nc;
    int psub;          // segment states in U per segment boundary (sub-segment prologue), >= 1
    int fuse_scan;     // 1: U holds the prologue's local states; each segment folds them itself
    int units;         // B * H (the per-chunk output kernel's grid)
    int out_xcd;       // output kernel: all chunks of a unit on one XCD (else chunk-major)
};

struct FwdPlan {
    int nc;          // chunks in the sequence
    int nseg;        // sequence segments run in parallel
    int seg_chunks;  // chunks per segment (the last segment may hold fewer)
    int psub;        // bf16 segments: the state-only prologue runs psub sub-segments per segment
    int chain;       // bf16 path: tiled state chain + per-chunk output instead of segments
    int fuse_scan;   // bf16 segments: no scan launch; each segment folds the (at most
                     // kFuseMaxStates) local states before it into its start state
    size_t ws_bytes; // segments: B*H*(nseg-1)*dk*dv fp32 (+ as many bf16 on the bf16 path);
                     // chain: B*H*nc*dk*dv bf16 chunk start states
};

// The tiled chain runs the chunk recurrence itself (sequential over chunks);
// it replaces the segment split only up to this many chunks.
constexpr int kChainMaxChunks = 64;

// Launch-plan choices a caller may fix (tests, sweeps); zero fields (chain: -1)
// leave the choice to fwd_plan.
struct PlanHint {
    int nseg;   // sequence segments, 1 .. kMaxSegments (0: default)
    int chain;  // 0: segment split, 1: tiled chain where it can run (-1: default)
    int psub;   // 1: one prologue workgroup per segment (0: default)
    int scan;   // 0: a scan launch between the state passes, 1: folded where allowed (-1: default)
};

// A segment folds the local states before it into its start state itself (no
// scan launch) when there are at most this many.
constexpr int kFuseMaxStates = 2;

// Token-major operands of one forward call (pointers and their strides).
struct FwdIO {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    Tok sq, sk, sv, so;
};

bool fwd_supported(bool bf16_io, int dk, int dv, int chunk);
FwdPlan fwd_plan(bool bf16_io, int B, int T, int H, int dk, int dv, int chunk, int num_cu,
                 const PlanHint* hint = nullptr);
// sbar (nullable): also store every chunk's start state, [B*H][nc][dk][dv] in
// the input dtype (the snapshots the backward consumes).
hipError_t launch_fwd(bool bf16_io, const FwdPlan& plan, int B, int T, int H, int dk, int dv, int chunk,
                      const FwdIO& io, const float* lambda, const float* S0, float scale, float* S_final, void* sbar,
                      void* ws, hipStream_t stream);

// bf16 forward (dk = 96, dv = 192, chunk 64 or 128): prologue, scan and main launches.
hipError_t launch_fwd_bf16(const FwdPlan& plan, int B, int T, int H, int chunk, const FwdIO& io, const float* lambda,
                           const float* S0, float scale, float* S_final, void* sbar, void* ws, hipStream_t stream);

// Sequence segments run in parallel (at most this many per sequence).
constexpr int kMaxSegments = 16;

// Turns segment-local end states U_0..U_{nseg-2} into start states of
// segments 1..nseg-1 in place (forward order), starting from S0 (or 0).
hipError_t launch_seg_scan(const float* S0, float* U, const float* lambda, int H, int nseg, int seg_tokens,
                           int dkdv, unsigned units, hipStream_t stream);

// dlam partials: [B*H][chunks][kNPart] fp32.  Slot 0 holds the chunk's term
// through lam^ceff, ceff lam^(ceff-1) <Gbar, Sbar> (from the fp32 path's reverse
// chain, or from the bf16 gradient kernels, which hold both snapshots), slots
// [kChainSlots, kChainSlots + 2 * tiles) the gradient kernels' other terms.
// All are summed per head in a fixed order.
constexpr int kChainSlots = 1;
constexpr int kNPart = 16;

struct StateArgs {
    int T, H;
    const void* x;        // [B][T][H][DK]: keys (forward pass) or queries (reverse pass)
    const void* y;        // [B][T][H][DV]: values (forward pass) or output gradients (reverse pass)
    Tok sx, sy;           // their element strides
    const float* lambda;
    float xscale;         // extra row factor on x: 1 (forward) or the readout scale (reverse)
    const float* S_edge;  // state entering the pass: S0 (forward) or dS_T (reverse); nullable
    float* U;             // [BH][nseg-1][DK][DV]: segment-local states, then segment start states
    void* snap;           // [BH][NC][DK][DV] (E): per-chunk snapshots written by the emit pass
    float* S_out;         // reverse emit pass: dS0 (nullable)
    const void* sbar;     // fp32 reverse emit pass: the forward snapshots (for <Gbar, Sbar>)
    float* part;          // fp32 reverse emit pass: dlam partials (slot 0)
    int nseg, seg_chunks, nc;
    int fuse_scan;        // emit passes: U holds the local passes' states, folded here
};

// bf16 chains (dk = 96, dv = 192, chunk 32, 64, 128 or 256); grid (grid_x, units).
hipError_t launch_chain_bf16(int chunk, bool rev, bool emit, const StateArgs& s, unsigned grid_x, unsigned units,
                             hipStream_t stream);

struct GradArgs {
    int T, H;
    const void* q;
    const void* k;
    const void* v;
    const void* d_o;
    Tok sq, sk, sv, sdo, sdq, sdk, sdv;   // element strides of the token-major tensors
    const float* lambda;
    float scale;
    const void* sbar;  // [BH][NC][DK][DV] (E): chunk start states
    const void* gbar;  // [BH][NC][DK][DV] (E): chunk end state gradients
    void* dq;
    void* dk;
    void* dv;
    float* part;       // [BH][NC][kNPart]
    int nc;
    int units;         // B * H
};

// bf16 gradient kernels (dk = 96, dv = 192, chunk 32, 64, 128 or 256): dQ, dK and dV of a chunk.
hipError_t launch_grad_bf16(int chunk, const GradArgs& ga, unsigned units, hipStream_t stream);

struct BwdPlan {
    int nc, nseg, seg_chunks;
    int fuse_scan;      // bf16: the emit passes fold the local states (no scan launches)
    bool saved;         // chunk start states come from the forward (no state snapshot array here)
    size_t snap_bytes;  // per-chunk snapshots: state gradients (and, unless saved, states)
    size_t u_bytes;     // segment states (fp32)
    size_t part_bytes;  // dlambda partials
    size_t ws_bytes;    // total
};

// Token-major operands of one backward call.
struct BwdIO {
    const void* q;
    const void* k;
    const void* v;
    const void* d_o;
    void* dq;
    void* dk;
    void* dv;
    Tok sq, sk, sv, sdo, sdq, sdk, sdv;
};

bool bwd_supported(bool bf16_io, int dk, int dv, int chunk);
// saved: the backward reads the chunk start states the forward saved.
BwdPlan bwd_plan(bool bf16_io, int B, int T, int H, int dk, int dv, int chunk, int num_cu, bool saved,
                 const PlanHint* hint = nullptr);
// sbar_in (non-null exactly when plan.saved): the chunk start states saved by
// the forward; the backward then skips its own forward state pass.
hipError_t launch_bwd(bool bf16_io, const BwdPlan& plan, int B, int T, int H, int dk, int dv, int chunk,
                      const BwdIO& io, const float* lambda, const float* S0, float scale, const float* dST,
                      float* dlambda, float* dS0, const void* sbar_in, void* ws, hipStream_t stream);

bool decode_supported(int dk, int dv);
// Mixer epilogue: device pointers, the tier map travels by value.
constexpr int kEpiMaxHeads = 64;

struct EpilogueArgs {
    long units;           // rows * H
    int H;
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* g;
    void* y;
    // element strides between consecutive rows (a packed [M][H][D] tensor: H * D);
    // the forward's output kernel reads the gate through sg instead
    int rq, rk, rv, ro, rg, ry;
    Tok sg;
    const float* aug_a;
    const float* norm_w;  // [n_tiers][dv]
    int n_tiers;
    float eps;
    int tier[kEpiMaxHeads];
};

bool epilogue_supported(int dk, int dv);
hipError_t launch_epilogue(bool bf16_io, int dk, int dv, const EpilogueArgs& a, hipStream_t stream);
// bf16 forward with the epilogue in the output kernel (tiled-chain plans only;
// hipErrorNotSupported for other plans); io.o is y
hipError_t launch_fwd_bf16_epilogue(const FwdPlan& plan, int B, int T, int H, int chunk, const FwdIO& io,
                                    const float* lambda, const float* S0, float scale, float* S_final, void* ws,
                                    const EpilogueArgs& ep, hipStream_t stream);

// Depth-wise causal conv + SiLU (width 4).  Prefill: x, y [B][T][D], windows
// [B][4][D] fp32 (win_in nullable).  Decode: x, y [N = B][D], win_out is the
// in/out window [N or P][4][D]; slots nullable (row n -> window slots[n]).
struct ConvArgs {
    int B;
    long T;
    int D;
    const void* x;
    const float* w;       // [D][4]
    const float* bias;    // [D] or nullptr
    const float* win_in;
    void* y;
    float* win_out;
    const int* slots;
    int P;
};
bool conv_supported(int D, int K);
hipError_t launch_conv_prefill(bool bf16_io, const ConvArgs& a, hipStream_t stream);
hipError_t launch_conv_decode(bool bf16_io, const ConvArgs& a, hipStream_t stream);

// slots == nullptr: row n uses page n of S; else page slots[n] of a P-page pool.
// epi == nullptr: o is the readout; else o receives the epilogue output y
// (epi->g the gate; q, k, v, o, y fields of epi unused).
hipError_t launch_decode(bool bf16_io, int N, int H, int dk, int dv, const void* q, const void* k,
                         const void* v, const float* lambda, float* S, const int* slots, int P, float scale,
                         void* o, const EpilogueArgs* epi, hipStream_t stream);

}  // namespace gla

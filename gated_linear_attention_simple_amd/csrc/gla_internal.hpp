// gla_internal.hpp -- launchers shared between the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gla {

struct FwdPlan {
    int nc;          // chunks in the sequence
    int nseg;        // sequence segments run in parallel
    int seg_chunks;  // chunks per segment (the last segment may hold fewer)
    size_t ws_bytes; // segment-local states: B*H*(nseg-1)*dk*dv fp32
};

bool fwd_supported(bool bf16_io, int dk, int dv, int chunk);
FwdPlan fwd_plan(int B, int T, int H, int dk, int dv, int chunk, int num_cu);
hipError_t launch_fwd(bool bf16_io, const FwdPlan& plan, int B, int T, int H, int dk, int dv,
                      int chunk, const void* q, const void* k, const void* v, const float* lambda,
                      const float* S0, float scale, void* o, float* S_final, void* ws,
                      hipStream_t stream);

bool decode_supported(int dk, int dv);
hipError_t launch_decode(bool bf16_io, int N, int H, int dk, int dv, const void* q, const void* k,
                         const void* v, const float* lambda, float* S, float scale, void* o,
                         hipStream_t stream);

}  // namespace gla

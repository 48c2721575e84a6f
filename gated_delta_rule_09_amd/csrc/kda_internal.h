// Internal launcher interface between the C ABI (kda_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
    const void* q; const void* k; const void* v;
    const float* log_alpha; const float* beta;
    float* state; void* o;
    int32_t N, H, d_k, d_v;
    bool bf16;
    hipStream_t stream;
};

struct PrefillArgs {
    const void* q; const void* k; const void* v;
    const float* log_alpha; const float* beta;
    const float* init_state; const int32_t* cu_seqlens;
    int32_t N; int64_t total_T; int32_t H, d_k, d_v;
    bool bf16;
    void* o; float* final_state;
    hipStream_t stream;
};

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_prefill(const PrefillArgs& a);

}  // namespace kda

// Internal launcher interface between the C ABI (kda_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// With `gated` set, `log_alpha` points at decay logits z in the element type
// of q (bf16 or fp32), `beta` at fp32 write-strength logits, and `a_log` at
// the per-head log-scales A_h [H]; the kernels apply the lower-bounded map
// g = -5 Sigmoid(e^{A_h} z), beta = Sigmoid(logit) on the fly.
struct DecodeArgs {
    const void* q; const void* k; const void* v;
    const void* log_alpha; const float* beta;
    float* state; void* o;
    int32_t N, H, d_k, d_v;
    bool bf16;
    hipStream_t stream;
    bool gated = false;
    const float* a_log = nullptr;
    // With `out_gate` set (gated decode only), `o` receives
    // y = Sigmoid(out_gate) * norm_weight * o / sqrt(mean(o^2) + eps) instead of o.
    const void* out_gate = nullptr;
    const float* norm_weight = nullptr;
    float eps = 0.f;
    // With `conv_w` set as well (gated decode with the epilogue only), q, k, v
    // are projection outputs and the input prologue runs first: width-4
    // convolution (taps [H, 2 d_k + d_v, 4] fp32, state [N, 3, H, 2 d_k + d_v]
    // in the element type, updated in place), Swish, L2 norm of q and k.
    const float* conv_w = nullptr;
    void* conv_state = nullptr;
};

struct PrefillArgs {
    const void* q; const void* k; const void* v;
    const void* log_alpha; const float* beta;
    const float* init_state; const int32_t* cu_seqlens;
    int32_t N; int64_t total_T; int32_t H, d_k, d_v;
    bool bf16;
    void* o; float* final_state;
    hipStream_t stream;
    bool gated = false;
    const float* a_log = nullptr;
};

// y = Sigmoid(gate) * weight * o / sqrt(mean(o^2) + eps) over rows of d_v
// values; weight may be null (ones); y may alias o or gate.
struct EpilogueArgs {
    const void* o; const void* gate; const float* weight;
    int64_t rows; int32_t d_v; float eps;
    bool bf16;
    void* y;
    hipStream_t stream;
};

// Input prologue: q = l2(swish(conv x_q)), k = l2(swish(conv x_k)),
// v = swish(conv x_v), width-4 depthwise causal convolution per head; weights
// [H, 2 d_k + d_v, 4] fp32, states [N, 3, H, 2 d_k + d_v] in the element type.
struct PrologueArgs {
    const void* x_q; const void* x_k; const void* x_v;
    const float* conv_w;
    const void* state_in;     // null: zeros
    void* state_out;          // null: not stored; must not overlap state_in
    const int32_t* cu_seqlens;
    int32_t N; int64_t total_T; int32_t H, d_k, d_v;
    bool bf16;
    void* q; void* k; void* v;
    hipStream_t stream;
};

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_prologue(const PrologueArgs& p);
bool prologue_grid_fits(int64_t total_T, int32_t H);
hipError_t launch_epilogue(const EpilogueArgs& a);
int64_t epilogue_max_rows();
hipError_t launch_prefill(const PrefillArgs& a);

}  // namespace kda

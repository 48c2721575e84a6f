// Internal launcher interface between the C ABI (kda_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// A dispatch's x size is a 32-bit count of work-items, and its block count is
// at most 2^31 - 1: host validation rejects anything larger before any HIP call.
constexpr int64_t kMaxGridItems = 0xffffffffll;
constexpr int64_t kMaxGridBlocks = 0x7fffffffll;
inline bool grid_fits(int64_t blocks, int64_t threads) {
    return blocks >= 0 && blocks <= kMaxGridBlocks && blocks * threads <= kMaxGridItems;
}

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

// One job of a prefill launch (a kernel argument): a set of sequences over the
// launch's q, k, decay and beta, with its own values, states and outputs.
enum : int32_t { kInitAll = 0, kInitFirst = 1, kInitIdentity = 2 };
struct PrefillJob {
    const void* v;               // [T, H, d_v]; null: every value is zero
    const float* init_state;     // kInitAll: [N, H, d_k, d_v]; kInitFirst: sequence 0 only; null: zeros
    const int32_t* cu_seqlens;   // sequence offsets; null: uniform segments (seg_len > 0) or all tokens
    void* o;                     // outputs; its first row holds token o_row0
    float* final_state;          // [N, H, d_k, d_v] end states; may be null
    int64_t seg_len;             // sequence n covers [(n + n_off) seg_len, + seg_len) clipped to T
    int64_t o_row0;
    int32_t n_off;
    int32_t units;               // N * H
    int32_t blocks;              // workgroups (set by the launcher)
    int32_t init_mode;           // kInitAll, kInitFirst (state of sequence 0 only), kInitIdentity (d_v = d_k)
};

// Time-split workspace of one sequence cut into `segments` runs of seg_len
// tokens (a multiple of the 64-token chunk).
struct SplitWork {
    int32_t segments;
    int64_t seg_len;
    float* ends;     // [segments, H, d_k, d_v] fp32: end state of each segment
    float* phis;     // [segments - 1, H, d_k, d_k] fp32: transition of segments 1..
    void* qt;        // [T - seg_len, H, d_k] element type: Phi_t^T q_t of tokens seg_len..T-1
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
bool decode_grid_fits(int64_t pairs, bool prologue);
hipError_t launch_prologue(const PrologueArgs& p);
bool prologue_grid_fits(int64_t N, int64_t total_T, int32_t H, int32_t d_k, int32_t d_v, bool bf16);
hipError_t launch_epilogue(const EpilogueArgs& a);
int64_t epilogue_max_rows(bool bf16, int32_t d_v);
hipError_t launch_prefill(const PrefillArgs& a);
// Whether a launch over `units` (sequence, head) pairs at d_v value columns
// fits a dispatch; for the time split, also the transition job of `trans_units`
// pairs at d_k columns.
bool prefill_grid_fits(int64_t units, int32_t d_v);
bool split_grid_fits(int64_t run_units, int64_t trans_units, int32_t d_k, int32_t d_v);
// The library's own split scratch on the current device (allocation-free entry
// point): its address (looked up once per device) and its size.
hipError_t split_scratch(void** ptr);
size_t split_scratch_bytes();
// Bounded in-kernel waits that ran out (a guard against a logic error: each
// wait's flag is written by a wave that does not wait itself), counted on the
// current device since the last reset.
hipError_t read_wait_giveups(uint32_t* count, bool reset);
// Time split of one sequence (N = 1): the segment runs, then the serial scan
// over segment end states, then the output correction.
hipError_t launch_prefill_split_runs(const PrefillArgs& a, const SplitWork& w);
hipError_t launch_split_scan(const PrefillArgs& a, const SplitWork& w);
hipError_t launch_split_correct(const PrefillArgs& a, const SplitWork& w);

}  // namespace kda

// C ABI of libkda: host-side argument validation and dispatch to the kernels.
// Every validation failure returns before any HIP runtime call.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

thread_local char g_last_error[256] = "";

void set_error(const char* what, hipError_t e) {
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool supported_d(int32_t d) { return d == 64 || d == 128; }

// gfx950 check, cached per device id.
constexpr int kMaxDevices = 64;
int g_arch_ok[kMaxDevices];      // 0 unknown, 1 ok, -1 not gfx950
std::mutex g_arch_mu;

kda_status check_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) {
        set_error("hipGetDevice", e);
        (void)hipGetLastError();
        return KDA_ERR_NO_DEVICE;
    }
    if (dev >= kMaxDevices) return KDA_ERR_NO_DEVICE;
    std::lock_guard<std::mutex> lk(g_arch_mu);
    if (g_arch_ok[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) {
            set_error("hipGetDeviceProperties", e);
            (void)hipGetLastError();
            return KDA_ERR_NO_DEVICE;
        }
        g_arch_ok[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
        if (g_arch_ok[dev] < 0)
            snprintf(g_last_error, sizeof(g_last_error), "device %d is %s, not gfx950", dev, prop.gcnArchName);
    }
    return g_arch_ok[dev] > 0 ? KDA_OK : KDA_ERR_NO_DEVICE;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "unsupported or inconsistent sizes";
        case KDA_ERR_DTYPE: return "unsupported dtype";
        case KDA_ERR_ALIGN: return "pointer not 16-byte aligned";
        case KDA_ERR_NO_DEVICE: return "no usable gfx950 HIP device";
        case KDA_ERR_HIP: return "HIP runtime error";
        case KDA_ERR_VALUE: return "an argument value is out of range";
    }
    return "unknown status";
}

const char* kda_last_error(void) { return g_last_error; }

kda_status kda_wait_giveups(uint32_t* count, int32_t reset, void* stream) {
    if (!count) return KDA_ERR_NULL;
    kda_status st = check_device();
    if (st != KDA_OK) return st;
    hipError_t e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = kda::read_wait_giveups(count, reset != 0);
    if (e != hipSuccess) {
        set_error("kda_wait_giveups", e);
        return KDA_ERR_HIP;
    }
    if (*count != 0)
        snprintf(g_last_error, sizeof(g_last_error),
                 "%u bounded in-kernel wait(s) of the prefill ran out: outputs since the last reset are suspect",
                 *count);
    return KDA_OK;
}

}  // extern "C"

namespace {

bool valid_eps(float eps) { return isfinite(eps) && eps >= 0.f; }

// `out_gate` non-null selects the fused output epilogue (gated decode only).
kda_status decode_impl(const char* name, const void* q, const void* k, const void* v, const void* decay,
                       const float* beta, const float* a_log, bool gated, float* state, int32_t N, int32_t H,
                       int32_t d_k, int32_t d_v, kda_dtype dtype, void* o, void* stream,
                       bool epilogue = false, const void* out_gate = nullptr, const float* norm_weight = nullptr,
                       float eps = 0.f, bool prologue = false, const float* conv_w = nullptr,
                       void* conv_state = nullptr) {
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_DTYPE;
    if (N < 0 || H < 1 || !supported_d(d_k) || !supported_d(d_v)) return KDA_ERR_SHAPE;
    if (!kda::decode_grid_fits((int64_t)N * H, prologue)) return KDA_ERR_SHAPE;
    if (epilogue && !valid_eps(eps)) return KDA_ERR_VALUE;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !decay || !beta || !state || !o || (gated && !a_log) || (epilogue && !out_gate) ||
        (prologue && (!conv_w || !conv_state)))
        return KDA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(decay) ||
        !aligned16(beta) || !aligned16(state) || !aligned16(o) || (gated && !aligned16(a_log)) ||
        (epilogue && !aligned16(out_gate)) || (norm_weight && !aligned16(norm_weight)) ||
        (prologue && (!aligned16(conv_w) || !aligned16(conv_state))))
        return KDA_ERR_ALIGN;
    kda_status st = check_device();
    if (st != KDA_OK) return st;
    kda::DecodeArgs a{q, k, v, decay, beta, state, o, N, H, d_k, d_v,
                      dtype == KDA_BF16, reinterpret_cast<hipStream_t>(stream), gated, a_log,
                      epilogue ? out_gate : nullptr, norm_weight, eps,
                      prologue ? conv_w : nullptr, prologue ? conv_state : nullptr};
    hipError_t e = kda::launch_decode(a);
    if (e != hipSuccess) {
        set_error(name, e);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

kda_status prefill_impl(const char* name, const void* q, const void* k, const void* v, const void* decay,
                        const float* beta, const float* a_log, bool gated, const float* init_state,
                        const int32_t* cu_seqlens, int32_t N, int64_t total_T, int32_t H, int32_t d_k,
                        int32_t d_v, kda_dtype dtype, void* o, float* final_state, void* stream) {
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_DTYPE;
    if (N < 1 || H < 1 || total_T < 0 || !supported_d(d_k) || !supported_d(d_v)) return KDA_ERR_SHAPE;
    if (cu_seqlens == nullptr && N != 1) return KDA_ERR_SHAPE;
    if (N > 65535 || H > 65535) return KDA_ERR_SHAPE;   // grid dimensions
    if (!kda::prefill_grid_fits((int64_t)N * H, d_v)) return KDA_ERR_SHAPE;
    if (total_T > 0 && (!q || !k || !v || !decay || !beta || !o || (gated && !a_log))) return KDA_ERR_NULL;
    const void* ptrs[] = {q, k, v, decay, beta, a_log, init_state, cu_seqlens, o, final_state};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    if (total_T == 0 && final_state == nullptr) return KDA_OK;
    kda_status st = check_device();
    if (st != KDA_OK) return st;
    kda::PrefillArgs a{q, k, v, decay, beta, init_state, cu_seqlens, N, total_T, H, d_k, d_v,
                       dtype == KDA_BF16, o, final_state, reinterpret_cast<hipStream_t>(stream), gated, a_log};
    hipError_t e = kda::launch_prefill(a);
    if (e != hipSuccess) {
        set_error(name, e);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

// ---- Time split of one sequence ------------------------------------------
constexpr int64_t kChunkTokens = 64;   // the prefill kernel's chunk

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Segments of a whole number of chunks: the requested count sets the segment
// length, and that length fixes how many segments there are (never more than
// requested; one when the sequence has at most one chunk).  Workspace: the
// segment end states, the transitions of segments 1.., and Phi_t^T q_t of
// tokens seg_len.., each at a 256-byte boundary.
struct SplitPlan {
    int32_t segments = 1;
    int64_t seg_len = 0;
    size_t phis = 0, qt = 0, bytes = 0;    // offsets (the end states start at 0) and total
};

SplitPlan split_plan(int64_t total_T, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype, int32_t segments) {
    SplitPlan p;
    const int64_t chunks = (total_T + kChunkTokens - 1) / kChunkTokens;
    if (chunks <= 1 || segments <= 1) return p;
    const int64_t per = (chunks + segments - 1) / segments;
    const int32_t n = (int32_t)((chunks + per - 1) / per);
    if (n <= 1) return p;
    p.segments = n;
    p.seg_len = per * kChunkTokens;
    const size_t es = dtype == KDA_BF16 ? 2 : 4;
    p.phis = round256((size_t)n * H * d_k * d_v * 4);
    p.qt = p.phis + round256((size_t)(n - 1) * H * d_k * d_k * 4);
    p.bytes = p.qt + round256((size_t)(total_T - p.seg_len) * H * d_k * es);
    return p;
}

// `noalloc`: the workspace is the library's own scratch (workspace and
// workspace_bytes are ignored); a plan larger than it is rejected.
kda_status split_impl(const char* name, const void* q, const void* k, const void* v, const void* decay,
                      const float* beta, const float* a_log, bool gated, const float* init_state, int64_t total_T,
                      int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype, int32_t segments, void* workspace,
                      size_t workspace_bytes, void* o, float* final_state, void* stream, bool noalloc = false) {
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_DTYPE;
    if (segments < 1) return KDA_ERR_VALUE;
    if (H < 1 || H > 65535 || total_T < 0 || !supported_d(d_k) || !supported_d(d_v)) return KDA_ERR_SHAPE;
    const SplitPlan p = split_plan(total_T, H, d_k, d_v, dtype, segments);
    if (p.segments == 1)
        return prefill_impl(name, q, k, v, decay, beta, a_log, gated, init_state, nullptr, 1, total_T, H, d_k, d_v,
                            dtype, o, final_state, stream);
    if (!kda::split_grid_fits((int64_t)p.segments * H, (int64_t)(p.segments - 1) * H, d_k, d_v)) return KDA_ERR_SHAPE;
    // The correction addresses the tokens of a head in pieces of at least 512
    // (its grid is two workgroups per CU) with 32-bit byte offsets.
    const int64_t es = dtype == KDA_BF16 ? 2 : 4;
    if (512 * (int64_t)H * (d_k > d_v ? d_k : d_v) * es > (int64_t)UINT32_MAX) return KDA_ERR_SHAPE;
    if (!q || !k || !v || !decay || !beta || !o || (gated && !a_log) || (!noalloc && !workspace)) return KDA_ERR_NULL;
    const void* ptrs[] = {q, k, v, decay, beta, a_log, init_state, o, final_state, noalloc ? nullptr : workspace};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return KDA_ERR_ALIGN;
    if (noalloc && p.bytes > kda::split_scratch_bytes()) {
        snprintf(g_last_error, sizeof(g_last_error),
                 "%s: this split needs %zu bytes of scratch; the library holds %zu (use fewer segments, or the "
                 "entry point that takes a workspace)", name, p.bytes, kda::split_scratch_bytes());
        return KDA_ERR_VALUE;
    }
    if (!noalloc && workspace_bytes < p.bytes) return KDA_ERR_VALUE;
    kda_status st = check_device();
    if (st != KDA_OK) return st;
    if (noalloc) {
        hipError_t e = kda::split_scratch(&workspace);
        if (e != hipSuccess) {
            set_error(name, e);
            return KDA_ERR_HIP;
        }
    }
    kda::PrefillArgs a{q, k, v, decay, beta, init_state, nullptr, 1, total_T, H, d_k, d_v,
                       dtype == KDA_BF16, o, final_state, reinterpret_cast<hipStream_t>(stream), gated, a_log};
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    const kda::SplitWork w{p.segments, p.seg_len, reinterpret_cast<float*>(ws), reinterpret_cast<float*>(ws + p.phis),
                           ws + p.qt};
    hipError_t e = kda::launch_prefill_split_runs(a, w);
    if (e == hipSuccess) e = kda::launch_split_scan(a, w);
    if (e == hipSuccess) e = kda::launch_split_correct(a, w);
    if (e != hipSuccess) {
        set_error(name, e);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

kda_status epilogue_checks(const void* o, const void* gate, const float* weight, int64_t rows, int32_t d_v,
                           float eps, kda_dtype dtype, const void* y) {
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_DTYPE;
    if (rows < 0 || !supported_d(d_v) || rows > kda::epilogue_max_rows(dtype == KDA_BF16, d_v)) return KDA_ERR_SHAPE;
    if (!valid_eps(eps)) return KDA_ERR_VALUE;
    if (rows == 0) return KDA_OK;
    if (!o || !gate || !y) return KDA_ERR_NULL;
    if (!aligned16(o) || !aligned16(gate) || !aligned16(y) || (weight && !aligned16(weight))) return KDA_ERR_ALIGN;
    return KDA_OK;
}

kda_status epilogue_launch(const char* name, const void* o, const void* gate, const float* weight, int64_t rows,
                           int32_t d_v, float eps, kda_dtype dtype, void* y, void* stream) {
    kda::EpilogueArgs a{o, gate, weight, rows, d_v, eps, dtype == KDA_BF16, y,
                        reinterpret_cast<hipStream_t>(stream)};
    hipError_t e = kda::launch_epilogue(a);
    if (e != hipSuccess) {
        set_error(name, e);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_decode_step(const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta,
                           float* state, int32_t N, int32_t H,
                           int32_t d_k, int32_t d_v, kda_dtype dtype,
                           void* o, void* stream) {
    return decode_impl("kda_decode_step launch", q, k, v, log_alpha, beta, nullptr, false, state, N, H, d_k, d_v,
                       dtype, o, stream);
}

kda_status kda_decode_step_gated(const void* q, const void* k, const void* v,
                                 const void* g_logits, const float* a_log, const float* beta_logits,
                                 float* state, int32_t N, int32_t H,
                                 int32_t d_k, int32_t d_v, kda_dtype dtype,
                                 void* o, void* stream) {
    return decode_impl("kda_decode_step_gated launch", q, k, v, g_logits, beta_logits, a_log, true, state, N, H,
                       d_k, d_v, dtype, o, stream);
}

kda_status kda_chunk_prefill(const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta,
                             const float* init_state, const int32_t* cu_seqlens,
                             int32_t N, int64_t total_T, int32_t H,
                             int32_t d_k, int32_t d_v, kda_dtype dtype,
                             void* o, float* final_state, void* stream) {
    return prefill_impl("kda_chunk_prefill launch", q, k, v, log_alpha, beta, nullptr, false, init_state,
                        cu_seqlens, N, total_T, H, d_k, d_v, dtype, o, final_state, stream);
}

kda_status kda_chunk_prefill_gated(const void* q, const void* k, const void* v,
                                   const void* g_logits, const float* a_log, const float* beta_logits,
                                   const float* init_state, const int32_t* cu_seqlens,
                                   int32_t N, int64_t total_T, int32_t H,
                                   int32_t d_k, int32_t d_v, kda_dtype dtype,
                                   void* o, float* final_state, void* stream) {
    return prefill_impl("kda_chunk_prefill_gated launch", q, k, v, g_logits, beta_logits, a_log, true, init_state,
                        cu_seqlens, N, total_T, H, d_k, d_v, dtype, o, final_state, stream);
}

int32_t kda_split_segments(int64_t total_T, int32_t H, int32_t d_k, int32_t d_v, int32_t num_cus) {
    if (total_T <= 0 || H < 1 || H > 65535 || !supported_d(d_k) || !supported_d(d_v) || num_cus < 1) return 1;
    const int64_t chunks = (total_T + kChunkTokens - 1) / kChunkTokens;
    // Workgroups of a job of `units` (sequence, head) pairs at `cols` value
    // columns: one per 64 columns, padded to groups of 16 for 128 columns.
    auto wgs = [](int64_t units, int32_t cols) { return cols == 128 ? 16 * ((units + 7) / 8) : units; };
    auto rounds = [&](int64_t w) { return (w + num_cus - 1) / num_cus; };
    // Cost in chunk steps of one workgroup (one workgroup per CU).  The segment
    // runs take rounds x (chunks per segment); with d_v = d_k both jobs share
    // one launch.  Each scan step costs about one chunk step, and the
    // correction streams qt and o once more: about 2 (d_k + 2 d_v) bytes per
    // token-head at some 5 TB/s, against about 3 us per chunk step.
    double best = (double)rounds(wgs(H, d_v)) * chunks;
    int32_t best_n = 1;
    for (int64_t n = 2; n <= 256 && n <= chunks; ++n) {
        const int64_t per = (chunks + n - 1) / n;
        if ((chunks + per - 1) / per != n) continue;    // this count is not reachable
        const int64_t run = wgs(n * H, d_v), trans = wgs((n - 1) * H, d_k);
        const int64_t r = d_v == d_k ? rounds(run + trans) : rounds(run) + rounds(trans);
        const double corr = (double)(total_T - per * kChunkTokens) * H * (d_k + 2 * d_v) * 2.0 / 5e12 / 3e-6;
        const double cost = (double)r * per + (double)(n - 1) + corr;
        if (cost < best * 0.95) {      // a split must gain at least 5%
            best = cost;
            best_n = (int32_t)n;
        }
    }
    return best_n;
}

size_t kda_split_workspace_bytes(int64_t total_T, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype,
                                 int32_t segments) {
    if (total_T < 0 || H < 1 || !supported_d(d_k) || !supported_d(d_v) || (dtype != KDA_F32 && dtype != KDA_BF16))
        return 0;
    return split_plan(total_T, H, d_k, d_v, dtype, segments).bytes;
}

kda_status kda_chunk_prefill_split(const void* q, const void* k, const void* v,
                                   const float* log_alpha, const float* beta, const float* init_state,
                                   int64_t total_T, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype,
                                   int32_t segments, void* workspace, size_t workspace_bytes,
                                   void* o, float* final_state, void* stream) {
    return split_impl("kda_chunk_prefill_split launch", q, k, v, log_alpha, beta, nullptr, false, init_state,
                      total_T, H, d_k, d_v, dtype, segments, workspace, workspace_bytes, o, final_state, stream);
}

kda_status kda_chunk_prefill_split_noalloc(const void* q, const void* k, const void* v,
                                           const float* log_alpha, const float* beta, const float* init_state,
                                           int64_t total_T, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype,
                                           int32_t segments, void* o, float* final_state, void* stream) {
    return split_impl("kda_chunk_prefill_split_noalloc", q, k, v, log_alpha, beta, nullptr, false, init_state,
                      total_T, H, d_k, d_v, dtype, segments, nullptr, 0, o, final_state, stream, true);
}

kda_status kda_chunk_prefill_gated_split(const void* q, const void* k, const void* v,
                                         const void* g_logits, const float* a_log, const float* beta_logits,
                                         const float* init_state, int64_t total_T, int32_t H,
                                         int32_t d_k, int32_t d_v, kda_dtype dtype,
                                         int32_t segments, void* workspace, size_t workspace_bytes,
                                         void* o, float* final_state, void* stream) {
    return split_impl("kda_chunk_prefill_gated_split launch", q, k, v, g_logits, beta_logits, a_log, true,
                      init_state, total_T, H, d_k, d_v, dtype, segments, workspace, workspace_bytes, o,
                      final_state, stream);
}

kda_status kda_output_gate_rmsnorm(const void* o, const void* gate_logits, const float* norm_weight,
                                   int64_t rows, int32_t d_v, float eps, kda_dtype dtype,
                                   void* y, void* stream) {
    kda_status st = epilogue_checks(o, gate_logits, norm_weight, rows, d_v, eps, dtype, y);
    if (st != KDA_OK || rows == 0) return st;
    st = check_device();
    if (st != KDA_OK) return st;
    return epilogue_launch("kda_output_gate_rmsnorm launch", o, gate_logits, norm_weight, rows, d_v, eps, dtype, y,
                           stream);
}

kda_status kda_chunk_prefill_gated_epilogue(const void* q, const void* k, const void* v,
                                            const void* g_logits, const float* a_log, const float* beta_logits,
                                            const void* out_gate_logits, const float* norm_weight, float eps,
                                            const float* init_state, const int32_t* cu_seqlens,
                                            int32_t N, int64_t total_T, int32_t H,
                                            int32_t d_k, int32_t d_v, kda_dtype dtype,
                                            void* y, float* final_state, void* stream) {
    // Everything is validated before the first launch, so a rejected call
    // leaves y and final_state untouched.
    if (total_T < 0 || H < 1 || total_T > INT64_MAX / H) return KDA_ERR_SHAPE;
    const int64_t rows = total_T * H;
    kda_status st = epilogue_checks(y, out_gate_logits, norm_weight, rows, d_v, eps, dtype, y);
    if (st != KDA_OK) return st;
    st = prefill_impl("kda_chunk_prefill_gated_epilogue launch", q, k, v, g_logits, beta_logits, a_log, true,
                      init_state, cu_seqlens, N, total_T, H, d_k, d_v, dtype, y, final_state, stream);
    if (st != KDA_OK || rows == 0) return st;
    return epilogue_launch("kda_chunk_prefill_gated_epilogue launch", y, out_gate_logits, norm_weight, rows, d_v,
                           eps, dtype, y, stream);
}

kda_status kda_decode_step_gated_epilogue(const void* q, const void* k, const void* v,
                                          const void* g_logits, const float* a_log, const float* beta_logits,
                                          const void* out_gate_logits, const float* norm_weight, float eps,
                                          float* state, int32_t N, int32_t H,
                                          int32_t d_k, int32_t d_v, kda_dtype dtype,
                                          void* y, void* stream) {
    return decode_impl("kda_decode_step_gated_epilogue launch", q, k, v, g_logits, beta_logits, a_log, true, state,
                       N, H, d_k, d_v, dtype, y, stream, true, out_gate_logits, norm_weight, eps);
}

kda_status kda_decode_step_fused(const void* x_q, const void* x_k, const void* x_v,
                                 const float* conv_w, void* conv_state,
                                 const void* g_logits, const float* a_log, const float* beta_logits,
                                 const void* out_gate_logits, const float* norm_weight, float eps,
                                 float* state, int32_t N, int32_t H,
                                 int32_t d_k, int32_t d_v, kda_dtype dtype,
                                 void* y, void* stream) {
    return decode_impl("kda_decode_step_fused launch", x_q, x_k, x_v, g_logits, beta_logits, a_log, true, state,
                       N, H, d_k, d_v, dtype, y, stream, true, out_gate_logits, norm_weight, eps, true, conv_w,
                       conv_state);
}

kda_status kda_short_conv_prologue(const void* x_q, const void* x_k, const void* x_v, const float* conv_w,
                                   const void* conv_state_in, const int32_t* cu_seqlens,
                                   int32_t N, int64_t total_T, int32_t H, int32_t d_k, int32_t d_v,
                                   kda_dtype dtype, void* q, void* k, void* v, void* conv_state_out,
                                   void* stream) {
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_DTYPE;
    if (N < 1 || H < 1 || total_T < 0 || !supported_d(d_k) || !supported_d(d_v)) return KDA_ERR_SHAPE;
    if (cu_seqlens == nullptr && N != 1) return KDA_ERR_SHAPE;
    if (H > 65535 || !kda::prologue_grid_fits(N, total_T, H, d_k, d_v, dtype == KDA_BF16)) return KDA_ERR_SHAPE;
    if (total_T > 0 && (!x_q || !x_k || !x_v || !conv_w || !q || !k || !v)) return KDA_ERR_NULL;
    const void* ptrs[] = {x_q, x_k, x_v, conv_w, conv_state_in, cu_seqlens, q, k, v, conv_state_out};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    if (conv_state_in && conv_state_out) {
        const uintptr_t bytes = (uintptr_t)N * 3 * H * (2 * d_k + d_v) * (dtype == KDA_BF16 ? 2 : 4);
        const uintptr_t a = reinterpret_cast<uintptr_t>(conv_state_in), b = reinterpret_cast<uintptr_t>(conv_state_out);
        if (a < b + bytes && b < a + bytes) return KDA_ERR_VALUE;     // the two states overlap
    }
    if (total_T == 0 && conv_state_out == nullptr) return KDA_OK;
    kda_status st = check_device();
    if (st != KDA_OK) return st;
    kda::PrologueArgs a{x_q, x_k, x_v, conv_w, conv_state_in, conv_state_out, cu_seqlens, N, total_T, H, d_k, d_v,
                        dtype == KDA_BF16, q, k, v, reinterpret_cast<hipStream_t>(stream)};
    hipError_t e = kda::launch_prologue(a);
    if (e != hipSuccess) {
        set_error("kda_short_conv_prologue launch", e);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

}  // extern "C"

/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library, libkda.so.
 *
 * The operation (one head; "Kimi K3 -- Architecture Notes", section 1.1):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * with S in R^{d_k x d_v} (the fixed-size state of the same section),
 * alpha_t = exp(log_alpha_t) in (0,1]^{d_k} a per-channel retention factor acting
 * on the d_k rows of S, and beta_t in [0,1] the write strength.  There is no
 * 1/sqrt(d_k) output scale.
 *
 * Memory layout (all arrays dense, row-major, innermost index last):
 *     q, k        [T, H, d_k]        element type given by `dtype`
 *     v           [T, H, d_v]        element type given by `dtype`
 *     log_alpha   [T, H, d_k]        float32
 *     beta        [T, H]             float32
 *     state       [N, H, d_k, d_v]   float32 (row index = key channel)
 *     o           [T, H, d_v]        element type given by `dtype`
 * For decode, T is replaced by N (one token per sequence).
 *
 * Ownership: every pointer is caller-owned device memory (any allocation the
 * HIP runtime can address from the current device).  The library neither
 * frees nor retains pointers after a call returns and allocates no device
 * memory of its own (the time-split prefill takes a caller-owned workspace).
 *
 * Asynchrony: calls validate their arguments on the host, enqueue kernels on
 * `stream` (a hipStream_t; NULL = the legacy default stream) and return; the
 * outputs are valid once the stream has been synchronised.
 *
 * Errors: host-side validation failures return a non-zero kda_status BEFORE any
 * HIP call is made.  A failed kernel launch returns KDA_ERR_HIP.  Errors raised
 * asynchronously by an earlier kernel surface as KDA_ERR_HIP on a later call or
 * on the caller's own synchronisation.  The library never aborts and never
 * lets an exception cross this interface.
 *
 * Value preconditions that are documented but not checked (checking them
 * would need an extra pass over device memory):
 *     log_alpha in [-5, 0]  (the lower bound of section 1.2 of the notes; the
 *                            prefill kernel relies on it to keep every
 *                            16-token rescale factor within e^80),
 *     beta in [0, 1], and q, k of unit L2 norm per token-head (section 1.1).
 * cu_seqlens is clamped on the device into [0, total_T] and made
 * non-decreasing, so malformed offsets cannot cause out-of-range accesses;
 * they do produce meaningless output.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,       /* a required pointer is NULL                        */
    KDA_ERR_SHAPE = 2,      /* unsupported or inconsistent sizes                 */
    KDA_ERR_DTYPE = 3,      /* dtype is not one of kda_dtype                     */
    KDA_ERR_ALIGN = 4,      /* a pointer is not 16-byte aligned                  */
    KDA_ERR_NO_DEVICE = 5,  /* no HIP device, or the current device is not gfx950 */
    KDA_ERR_HIP = 6,        /* a HIP runtime call failed                          */
    KDA_ERR_VALUE = 7       /* a scalar argument is out of range (e.g. eps < 0)   */
} kda_status;

typedef enum {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype;

/* Version of this interface; bumped on any incompatible change. */
#define KDA_ABI_VERSION 4
int kda_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* kda_status_string(kda_status s);

/* Text of the last HIP error seen by the library on this thread ("" if none). */
const char* kda_last_error(void);

/*
 * kda_wait_giveups -- count of bounded in-kernel waits that ran out.
 *
 * The prefill kernel's state waves wait on a flag in LDS before reading a
 * triangular inverse that another wave of the workgroup publishes.  Every such
 * flag is written by a wave whose own path to that write has no waits, so the
 * wait always ends; its bound (2^22 polls) only guards against a logic error.
 * A wait that reaches the bound does not hang the GPU: the wave goes on with
 * whatever the LDS holds and adds one to a counter in device memory, and the
 * outputs of that launch are then not to be trusted.
 *
 *   count  : (host) receives the counter of the current device.
 *   reset  : non-zero sets the counter back to zero after reading it.
 *   stream : synchronised before the read (NULL: the default stream).  This
 *            call blocks the host; it is meant for checks after a batch of
 *            work, not for every launch.
 *
 * Returns KDA_ERR_NULL for a NULL count and KDA_ERR_HIP when the read fails.
 * A non-zero count returns KDA_OK and also sets kda_last_error's text.
 */
kda_status kda_wait_giveups(uint32_t* count, int32_t reset, void* stream);

/*
 * kda_chunk_prefill -- KDA over a packed batch of N sequences.
 *
 * Implements the section-1.1 recurrence chunkwise (section 1.2 of the notes): the
 * state passes serially from one chunk to the next while the tokens inside a
 * chunk are processed together, with 64-token chunks
 * split into 16-token tiles whose decay is taken relative to the tile start in
 * log space.  The result equals the token-by-token recurrence up to rounding.
 *
 *   q, k, v, log_alpha, beta : inputs, layouts above, total_T tokens.
 *   init_state  : [N, H, d_k, d_v] fp32 initial state per sequence, or NULL for
 *                 zeros.  May alias final_state (each sequence reads its slab
 *                 before writing it).
 *   cu_seqlens  : device int32 [N + 1]; sequence n owns tokens
 *                 [cu_seqlens[n], cu_seqlens[n+1]).  Requires cu[0] = 0,
 *                 non-decreasing, cu[N] = total_T.  NULL means N must be 1 and
 *                 the single sequence covers all total_T tokens.
 *                 Zero-length sequences are allowed (final = init).
 *   N           : number of sequences, >= 1.
 *   total_T     : total tokens, >= 0 (0 copies init to final).
 *   H           : heads, >= 1.
 *   d_k, d_v    : 64 or 128 each, for both dtypes.
 *   dtype       : element type of q, k, v and o.  The state is always fp32.
 *   o           : [total_T, H, d_v] output (required when total_T > 0).
 *   final_state : [N, H, d_k, d_v] fp32 output, or NULL to skip storing it.
 *   stream      : hipStream_t to enqueue on.
 */
kda_status kda_chunk_prefill(const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta,
                             const float* init_state, const int32_t* cu_seqlens,
                             int32_t N, int64_t total_T, int32_t H,
                             int32_t d_k, int32_t d_v, kda_dtype dtype,
                             void* o, float* final_state, void* stream);

/*
 * kda_decode_step -- advance N independent sequences by one token each.
 *
 * Per (sequence, head) one pass over the state: with a = exp(log_alpha),
 *     w  = beta (v - S^T (a * k)),
 *     o  = S^T (a * q) + w (k^T q),
 *     S <- Diag(a) S + k w^T            (written back in place),
 * which is the section-1.1 recurrence for a single token, rearranged so that S
 * is read once and written once.
 *
 *   q, k, v, log_alpha, beta : [N, H, d_k] / [N, H, d_v] / [N, H, d_k] / [N, H].
 *   state  : [N, H, d_k, d_v] fp32, read and overwritten in place.
 *   N, H   : >= 1 (N = 0 is a no-op).  d_k, d_v: 64 or 128.
 *   dtype  : element type of q, k, v and o.
 *   o      : [N, H, d_v] output.
 *   stream : hipStream_t to enqueue on.
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta,
                           float* state, int32_t N, int32_t H,
                           int32_t d_k, int32_t d_v, kda_dtype dtype,
                           void* o, void* stream);

/*
 * Gated variants: the decay and the write strength are given as logits and
 * mapped inside the kernels by the lower-bounded decay of section 1.2 of the
 * notes (the Kimi K3 row of its table of decay mappings):
 *
 *     log_alpha = g_min * Sigmoid(exp(A_h) * z),   g_min = -5,
 *     beta      = Sigmoid(b),
 *
 * so log_alpha lies in (-5, 0) by construction and the section-1.2 bound needs
 * no precondition.  A_h is the per-head log-scale of that section; z and b are
 * the outputs of the decay and write-strength projections, which stay outside
 * this library.  Everything else (layouts, ownership, asynchrony, errors,
 * shapes) is as for the ungated calls; the extra arguments are
 *
 *   g_logits    : [T, H, d_k] decay logits z, element type given by `dtype`
 *                 (bf16 halves the bytes of the fp32 log_alpha input).
 *   a_log       : [H] float32, A_h per head (16-byte aligned; required).
 *   beta_logits : [T, H] float32 write-strength logits b.
 *
 * For decode, T is replaced by N.
 */
kda_status kda_chunk_prefill_gated(const void* q, const void* k, const void* v,
                                   const void* g_logits, const float* a_log, const float* beta_logits,
                                   const float* init_state, const int32_t* cu_seqlens,
                                   int32_t N, int64_t total_T, int32_t H,
                                   int32_t d_k, int32_t d_v, kda_dtype dtype,
                                   void* o, float* final_state, void* stream);

kda_status kda_decode_step_gated(const void* q, const void* k, const void* v,
                                 const void* g_logits, const float* a_log, const float* beta_logits,
                                 float* state, int32_t N, int32_t H,
                                 int32_t d_k, int32_t d_v, kda_dtype dtype,
                                 void* o, void* stream);

/*
 * kda_chunk_prefill_split -- the prefill of ONE sequence, cut in time into
 * segments that run at the same time, for shapes whose heads alone would leave
 * most of the GPU idle (few heads per GPU, e.g. one GPU's share of a head
 * split across GPUs).
 *
 * The section-1.1 recurrence is affine in the state: a run of tokens maps a
 * start state S to Phi S + B, with Phi the product of the step matrices
 * (I - beta_t k_t k_t^T) Diag(alpha_t) and B the end state from a zero start.
 * The call
 *   1. runs every segment from a zero state (the first from init_state), and
 *      every segment after the first also from the identity with no values,
 *      which gives its Phi and Phi_t^T q_t for each of its tokens (Phi_t: the
 *      product up to token t);
 *   2. chains the segment end states, S_p = Phi_p S_{p-1} + B_p (fp32);
 *   3. adds S_{p-1}^T Phi_t^T q_t to the outputs of segment p >= 1.
 * The result equals kda_chunk_prefill on the same sequence up to rounding
 * (the correction rounds Phi_t^T q_t to the element type once more).
 *
 *   q, k, v, log_alpha, beta, init_state, total_T, H, d_k, d_v, dtype, o,
 *   final_state : as for kda_chunk_prefill with N = 1 and cu_seqlens NULL.
 *                 init_state may alias final_state.
 *   segments    : requested number of segments, >= 1.  Segments are whole
 *                 64-token chunks; the count actually used is the one that
 *                 length gives (at most `segments`).  With one segment the call
 *                 is kda_chunk_prefill (the workspace is not touched and may be
 *                 NULL).
 *   workspace   : caller-owned device memory of at least
 *                 kda_split_workspace_bytes(...) bytes, 16-byte aligned, not
 *                 overlapping any other argument; its contents on entry do not
 *                 matter and on return are unspecified.  Calls that share a
 *                 workspace must be ordered on one stream.
 *   Returns KDA_ERR_VALUE for segments < 1 or a workspace that is too small,
 *   KDA_ERR_NULL for a missing workspace when more than one segment is used,
 *   KDA_ERR_SHAPE when 512 * H * max(d_k, d_v) * (element bytes) exceeds
 *   2^32 - 1 (the correction's 32-bit offsets).
 */
kda_status kda_chunk_prefill_split(const void* q, const void* k, const void* v,
                                   const float* log_alpha, const float* beta, const float* init_state,
                                   int64_t total_T, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype,
                                   int32_t segments, void* workspace, size_t workspace_bytes,
                                   void* o, float* final_state, void* stream);

/* The same from decay / write-strength logits (see the gated calls above). */
/*
 * kda_chunk_prefill_split_noalloc -- kda_chunk_prefill_split without a
 * caller-owned workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).
 *
 * Same arguments, results and errors as kda_chunk_prefill_split, except that
 * the workspace is scratch the library holds in its code object:
 * KDA_SPLIT_SCRATCH_BYTES (64 MiB) on each device the library runs on, kept
 * until the process ends.  The call itself allocates nothing (no hipMalloc or
 * allocating library routine).  A split whose kda_split_workspace_bytes exceeds
 * KDA_SPLIT_SCRATCH_BYTES returns KDA_ERR_VALUE (with kda_last_error naming both
 * sizes) before any HIP call; fewer segments need less.  No byte of the scratch
 * has to start at zero: every byte a call reads was written by the same call.
 * Every call on one device shares that device's scratch: calls that overlap on
 * one device (other streams, other threads) race and must be ordered by the
 * caller.
 */
#define KDA_SPLIT_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_chunk_prefill_split_noalloc(const void* q, const void* k, const void* v,
                                           const float* log_alpha, const float* beta, const float* init_state,
                                           int64_t total_T, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype,
                                           int32_t segments, void* o, float* final_state, void* stream);

kda_status kda_chunk_prefill_gated_split(const void* q, const void* k, const void* v,
                                         const void* g_logits, const float* a_log, const float* beta_logits,
                                         const float* init_state, int64_t total_T, int32_t H,
                                         int32_t d_k, int32_t d_v, kda_dtype dtype,
                                         int32_t segments, void* workspace, size_t workspace_bytes,
                                         void* o, float* final_state, void* stream);

/*
 * Workspace bytes of a split prefill with these sizes and `segments` requested
 * (0 when one segment is used or the sizes are invalid).  Host-only; no HIP call.
 */
size_t kda_split_workspace_bytes(int64_t total_T, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype,
                                 int32_t segments);

/*
 * A segment count for kda_chunk_prefill_split on a GPU with `num_cus` compute
 * units, from a cost model of the three steps (one prefill workgroup per CU):
 * 1 when splitting would not pay, e.g. when the heads already fill the GPU.
 * Host-only; no HIP call.
 */
int32_t kda_split_segments(int64_t total_T, int32_t H, int32_t d_k, int32_t d_v, int32_t num_cus);

/*
 * Output epilogue (section 1.3 of the notes, full-rank output gate): the
 * recurrent output is normalised head-wise with RMSNorm and multiplied by a
 * sigmoid gate computed from the layer input, before the output projection:
 *
 *     y = Sigmoid(gate) * w * o / sqrt(mean(o^2) + eps)
 *
 * over the d_v channels of every (token, head) row.  The norm is the one of
 * the "MoE RMSNorm" page (mean of squares plus eps under the root, a learned
 * per-channel gain w; the model uses eps = 1e-5), with fp32 arithmetic.  The
 * gate logits are the output of the projection W_g x (outside this library),
 * laid out like o.
 *
 *   o, gate_logits : [rows, d_v] (rows = T * H; [T, H, d_v] is the same
 *                    memory), element type given by `dtype`.
 *   norm_weight    : [d_v] float32 gain shared by the heads, or NULL for 1.
 *   rows           : >= 0 (0 is a no-op).   d_v: 64 or 128.
 *   eps            : finite, >= 0, else KDA_ERR_VALUE.  With eps = 0 an
 *                    all-zero row gives NaN, as the formula does.
 *   y              : [rows, d_v] output, element type `dtype`.  May alias o or
 *                    gate_logits exactly (in place); no other overlap.
 *   stream         : hipStream_t to enqueue on.
 */
kda_status kda_output_gate_rmsnorm(const void* o, const void* gate_logits, const float* norm_weight,
                                   int64_t rows, int32_t d_v, float eps, kda_dtype dtype,
                                   void* y, void* stream);

/*
 * The gated prefill followed by the output epilogue: y receives the epilogue
 * of the prefill's o (o itself is not returned).  Arguments as for
 * kda_chunk_prefill_gated and kda_output_gate_rmsnorm; out_gate_logits is
 * [total_T, H, d_v] in `dtype` and must not overlap y.  Two kernels on
 * `stream`: the prefill writes o into y, the epilogue rewrites y in place, so
 * no memory beyond the caller's is used.  All arguments are validated before
 * the first launch.
 */
kda_status kda_chunk_prefill_gated_epilogue(const void* q, const void* k, const void* v,
                                            const void* g_logits, const float* a_log, const float* beta_logits,
                                            const void* out_gate_logits, const float* norm_weight, float eps,
                                            const float* init_state, const int32_t* cu_seqlens,
                                            int32_t N, int64_t total_T, int32_t H,
                                            int32_t d_k, int32_t d_v, kda_dtype dtype,
                                            void* y, float* final_state, void* stream);

/*
 * The gated decode step with the output epilogue fused into the same kernel
 * (a pair's whole output row lives in one workgroup): y [N, H, d_v] receives
 * Sigmoid(out_gate) * w * o / sqrt(mean(o^2) + eps) of the step's o; the
 * state is updated in place as by kda_decode_step_gated.  out_gate_logits is
 * [N, H, d_v] in `dtype`; norm_weight, eps as for kda_output_gate_rmsnorm.
 */
kda_status kda_decode_step_gated_epilogue(const void* q, const void* k, const void* v,
                                          const void* g_logits, const float* a_log, const float* beta_logits,
                                          const void* out_gate_logits, const float* norm_weight, float eps,
                                          float* state, int32_t N, int32_t H,
                                          int32_t d_k, int32_t d_v, kda_dtype dtype,
                                          void* y, void* stream);

/*
 * Input prologue (section 1.1 of the notes; the width comes from the "Kimi
 * Delta Attention (KDA)" box of the "Kimi K3" visualiser page): each of the q, k, v projection outputs passes a depthwise causal
 * convolution of width 4 and Swish, and q and k are then L2-normalised:
 *
 *     conv(x)_t = sum_{j=0..3} w[c, j] x_{t-3+j}[c]   (per head and channel c)
 *     q = l2(swish(conv x_q)),  k = l2(swish(conv x_k)),  v = swish(conv x_v),
 *     swish(u) = u Sigmoid(u),  l2(u) = u / sqrt(sum u^2 + 1e-6).
 *
 * Inputs before a sequence's first token come from its convolution state:
 * the last 3 inputs of the previous segment, oldest first (zeros if NULL).
 * Per head the packed channel order of weights and states is q (d_k
 * channels), then k (d_k), then v (d_v); C = 2 d_k + d_v.  fp32 arithmetic.
 *
 *   x_q, x_k       : [total_T, H, d_k] projection outputs, element type `dtype`.
 *   x_v            : [total_T, H, d_v].
 *   conv_w         : [H, C, 4] float32 taps (tap 3 meets the current input).
 *   conv_state_in  : [N, 3, H, C] in `dtype`, or NULL for zeros.
 *   cu_seqlens, N, total_T, H, d_k, d_v, dtype : as for kda_chunk_prefill.
 *   q, k, v        : outputs, shaped like x_q, x_k, x_v (the inputs of
 *                    kda_chunk_prefill_gated).
 *   conv_state_out : [N, 3, H, C] final state per sequence (the last 3 inputs,
 *                    filled from the initial state for sequences shorter than
 *                    3), or NULL.  It must not overlap conv_state_in
 *                    (KDA_ERR_VALUE); to continue in place, alternate two
 *                    buffers.
 *   stream         : hipStream_t to enqueue on.
 */
kda_status kda_short_conv_prologue(const void* x_q, const void* x_k, const void* x_v, const float* conv_w,
                                   const void* conv_state_in, const int32_t* cu_seqlens,
                                   int32_t N, int64_t total_T, int32_t H, int32_t d_k, int32_t d_v,
                                   kda_dtype dtype, void* q, void* k, void* v, void* conv_state_out,
                                   void* stream);

/*
 * One whole decode step of a KDA layer between its projections: the input
 * prologue (as kda_short_conv_prologue, one token per sequence, the
 * convolution state updated in place), the gate maps and the recurrence (as
 * kda_decode_step_gated) and the output epilogue (as kda_output_gate_rmsnorm),
 * in one kernel launch; every step of a pair runs in one workgroup.
 *
 *   x_q, x_k    : [N, H, d_k] projection outputs, element type `dtype`.
 *   x_v         : [N, H, d_v].
 *   conv_w      : [H, 2 d_k + d_v, 4] float32 convolution taps.
 *   conv_state  : [N, 3, H, 2 d_k + d_v] in `dtype`, read and overwritten in
 *                 place (the oldest input dropped, this token's appended).
 *   g_logits, a_log, beta_logits : as for kda_decode_step_gated.
 *   out_gate_logits, norm_weight, eps : as for kda_decode_step_gated_epilogue.
 *   state       : [N, H, d_k, d_v] fp32, updated in place.
 *   y           : [N, H, d_v] output in `dtype`.
 * No two of x_q, x_k, x_v, conv_state, y may overlap.
 */
kda_status kda_decode_step_fused(const void* x_q, const void* x_k, const void* x_v,
                                 const float* conv_w, void* conv_state,
                                 const void* g_logits, const float* a_log, const float* beta_logits,
                                 const void* out_gate_logits, const float* norm_weight, float eps,
                                 float* state, int32_t N, int32_t H,
                                 int32_t d_k, int32_t d_v, kda_dtype dtype,
                                 void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */

// KDA single-token decode: one read-modify-write pass over each fp32 state.
//
// For one (sequence, head) the recurrence of "Kimi K3 -- Architecture Notes"
// section 1.1 applied to a single token is rearranged as
//     a  = exp(log_alpha)                       (retention, per key channel c)
//     e  = S^T (a * k)      o' = S^T (a * q)    (two reductions over c)
//     w  = beta (v - e)
//     o  = o' + w (k^T q)
//     S <- Diag(a) S + k w^T
// so the state is read once and written once: the kernel is HBM-bound
// (2 * d_k * d_v * 4 bytes per pair against ~7 d_k d_v flops).
//
// One workgroup of NT threads per pair (1024; 512 with the input prologue).
// Thread t owns a 4-column slice (columns 4*(t % (DV/4)) .. +3) of ROWS state
// rows, rows interleaved so that each load instruction of a wave covers whole
// adjacent rows (coalesced 16-byte accesses).  The state slice stays in
// registers between the read and the write.  The state is touched once per
// step and is far larger than the caches, so its loads and stores are
// non-temporal (streaming).  At 512 x 96 pairs, 1024 threads per pair measured
// 6.0 TB/s against 5.5 TB/s with 256 (and less with 128 or 512): the whole
// 64 KB of a pair is requested by 16 waves at once, and the two reductions
// are shallow.  With the prologue the per-channel work before the first
// barrier is longer, and 512 threads (four workgroups per CU, whose state
// streams cover each other's latency) measured 1.11 ms against 1.28 at 1024.
//
// The few per-channel loads (q, k, v or the projection outputs with their
// convolution state and taps, the decay input) are issued before the state
// loads and without branches, so the first phase waits for them alone while
// the state is still streaming in (the vector memory counter retires loads
// in order).

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kDecodeThreads = 1024;      // workgroup size without the prologue
constexpr int kDecodeThreadsPro = 512;     // with the input prologue
constexpr float kL2EpsDecode = 1e-6f;

__device__ __forceinline__ float to_f(uint16_t r) { return bf16_to_f32(r); }
__device__ __forceinline__ float to_f(float r) { return r; }

__device__ __forceinline__ float swish_d(float u) { return u / (1.f + __expf(-u)); }

// Per-channel loads of a pair go through range-checked buffer loads: a lane
// with no channel passes an offset past the range and reads 0 without a
// memory access, so the loads need no branch.  (Loads inside a divergent
// branch make the compiler wait for them where the branch joins, which
// would hold back the state loads issued after them.)
constexpr uint32_t kNoLoad = 0x7ffffff0u;

template <typename T>
__device__ __forceinline__ T ld_ch(const T* base, uint32_t n, uint32_t i, bool ok) {
    const Rsrc r = make_rsrc(base, n * (uint32_t)sizeof(T));
    const uint32_t off = ok ? i * (uint32_t)sizeof(T) : kNoLoad;
    if constexpr (sizeof(T) == 2) return (T)buf_ld16(r, off);
    else return __uint_as_float(buf_ld32(r, off));
}

// One token of the width-4 causal convolution on one channel: the channel's
// three state entries (oldest first, `stride` elements apart) and the new
// input meet taps 0..3; the state then drops its oldest entry and appends the
// input, copied exactly.  Split into the loads (issued early) and the rest.
template <typename T> struct ConvIn { T r[4]; f32x4 w; };

// x: the pair's inputs of this projection (n channels); cs: slot 0 of the
// pair's state at this projection's first channel; w: the head's taps of that
// channel block; i: the channel; ok: whether this lane has one.
template <typename T>
__device__ __forceinline__ ConvIn<T> conv_load(const T* x, const T* cs, int64_t stride, const float* w, uint32_t n,
                                               uint32_t i, bool ok) {
    ConvIn<T> c;
    c.r[0] = ld_ch(cs, n, i, ok);
    c.r[1] = ld_ch(cs + stride, n, i, ok);
    c.r[2] = ld_ch(cs + 2 * stride, n, i, ok);
    c.r[3] = ld_ch(x, n, i, ok);
    const Rsrc rw = make_rsrc(w, n * 16u);
    c.w = __builtin_bit_cast(f32x4, buf_ld128(rw, ok ? i * 16u : kNoLoad));
    return c;
}

template <typename T>
__device__ __forceinline__ float conv_apply(const ConvIn<T>& c, T* __restrict__ cs, int64_t c0, int64_t stride) {
    cs[c0] = c.r[1];
    cs[c0 + stride] = c.r[2];
    cs[c0 + 2 * stride] = c.r[3];
    return c.w[0] * to_f(c.r[0]) + c.w[1] * to_f(c.r[1]) + c.w[2] * to_f(c.r[2]) + c.w[3] * to_f(c.r[3]);
}

// GATED: `decay` holds decay logits z (element type T) and `beta` the
// write-strength logits; the lower-bounded map of section 1.2 of the notes
// (Kimi K3 row of its table), log alpha = -5 Sigmoid(e^{A_h} z) and
// beta = Sigmoid(logit), is applied on the fly.  Otherwise `decay` holds fp32
// log alpha and `beta` beta.
// NORM: the output epilogue of section 1.3 is applied before the store,
// y = Sigmoid(og) * nw * o / sqrt(mean(o^2) + eps) over the pair's d_v
// channels (nw null: gain 1); the pair's whole o lives in this workgroup, so
// it costs one more reduction and no extra pass.
// PRO: q, k, v hold the projection outputs and the input prologue of section
// 1.1 runs first: a width-4 causal convolution per channel (taps cw
// [H, 2 d_k + d_v, 4], state cs [N, 3, H, 2 d_k + d_v] updated in place), Swish,
// and the L2 norm of q and k.  The norms are folded in after the reductions
// (e and o' are linear in k and q, k^T q is bilinear), so they add two wave
// sums and no barrier.
template <typename T, int DK, int DV, bool GATED, bool NORM, bool PRO, int NT>
__global__ __launch_bounds__(NT) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const void* __restrict__ decay, const float* __restrict__ beta, const float* __restrict__ a_log,
    float* state, T* __restrict__ o, int32_t H, int64_t pairs,
    const T* __restrict__ og, const float* __restrict__ nw, float eps,
    const float* __restrict__ cw, T* __restrict__ cs) {
    constexpr int QUADS = DV / 4;          // threads per state row
    constexpr int RG = NT / QUADS;         // row groups
    constexpr int ROWS = DK / RG;          // rows per thread
    static_assert(DK % RG == 0, "shape");

    __shared__ float s_a[DK], s_ak[DK], s_aq[DK], s_k[DK];
    __shared__ f32x4 s_red[2][RG][QUADS];
    __shared__ float s_w[DV];
    __shared__ float s_kq[NT / kWave];
    __shared__ float s_ss[DV / kWave];
    __shared__ float s_qsq[PRO ? NT / kWave : 1], s_ksq[PRO ? NT / kWave : 1], s_rk[1];

    const int64_t pair = blockIdx.x;
    if (pair >= pairs) return;
    const int t = threadIdx.x;
    const int vq = t % QUADS;
    const int rg = t / QUADS;

    float* S = state + pair * (int64_t)(DK * DV);

    // The few per-channel loads go first: the vector memory counter retires
    // loads in order, so their consumers then wait only for them while the
    // state loads, the bulk of the traffic, are still in flight.
    constexpr int C = 2 * DK + DV;
    const int h = (int)(pair % H);
    const int64_t cs0 = (pair / H) * 3 * (int64_t)H * C + (int64_t)h * C;   // slot 0 of this pair, channel 0
    const int64_t cstride = (int64_t)H * C;                                 // between slots
    const bool hk = t < DK, hv = t < DV;
    T dec_raw{};
    float dec_f = 0.f;
    if constexpr (GATED) dec_raw = ld_ch(reinterpret_cast<const T*>(decay) + pair * DK, DK, t, hk);
    else dec_f = ld_ch(reinterpret_cast<const float*>(decay) + pair * DK, DK, t, hk);
    T qraw{}, kraw{};
    ConvIn<T> cin_q{}, cin_k{}, cin_v{};
    if constexpr (PRO) {
        const float* wh = cw + (int64_t)h * C * 4;
        cin_q = conv_load(q + pair * DK, cs + cs0, cstride, wh, DK, t, hk);
        cin_k = conv_load(k + pair * DK, cs + cs0 + DK, cstride, wh + DK * 4, DK, t, hk);
        cin_v = conv_load(v + pair * DV, cs + cs0 + 2 * DK, cstride, wh + 2 * DK * 4, DV, t, hv);
    } else {
        qraw = ld_ch(q + pair * DK, DK, t, hk);
        kraw = ld_ch(k + pair * DK, DK, t, hk);
    }
    const float scale = GATED ? a_log[h] : 0.f;
    // Keep the state loads after these: instruction selection schedules each
    // basic block on its own, so a (never taken, wave-uniform) branch on a
    // kernel argument fences the two groups of loads.
    if (__builtin_expect(H < 0, 0)) asm volatile("s_nop 0");

    f32x4 s[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int row = i * RG + rg;
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + row * DV + 4 * vq));
    }

    // Per-channel vectors.
    float kq_part = 0.f, qsq_part = 0.f, ksq_part = 0.f, vv = 0.f;
    if (t < DK) {
        float a;
        if constexpr (GATED) {
            const float u = __expf(scale) * to_f(dec_raw);
            a = __expf(-5.f / (1.f + __expf(-u)));
        } else {
            a = __expf(dec_f);
        }
        float kk, qq;
        if constexpr (PRO) {
            qq = swish_d(conv_apply(cin_q, cs, cs0 + t, cstride));
            kk = swish_d(conv_apply(cin_k, cs, cs0 + DK + t, cstride));
            qsq_part = qq * qq;
            ksq_part = kk * kk;
        } else {
            kk = to_f(kraw);
            qq = to_f(qraw);
        }
        s_a[t] = a;
        s_ak[t] = a * kk;
        s_aq[t] = a * qq;
        s_k[t] = kk;
        kq_part = kk * qq;
    }
    kq_part = wave_sum(kq_part);
    if ((t % kWave) == 0) s_kq[t / kWave] = kq_part;
    if constexpr (PRO) {
        qsq_part = wave_sum(qsq_part);
        ksq_part = wave_sum(ksq_part);
        if ((t % kWave) == 0) {
            s_qsq[t / kWave] = qsq_part;
            s_ksq[t / kWave] = ksq_part;
        }
    }
    __syncthreads();

    // Partial reductions over this thread's rows.
    f32x4 e = {0.f, 0.f, 0.f, 0.f}, op = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int row = i * RG + rg;
        e += s[i] * s_ak[row];
        op += s[i] * s_aq[row];
    }
    s_red[0][rg][vq] = e;
    s_red[1][rg][vq] = op;
    __syncthreads();

    float out = 0.f;
    if (t < DV) {
        const int cq = t / 4, cl = t % 4;
        float es = 0.f, os = 0.f;
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            es += s_red[0][g][cq][cl];
            os += s_red[1][g][cq][cl];
        }
        float kq = 0.f;
#pragma unroll
        for (int i = 0; i < NT / kWave; ++i) kq += s_kq[i];
        if constexpr (PRO) {
            float qs = 0.f, ks = 0.f;
#pragma unroll
            for (int i = 0; i < NT / kWave; ++i) {
                qs += s_qsq[i];
                ks += s_ksq[i];
            }
            const float rq = rsqrtf(qs + kL2EpsDecode), rk = rsqrtf(ks + kL2EpsDecode);
            es *= rk;
            os *= rq;
            kq *= rq * rk;
            if (t == 0) s_rk[0] = rk;
            vv = swish_d(conv_apply(cin_v, cs, cs0 + 2 * DK + t, cstride));
        } else {
            vv = Elem<T>::load(v, pair * DV + t);
        }
        const float b = GATED ? 1.f / (1.f + __expf(-beta[pair])) : beta[pair];
        const float w = b * (vv - es);
        s_w[t] = w;
        out = os + w * kq;
        if constexpr (NORM) {
            const float ss = wave_sum(out * out);      // DV is a multiple of the wave size
            if ((t % kWave) == 0) s_ss[t / kWave] = ss;
        } else {
            Elem<T>::store(o, pair * DV + t, out);
        }
    }
    __syncthreads();

    if constexpr (NORM) {
        if (t < DV) {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < DV / kWave; ++i) ss += s_ss[i];
            const float gate = 1.f / (1.f + __expf(-Elem<T>::load(og, pair * DV + t)));
            const float gain = nw ? nw[t] : 1.f;
            Elem<T>::store(o, pair * DV + t, out * rsqrtf(ss * (1.f / DV) + eps) * gain * gate);
        }
    }

    const f32x4 w4 = {s_w[4 * vq], s_w[4 * vq + 1], s_w[4 * vq + 2], s_w[4 * vq + 3]};
    const float kscale = PRO ? s_rk[0] : 1.f;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int row = i * RG + rg;
        const f32x4 nv = s[i] * s_a[row] + (s_k[row] * kscale) * w4;
        __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(S + row * DV + 4 * vq));
    }
}

template <typename T, int DK, int DV, bool GATED, bool NORM, bool PRO = false>
static void launch_decode_v(const DecodeArgs& a, int64_t pairs) {
    constexpr int NT = PRO ? kDecodeThreadsPro : kDecodeThreads;
    hipLaunchKernelGGL((decode_kernel<T, DK, DV, GATED, NORM, PRO, NT>), dim3((unsigned)pairs), dim3(NT), 0,
                       a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.log_alpha, a.beta, a.a_log,
                       a.state, (T*)a.o, a.H, pairs, (const T*)a.out_gate, a.norm_weight, a.eps, a.conv_w,
                       (T*)a.conv_state);
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a) {
    const int64_t pairs = (int64_t)a.N * a.H;
    if (pairs == 0) return hipSuccess;
    if (a.gated && a.out_gate && a.conv_w) launch_decode_v<T, DK, DV, true, true, true>(a, pairs);
    else if (a.gated && a.out_gate) launch_decode_v<T, DK, DV, true, true>(a, pairs);
    else if (a.gated) launch_decode_v<T, DK, DV, true, false>(a, pairs);
    else launch_decode_v<T, DK, DV, false, false>(a, pairs);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_dtype(const DecodeArgs& a) {
    if (a.d_k == 128 && a.d_v == 128) return launch_decode_t<T, 128, 128>(a);
    if (a.d_k == 128 && a.d_v == 64) return launch_decode_t<T, 128, 64>(a);
    if (a.d_k == 64 && a.d_v == 128) return launch_decode_t<T, 64, 128>(a);
    return launch_decode_t<T, 64, 64>(a);
}

bool decode_grid_fits(int64_t pairs, bool prologue) {
    return grid_fits(pairs, prologue ? kDecodeThreadsPro : kDecodeThreads);
}

hipError_t launch_decode(const DecodeArgs& a) {
    return a.bf16 ? launch_decode_dtype<uint16_t>(a) : launch_decode_dtype<float>(a);
}

}  // namespace kda

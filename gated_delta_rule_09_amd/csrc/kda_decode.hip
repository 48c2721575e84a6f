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
// One 1024-thread workgroup per pair.  Thread t owns a 4-column slice
// (columns 4*(t % (DV/4)) .. +3) of ROWS state rows (4 at d_k = 128), rows
// interleaved so that each load instruction of a wave covers whole adjacent
// rows (coalesced 16-byte accesses).  The state slice stays in registers
// between the read and the write.  The state is touched once per step and is
// far larger than the caches, so its loads and stores are non-temporal
// (streaming).  At 512 x 96 pairs, 1024 threads per pair measured 6.0 TB/s
// against 5.5 TB/s with 256 (and less with 128 or 512): the whole 64 KB of a
// pair is requested by 16 waves at once, and the two reductions are shallow.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kDecodeThreads = 1024;

// GATED: `decay` holds decay logits z (element type T) and `beta` the
// write-strength logits; the lower-bounded map of section 1.2 of the notes
// (Kimi K3 row of its table), log alpha = -5 Sigmoid(e^{A_h} z) and
// beta = Sigmoid(logit), is applied on the fly.  Otherwise `decay` holds fp32
// log alpha and `beta` beta.
// NORM: the output epilogue of section 1.3 is applied before the store,
// y = Sigmoid(og) * nw * o / sqrt(mean(o^2) + eps) over the pair's d_v
// channels (nw null: gain 1); the pair's whole o lives in this workgroup, so
// it costs one more reduction and no extra pass.
template <typename T, int DK, int DV, bool GATED, bool NORM>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const void* __restrict__ decay, const float* __restrict__ beta, const float* __restrict__ a_log,
    float* __restrict__ state, T* __restrict__ o, int32_t H, int64_t pairs,
    const T* __restrict__ og, const float* __restrict__ nw, float eps) {
    constexpr int NT = kDecodeThreads;
    constexpr int QUADS = DV / 4;          // threads per state row
    constexpr int RG = NT / QUADS;         // row groups
    constexpr int ROWS = DK / RG;          // rows per thread
    static_assert(DK % RG == 0, "shape");

    __shared__ float s_a[DK], s_ak[DK], s_aq[DK], s_k[DK];
    __shared__ f32x4 s_red[2][RG][QUADS];
    __shared__ float s_w[DV];
    __shared__ float s_kq[NT / kWave];
    __shared__ float s_ss[DV / kWave];

    const int64_t pair = blockIdx.x;
    if (pair >= pairs) return;
    const int t = threadIdx.x;
    const int vq = t % QUADS;
    const int rg = t / QUADS;

    float* S = state + pair * (int64_t)(DK * DV);

    // Issue the state loads first: they are the bulk of the traffic.
    f32x4 s[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int row = i * RG + rg;
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + row * DV + 4 * vq));
    }

    // Per-channel vectors.
    float kq_part = 0.f;
    if (t < DK) {
        float a;
        if constexpr (GATED) {
            const float u = __expf(a_log[pair % H]) * Elem<T>::load(reinterpret_cast<const T*>(decay), pair * DK + t);
            a = __expf(-5.f / (1.f + __expf(-u)));
        } else {
            a = __expf(reinterpret_cast<const float*>(decay)[pair * DK + t]);
        }
        const float kk = Elem<T>::load(k, pair * DK + t);
        const float qq = Elem<T>::load(q, pair * DK + t);
        s_a[t] = a;
        s_ak[t] = a * kk;
        s_aq[t] = a * qq;
        s_k[t] = kk;
        kq_part = kk * qq;
    }
    kq_part = wave_sum(kq_part);
    if ((t % kWave) == 0) s_kq[t / kWave] = kq_part;
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
        const float b = GATED ? 1.f / (1.f + __expf(-beta[pair])) : beta[pair];
        const float w = b * (Elem<T>::load(v, pair * DV + t) - es);
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
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int row = i * RG + rg;
        const f32x4 nv = s[i] * s_a[row] + s_k[row] * w4;
        __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(S + row * DV + 4 * vq));
    }
}

template <typename T, int DK, int DV, bool GATED, bool NORM>
static void launch_decode_v(const DecodeArgs& a, int64_t pairs) {
    hipLaunchKernelGGL((decode_kernel<T, DK, DV, GATED, NORM>), dim3((unsigned)pairs), dim3(kDecodeThreads), 0,
                       a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.log_alpha, a.beta, a.a_log,
                       a.state, (T*)a.o, a.H, pairs, (const T*)a.out_gate, a.norm_weight, a.eps);
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a) {
    const int64_t pairs = (int64_t)a.N * a.H;
    if (pairs == 0) return hipSuccess;
    if (a.gated && a.out_gate) launch_decode_v<T, DK, DV, true, true>(a, pairs);
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

hipError_t launch_decode(const DecodeArgs& a) {
    return a.bf16 ? launch_decode_dtype<uint16_t>(a) : launch_decode_dtype<float>(a);
}

}  // namespace kda

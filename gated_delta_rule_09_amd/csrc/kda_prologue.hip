// Input prologue of KDA ("Kimi K3 -- Architecture Notes", section 1.1; the
// "Kimi Delta Attention (KDA)" box of the "Kimi K3" visualiser page gives the
// width): each of the q, k, v projections passes a
// depthwise causal convolution of width 4 and Swish, and q and k are then
// L2-normalised over their d_k channels:
//
//     conv(x)_t = sum_j w[., j] x_{t-3+j}        (the newest input meets tap 3)
//     swish(u) = u Sigmoid(u),   l2(u) = u / sqrt(|u|^2 + eps),  eps = 1e-6
//     q = l2(swish(conv x_q)),  k = l2(swish(conv x_k)),  v = swish(conv x_v).
//
// Inputs before a sequence's first token come from its convolution state
// (the last 3 inputs of the previous segment, oldest first) or are zero.
//
// Streaming and HBM-bound: every input and output element moves once
// (2 * (2 d_k + d_v) * sizeof(T) bytes per token-head).  A wave owns one
// projection, a group of RPW = 64 / LPR consecutive heads (LPR lanes of one
// 16-byte piece each cover a head's row, as in the output epilogue) and a
// strip of kStrip tokens; neighbouring workgroups take neighbouring head
// groups, so the waves in flight together read whole token rows.  A wave
// walks its strip in groups of kAhead tokens whose loads are issued before
// their arithmetic, with the 3-token window of earlier inputs in registers
// (inside one sequence the window and the group share one register array,
// so nothing moves per token); only the 3-token halo before the strip is
// read twice (from L2).  Sequence starts reload the window from the state;
// the wave that handles a sequence's last token writes its final state (so
// the final state must not overlap the initial state); empty sequences are
// handled by a second, small kernel.
// Measured on 65,536 tokens x 96 heads x 3 projections of 128 bf16: strips of
// 16 tokens with 8 in flight, 1.67-1.69 ms (5.7-5.8 TB/s); strips of 32, 64,
// 128: 1.73, 1.78, 1.86 ms; 4 in flight 1.73-1.75 ms; 16 in flight about
// 2.9 ms; head-group-major block order instead of row order 1.92 ms.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kProThreads = 64;    // one wave per workgroup
constexpr int kStrip = 16;         // tokens per wave
constexpr int kAhead = 8;          // tokens whose loads are in flight together
constexpr float kL2Eps = 1e-6f;
constexpr float kLog2eP = 1.4426950408889634f;

template <int CTRL>
__device__ __forceinline__ float dppm(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of L lanes (8, 16 or 32), in every lane of the group
// (quad permutes, then mirrors inside 8 and 16 lanes, then the row-pair swap).
template <int L>
__device__ __forceinline__ float lane_group_sum(float x) {
    x += dppm<0xB1>(x);
    x += dppm<0x4E>(x);
    x += dppm<0x141>(x);
    if constexpr (L >= 16) x += dppm<0x140>(x);
    if constexpr (L >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    static_assert(L == 8 || L == 16 || L == 32, "group size");
    return x;
}

// Buffer access with the non-temporal hint (cache-policy bit 1): the strip's
// data are touched once.
constexpr uint32_t kNoAccess = 0x80000000u;   // past every range (at most 64 * 65535 * 512 bytes): reads 0, writes nothing
__device__ __forceinline__ u32x4 ld_nt(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ void st_nt(u32x4 v, Rsrc r, uint32_t off) {
    typedef unsigned int v4u __attribute__((__vector_size__(16)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, off, 0, 2);
}

__device__ __forceinline__ float swish(float u) {
    return u * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2eP * u));
}

template <typename T> struct Pc;
template <> struct Pc<uint16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void unpack(u32x4 p, float* x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(p[i]); x[2 * i + 1] = bf16_hi(p[i]); }
    }
    static __device__ __forceinline__ u32x4 pack(const float* x) {
        u32x4 p;
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        return p;
    }
};
template <> struct Pc<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void unpack(u32x4 p, float* x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(p[i]);
    }
    static __device__ __forceinline__ u32x4 pack(const float* x) {
        u32x4 p;
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __float_as_uint(x[i]);
        return p;
    }
};

// Sequence boundaries, clamped into [0, total_T]; offsets are assumed
// non-decreasing (malformed ones give meaningless output, never an access
// out of range).
__device__ __forceinline__ int64_t cu_at(const int32_t* cu, int32_t i, int32_t N, int64_t total_T) {
    if (cu == nullptr) return i == 0 ? 0 : total_T;
    int64_t c = cu[i];
    c = c < 0 ? 0 : c;
    return c > total_T ? total_T : c;
}

struct ProjArgs {
    const void* x; void* out;
    int32_t c0;          // first packed channel of this projection within a head
    bool normalize;
};

struct ProKernelArgs {
    ProjArgs proj[3];
    const float* w;      // [H, C, 4]
    const void* st_in;   // [N, 3, H, C] or null
    void* st_out;        // [N, 3, H, C] or null
    const int32_t* cu;
    int32_t N; int64_t total_T; int32_t H, C;
    int32_t strips, head_groups;
};

template <typename T, int D>
__global__ __launch_bounds__(kProThreads) void prologue_kernel(ProKernelArgs a) {
    constexpr int VE = Pc<T>::N;
    constexpr int LPR = D / VE;
    constexpr int RPW = kWave / LPR;
    const ProjArgs& pj = a.proj[blockIdx.y];
    const int lane = threadIdx.x;
    const int l = lane % LPR;
    const int hg = blockIdx.x % a.head_groups;      // neighbouring waves cover one token row together
    const int strip = blockIdx.x / a.head_groups;
    const int h = hg * RPW + lane / LPR;
    const bool hv = h < a.H;
    const int hc = hv ? h : 0;                   // clamped head for addresses
    const int ch = pj.c0 + l * VE;               // first packed channel of this lane
    const int64_t t0 = (int64_t)strip * kStrip;
    if (t0 >= a.total_T) return;
    const int64_t t1 = t0 + kStrip < a.total_T ? t0 + kStrip : a.total_T;
    const int64_t rowstride = (int64_t)a.H * LPR;          // 16-byte pieces per token
    const u32x4* x = reinterpret_cast<const u32x4*>(pj.x);
    u32x4* out = reinterpret_cast<u32x4*>(pj.out);
    const T* st_in = reinterpret_cast<const T*>(a.st_in);
    T* st_out = reinterpret_cast<T*>(a.st_out);

    float w[4][VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) {
        const f32x4 t4 = *reinterpret_cast<const f32x4*>(a.w + ((int64_t)hc * a.C + ch + i) * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j][i] = t4[j];
    }

    // sequence holding t0: the first n with cu[n + 1] > t0
    int32_t lo = 0, hi = a.N - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi) / 2;
        if (cu_at(a.cu, mid + 1, a.N, a.total_T) > t0) hi = mid; else lo = mid + 1;
    }
    int32_t n = lo;
    int64_t s = cu_at(a.cu, n, a.N, a.total_T), e = cu_at(a.cu, n + 1, a.N, a.total_T);

    // state entry `slot` (0 = oldest) of sequence n for this lane's channels
    auto state_piece = [&](int32_t nn, int slot, float* v) {
        if (st_in != nullptr && hv) {
            const int64_t off = (((int64_t)nn * 3 + slot) * a.H + h) * a.C + ch;
            Pc<T>::unpack(*reinterpret_cast<const u32x4*>(st_in + off), v);
        } else {
#pragma unroll
            for (int i = 0; i < VE; ++i) v[i] = 0.f;
        }
    };
    auto load_window = [&](int64_t t, float (*win)[VE]) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int64_t p = t - 3 + j;
            if (p >= s) {
                Pc<T>::unpack(hv ? x[p * rowstride + (int64_t)hc * LPR + l] : u32x4{0u, 0u, 0u, 0u}, win[j]);
            } else {
                state_piece(n, (int)(p - (s - 3)), win[j]);
            }
        }
    };

    // This strip's rows through buffer resources: offsets are 32-bit, and a
    // token past the strip's end or a lane past the last head is outside the
    // range (reads 0, writes nothing) without a branch.
    const int64_t strip_base = t0 * rowstride;
    const uint32_t row_bytes = (uint32_t)(rowstride * 16);
    const Rsrc rx = make_rsrc(x + strip_base, (uint32_t)(t1 - t0) * row_bytes);
    const Rsrc ro = make_rsrc(out + strip_base, (uint32_t)(t1 - t0) * row_bytes);
    const uint32_t lane_base = (uint32_t)((hc * LPR + l) * 16);

    auto convolve = [&](const float* x0, const float* x1, const float* x2, const float* x3, uint32_t off) {
        float y[VE];
#pragma unroll
        for (int i = 0; i < VE; ++i) y[i] = swish(w[0][i] * x0[i] + w[1][i] * x1[i] + w[2][i] * x2[i] + w[3][i] * x3[i]);
        if (pj.normalize) {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < VE; ++i) ss += y[i] * y[i];
            const float r = __builtin_amdgcn_rsqf(lane_group_sum<LPR>(ss) + kL2Eps);
#pragma unroll
            for (int i = 0; i < VE; ++i) y[i] *= r;
        }
        st_nt(Pc<T>::pack(y), ro, hv ? off : kNoAccess);
    };
    auto write_final = [&](const float* a0, const float* a1, const float* a2) {
        if (st_out == nullptr || !hv) return;
        const float* src[3] = {a0, a1, a2};
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int64_t off = (((int64_t)n * 3 + j) * a.H + h) * a.C + ch;
            *reinterpret_cast<u32x4*>(st_out + off) = Pc<T>::pack(src[j]);
        }
    };

    // xs[0..2]: inputs at the three positions before the group (the window);
    // xs[3..]: the group's inputs.
    constexpr int A = kAhead;
    float xs[3 + A][VE];
    load_window(t0, xs);

    for (int64_t tb = t0; tb < t1; tb += A) {
        const uint32_t gb = (uint32_t)(tb - t0) * row_bytes + lane_base;
        u32x4 px[A];
#pragma unroll
        for (int u = 0; u < A; ++u) px[u] = ld_nt(rx, hv ? gb + u * row_bytes : kNoAccess);
        while (tb >= e && n < a.N - 1) {          // next non-empty sequence
            ++n;
            s = e;
            e = cu_at(a.cu, n + 1, a.N, a.total_T);
        }
        if (tb == s) load_window(tb, xs);
        if (tb + A <= e && tb + A <= t1) {
            // the whole group lies inside sequence n: no window shifts per token
#pragma unroll
            for (int u = 0; u < A; ++u) Pc<T>::unpack(px[u], xs[3 + u]);
#pragma unroll
            for (int u = 0; u < A; ++u) convolve(xs[u], xs[u + 1], xs[u + 2], xs[u + 3], gb + u * row_bytes);
            if (tb + A == e) write_final(xs[A], xs[A + 1], xs[A + 2]);
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
                for (int i = 0; i < VE; ++i) xs[j][i] = xs[A + j][i];
        } else {
            // a sequence starts or ends inside the group, or the strip does: token by token
#pragma unroll
            for (int u = 0; u < A; ++u) {
                const int64_t t = tb + u;
                if (t >= t1) break;
                while (t >= e && n < a.N - 1) {
                    ++n;
                    s = e;
                    e = cu_at(a.cu, n + 1, a.N, a.total_T);
                }
                if (t == s) load_window(t, xs);
                float cur[VE];
                Pc<T>::unpack(px[u], cur);
                convolve(xs[0], xs[1], xs[2], cur, gb + u * row_bytes);
#pragma unroll
                for (int i = 0; i < VE; ++i) {
                    xs[0][i] = xs[1][i];
                    xs[1][i] = xs[2][i];
                    xs[2][i] = cur[i];
                }
                if (t == e - 1) write_final(xs[0], xs[1], xs[2]);
            }
        }
    }
}

// Final state of every empty sequence: its initial state (or zeros).
template <typename T>
__global__ __launch_bounds__(256) void prologue_empty_kernel(const T* st_in, T* st_out, const int32_t* cu,
                                                             int32_t N, int64_t total_T, int32_t H, int32_t C) {
    const int32_t n = blockIdx.x;
    if (cu_at(cu, n, N, total_T) != cu_at(cu, n + 1, N, total_T)) return;
    const int64_t len = (int64_t)3 * H * C;
    const int64_t base = (int64_t)n * len;
    for (int64_t i = threadIdx.x; i < len; i += blockDim.x)
        st_out[base + i] = st_in ? st_in[base + i] : T(0);
}

template <typename T, int DK, int DV>
hipError_t launch_t(const PrologueArgs& p) {
    constexpr int VE = Pc<T>::N;
    const int32_t C = 2 * p.d_k + p.d_v;
    ProKernelArgs a{};
    a.w = p.conv_w; a.st_in = p.state_in; a.st_out = p.state_out; a.cu = p.cu_seqlens;
    a.N = p.N; a.total_T = p.total_T; a.H = p.H; a.C = C;
    a.strips = (int32_t)((p.total_T + kStrip - 1) / kStrip);
    if (p.total_T > 0) {
        constexpr int RPWK = kWave / (DK / VE);
        a.head_groups = (p.H + RPWK - 1) / RPWK;
        a.proj[0] = ProjArgs{p.x_q, p.q, 0, true};
        a.proj[1] = ProjArgs{p.x_k, p.k, DK, true};
        a.proj[2] = ProjArgs{p.x_v, p.v, 2 * DK, false};
        if constexpr (DK == DV) {
            // one launch for the three projections (the grid's y index)
            hipLaunchKernelGGL((prologue_kernel<T, DK>), dim3((unsigned)a.strips * a.head_groups, 3),
                               dim3(kProThreads), 0, p.stream, a);
        } else {
            hipLaunchKernelGGL((prologue_kernel<T, DK>), dim3((unsigned)a.strips * a.head_groups, 2),
                               dim3(kProThreads), 0, p.stream, a);
            constexpr int RPWV = kWave / (DV / VE);
            a.head_groups = (p.H + RPWV - 1) / RPWV;
            a.proj[0] = a.proj[2];
            hipLaunchKernelGGL((prologue_kernel<T, DV>), dim3((unsigned)a.strips * a.head_groups, 1),
                               dim3(kProThreads), 0, p.stream, a);
        }
    }
    if (p.state_out != nullptr)
        hipLaunchKernelGGL((prologue_empty_kernel<T>), dim3((unsigned)p.N), dim3(256), 0, p.stream,
                           (const T*)p.state_in, (T*)p.state_out, p.cu_seqlens, p.N, p.total_T, p.H, C);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const PrologueArgs& p) {
    if (p.d_k == 128 && p.d_v == 128) return launch_t<T, 128, 128>(p);
    if (p.d_k == 128 && p.d_v == 64) return launch_t<T, 128, 64>(p);
    if (p.d_k == 64 && p.d_v == 128) return launch_t<T, 64, 128>(p);
    return launch_t<T, 64, 64>(p);
}

}  // namespace

bool prologue_grid_fits(int64_t N, int64_t total_T, int32_t H, int32_t d_k, int32_t d_v, bool bf16) {
    // strips x head groups is the grid's x dimension (one wave per workgroup); a
    // head group is the heads one wave covers, kWave / (d / elements per lane)
    const int64_t ve = bf16 ? Pc<uint16_t>::N : Pc<float>::N;
    const int64_t strips = (total_T + kStrip - 1) / kStrip;
    for (int32_t d : {d_k, d_v}) {
        const int64_t per_wave = kWave / (d / ve);
        if (!grid_fits(strips * ((H + per_wave - 1) / per_wave), kProThreads)) return false;
    }
    return grid_fits(N, 256);     // the kernel that passes the states of empty sequences
}

hipError_t launch_prologue(const PrologueArgs& p) {
    return p.bf16 ? launch_dtype<uint16_t>(p) : launch_dtype<float>(p);
}

}  // namespace kda

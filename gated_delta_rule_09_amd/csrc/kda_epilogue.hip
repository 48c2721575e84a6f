// Output epilogue of a KDA layer ("Kimi K3 -- Architecture Notes", section
// 1.3, full-rank output gate): for every (token, head) row of d_v channels
//
//     y = Sigmoid(gate) * w * o / sqrt(mean(o^2) + eps),
//
// the head-wise RMSNorm of the recurrent output (the "MoE RMSNorm" page: the
// mean of squares plus epsilon under the root, a per-channel gain w, fp32
// arithmetic) times a sigmoid of the gate projection W_g x.
//
// A pure stream: each row is read once from o and from the gate logits and
// written once, 3 * d_v * sizeof(T) bytes against ~8 d_v flops, so the kernel
// is HBM-bound and built like a copy: every lane moves 16-byte pieces, a row
// is spread over LPR = d_v * sizeof(T) / 16 adjacent lanes (8, 16 or 32), a
// wave covers 64 / LPR whole rows per load instruction and U such row groups
// back to back, all loads issued before any arithmetic.  The row's sum of
// squares is reduced across its lanes with DPP moves and the gfx950 row swap
// (no LDS).  Loads and stores are non-temporal: nothing is reused.
// Launch shape, measured on 65,536 x 96 rows of 128 bf16: one wave per
// workgroup and U = 1 move 6.7 TB/s; 256 threads 6.5, U = 2 6.1 to 6.2, U = 8
// 5.6, and plain (temporal) loads and stores 6.05.
//
// y may alias o or the gate logits: every 16-byte piece is read and written
// by the same lane, reads first.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kEpiThreads = 64;       // one wave per workgroup
constexpr int kEpiRowGroups = 1;      // U: row groups per wave

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of L lanes (L = 8, 16 or 32), in every lane of the
// group.  After the two quad steps each quad holds its sum in all four lanes,
// so a mirror inside 8 lanes (lane i takes lane 7 - i, in the other quad)
// adds the neighbouring quad, and a mirror inside the 16-lane row adds the
// other half-row.  With both operands equal, v_permlane16_swap returns the
// even row's and the odd row's value of a row pair.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);   // row_half_mirror
    if constexpr (L >= 16) x += dpp<0x140>(x);   // row_mirror
    if constexpr (L >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    static_assert(L == 8 || L == 16 || L == 32, "group size");
    return x;
}

constexpr float kLog2eEpi = 1.4426950408889634f;

// Sigmoid(u) = 1 / (1 + 2^(-u log2 e)); saturates to 0 and 1 at the ends.
__device__ __forceinline__ float sigmoid_fast(float u) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2eEpi * u));
}

// Eight bf16 (four words) or four fp32 values per 16-byte piece.
template <typename T> struct Piece;
template <> struct Piece<uint16_t> {
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
template <> struct Piece<float> {
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

template <typename T, int DV>
__global__ __launch_bounds__(kEpiThreads) void gate_rmsnorm_kernel(
    const u32x4* o, const u32x4* g, const float* __restrict__ w, int64_t rows, float eps, u32x4* y) {
    constexpr int VE = Piece<T>::N;              // values per lane
    constexpr int LPR = DV / VE;                 // lanes per row
    constexpr int RPW = kWave / LPR;             // rows per wave and load instruction
    constexpr int U = kEpiRowGroups;
    constexpr int WAVES = kEpiThreads / kWave;

    const int lane = threadIdx.x % kWave;
    const int l = lane % LPR;
    const int64_t wave = (int64_t)blockIdx.x * WAVES + threadIdx.x / kWave;
    const int64_t row0 = wave * (RPW * U) + lane / LPR;

    u32x4 po[U], pg[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t row = row0 + u * RPW;
        po[u] = u32x4{0u, 0u, 0u, 0u};
        pg[u] = u32x4{0u, 0u, 0u, 0u};
        if (row < rows) {
            po[u] = __builtin_nontemporal_load(o + row * LPR + l);
            pg[u] = __builtin_nontemporal_load(g + row * LPR + l);
        }
    }

    float wv[VE];
    if (w) {
#pragma unroll
        for (int i = 0; i < VE; i += 4) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(w + l * VE + i);
            wv[i] = t[0]; wv[i + 1] = t[1]; wv[i + 2] = t[2]; wv[i + 3] = t[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < VE; ++i) wv[i] = 1.f;
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VE], gl[VE];
        Piece<T>::unpack(po[u], x);
        Piece<T>::unpack(pg[u], gl);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < VE; ++i) ss += x[i] * x[i];
        ss = group_sum<LPR>(ss);
        const float r = __builtin_amdgcn_rsqf(ss * (1.f / DV) + eps);
#pragma unroll
        for (int i = 0; i < VE; ++i) x[i] = (x[i] * r) * wv[i] * sigmoid_fast(gl[i]);
        const int64_t row = row0 + u * RPW;
        if (row < rows) __builtin_nontemporal_store(Piece<T>::pack(x), y + row * LPR + l);
    }
}

template <typename T, int DV>
constexpr int64_t epi_rows_per_block() {
    return (int64_t)(kEpiThreads / kWave) * (kWave / (DV / Piece<T>::N)) * kEpiRowGroups;
}

template <typename T, int DV>
static hipError_t launch_epi_t(const EpilogueArgs& a) {
    constexpr int64_t RPB = epi_rows_per_block<T, DV>();
    const int64_t blocks = (a.rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((gate_rmsnorm_kernel<T, DV>), dim3((unsigned)blocks), dim3(kEpiThreads), 0, a.stream,
                       (const u32x4*)a.o, (const u32x4*)a.gate, a.weight, a.rows, a.eps, (u32x4*)a.y);
    return hipGetLastError();
}

int64_t epilogue_max_rows(bool bf16, int32_t d_v) {
    // the largest row count whose grid (rows per block x blocks of kEpiThreads) fits a dispatch
    int64_t rpb;
    if (bf16) rpb = d_v == 128 ? epi_rows_per_block<uint16_t, 128>() : epi_rows_per_block<uint16_t, 64>();
    else rpb = d_v == 128 ? epi_rows_per_block<float, 128>() : epi_rows_per_block<float, 64>();
    int64_t blocks = kMaxGridItems / kEpiThreads;
    if (blocks > kMaxGridBlocks) blocks = kMaxGridBlocks;
    return blocks * rpb;
}

hipError_t launch_epilogue(const EpilogueArgs& a) {
    if (a.rows == 0) return hipSuccess;
    if (a.bf16) return a.d_v == 128 ? launch_epi_t<uint16_t, 128>(a) : launch_epi_t<uint16_t, 64>(a);
    return a.d_v == 128 ? launch_epi_t<float, 128>(a) : launch_epi_t<float, 64>(a);
}

}  // namespace kda

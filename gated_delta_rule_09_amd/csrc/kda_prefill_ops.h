// Building blocks shared by the two prefill kernels of this library (the
// single-workgroup kernel in kda_prefill.hip and the producer/state pair in
// kda_prefill_pair.hip): chunk geometry, the gfx950 row-swap butterfly, the
// MFMA operand helpers and the packed input words.  Device code only.
#pragma once

#include <type_traits>

#include "kda_device.h"

namespace kda {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kC = 64;        // chunk length (tokens per pipeline step)
constexpr int kTiles = 4;     // 16-token tiles per chunk

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// For blocks of D lanes (D = 8, 16, 32) paired as (2b, 2b + 1): the value
// that the lower and the upper block of this lane's pair hold, in every lane
// of the pair.  For D = 16 and 32 this is one gfx950 row swap (plain VALU):
// with both operands equal, v_permlane16_swap returns the even row's value in
// its first result and the odd row's in its second, in both rows of a pair;
// v_permlane32_swap does the same for the two halves of the wave.
struct LoHi { float lo, hi; };
template <int D>
__device__ __forceinline__ LoHi block_pair(float v) {
    const uint32_t u = __float_as_uint(v);
    if constexpr (D == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return {__uint_as_float(r[0]), __uint_as_float(r[1])};
    } else if constexpr (D == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return {__uint_as_float(r[0]), __uint_as_float(r[1])};
    } else {
        const float other = __shfl_xor(v, D, 64);
        const bool upper = (threadIdx.x & D) != 0;
        return {upper ? other : v, upper ? v : other};
    }
}

// Order this wave's earlier LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// MFMA helpers.  Accumulator layout (CDNA 16x16): lane l, register e holds
// D[4*(l/16) + e][l % 16].  An "acc tile" X is such a 16x16 fp32 tile; an "LDS
// row" is a pointer to the 16-wide K segment of the row that this lane's M (or
// N) index selects.  Every product pairs, for lane group g = l/16 and slot e,
// row 4g+e of the accumulator tile with column 4g+e of the LDS row, so the
// contraction is complete whatever order the hardware assigns to K.
// ---------------------------------------------------------------------------
template <typename OT> struct Op;

template <> struct Op<uint16_t> {    // bf16 operands
    static constexpr int KS = 32;    // K of an LDS x LDS product step
    typedef bf16x8 Frag;
    typedef u32x2 Xop;               // an acc tile as a bf16 operand (4 values)
    static __device__ __forceinline__ Frag frag(const uint16_t* base, int ld, int k0) {
        const int lane = threadIdx.x & 63;
        // Two 8-byte halves: rows are only 8-byte aligned (see the LDS plan).
        const uint16_t* p = base + (lane & 15) * ld + 8 * (lane >> 4) + k0;
        const u32x2 lo = ld4(p), hi = ld4(p + 4);
        return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    static __device__ __forceinline__ Xop cvt(f32x4 x) {
        return u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    }
    static __device__ __forceinline__ u32x2 ld4(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }
    // K = 16: D += A(LDS row) * X (acc tile as B, K = its rows)
    static __device__ __forceinline__ f32x4 lds_acc16(const uint16_t* arow, Xop xb, f32x4 acc) {
        const int g = (threadIdx.x & 63) >> 4;
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, ld4(arow + 4 * g)),
                                                         __builtin_bit_cast(s16x4, xb), acc, 0, 0, 0);
    }
    // K = 16: D += X^T (acc tile as A, K = its rows) * B(LDS row)
    static __device__ __forceinline__ f32x4 acc_lds16(Xop xa, const uint16_t* brow, f32x4 acc) {
        const int g = (threadIdx.x & 63) >> 4;
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, xa),
                                                         __builtin_bit_cast(s16x4, ld4(brow + 4 * g)), acc, 0, 0, 0);
    }
    // K = 32 from two 16-wide segments of the LDS row and two acc tiles.
    static __device__ __forceinline__ f32x4 lds_acc32(const uint16_t* arow1, const uint16_t* arow2, Xop x1, Xop x2,
                                                      f32x4 acc) {
        const int g = (threadIdx.x & 63) >> 4;
        const u32x2 a1 = ld4(arow1 + 4 * g), a2 = ld4(arow2 + 4 * g);
        const u32x4 a = {a1[0], a1[1], a2[0], a2[1]}, b = {x1[0], x1[1], x2[0], x2[1]};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       acc, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 acc_lds32(Xop x1, Xop x2, const uint16_t* brow1, const uint16_t* brow2,
                                                      f32x4 acc) {
        const int g = (threadIdx.x & 63) >> 4;
        const u32x2 b1 = ld4(brow1 + 4 * g), b2 = ld4(brow2 + 4 * g);
        const u32x4 a = {x1[0], x1[1], x2[0], x2[1]}, b = {b1[0], b1[1], b2[0], b2[1]};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       acc, 0, 0, 0);
    }
    // Segments: the 4 consecutive K elements of an LDS row that lane group g
    // supplies (row + 4g), loaded ahead of the MFMA that consumes them.
    typedef u32x2 Seg;
    static __device__ __forceinline__ Seg seg(const uint16_t* row) {
        return ld4(row + 4 * ((threadIdx.x & 63) >> 4));
    }
    // Transposed segment of a row-major [K][16] block X (row stride ld): lane
    // (g, t) gets X[4g + e][t], e = 0..3, i.e. the segment of row t of X^T.
    // ds_read_b64_tr_b16 hands lane t of each 16-lane group element t % 4 of
    // the 8-byte pieces read by lanes 4e + t / 4 of its group, so lane (g, t)
    // points at row 4g + t / 4, columns 4 (t % 4) .. 4 (t % 4) + 3.
    static __device__ __forceinline__ int seg_t_offset(int ld) {
        const int lane = threadIdx.x & 63, t = lane & 15;
        return (4 * (lane >> 4) + (t >> 2)) * ld + 4 * (t & 3);
    }
    static __device__ __forceinline__ Seg seg_t(const uint16_t* blk, int off, int /*ld*/) {
        typedef short s16x4t __attribute__((ext_vector_type(4)));
        const s16x4t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4t*)(blk + off));
        return __builtin_bit_cast(Seg, r);
    }
    static __device__ __forceinline__ f32x4 seg_acc16(Seg a, Xop xb, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, xb),
                                                         acc, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 seg_acc32(Seg a1, Seg a2, Xop x1, Xop x2, f32x4 acc) {
        const u32x4 a = {a1[0], a1[1], a2[0], a2[1]}, b = {x1[0], x1[1], x2[0], x2[1]};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       acc, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 acc_seg32(Xop x1, Xop x2, Seg b1, Seg b2, f32x4 acc) {
        const u32x4 a = {x1[0], x1[1], x2[0], x2[1]}, b = {b1[0], b1[1], b2[0], b2[1]};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       acc, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 acc_seg16_k32(Xop xa, Seg b1, f32x4 acc) {
        const u32x4 a = {xa[0], xa[1], 0u, 0u}, b = {b1[0], b1[1], 0u, 0u};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       acc, 0, 0, 0);
    }
    // K = 16 product issued as a K = 32 MFMA with the second half zero, for
    // accumulators that also receive 16x16x32 products: every MFMA that
    // accumulates into one register tile then has the same shape.
    static __device__ __forceinline__ f32x4 acc_lds16_k32(Xop xa, const uint16_t* brow, f32x4 acc) {
        const int g = (threadIdx.x & 63) >> 4;
        const u32x2 b1 = ld4(brow + 4 * g);
        const u32x4 a = {xa[0], xa[1], 0u, 0u}, b = {b1[0], b1[1], 0u, 0u};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       acc, 0, 0, 0);
    }
    static __device__ __forceinline__ void put(uint16_t* p, float x) { *p = f32_to_bf16(x); }
    static __device__ __forceinline__ void put2(uint16_t* p, float x0, float x1) {
        *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(x0, x1);
    }
    static __device__ __forceinline__ void put4(uint16_t* p, f32x4 x) { *reinterpret_cast<u32x2*>(p) = cvt(x); }
    static __device__ __forceinline__ void put8(uint16_t* p, f32x4 a, f32x4 b) {   // two 8-byte stores
        *reinterpret_cast<u32x2*>(p) = cvt(a);
        *reinterpret_cast<u32x2*>(p + 4) = cvt(b);
    }
};

template <> struct Op<float> {       // fp32 operands
    static constexpr int KS = 4;
    typedef float Frag;
    typedef f32x4 Xop;
    static __device__ __forceinline__ Frag frag(const float* base, int ld, int k0) {
        const int lane = threadIdx.x & 63;
        return base[(lane & 15) * ld + (lane >> 4) + k0];
    }
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
    static __device__ __forceinline__ Xop cvt(f32x4 x) { return x; }
    static __device__ __forceinline__ f32x4 lds_acc16(const float* arow, Xop xb, f32x4 acc) {
        const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(arow[4 * g + e], xb[e], acc, 0, 0, 0);
        return acc;
    }
    static __device__ __forceinline__ f32x4 acc_lds16(Xop xa, const float* brow, f32x4 acc) {
        const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[e], brow[4 * g + e], acc, 0, 0, 0);
        return acc;
    }
    static __device__ __forceinline__ f32x4 lds_acc32(const float* arow1, const float* arow2, Xop x1, Xop x2,
                                                      f32x4 acc) {
        return lds_acc16(arow2, x2, lds_acc16(arow1, x1, acc));
    }
    static __device__ __forceinline__ f32x4 acc_lds32(Xop x1, Xop x2, const float* brow1, const float* brow2,
                                                      f32x4 acc) {
        return acc_lds16(x2, brow2, acc_lds16(x1, brow1, acc));
    }
    static __device__ __forceinline__ f32x4 acc_lds16_k32(Xop xa, const float* brow, f32x4 acc) {
        return acc_lds16(xa, brow, acc);
    }
    typedef f32x4 Seg;
    static __device__ __forceinline__ Seg seg(const float* row) {
        return *reinterpret_cast<const f32x4*>(row + 4 * ((threadIdx.x & 63) >> 4));
    }
    // Transposed segment of a row-major [K][16] block X: lane (g, t) gets
    // X[4g + e][t], e = 0..3 (four scalar reads; there is no 32-bit transpose read).
    static __device__ __forceinline__ int seg_t_offset(int ld) {
        const int lane = threadIdx.x & 63;
        return 4 * (lane >> 4) * ld + (lane & 15);
    }
    static __device__ __forceinline__ Seg seg_t(const float* blk, int off, int ld) {
        return f32x4{blk[off], blk[off + ld], blk[off + 2 * ld], blk[off + 3 * ld]};
    }
    static __device__ __forceinline__ f32x4 seg_acc16(Seg a, Xop xb, f32x4 acc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], xb[e], acc, 0, 0, 0);
        return acc;
    }
    static __device__ __forceinline__ f32x4 acc_seg16(Xop xa, Seg b, f32x4 acc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[e], b[e], acc, 0, 0, 0);
        return acc;
    }
    static __device__ __forceinline__ f32x4 seg_acc32(Seg a1, Seg a2, Xop x1, Xop x2, f32x4 acc) {
        return seg_acc16(a2, x2, seg_acc16(a1, x1, acc));
    }
    static __device__ __forceinline__ f32x4 acc_seg32(Xop x1, Xop x2, Seg b1, Seg b2, f32x4 acc) {
        return acc_seg16(x2, b2, acc_seg16(x1, b1, acc));
    }
    static __device__ __forceinline__ f32x4 acc_seg16_k32(Xop xa, Seg b, f32x4 acc) { return acc_seg16(xa, b, acc); }
    static __device__ __forceinline__ void put(float* p, float x) { *p = x; }
    static __device__ __forceinline__ void put2(float* p, float x0, float x1) {
        *reinterpret_cast<f32x2*>(p) = f32x2{x0, x1};
    }
    static __device__ __forceinline__ void put4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
    static __device__ __forceinline__ void put8(float* p, f32x4 a, f32x4 b) {
        *reinterpret_cast<f32x4*>(p) = a;
        *reinterpret_cast<f32x4*>(p + 4) = b;
    }
};

// Raw input words: CPT packed elements (a bf16 pair, or one bf16 / fp32 element).
template <typename T, int CPT>
__device__ __forceinline__ uint32_t load_word(const T* p) {
    if constexpr (sizeof(T) == 2 && CPT == 2) return *reinterpret_cast<const uint32_t*>(p);
    else if constexpr (sizeof(T) == 2) return (uint32_t)(*reinterpret_cast<const uint16_t*>(p));
    else return __float_as_uint(*reinterpret_cast<const float*>(p));
}

template <typename T>
__device__ __forceinline__ float word_elem(uint32_t w, int cc) {
    if constexpr (sizeof(T) == 2) return cc == 0 ? bf16_lo(w) : bf16_hi(w);
    else return __uint_as_float(w);
}

// Element cc of a lane's packed words (bf16: two per word; fp32: one per word).
template <typename T, int N>
__device__ __forceinline__ float lane_elem(const uint32_t (&w)[N], int cc) {
    if constexpr (sizeof(T) == 2) return word_elem<T>(w[cc / 2], cc % 2);
    else return __uint_as_float(w[cc]);
}


}  // namespace
}  // namespace kda

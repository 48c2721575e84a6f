// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bf16 <-> fp32.  Widening is exact (the bf16 bits are the high half of the
// fp32 word); narrowing rounds to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Element access for the two input dtypes.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, int64_t i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {   // bf16 stored as raw 16-bit words
    static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float x) { p[i] = f32_to_bf16(x); }
};

// Value of lane Q of this lane's quad (DPP quad_perm broadcast).
template <int Q>
__device__ __forceinline__ float quad_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x55 * Q, 0xf, 0xf, false));
}
__device__ __forceinline__ float quad_bcast(float v, int q) {   // q is a constant after unrolling
    switch (q) {
        case 0: return quad_bcast<0>(v);
        case 1: return quad_bcast<1>(v);
        case 2: return quad_bcast<2>(v);
        default: return quad_bcast<3>(v);
    }
}

// Value of lane K of this lane's 16-lane row (DPP row_newbcast, gfx90a and
// later); folded by the compiler into the consuming VALU instruction.
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + K, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_bcast(float v, int k) {   // k is a constant after unrolling
    switch (k) {
        case 0: return row_bcast<0>(v);   case 1: return row_bcast<1>(v);
        case 2: return row_bcast<2>(v);   case 3: return row_bcast<3>(v);
        case 4: return row_bcast<4>(v);   case 5: return row_bcast<5>(v);
        case 6: return row_bcast<6>(v);   case 7: return row_bcast<7>(v);
        case 8: return row_bcast<8>(v);   case 9: return row_bcast<9>(v);
        case 10: return row_bcast<10>(v); case 11: return row_bcast<11>(v);
        case 12: return row_bcast<12>(v); case 13: return row_bcast<13>(v);
        case 14: return row_bcast<14>(v); default: return row_bcast<15>(v);
    }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

}  // namespace kda

namespace kda {

// Raw buffer access (gfx9 buffer descriptor, stride 0).  The base is
// wave-uniform; `bytes` bounds the range: a load at a byte offset at or past
// it returns zero and a store there is dropped.  Every offset that has to be
// range-checked is passed as the per-lane offset (the scalar offset is zero).
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t buf_ld16(Rsrc r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_ld32(Rsrc r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_ld64(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ u32x4 buf_ld128(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void buf_st64(u32x2 x, Rsrc r, uint32_t off) {
    typedef unsigned int v2u __attribute__((__vector_size__(8)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, x), r, off, 0, 0);
}
__device__ __forceinline__ void buf_st128(u32x4 x, Rsrc r, uint32_t off) {
    typedef unsigned int v4u __attribute__((__vector_size__(16)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, x), r, off, 0, 0);
}

}  // namespace kda

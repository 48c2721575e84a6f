// KDA chunkwise prefill for gfx950 (CDNA4): one fused kernel.
//
// The recurrence of "Kimi K3 -- Architecture Notes", section 1.1,
//     S_t = (I - b_t k_t k_t^T) Diag(alpha_t) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t,
// is evaluated chunkwise as section 1.2 describes it: the state is carried
// serially from chunk to chunk, and the work inside a chunk is parallel.  Tokens are streamed in chunks of 64, and each chunk is cut
// into four 16-token tiles ("secondary tiles", section 1.2).  The state is
// carried from tile to tile.  For one tile of positions r = 1..16 starting from
// state S (d_k x d_v), with x_r = sum_{s<=r} log2-decay (per key channel),
// X = x_16, e1_r = 2^{x_r}, e2_r = 2^{X - x_r}:
//
//   P_rs = sum_c q_rc e1_rc * k_sc 2^{-x_sc}       (s <= r)   decayed query-key Gram
//   M_rs = sum_c k_rc e1_rc * k_sc 2^{-x_sc}       (s <  r)   decayed key Gram
//   A    = (I + Diag(b) M)^{-1} Diag(b)                      unit-lower-triangular solve
//   W    = A (V - (K * e1) S)                                pseudo-values
//   O    = (Q * e1) S + P W                                  tile output
//   S   <- Diag(2^X) S + (K * e2)^T W                        state after the tile
//
// which is the token recurrence regrouped exactly: the delta correction of
// token r sees the decayed state and the corrections of the tile's earlier
// tokens, which gives the triangular system.
//
// Range control (section 1.2 of the notes): log alpha >= -5, so within a
// 16-token tile x lies in [-115.4, 0] (base 2, i.e. [-80, 0] in base e):
// e1, e2 lie in [2^-115, 1] and the column factor 2^{-x} in [1, 2^115], all
// representable in fp32 and bf16 (8-bit exponent).  Every factor is a running
// product of alpha = 2^{log2-decay} within the tile (one v_exp_f32 per
// element); no pairwise exponentials are needed and no factor spans more than
// one tile.
//
// Work decomposition: one workgroup of eight waves per (sequence, head, block
// of 64 value columns); the recurrence is independent across value columns.
// The waves take one of two roles, and in every chunk iteration both run at
// once on different chunks:
//   SI  (state-independent, waves 0-3, chunk c+1): wave i owns tile i.  A lane
//       owns 8 consecutive key channels (one 16-byte bf16 load) of RP
//       consecutive positions (d_k = 128: 16 lanes per token row, 4 position
//       groups of 4 positions); the running products are formed in registers
//       and joined across the position groups with a butterfly of row swaps.
//       The wave writes the tile's scaled operands, its P and M (MFMA) and beta
//       to one of two LDS buffers, selected by chunk parity.
//   SD  (state-dependent, waves 4-7, chunk c): wave w owns 16 value columns and
//       walks the chunk's four tiles.  Wave 4 + i first forms the 16x16 inverse
//       of tile i (fp32 substitution on all 64 lanes) and publishes it through
//       an LDS flag, so the four inverses of a chunk are built in parallel.  Its slab of S, and U and W, live in MFMA
//       accumulators and are fed back as MFMA operands directly (an accumulator
//       tile holds 4 consecutive rows per lane, the K-layout of an operand);
//       the LDS operands are read with the matching row permutation.
// One workgroup barrier per chunk hands the SI buffer to SD and frees the
// other buffer.  Global loads run one chunk ahead of their consumer.  The two
// value-column workgroups of a head are placed 8 workgroups apart so that they
// land on the same XCD and share its L2.
//
// A launch runs one or two jobs (PrefillJob) over the same q, k, decay and
// beta: the plain entry point runs one; the time split of one sequence runs
// its zero-state segment runs and its identity-state transition runs as two
// jobs of one launch (kda_split.hip has the other two steps).
//
// One MFMA shape per accumulator chain: on gfx950, a 16x16x16 bf16 MFMA that
// accumulates directly onto the result of a 16x16x32 bf16 MFMA was seen to
// read stale accumulator registers.  Every chain that mixes K = 16 and K = 32
// terms therefore issues the K = 16 term as a K = 32 MFMA with a zero half.
//
// Operand precision: bf16 inputs use bf16 MFMA operands with fp32 accumulation
// (v_mfma_f32_16x16x32_bf16 / 16x16x16_bf16); fp32 inputs use
// v_mfma_f32_16x16x4_f32.  The state, the decay arithmetic and the inverse are
// fp32 throughout.

#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Bounded flag waits that ran out on this device (see wait_a); read and reset
// by the host through read_wait_giveups.
__device__ uint32_t g_prefill_wait_giveups;

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kC = 64;        // chunk length (tokens per pipeline step)
constexpr int kTiles = 4;     // 16-token tiles per chunk
constexpr int kSIW = 4;       // state-independent waves (one per 16-token tile)
constexpr int kSDW = 4;       // state-dependent waves (16 value columns each)
constexpr int kNW = kSIW + kSDW;
constexpr int kBV = 16 * kSDW; // value columns per workgroup

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

// ---------------------------------------------------------------------------
// LDS plan.  Two buffers (chunk parity) of the state-independent results that
// the state-dependent half consumes, plus scratch used only inside SI.  fp32
// operands with d_k = 128 do not fit twice in 160 KB: they get one buffer, and
// the two roles then take turns on it instead of overlapping.
// ---------------------------------------------------------------------------
template <typename OT, int DK, bool GATED>
struct Plan {
    static constexpr int NBUF = (sizeof(OT) == 4 && DK == 128) ? 1 : 2;
    static constexpr int ES = sizeof(OT);
    // Row padding, chosen against LDS bank conflicts (32 banks of 4 bytes).
    // The state-dependent waves read 8 bytes from each of 16 consecutive rows
    // at one column: with bf16 rows of DK + 4 elements (DK/2 + 2 words) those
    // land on 16 distinct bank pairs.  Such rows are only 8-byte aligned, so
    // every access to them is at most 8 bytes wide.  fp32 rows keep 16 bytes
    // of padding (16-byte aligned).
    static constexpr int PAD = 4;
    static constexpr int LDK = DK + PAD;            // stride of [*, DK] rows
    // Stride of the k * e2 rows (72 words for DK = 128 bf16 or DK = 64 fp32),
    // read only through transposed segments: the four rows one lane group
    // reads then fall 8 banks apart.
    static constexpr int LDK2 = DK + 32 / ES;
    static constexpr int LD16 = 16 + PAD;           // stride of 16x16 blocks (10 words for bf16)
    // one buffer
    static constexpr int QE1 = 0;                                  // [C][LDK]   q * e1
    static constexpr int KE1 = QE1 + kC * LDK * ES;                // [C][LDK]   k * e1
    static constexpr int KE2 = KE1 + kC * LDK * ES;                // [C][LDK2]  k * e2
    static constexpr int PD = KE2 + kC * LDK2 * ES;                // [4][16][LD16] P per tile
    static constexpr int AD = PD + kTiles * 16 * LD16 * ES;        // [4][16][LD16] A per tile
    static constexpr int DEC = AD + kTiles * 16 * LD16 * ES;       // [4][DK] fp32 2^X per tile
    static constexpr int MSTR = 20;                                // fp32 stride of M^T rows (16-byte aligned)
    static constexpr int MS = DEC + kTiles * DK * 4;               // [4][16][MSTR] fp32 M^T per tile
    static constexpr int BS = MS + kTiles * 16 * MSTR * 4;         // [4][16] fp32 beta per tile
    // Gated bf16: both Gram products of a tile (P and M) are formed by the
    // state wave that inverts it, one chunk after the producer wave wrote the
    // column operand, so that operand is kept per buffer.  The gated producer
    // waves also map every decay logit (a sigmoid each), and moving the Grams
    // off them measured 5-8% faster at 64K x 96; with plain log-decay inputs
    // it measured 3-7% slower, and fp32 has no room for a second copy, so
    // there the producer waves form them.
    static constexpr bool GSD = ES == 2 && GATED;
    static constexpr int KBIN = BS + kTiles * 16 * 4;              // [C][LDK]   k * 2^{-x} (GSD)
    static constexpr int BUF = GSD ? KBIN + kC * LDK * ES : KBIN;
    // scratch (producer waves only)
    static constexpr int KB = NBUF * BUF;                          // [C][LDK]   k * 2^{-x} (not GSD)
    static constexpr int FLAG = GSD ? KB : KB + kC * LDK * ES;     // [4] int: chunk whose A of tile i is ready
    static constexpr int TOTAL = FLAG + 16;
    static_assert(BUF % 16 == 0 && KB % 16 == 0 && KBIN % 16 == 0, "alignment");
    static_assert(TOTAL <= 160 * 1024, "LDS plan exceeds 160 KB");
};

// GATED: `decay` holds the decay logits z (element type T) and `beta` the
// write-strength logits; the lower-bounded map of section 1.2 of the notes
// (Kimi K3 row of its table), g = -5 Sigmoid(e^{A_h} z), beta = Sigmoid(logit),
// is applied on the fly.  Otherwise `decay` holds log alpha (fp32) and `beta`
// beta.
//
// A launch runs one or two jobs over the same q, k, decay and beta (the
// workgroups of j1 follow those of j0); each job is a set of sequences with
// their own values, initial states and outputs (PrefillJob).
template <typename T, int DK, int DV, bool GATED>
__global__ __launch_bounds__(64 * kNW, 1) void prefill_kernel(
    const T* __restrict__ q, const T* __restrict__ k,
    const void* __restrict__ decay, const float* __restrict__ beta, const float* __restrict__ a_log,
    int64_t total_T, int H, PrefillJob j0, PrefillJob j1) {
    // Decay input: fp32 log alpha, or decay logits of type T (GATED).
    using DT = typename std::conditional<GATED, T, float>::type;
    const DT* log_alpha = reinterpret_cast<const DT*>(decay);
    const bool second = (int)blockIdx.x >= j0.blocks;
    const PrefillJob& J = second ? j1 : j0;
    const T* __restrict__ v = reinterpret_cast<const T*>(J.v);
    const float* __restrict__ init_state = J.init_state;
    const int32_t* __restrict__ cu_seqlens = J.cu_seqlens;
    T* __restrict__ o = reinterpret_cast<T*>(J.o);
    float* __restrict__ final_state = J.final_state;
    const int units = J.units;
    using OT = T;
    using OP = Op<OT>;
    using PL = Plan<OT, DK, GATED>;
    using Xop = typename OP::Xop;
    constexpr int KS = OP::KS;
    constexpr int CPL = 8;                // SI: key channels per lane (16-byte loads of bf16 q, k)
    constexpr int LPR = DK / CPL;         // SI: lanes per token row
    constexpr int NG = 64 / LPR;          // SI: position groups of a tile
    constexpr int RP = 16 / NG;           // SI: consecutive tile positions per lane
    constexpr int QWN = CPL * (int)sizeof(T) / 4;   // 32-bit words holding CPL q (or k) elements
    constexpr int NCT = DK / 16;          // 16-row channel tiles of the state
    constexpr int NKS = DK / KS;          // K-steps of the Gram products
    constexpr int NV = DV / kBV;          // value-column workgroups per (sequence, head)
    static_assert((LPR == 8 || LPR == 16) && RP >= 2, "SI mapping");
    static_assert(NV == 1 || NV == 2, "value blocking");

    // Workgroup -> (unit = sequence * H + head, value block); in the jobs of a
    // time split a "sequence" is one segment.  With two value blocks, the pair
    // of a unit sits 8 workgroups apart (same XCD).
    const int lid = (int)blockIdx.x - (second ? j0.blocks : 0);
    int unit, vblk;
    if constexpr (NV == 2) {
        unit = 8 * (lid >> 4) + (lid & 7);
        vblk = (lid >> 3) & 1;
    } else {
        unit = lid;
        vblk = 0;
    }
    if (unit >= units) return;
    const int n = unit / H;
    const int h = unit - n * H;
    const float eA = GATED ? __expf(a_log[h]) : 1.f;    // e^{A_h}, the per-head logit scale

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int* sFLAG = reinterpret_cast<int*>(smem + PL::FLAG);
    OT* sKB = reinterpret_cast<OT*>(smem + PL::KB);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int vcol = vblk * kBV + 16 * (wave - kSIW);   // SD waves: first value column
    const int tro = OP::seg_t_offset(PL::LDK2);          // SD: lane offset of transposed reads
    const int cb = (lane % LPR) * CPL;           // SI: first key channel of this lane
    const int pg = lane / LPR;                   // SI: position group (positions RP pg .. RP pg + RP - 1)

    // Sequence range, clamped so malformed offsets cannot address out of range:
    // from the offsets, or segment n + n_off of seg_len tokens, or every token.
    int64_t seq0 = 0, seq1 = total_T;
    if (cu_seqlens != nullptr) {
        seq0 = cu_seqlens[n];
        seq1 = cu_seqlens[n + 1];
    } else if (J.seg_len > 0) {
        seq0 = (int64_t)(n + J.n_off) * J.seg_len;
        seq1 = seq0 + J.seg_len;
    }
    seq0 = seq0 < 0 ? 0 : (seq0 > total_T ? total_T : seq0);
    seq1 = seq1 < seq0 ? seq0 : (seq1 > total_T ? total_T : seq1);
    const int64_t len = seq1 - seq0;
    const int64_t nchunks = (len + kC - 1) / kC;

    // ---- prefetch registers (one chunk ahead).  Loads go through buffer
    // descriptors whose range ends after the chunk's last valid token, so rows
    // past a sequence's end read as zero (decay 1, key, query, value and beta
    // 0) and output rows past it are not written.
    constexpr int LAW = CPL * (int)sizeof(DT) / 4;   // 32-bit words holding CPL decay inputs
    uint32_t la_w[RP][LAW];      // raw words: fp32 log alpha, or decay logits (GATED)
    uint32_t qw_r[RP][QWN], kw_r[RP][QWN];
    float beta_r;
    uint32_t v_r[kTiles][4];     // v[16 i + 4 lg + e][vcol + l16], raw words
    auto chunk_len = [&](int64_t c) { return (int)((len - c * kC) < kC ? (len - c * kC) : kC); };
    // Rows of the [tokens, H] layout from a head's first valid row to the end
    // of its last valid row: (Lc - 1) * H + 1.
    // Beyond the last chunk the range is empty (every load returns zero and
    // touches no memory), so prefetches can be issued unconditionally and the
    // compiler's in-order wait counts never include them.
    auto valid_rows = [&](int64_t c) {
        return c < nchunks ? (uint32_t)(chunk_len(c) - 1) * (uint32_t)H + 1u : 0u;
    };
    auto row_of = [&](int64_t c) { return (seq0 + (c < nchunks ? c : 0) * kC) * H + h; };
    const uint32_t p0 = 16 * wave + RP * pg;    // SI: chunk position of this lane's first row
    // The state-independent prefetch comes in two parts, each issued as soon
    // as its registers are free: log-decay after the exponentials, q, k and
    // beta after the products of the tile.
    auto load_la = [&](int64_t c) {
        const Rsrc rla = make_rsrc(log_alpha + row_of(c) * DK, valid_rows(c) * (DK * (uint32_t)sizeof(DT)));
        const uint32_t rs = (uint32_t)H * DK;
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const uint32_t el = (p0 + r) * rs + cb;
#pragma unroll
            for (int u = 0; u < LAW / 4; ++u) {
                const u32x4 a = buf_ld128(rla, el * (uint32_t)sizeof(DT) + 16 * u);
#pragma unroll
                for (int j = 0; j < 4; ++j) la_w[r][4 * u + j] = a[j];
            }
        }
    };
    struct QKRes { Rsrc q, k; };
    auto qk_rsrc = [&](int64_t c) {
        const uint32_t nb = valid_rows(c) * (DK * (uint32_t)sizeof(T));
        const int64_t row0 = row_of(c);
        return QKRes{make_rsrc(q + row0 * DK, nb), make_rsrc(k + row0 * DK, nb)};
    };
    auto load_qk_row = [&](const QKRes& rr, int r) {
        const uint32_t el = (p0 + r) * ((uint32_t)H * DK) + cb;
#pragma unroll
        for (int u = 0; u < QWN / 4; ++u) {
            const u32x4 qv = buf_ld128(rr.q, el * (uint32_t)sizeof(T) + 16 * u);
            const u32x4 kv = buf_ld128(rr.k, el * (uint32_t)sizeof(T) + 16 * u);
#pragma unroll
            for (int j = 0; j < 4; ++j) { qw_r[r][4 * u + j] = qv[j]; kw_r[r][4 * u + j] = kv[j]; }
        }
    };
    auto load_beta = [&](int64_t c) {
        beta_r = __uint_as_float(buf_ld32(make_rsrc(beta + row_of(c), valid_rows(c) * 4),
                                          (16 * wave + l16) * (uint32_t)H * 4));
    };
    // No values (v null): an empty range, so every value reads as zero.
    auto v_rsrc = [&](int64_t c) {
        return v != nullptr ? make_rsrc(v + row_of(c) * DV + vcol, valid_rows(c) * (DV * (uint32_t)sizeof(T)))
                            : make_rsrc(nullptr, 0u);
    };
    auto load_v_tile = [&](Rsrc rv, int i) {
        const uint32_t rs = (uint32_t)H * DV;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t el = (16 * i + 4 * lg + e) * rs + l16;
            // Raw words: widening happens at the use, so that the load is not waited for here.
            if constexpr (sizeof(T) == 2) v_r[i][e] = buf_ld16(rv, el * 2);
            else v_r[i][e] = buf_ld32(rv, el * 4);
        }
    };

    // ---- SI: state-independent results of chunk c into buffer (c & 1).  Wave i = tile i.
    auto si = [&](int64_t c) {
        unsigned char* buf = smem + (c % PL::NBUF) * PL::BUF;
        OT* sQE1 = reinterpret_cast<OT*>(buf + PL::QE1);
        OT* sKE1 = reinterpret_cast<OT*>(buf + PL::KE1);
        OT* sKE2 = reinterpret_cast<OT*>(buf + PL::KE2);
        OT* sPD = reinterpret_cast<OT*>(buf + PL::PD);
        float* sDEC = reinterpret_cast<float*>(buf + PL::DEC);
        float* sMS = reinterpret_cast<float*>(buf + PL::MS);
        float* sBS = reinterpret_cast<float*>(buf + PL::BS);
        OT* sKBc = PL::GSD ? reinterpret_cast<OT*>(buf + PL::KBIN) : sKB;
        const int ti = wave;
        // Lane = (key channels cb .. cb+7; tile positions pb .. pb+RP-1).
        // alpha = 2^{l2}; e1 = prefix products over the tile, e2 = suffix
        // products excluding r, dec = the product over the whole tile.  Each
        // lane forms the running products of its RP positions; a butterfly
        // over the position groups then supplies the product of the groups
        // before (pre) and after (post) this lane's, and the tile total.
        const int pb = (int)p0;
        const QKRes rq_next = qk_rsrc(c + 1);
        float al[RP][CPL], dec[CPL];
        // Base-2 log-decay of each element.  GATED: g = -5 Sigmoid(e^{A_h} z);
        // rows past the end of a partial chunk get g = 0 (their logits read
        // as 0, which the map does not send to 0).
        float l2[RP][CPL];
#pragma unroll
        for (int r = 0; r < RP; ++r)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                if constexpr (GATED) {
                    const float u = eA * lane_elem<T>(la_w[r], cc);
                    l2[r][cc] = (-5.f * kLog2e) * __builtin_amdgcn_rcpf(1.f + fexp2(-kLog2e * u));
                } else {
                    l2[r][cc] = __uint_as_float(la_w[r][cc]) * kLog2e;
                }
            }
        if constexpr (GATED) {
            const int lc = chunk_len(c);
            if (lc < kC) {
#pragma unroll
                for (int r = 0; r < RP; ++r)
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc) l2[r][cc] = (int)p0 + r < lc ? l2[r][cc] : 0.f;
            }
        }
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
            for (int r = 0; r < RP; ++r) al[r][cc] = fexp2(l2[r][cc]);
            float t = al[0][cc];
#pragma unroll
            for (int r = 1; r < RP; ++r) t *= al[r][cc];
            dec[cc] = t;                       // product over this lane's positions
        }
        load_la(c + 1);
        __builtin_amdgcn_sched_barrier(0);
        // Butterfly over the position groups (blocks of LPR lanes, then 2 LPR,
        // ...): pre = product of the groups before this lane's, post = of the
        // groups after it, dec = of all (the same value in every lane).
        float pre[CPL], post[CPL];
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) { pre[cc] = 1.f; post[cc] = 1.f; }
        auto level = [&](auto dtag) {
            constexpr int D = decltype(dtag)::value;
            const bool upper = (lane & D) != 0;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const LoHi b = block_pair<D>(dec[cc]);
                pre[cc] *= upper ? b.lo : 1.f;
                post[cc] *= upper ? 1.f : b.hi;
                dec[cc] = b.lo * b.hi;
            }
        };
        if constexpr (LPR == 8) level(std::integral_constant<int, 8>{});
        level(std::integral_constant<int, 16>{});
        level(std::integral_constant<int, 32>{});
        // Running products seeded with pre and post.
        float e1[RP][CPL], e2[RP][CPL], fB[CPL];
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            float p = pre[cc];
#pragma unroll
            for (int r = 0; r < RP; ++r) { p *= al[r][cc]; e1[r][cc] = p; }
            float sfx = post[cc];
#pragma unroll
            for (int r = RP - 1; r >= 0; --r) { e2[r][cc] = sfx; if (r > 0) sfx *= al[r][cc]; }
            fB[cc] = __builtin_amdgcn_rcpf(dec[cc]);
        }
        if (pg == 0) {
#pragma unroll
            for (int u = 0; u < CPL / 4; ++u)
                *reinterpret_cast<f32x4*>(sDEC + ti * DK + cb + 4 * u) =
                    f32x4{dec[4 * u], dec[4 * u + 1], dec[4 * u + 2], dec[4 * u + 3]};
        }
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const int orow = (pb + r) * PL::LDK + cb;
            f32x4 qe1[2], ke1[2], ke2[2], kb[2];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const float qv = lane_elem<T>(qw_r[r], cc);
                const float kv = lane_elem<T>(kw_r[r], cc);
                qe1[cc / 4][cc % 4] = qv * e1[r][cc];
                ke1[cc / 4][cc % 4] = kv * e1[r][cc];
                ke2[cc / 4][cc % 4] = kv * e2[r][cc];
                kb[cc / 4][cc % 4] = ke2[cc / 4][cc % 4] * fB[cc];
            }
            OP::put8(sQE1 + orow, qe1[0], qe1[1]);
            OP::put8(sKE1 + orow, ke1[0], ke1[1]);
            OP::put8(sKE2 + (pb + r) * PL::LDK2 + cb, ke2[0], ke2[1]);
            OP::put8(sKBc + orow, kb[0], kb[1]);
            // Row r of q and k is consumed: load the same row of the next chunk.
            load_qk_row(rq_next, r);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (lane < 16) {
            if constexpr (GATED)   // beta = Sigmoid(logit); 0 past the end of the sequence
                sBS[ti * 16 + lane] = 16 * ti + lane < chunk_len(c)
                                          ? __builtin_amdgcn_rcpf(1.f + fexp2(-kLog2e * beta_r)) : 0.f;
            else
                sBS[ti * 16 + lane] = beta_r;
        }
        load_beta(c + 1);
        wave_lds_sync();

        // P and M of the tile, transposed (D[s][r] = sum_c Kb[s][c] X[r][c]):
        // lane holds row r = l16, columns s = 4 lg + e.  (bf16: M is formed by
        // the state wave that inverts the tile.)
        if constexpr (!PL::GSD) {
            const OT* rq = sQE1 + 16 * ti * PL::LDK;
            const OT* rk = sKE1 + 16 * ti * PL::LDK;
            const OT* rb = sKBc + 16 * ti * PL::LDK;
            f32x4 accP = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const typename OP::Frag fb = OP::frag(rb, PL::LDK, ks * KS);
                accP = OP::mma(fb, OP::frag(rq, PL::LDK, ks * KS), accP);
                if constexpr (!PL::GSD) accM = OP::mma(fb, OP::frag(rk, PL::LDK, ks * KS), accM);
            }
            f32x4 vp;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 4 * lg + e;
                vp[e] = s <= l16 ? accP[e] : 0.f;
                // M^T[s][r], columns in (r % 4, r / 4) order
                if constexpr (!PL::GSD)
                    sMS[(ti * 16 + s) * PL::MSTR + 4 * (l16 & 3) + (l16 >> 2)] = s < l16 ? accM[e] : 0.f;
            }
            OP::put4(sPD + (ti * 16 + l16) * PL::LD16 + 4 * lg, vp);
        }
    };

    // ---- Inverse of tile ti of chunk c (run by the state-dependent waves, one
    // tile each, on the M and beta the producer waves left in buffer c & 1).
    auto inverse = [&](int64_t c, int ti) {
        unsigned char* buf = smem + (c % PL::NBUF) * PL::BUF;
        OT* sAD = reinterpret_cast<OT*>(buf + PL::AD);
        float* sMS = reinterpret_cast<float*>(buf + PL::MS);
        const float* sBS = reinterpret_cast<const float*>(buf + PL::BS);
        if constexpr (PL::GSD) {
            // P and M of the tile (transposed, as the producer waves would store
            // them); P is published with A (it is written before A's flag).
            const OT* rq = reinterpret_cast<const OT*>(buf + PL::QE1) + 16 * ti * PL::LDK;
            const OT* rk = reinterpret_cast<const OT*>(buf + PL::KE1) + 16 * ti * PL::LDK;
            const OT* rb = reinterpret_cast<const OT*>(buf + PL::KBIN) + 16 * ti * PL::LDK;
            OT* sPD = reinterpret_cast<OT*>(buf + PL::PD);
            f32x4 accP = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const typename OP::Frag fb = OP::frag(rb, PL::LDK, ks * KS);
                accP = OP::mma(fb, OP::frag(rq, PL::LDK, ks * KS), accP);
                accM = OP::mma(fb, OP::frag(rk, PL::LDK, ks * KS), accM);
            }
            f32x4 vp;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 4 * lg + e;
                vp[e] = s <= l16 ? accP[e] : 0.f;
                sMS[(ti * 16 + s) * PL::MSTR + 4 * (l16 & 3) + (l16 >> 2)] = s < l16 ? accM[e] : 0.f;
            }
            OP::put4(sPD + (ti * 16 + l16) * PL::LD16 + 4 * lg, vp);
            wave_lds_sync();
        }
        // A = (I + Diag(b) M)^{-1} Diag(b) by right-looking substitution on
        // all 64 lanes: lane = (column j = lane / 4, row residue q = lane % 4)
        // and holds rows r = 4 m + q, m = 0..3, of column j of X = (I +
        // Diag(b) M)^{-1}:  x_s = [s == j] - b_s sum_{s' < s} M_{s s'} x_{s'}.
        // At step s the lane that owns row s forms x_s, a quad broadcast (DPP)
        // hands it to the other three lanes of its column, and every lane adds
        // M_{r s} x_s to its rows.  Row s of M^T is stored with its columns in
        // (q, m) order, so one 16-byte read gives a lane its four M_{r s}.
        {
            const int j = lane >> 2, q = lane & 3;
            const float* MT = sMS + ti * 16 * PL::MSTR + 4 * q;
            float bt[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 b4 = *reinterpret_cast<const f32x4*>(sBS + ti * 16 + 4 * q4);
#pragma unroll
                for (int e = 0; e < 4; ++e) bt[4 * q4 + e] = b4[e];
            }
            f32x4 mr[16];
#pragma unroll
            for (int s2 = 0; s2 < 16; ++s2) mr[s2] = *reinterpret_cast<const f32x4*>(MT + s2 * PL::MSTR);
            float acc[4], xs[4], one[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) { acc[m] = 0.f; xs[m] = 0.f; one[m] = (4 * m + q == j) ? 1.f : 0.f; }
#pragma unroll
            for (int s2 = 0; s2 < 16; ++s2) {
                const int ms = s2 >> 2, qs = s2 & 3;
                const float cand = fmaf(-bt[s2], acc[ms], one[ms]);   // x_s in the lanes with q == s % 4
                if (q == qs) xs[ms] = cand;
                const float x = quad_bcast(cand, qs);
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (4 * m + 3 > s2) acc[m] = fmaf(mr[s2][m], x, acc[m]);
            }
            const float bj = sBS[ti * 16 + j];
#pragma unroll
            for (int m = 0; m < 4; ++m) OP::put(sAD + (ti * 16 + 4 * m + q) * PL::LD16 + j, xs[m] * bj);
        }
        // Publish: every write of A is complete before the flag names chunk c.
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) __hip_atomic_store(sFLAG + ti, (int)c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    // Wait until the A of tile i of chunk c is published.  Each flag is written
    // by a wave whose own path up to that write has no waits, so the loop
    // ends; the bound only guards against a logic error.
    // A wait that runs out is counted in a device word the host can read (the
    // outputs of that workgroup are then not to be trusted).
    auto wait_a = [&](int64_t c, int i) {
        bool ready = false;
        for (int spin = 0; spin < (1 << 22) && !ready; ++spin) {
            ready = __hip_atomic_load(sFLAG + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == (int)c;
            if (!ready) __builtin_amdgcn_s_sleep(1);
        }
        if (!ready && lane == 0) atomicAdd(&g_prefill_wait_giveups, 1u);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    // ---- SD: state-dependent part of chunk c from buffer (c & 1).  Wave w = value columns.
    auto sd = [&](int64_t c, f32x4 (&Sacc)[NCT]) {
        const Rsrc rv_next = v_rsrc(c + 1);
        const unsigned char* buf = smem + (c % PL::NBUF) * PL::BUF;
        const OT* sQE1 = reinterpret_cast<const OT*>(buf + PL::QE1);
        const OT* sKE1 = reinterpret_cast<const OT*>(buf + PL::KE1);
        const OT* sKE2 = reinterpret_cast<const OT*>(buf + PL::KE2);
        const OT* sPD = reinterpret_cast<const OT*>(buf + PL::PD);
        const OT* sAD = reinterpret_cast<const OT*>(buf + PL::AD);
        const float* sDEC = reinterpret_cast<const float*>(buf + PL::DEC);
        const Rsrc ro = make_rsrc(o + (row_of(c) - J.o_row0 * H) * DV + vcol, valid_rows(c) * (DV * (uint32_t)sizeof(T)));
        inverse(c, wave - kSIW);
        // LDS operands of one tile (A excepted: it is read after its flag).
        // Tile decay of the state rows 16 ct + 4 lg + e: the 4 NCT values a
        // 16-lane row needs are spread over its lanes (VPL each) and broadcast
        // into the multiplies.
        using Seg = typename OP::Seg;
        constexpr int VPL = NCT / 4;
        struct TileOps { Seg kseg[NCT], qseg[NCT], eseg[NCT], pseg; float decv[VPL]; };
        auto load_ops = [&](int i, TileOps& t) {
            const OT* krow = sKE1 + (16 * i + l16) * PL::LDK;
            const OT* qrow = sQE1 + (16 * i + l16) * PL::LDK;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) t.kseg[ct] = OP::seg(krow + 16 * ct);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) t.qseg[ct] = OP::seg(qrow + 16 * ct);
            if constexpr (!PL::GSD) t.pseg = OP::seg(sPD + (16 * i + l16) * PL::LD16);   // (GSD: after A's flag)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) t.eseg[ct] = OP::seg_t(sKE2 + 16 * i * PL::LDK2 + 16 * ct, tro, PL::LDK2);
            const float* dp = sDEC + i * DK + 16 * ((VPL * l16) >> 2) + 4 * lg + ((VPL * l16) & 3);
#pragma unroll
            for (int u = 0; u < VPL; ++u) t.decv[u] = dp[u];
        };
        // Software pipeline over the tiles: the operands of tile i + 1 are read
        // while tile i computes.  A of tile i is read first (after its flag), so
        // that waiting for it never waits for the prefetch (LDS returns in order).
        // fp32 operands with d_k = 128 would need too many registers for two
        // sets: their tiles read their own operands.
        constexpr int NOPS = (sizeof(OT) == 4 && DK == 128) ? 1 : 2;
        TileOps ops[NOPS];
        if constexpr (NOPS == 2) load_ops(0, ops[0]);
#pragma unroll
        for (int i = 0; i < kTiles; ++i) {
            if (i != wave - kSIW) wait_a(c, i);
            const Seg aseg = OP::seg(sAD + (16 * i + l16) * PL::LD16);
            Seg pseg_f{};
            if constexpr (PL::GSD) pseg_f = OP::seg(sPD + (16 * i + l16) * PL::LD16);   // P is published with A
            if constexpr (NOPS == 2) {
                if (i + 1 < kTiles) load_ops(i + 1, ops[(i + 1) & 1]);
            } else {
                load_ops(i, ops[0]);
            }
            const TileOps& cur = ops[i % NOPS];
            const auto& kseg = cur.kseg;
            const auto& qseg = cur.qseg;
            const auto& eseg = cur.eseg;
            const Seg pseg = PL::GSD ? pseg_f : cur.pseg;
            const auto& decv = cur.decv;
            Xop Sop[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) Sop[ct] = OP::cvt(Sacc[ct]);
            // U = V_i - (K e1)_i S   (D[r][v]: lane v = l16, rows r = 4 lg + e)
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ct = 0; ct < NCT; ct += 2) acc = OP::seg_acc32(kseg[ct], kseg[ct + 1], Sop[ct], Sop[ct + 1], acc);
            f32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                y[e] = word_elem<T>(v_r[i][e], 0) - acc[e];
            }
            // v of this tile is consumed: load the same tile of the next chunk.
            load_v_tile(rv_next, i);
            __builtin_amdgcn_sched_barrier(0);   // keep the prefetch here, early in the chunk
            // W = A U
            f32x4 w = {0.f, 0.f, 0.f, 0.f};
            w = OP::seg_acc16(aseg, OP::cvt(y), w);
            const Xop Wop = OP::cvt(w);
            // O^T = S^T (Q e1)^T + W^T P^T   (lane: row r = l16, columns 4 lg + e)
            f32x4 oacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ct = 0; ct < NCT; ct += 2) oacc = OP::acc_seg32(Sop[ct], Sop[ct + 1], qseg[ct], qseg[ct + 1], oacc);
            oacc = OP::acc_seg16_k32(Wop, pseg, oacc);
            // S <- Diag(2^X) S + (K e2)^T W   (lane v = l16, rows c = 16 ct + 4 lg + e)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 sd4;
#pragma unroll
                for (int e = 0; e < 4; ++e) sd4[e] = Sacc[ct][e] * row_bcast(decv[(4 * ct + e) % VPL], (4 * ct + e) / VPL);
                Sacc[ct] = OP::seg_acc16(eseg[ct], Wop, sd4);
            }
            const uint32_t ooff = ((16 * i + l16) * (uint32_t)H * DV + 4 * lg) * (uint32_t)sizeof(T);
            if constexpr (sizeof(T) == 2) buf_st64(OP::cvt(oacc), ro, ooff);
            else buf_st128(__builtin_bit_cast(u32x4, oacc), ro, ooff);
        }
    };

    // Waves 0..3 produce chunk c+1's state-independent results while waves
    // 4..7 consume chunk c's.  Both roles pass the same barriers: one after
    // the first chunk's results, then one per chunk.
    if (wave < kSIW) {
        if (nchunks > 0) {
            load_la(0);
            {
                const QKRes r0 = qk_rsrc(0);
#pragma unroll
                for (int r = 0; r < RP; ++r) load_qk_row(r0, r);
                load_beta(0);
            }
            si(0);
            __syncthreads();
            for (int64_t c = 0; c < nchunks; ++c) {
                if constexpr (PL::NBUF == 1) __syncthreads();   // the state waves are done with the buffer
                if (c + 1 < nchunks) si(c + 1);
                __syncthreads();
            }
        }
    } else {
        // The state-dependent waves carry the serial chain of the recurrence:
        // they take issue priority over the producer waves on their SIMD.
        __builtin_amdgcn_s_setprio(2);
        // This wave's state slab: Sacc[ct][e] = S[16 ct + 4 lg + e][vcol + l16].
        f32x4 Sacc[NCT];
        const int64_t sbase = ((int64_t)n * H + h) * DK * DV;
    #pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
    #pragma unroll
            for (int e = 0; e < 4; ++e)
                Sacc[ct][e] = J.init_mode == kInitIdentity ? (16 * ct + 4 * lg + e == vcol + l16 ? 1.f : 0.f)
                              : (init_state != nullptr && (J.init_mode == kInitAll || n == 0))
                                  ? init_state[sbase + (int64_t)(16 * ct + 4 * lg + e) * DV + vcol + l16] : 0.f;
        if (wave == kSIW && lane < kTiles) __hip_atomic_store(sFLAG + lane, -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (nchunks > 0) {
            {
                const Rsrc rv0 = v_rsrc(0);
#pragma unroll
                for (int i = 0; i < kTiles; ++i) load_v_tile(rv0, i);
            }
            __syncthreads();
            for (int64_t c = 0; c < nchunks; ++c) {
                sd(c, Sacc);
                if constexpr (PL::NBUF == 1) __syncthreads();
                __syncthreads();
            }
        }
        if (final_state != nullptr) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    final_state[sbase + (int64_t)(16 * ct + 4 * lg + e) * DV + vcol + l16] = Sacc[ct][e];
        }
    }
}

// Workgroups of a job: with two value blocks, the pair of a unit sits 8
// workgroups apart (the grid is padded to whole groups of 16).
template <int DV>
int64_t job_blocks(int64_t units) {
    return DV / kBV == 2 ? 16 * ((units + 7) / 8) : units;
}

// One launch of the jobs j0 and j1 (j1.units may be 0).
template <typename T, int DK, int DV, bool GATED>
hipError_t launch_jobs(const PrefillArgs& a, PrefillJob j0, PrefillJob j1) {
    using PL = Plan<T, DK, GATED>;
    auto kern = prefill_kernel<T, DK, DV, GATED>;
    // The dynamic-LDS limit is set on every launch: it is a host-side property of
    // the function on the current device, cheap to set, and no cached flag can
    // then miss a second device or race between threads.
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       PL::TOTAL);
    if (e != hipSuccess) return e;
    j0.blocks = (int32_t)job_blocks<DV>(j0.units);
    j1.blocks = (int32_t)job_blocks<DV>(j1.units);
    const int64_t blocks = (int64_t)j0.blocks + j1.blocks;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kNW), PL::TOTAL, a.stream,
                       (const T*)a.q, (const T*)a.k, a.log_alpha, a.beta, a.a_log, a.total_T, a.H, j0, j1);
    return hipGetLastError();
}

template <typename T, int DK, int DV, bool GATED>
hipError_t launch_t(const PrefillArgs& a) {
    PrefillJob j0{a.v, a.init_state, a.cu_seqlens, a.o, a.final_state, 0, 0, 0, a.N * a.H, 0, kInitAll};
    PrefillJob none{};
    return launch_jobs<T, DK, DV, GATED>(a, j0, none);
}

// Time split of one sequence into `segments` runs of seg_len tokens (phase 1):
// every segment from a zero state (the first from the initial state), giving
// its outputs in o and its end state in ends[p]; and every segment after the
// first from the identity with no values (d_k value columns), giving the
// outputs Phi_t^T q_t in qt (rows from token seg_len on) and its transition
// in phis[p - 1].  One launch when d_v = d_k, else two.
template <typename T, int DK, int DV, bool GATED>
hipError_t launch_split_t(const PrefillArgs& a, const SplitWork& w) {
    PrefillJob run{a.v, a.init_state, nullptr, a.o, w.ends, w.seg_len, 0, 0, w.segments * a.H, 0, kInitFirst};
    PrefillJob trans{nullptr, nullptr, nullptr, w.qt, w.phis, w.seg_len, w.seg_len, 1,
                     (w.segments - 1) * a.H, 0, kInitIdentity};
    if constexpr (DV == DK) {
        return launch_jobs<T, DK, DV, GATED>(a, run, trans);
    } else {
        PrefillJob none{};
        hipError_t e = launch_jobs<T, DK, DV, GATED>(a, run, none);
        if (e != hipSuccess) return e;
        return launch_jobs<T, DK, DK, GATED>(a, trans, none);
    }
}

}  // namespace

bool prefill_grid_fits(int64_t units, int32_t d_v) {
    return grid_fits(d_v == 128 ? job_blocks<128>(units) : job_blocks<64>(units), 64 * kNW);
}

bool split_grid_fits(int64_t run_units, int64_t trans_units, int32_t d_k, int32_t d_v) {
    auto blocks = [](int64_t u, int32_t d) { return d == 128 ? job_blocks<128>(u) : job_blocks<64>(u); };
    if (d_k == d_v) return grid_fits(blocks(run_units, d_v) + blocks(trans_units, d_k), 64 * kNW);
    return grid_fits(blocks(run_units, d_v), 64 * kNW) && grid_fits(blocks(trans_units, d_k), 64 * kNW);
}

hipError_t read_wait_giveups(uint32_t* count, bool reset) {
    hipError_t e = hipMemcpyFromSymbol(count, HIP_SYMBOL(g_prefill_wait_giveups), sizeof(uint32_t));
    if (e == hipSuccess && reset) {
        const uint32_t zero = 0;
        e = hipMemcpyToSymbol(HIP_SYMBOL(g_prefill_wait_giveups), &zero, sizeof(uint32_t));
    }
    return e;
}

template <bool GATED>
hipError_t launch_prefill_g(const PrefillArgs& a) {
    if (a.bf16) {
        if (a.d_k == 128)
            return a.d_v == 128 ? launch_t<uint16_t, 128, 128, GATED>(a) : launch_t<uint16_t, 128, 64, GATED>(a);
        return a.d_v == 128 ? launch_t<uint16_t, 64, 128, GATED>(a) : launch_t<uint16_t, 64, 64, GATED>(a);
    }
    if (a.d_k == 128)
        return a.d_v == 128 ? launch_t<float, 128, 128, GATED>(a) : launch_t<float, 128, 64, GATED>(a);
    return a.d_v == 128 ? launch_t<float, 64, 128, GATED>(a) : launch_t<float, 64, 64, GATED>(a);
}

hipError_t launch_prefill(const PrefillArgs& a) {
    return a.gated ? launch_prefill_g<true>(a) : launch_prefill_g<false>(a);
}

template <bool GATED>
hipError_t launch_split_g(const PrefillArgs& a, const SplitWork& w) {
    if (a.bf16) {
        if (a.d_k == 128)
            return a.d_v == 128 ? launch_split_t<uint16_t, 128, 128, GATED>(a, w)
                                : launch_split_t<uint16_t, 128, 64, GATED>(a, w);
        return a.d_v == 128 ? launch_split_t<uint16_t, 64, 128, GATED>(a, w) : launch_split_t<uint16_t, 64, 64, GATED>(a, w);
    }
    if (a.d_k == 128)
        return a.d_v == 128 ? launch_split_t<float, 128, 128, GATED>(a, w)
                            : launch_split_t<float, 128, 64, GATED>(a, w);
    return a.d_v == 128 ? launch_split_t<float, 64, 128, GATED>(a, w) : launch_split_t<float, 64, 64, GATED>(a, w);
}

hipError_t launch_prefill_split_runs(const PrefillArgs& a, const SplitWork& w) {
    return a.gated ? launch_split_g<true>(a, w) : launch_split_g<false>(a, w);
}

}  // namespace kda

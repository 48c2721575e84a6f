// KDA chunkwise prefill for gfx950 (CDNA4): one fused kernel.
//
// The recurrence of "Kimi K3 -- Architecture Notes", section 1.1,
//     S_t = (I - b_t k_t k_t^T) Diag(alpha_t) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t,
// is evaluated "recurrent across chunks and parallel within each chunk"
// (section 1.2).  For a chunk of C = 64 tokens starting from state S0, with
// g_r = sum_{s<=r} log alpha_s (per key channel) and Gamma_r = exp(g_r):
//
//   M_rs = sum_c k_rc k_sc e^{g_rc - g_sc}   (s < r)     decayed key Gram
//   P_rs = sum_c q_rc k_sc e^{g_rc - g_sc}   (s <= r)    decayed query-key Gram
//   W    = (I + Diag(b) M)^{-1} Diag(b) (V - K_Gamma S0) pseudo-values, K_Gamma = K * Gamma
//   O    = Q_Gamma S0 + P W                              chunk output, Q_Gamma = Q * Gamma
//   S    = Diag(Gamma_C) S0 + (K * Gamma_C / Gamma)^T W  next chunk's state
//
// which follows from unrolling the recurrence inside the chunk: the delta
// correction of token r sees the decayed state and the corrections of the
// chunk's earlier tokens, which gives the unit-lower-triangular system.  The
// system is solved by blocks of 16 tokens: with A_ii = (I + Diag(b_i) M_ii)^{-1}
// Diag(b_i) for the four diagonal blocks,
//   W_i = A_ii (U_i - sum_{j<i} M_ij W_j),   U = V - K_Gamma S0.
//
// Range control (section 1.2 of the notes): every factor e^{g_r - g_s} with
// s <= r is at most 1, but splitting it into a row part and a column part for a
// matrix product needs a reference point.  The chunk is cut into four 16-token
// tiles; tile i has reference rho_i = g just before the tile.  Because
// log alpha >= -5, a tile's cumulative log-decay lies in [-80, 0], so
//   row factor    e^{g_r - rho_i}        in [e^-80, 1]
//   column factor e^{rho_i - g_s}        in [1, e^80]   (s in the same tile)
//                                        in [0, 1]      (s in an earlier tile)
// all representable in fp32 and bf16 (8-bit exponent).  Every tile pair,
// diagonal or not, is then a dense MFMA product.  Decay arithmetic runs in
// base 2 (log alpha * log2 e) so that v_exp_f32 is used directly; within a
// tile the factors are running products of alpha (one exponential per
// element), across tiles they come from sums of log alpha.
//
// Work decomposition: one workgroup of NW waves per (sequence, head, V-block
// of BV = 16 NW value columns); the recurrence is independent across value
// columns.  Per chunk:
//   E  elementwise: per-tile decay factors and scaled operands, written to LDS
//      row-major with the contraction index contiguous.  Thread = (tile,
//      channels), so the running products are sequential in registers;
//   G  the P and M tile products (MFMA, row fragments reused across columns);
//   S  the four diagonal 16x16 inverses, fp32 right-looking substitution;
//   SD the state-dependent part, wave-local: wave w owns value columns
//      16w .. 16w+15.  Its slab of S, and U and W, live in MFMA accumulators
//      and are fed back directly as MFMA operands (an accumulator tile holds 4
//      consecutive rows per lane, exactly the K-layout of an operand); the
//      LDS operands are read with the matching row permutation.  No LDS writes
//      and no barriers inside SD.
// The global loads of chunk c+1 are issued while chunk c is being processed.
//
// Operand precision: bf16 inputs use bf16 MFMA operands with fp32
// accumulation (v_mfma_f32_16x16x32_bf16 / 16x16x16_bf16); fp32 inputs use
// v_mfma_f32_16x16x4_f32.  The state, the decay arithmetic and the diagonal
// inverses are fp32 throughout.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kC = 64;        // chunk length
constexpr int kTiles = 4;     // 16-token tiles per chunk

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// MFMA helpers.  Accumulator layout (CDNA 16x16): lane l, register e holds
// D[4*(l/16) + e][l % 16].  Below, "acc tile" X is such a 16x16 fp32 tile and
// "row of an LDS operand" is a pointer to the 16-wide K segment of the row
// that this lane's M (or N) index selects.  Every product pairs, for lane
// group g = l/16 and slot e, row 4g+e of the accumulator tile with column
// 4g+e of the LDS row, so the contraction is complete whatever order the
// hardware assigns to K.
// ---------------------------------------------------------------------------
template <typename OT> struct Op;

template <> struct Op<uint16_t> {    // bf16 operands
    static constexpr int KS = 32;    // K of the LDS x LDS product
    typedef bf16x8 Frag;
    static __device__ __forceinline__ Frag frag(const uint16_t* base, int ld, int k0) {
        const int lane = threadIdx.x & 63;
        return *reinterpret_cast<const bf16x8*>(base + (lane & 15) * ld + 8 * (lane >> 4) + k0);
    }
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    static __device__ __forceinline__ u32x2 cvt(f32x4 x) {
        return u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    }
    static __device__ __forceinline__ u32x2 ld4(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }
    // K = 16: D += A(lds row, 16 cols) * X (acc tile as B, K = its rows)
    static __device__ __forceinline__ f32x4 lds_acc16(const uint16_t* arow, u32x2 xb, f32x4 acc) {
        const int g = (threadIdx.x & 63) >> 4;
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, ld4(arow + 4 * g)),
                                                         __builtin_bit_cast(s16x4, xb), acc, 0, 0, 0);
    }
    // K = 16: D += X^T (acc tile as A, K = its rows) * B(lds row, 16 cols)
    static __device__ __forceinline__ f32x4 acc_lds16(u32x2 xa, const uint16_t* brow, f32x4 acc) {
        const int g = (threadIdx.x & 63) >> 4;
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, xa),
                                                         __builtin_bit_cast(s16x4, ld4(brow + 4 * g)), acc, 0, 0, 0);
    }
    // K = 32 from two 16-row groups (t1, t2) of the LDS row and two acc tiles.
    static __device__ __forceinline__ f32x4 lds_acc32(const uint16_t* arow1, const uint16_t* arow2, u32x2 x1, u32x2 x2,
                                                      f32x4 acc) {
        const int g = (threadIdx.x & 63) >> 4;
        const u32x2 a1 = ld4(arow1 + 4 * g), a2 = ld4(arow2 + 4 * g);
        const u32x4 a = {a1[0], a1[1], a2[0], a2[1]}, b = {x1[0], x1[1], x2[0], x2[1]};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       acc, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 acc_lds32(u32x2 x1, u32x2 x2, const uint16_t* brow1, const uint16_t* brow2,
                                                      f32x4 acc) {
        const int g = (threadIdx.x & 63) >> 4;
        const u32x2 b1 = ld4(brow1 + 4 * g), b2 = ld4(brow2 + 4 * g);
        const u32x4 a = {x1[0], x1[1], x2[0], x2[1]}, b = {b1[0], b1[1], b2[0], b2[1]};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       acc, 0, 0, 0);
    }
    static __device__ __forceinline__ void put(uint16_t* p, float x) { *p = f32_to_bf16(x); }
    static __device__ __forceinline__ void put2(uint16_t* p, float x0, float x1) {
        *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(x0, x1);
    }
    static __device__ __forceinline__ void put4(uint16_t* p, f32x4 x) { *reinterpret_cast<u32x2*>(p) = cvt(x); }
    static __device__ __forceinline__ float get(const uint16_t* p) { return bf16_to_f32(*p); }
};

template <> struct Op<float> {       // fp32 operands
    static constexpr int KS = 4;
    typedef float Frag;
    static __device__ __forceinline__ Frag frag(const float* base, int ld, int k0) {
        const int lane = threadIdx.x & 63;
        return base[(lane & 15) * ld + (lane >> 4) + k0];
    }
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 cvt(f32x4 x) { return x; }
    static __device__ __forceinline__ f32x4 lds_acc16(const float* arow, f32x4 xb, f32x4 acc) {
        const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(arow[4 * g + e], xb[e], acc, 0, 0, 0);
        return acc;
    }
    static __device__ __forceinline__ f32x4 acc_lds16(f32x4 xa, const float* brow, f32x4 acc) {
        const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[e], brow[4 * g + e], acc, 0, 0, 0);
        return acc;
    }
    static __device__ __forceinline__ f32x4 lds_acc32(const float* arow1, const float* arow2, f32x4 x1, f32x4 x2,
                                                      f32x4 acc) {
        return lds_acc16(arow2, x2, lds_acc16(arow1, x1, acc));
    }
    static __device__ __forceinline__ f32x4 acc_lds32(f32x4 x1, f32x4 x2, const float* brow1, const float* brow2,
                                                      f32x4 acc) {
        return acc_lds16(x2, brow2, acc_lds16(x1, brow1, acc));
    }
    static __device__ __forceinline__ void put(float* p, float x) { *p = x; }
    static __device__ __forceinline__ void put2(float* p, float x0, float x1) {
        *reinterpret_cast<f32x2*>(p) = f32x2{x0, x1};
    }
    static __device__ __forceinline__ void put4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
    static __device__ __forceinline__ float get(const float* p) { return *p; }
};

// Index of tile-pair block (i, j), j <= i, among the 10 lower blocks.
__device__ __forceinline__ constexpr int blk(int i, int j) { return i * (i + 1) / 2 + j; }

// ---------------------------------------------------------------------------
// Raw input words.  q/k words hold CPT packed elements (a bf16 pair, or one
// bf16 / fp32 element).
// ---------------------------------------------------------------------------
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

// ---------------------------------------------------------------------------
// LDS plan (all buffers live for the whole chunk).
// ---------------------------------------------------------------------------
template <typename OT, int DK>
struct Plan {
    static constexpr int ES = sizeof(OT);
    static constexpr int PAD = (ES == 2) ? 8 : 2;   // row padding (elements)
    static constexpr int LDK = DK + PAD;            // stride of [*, DK] buffers
    static constexpr int LDC = kC + PAD;            // stride of [*, C] buffers
    static constexpr int QE1 = 0;                                  // [C][LDK]  q * e^{g - rho_i}
    static constexpr int KE1 = QE1 + kC * LDK * ES;                // [C][LDK]  k * e^{g - rho_i}
    static constexpr int KCOL = KE1 + kC * LDK * ES;               // 10 x [16][LDK] column operands
    static constexpr int QG = KCOL + 10 * 16 * LDK * ES;           // [C][LDK]  q * e^{g}
    static constexpr int KG = QG + kC * LDK * ES;                  // [C][LDK]  k * e^{g}
    static constexpr int KDT = KG + kC * LDK * ES;                 // [DK][LDC] (k * e^{g_C - g})^T
    static constexpr int PB = KDT + DK * LDC * ES;                 // [C][LDC]  P (lower incl. diagonal)
    static constexpr int MB = PB + kC * LDC * ES;                  // [C][LDC]  M below the diagonal blocks,
                                                                   //           A_ii in the diagonal blocks
    static constexpr int BETA = MB + kC * LDC * ES;                // [C] fp32
    static constexpr int SX = BETA + kC * 4;                       // [4][DK] fp32 tile log2-decay totals
    static constexpr int DECAY = SX + kTiles * DK * 4;             // [DK] fp32 e^{g_C}
    static constexpr int TOTAL = DECAY + DK * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS plan exceeds 160 KB");
};

// Gram work list: wave w computes the tile pairs (i, j0 .. j0 + cnt - 1) of row tile i,
// then (i2, j2 .. ) when it has a second row.  Pairs (i, j), j <= i, 10 in total.
template <int NW> struct GramSched;
template <> struct GramSched<4> {   // w0: (0,0) (1,0) (1,1)  w1: (2,0..2)  w2: (3,0) (3,1)  w3: (3,2) (3,3)
    static __device__ __forceinline__ void pair(int w, int p, int& i, int& j, int& cnt) {
        cnt = w < 2 ? 3 : 2;
        if (w == 0) { i = p == 0 ? 0 : 1; j = p == 0 ? 0 : p - 1; }
        else if (w == 1) { i = 2; j = p; }
        else { i = 3; j = (w == 2 ? 0 : 2) + p; }
    }
};
template <> struct GramSched<8> {   // w0: (0,0)  w1: (1,0) (1,1)  w2: (2,0)  w3: (2,1) (2,2)  w4..w7: (3,0) .. (3,3)
    static __device__ __forceinline__ void pair(int w, int p, int& i, int& j, int& cnt) {
        cnt = (w == 1 || w == 3) ? 2 : 1;
        if (w == 0) { i = 0; j = 0; }
        else if (w == 1) { i = 1; j = p; }
        else if (w == 2) { i = 2; j = 0; }
        else if (w == 3) { i = 2; j = 1 + p; }
        else { i = 3; j = w - 4; }
    }
};

template <typename T, int DK, int DV, int NW>
__global__ __launch_bounds__(64 * NW, 1) void prefill_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const float* __restrict__ init_state, const int32_t* __restrict__ cu_seqlens,
    int64_t total_T, int H, T* __restrict__ o, float* __restrict__ final_state) {
    using OT = T;
    using OP = Op<OT>;
    using PL = Plan<OT, DK>;
    constexpr int KS = OP::KS;
    constexpr int WPT = NW / kTiles;      // phase E: waves per 16-token tile
    constexpr int CPT = DK / (64 * WPT);  // phase E: channels per thread
    constexpr int NCT = DK / 16;          // 16-row channel tiles of the state
    constexpr int NKS = DK / KS;          // K-steps of the Gram products
    constexpr int BV = 16 * NW;           // value columns per workgroup
    static_assert(CPT == 1 || CPT == 2, "phase E mapping");
    static_assert(DV % BV == 0, "value blocking");

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    OT* sQE1 = reinterpret_cast<OT*>(smem + PL::QE1);
    OT* sKE1 = reinterpret_cast<OT*>(smem + PL::KE1);
    OT* sKCOL = reinterpret_cast<OT*>(smem + PL::KCOL);
    OT* sQG = reinterpret_cast<OT*>(smem + PL::QG);
    OT* sKG = reinterpret_cast<OT*>(smem + PL::KG);
    OT* sKDT = reinterpret_cast<OT*>(smem + PL::KDT);
    OT* sP = reinterpret_cast<OT*>(smem + PL::PB);
    OT* sM = reinterpret_cast<OT*>(smem + PL::MB);
    float* sBeta = reinterpret_cast<float*>(smem + PL::BETA);
    float* sX = reinterpret_cast<float*>(smem + PL::SX);
    float* sDecay = reinterpret_cast<float*>(smem + PL::DECAY);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int h = blockIdx.y;
    const int n = blockIdx.z;
    const int vcol = blockIdx.x * BV + 16 * wave;    // this wave's first value column
    const int ti = wave / WPT;                        // phase E: tile
    const int cb = (wave % WPT) * (64 * CPT) + lane * CPT;   // phase E: first channel

    // Sequence range, clamped so malformed offsets cannot address out of range.
    int64_t seq0 = 0, seq1 = total_T;
    if (cu_seqlens != nullptr) {
        seq0 = cu_seqlens[n];
        seq1 = cu_seqlens[n + 1];
        seq0 = seq0 < 0 ? 0 : (seq0 > total_T ? total_T : seq0);
        seq1 = seq1 < seq0 ? seq0 : (seq1 > total_T ? total_T : seq1);
    }
    const int64_t len = seq1 - seq0;

    // This wave's state slab: Sacc[ct][e] = S[16 ct + 4 lg + e][vcol + l16].
    f32x4 Sacc[NCT];
    const int64_t sbase = ((int64_t)n * H + h) * DK * DV;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            Sacc[ct][e] = init_state ? init_state[sbase + (int64_t)(16 * ct + 4 * lg + e) * DV + vcol + l16] : 0.f;

    // Raw-input prefetch registers.  Positions past the chunk's end are
    // clamped to its last token (always a valid address) and zeroed when used.
    float la_r[16][CPT];
    uint32_t qw_r[16], kw_r[16];
    float beta_r;
    uint32_t v_r[kTiles][4];   // v[16 i + 4 lg + e][vcol + l16]
    auto load_e = [&](int64_t c0n) {
        const int Ln = (int)((len - c0n) < kC ? (len - c0n) : kC);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int pos = 16 * ti + r < Ln ? 16 * ti + r : Ln - 1;
            const int64_t row = (seq0 + c0n + pos) * H + h;
            if constexpr (CPT == 2) {
                const f32x2 la2 = *reinterpret_cast<const f32x2*>(log_alpha + row * DK + cb);
                la_r[r][0] = la2[0];
                la_r[r][CPT - 1] = la2[1];
            } else {
                la_r[r][0] = log_alpha[row * DK + cb];
            }
            qw_r[r] = load_word<T, CPT>(q + row * DK + cb);
            kw_r[r] = load_word<T, CPT>(k + row * DK + cb);
        }
        const int bp = tid < Ln ? tid : Ln - 1;
        beta_r = tid < kC ? beta[(seq0 + c0n + bp) * H + h] : 0.f;
    };
    auto load_v = [&](int64_t c0n) {
        const int Ln = (int)((len - c0n) < kC ? (len - c0n) : kC);
#pragma unroll
        for (int i = 0; i < kTiles; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int p = 16 * i + 4 * lg + e;
                const int pos = p < Ln ? p : Ln - 1;
                v_r[i][e] = load_word<T, 1>(v + ((seq0 + c0n + pos) * H + h) * DV + vcol + l16);
            }
    };
    if (len > 0) {
        load_e(0);
        load_v(0);
    }

    for (int64_t c0 = 0; c0 < len; c0 += kC) {
        const int L = (int)((len - c0) < kC ? (len - c0) : kC);
        const int64_t tok0 = seq0 + c0;
        const bool has_next = c0 + kC < len;

        // ---------------- phase E: decay factors and scaled operands ----------------
        {
            float al[16][CPT], xs[CPT];
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) xs[cc] = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const bool ok = 16 * ti + r < L;
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) {
                    const float l2 = ok ? la_r[r][cc] * kLog2e : 0.f;
                    xs[cc] += l2;
                    al[r][cc] = fexp2(l2);
                }
            }
            if (tid < kC) sBeta[tid] = tid < L ? beta_r : 0.f;
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) sX[ti * DK + cb + cc] = xs[cc];
            // e1[r] = prod_{s<=r} alpha_s (relative to the tile start),
            // e2[r] = prod_{s>r} alpha_s  (remaining decay to the tile end).
            float e1[16][CPT], e2[16][CPT];
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) {
                float p = 1.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) { p *= al[r][cc]; e1[r][cc] = p; }
                p = 1.f;
#pragma unroll
                for (int r = 15; r >= 0; --r) { e2[r][cc] = p; p *= al[r][cc]; }
            }
            __syncthreads();

            // Per-channel factors from the tiles' log2-decay totals.
            float fG[CPT], fD[CPT], F[kTiles][CPT];
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) {
                float rho[kTiles + 1];
                rho[0] = 0.f;
#pragma unroll
                for (int j = 0; j < kTiles; ++j) rho[j + 1] = rho[j] + sX[j * DK + cb + cc];
                if (ti == 0) sDecay[cb + cc] = fexp2(rho[kTiles]);
                fG[cc] = fexp2(rho[ti]);                               // e^{rho_i}
                fD[cc] = fexp2(rho[kTiles] - rho[ti + 1]);             // e^{g_C - rho_{i+1}}
#pragma unroll
                for (int ip = 0; ip < kTiles; ++ip)                    // column factor for row tile ip
                    F[ip][cc] = (ip == ti) ? fexp2(-xs[cc]) : (ip > ti + 1 ? fexp2(rho[ip] - rho[ti + 1]) : 1.f);
            }
            float kd[CPT][16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int pos = 16 * ti + r;
                const bool ok = pos < L;
                float qe1[CPT], ke1[CPT], ke2[CPT];
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) {
                    const float qv = ok ? word_elem<T>(qw_r[r], cc) : 0.f;
                    const float kv = ok ? word_elem<T>(kw_r[r], cc) : 0.f;
                    qe1[cc] = qv * e1[r][cc];
                    ke1[cc] = kv * e1[r][cc];
                    ke2[cc] = kv * e2[r][cc];
                    kd[cc][r] = ke2[cc] * fD[cc];
                }
                const int o_row = pos * PL::LDK + cb;
                if constexpr (CPT == 2) {
                    OP::put2(sQE1 + o_row, qe1[0], qe1[CPT - 1]);
                    OP::put2(sKE1 + o_row, ke1[0], ke1[CPT - 1]);
                    OP::put2(sQG + o_row, qe1[0] * fG[0], qe1[CPT - 1] * fG[CPT - 1]);
                    OP::put2(sKG + o_row, ke1[0] * fG[0], ke1[CPT - 1] * fG[CPT - 1]);
#pragma unroll
                    for (int ip = 0; ip < kTiles; ++ip)
                        if (ip >= ti)
                            OP::put2(sKCOL + (blk(ip, ti) * 16 + r) * PL::LDK + cb, ke2[0] * F[ip][0],
                                     ke2[CPT - 1] * F[ip][CPT - 1]);
                } else {
                    OP::put(sQE1 + o_row, qe1[0]);
                    OP::put(sKE1 + o_row, ke1[0]);
                    OP::put(sQG + o_row, qe1[0] * fG[0]);
                    OP::put(sKG + o_row, ke1[0] * fG[0]);
#pragma unroll
                    for (int ip = 0; ip < kTiles; ++ip)
                        if (ip >= ti) OP::put(sKCOL + (blk(ip, ti) * 16 + r) * PL::LDK + cb, ke2[0] * F[ip][0]);
                }
            }
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc)
#pragma unroll
                for (int r = 0; r < 16; r += 4) {
                    f32x4 w4 = {kd[cc][r], kd[cc][r + 1], kd[cc][r + 2], kd[cc][r + 3]};
                    OP::put4(sKDT + (cb + cc) * PL::LDC + 16 * ti + r, w4);
                }
        }
        if (has_next) load_e(c0 + kC);      // prefetch: in flight during phases G..SD
        __syncthreads();

        // ---------------- phase G: P and M tile products ----------------
        // Both computed transposed (D[s][r] = sum_c Kcol[s][c] X[r][c]) so that
        // each lane holds 4 consecutive columns s of one row r, stored row-major.
        {
            int ci, cj, cnt;
            GramSched<NW>::pair(wave, 0, ci, cj, cnt);
            typename OP::Frag fq[NKS], fk[NKS];
            int loaded_i = -1;
            for (int p = 0; p < cnt; ++p) {
                GramSched<NW>::pair(wave, p, ci, cj, cnt);
                if (ci != loaded_i) {
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        fq[ks] = OP::frag(sQE1 + 16 * ci * PL::LDK, PL::LDK, ks * KS);
                        fk[ks] = OP::frag(sKE1 + 16 * ci * PL::LDK, PL::LDK, ks * KS);
                    }
                    loaded_i = ci;
                }
                const OT* colb = sKCOL + blk(ci, cj) * 16 * PL::LDK;
                f32x4 accP = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const typename OP::Frag fc = OP::frag(colb, PL::LDK, ks * KS);
                    accP = OP::mma(fc, fq[ks], accP);
                    accM = OP::mma(fc, fk[ks], accM);
                }
                // row r = l16 of tile ci, columns s = 4 lg + e of tile cj
                f32x4 vp, vm;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vp[e] = (ci > cj || 4 * lg + e <= l16) ? accP[e] : 0.f;
                    vm[e] = (ci > cj || 4 * lg + e < l16) ? accM[e] : 0.f;
                }
                OP::put4(sP + (16 * ci + l16) * PL::LDC + 16 * cj + 4 * lg, vp);
                OP::put4(sM + (16 * ci + l16) * PL::LDC + 16 * cj + 4 * lg, vm);
            }
        }
        __syncthreads();

        // ---------------- phase S: diagonal blocks A_ii = (I + Diag(b_i) M_ii)^{-1} Diag(b_i) ----------------
        // Wave i < 4 inverts block i, lane j < 16 owns column j of T_ii:
        //   t_r = [r == j] - b_r sum_{s<r} M_rs t_s   (right-looking), A_ii[r][j] = t_r b_j.
        if (wave < kTiles && lane < 16) {
            const int base = 16 * wave;
            const int j = lane;
            float acc[16], t[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                t[s] = (s == j ? 1.f : 0.f) - sBeta[base + s] * acc[s];
#pragma unroll
                for (int r = s + 1; r < 16; ++r) acc[r] += OP::get(sM + (base + r) * PL::LDC + base + s) * t[s];
            }
            const float bj = sBeta[base + j];
#pragma unroll
            for (int r = 0; r < 16; ++r) OP::put(sM + (base + r) * PL::LDC + base + j, t[r] * bj);
        }
        __syncthreads();

        // ---------------- phase SD: state-dependent part, wave-local ----------------
        {
            typedef decltype(OP::cvt(Sacc[0])) Xop;
            Xop Sop[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) Sop[ct] = OP::cvt(Sacc[ct]);

            // U_i = V_i - K_Gamma,i S0;  W_i = A_ii (U_i - sum_{j<i} M_ij W_j).
            // Tiles hold D[r][v]: lane (v = l16, r = 16 i + 4 lg + e).
            Xop Wop[kTiles];
#pragma unroll
            for (int i = 0; i < kTiles; ++i) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const OT* kgrow = sKG + (16 * i + l16) * PL::LDK;
#pragma unroll
                for (int ct = 0; ct < NCT; ct += 2)
                    acc = OP::lds_acc32(kgrow + 16 * ct, kgrow + 16 * (ct + 1), Sop[ct], Sop[ct + 1], acc);
                const OT* mrow = sM + (16 * i + l16) * PL::LDC;
#pragma unroll
                for (int j = 0; j < i; ++j) acc = OP::lds_acc16(mrow + 16 * j, Wop[j], acc);
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float vv = (16 * i + 4 * lg + e < L) ? word_elem<T>(v_r[i][e], 0) : 0.f;
                    y[e] = vv - acc[e];
                }
                f32x4 w = {0.f, 0.f, 0.f, 0.f};
                w = OP::lds_acc16(mrow + 16 * i, OP::cvt(y), w);
                Wop[i] = OP::cvt(w);
            }
            if (has_next) load_v(c0 + kC);

            // O_i^T = S0^T Q_Gamma,i^T + sum_{j<=i} W_j^T P_ij^T: lane (r = l16, v = 4 lg + e).
#pragma unroll
            for (int i = 0; i < kTiles; ++i) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const OT* qgrow = sQG + (16 * i + l16) * PL::LDK;
#pragma unroll
                for (int ct = 0; ct < NCT; ct += 2)
                    acc = OP::acc_lds32(Sop[ct], Sop[ct + 1], qgrow + 16 * ct, qgrow + 16 * (ct + 1), acc);
                const OT* prow = sP + (16 * i + l16) * PL::LDC;
#pragma unroll
                for (int j = 0; j <= i; ++j) acc = OP::acc_lds16(Wop[j], prow + 16 * j, acc);
                const int pos = 16 * i + l16;
                if (pos < L) {
                    T* dst = o + ((tok0 + pos) * H + h) * DV + vcol + 4 * lg;
                    if constexpr (sizeof(T) == 2) *reinterpret_cast<u32x2*>(dst) = OP::cvt(acc);
                    else *reinterpret_cast<f32x4*>(dst) = acc;
                }
            }

            // S <- Diag(Gamma_C) S0 + Kd^T W: lane (v = l16, c = 16 ct + 4 lg + e).
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 acc;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = Sacc[ct][e] * sDecay[16 * ct + 4 * lg + e];
                const OT* kdrow = sKDT + (16 * ct + l16) * PL::LDC;
                acc = OP::lds_acc32(kdrow, kdrow + 16, Wop[0], Wop[1], acc);
                acc = OP::lds_acc32(kdrow + 32, kdrow + 48, Wop[2], Wop[3], acc);
                Sacc[ct] = acc;
            }
        }
        __syncthreads();
    }

    if (final_state != nullptr) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                final_state[sbase + (int64_t)(16 * ct + 4 * lg + e) * DV + vcol + l16] = Sacc[ct][e];
    }
}

template <typename T, int DK, int DV, int NW>
hipError_t launch_t(const PrefillArgs& a) {
    using PL = Plan<T, DK>;
    auto kern = prefill_kernel<T, DK, DV, NW>;
    static bool attr_set = false;   // per instantiation; the attribute is a property of the function
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, PL::TOTAL);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    dim3 grid(DV / (16 * NW), a.H, a.N);
    hipLaunchKernelGGL(kern, grid, dim3(64 * NW), PL::TOTAL, a.stream,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, a.log_alpha, a.beta, a.init_state,
                       a.cu_seqlens, a.total_T, a.H, (T*)a.o, a.final_state);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a) {
    if (a.bf16) {
        if (a.d_k == 128) return a.d_v == 128 ? launch_t<uint16_t, 128, 128, 4>(a) : launch_t<uint16_t, 128, 64, 4>(a);
        return a.d_v == 128 ? launch_t<uint16_t, 64, 128, 4>(a) : launch_t<uint16_t, 64, 64, 4>(a);
    }
    // fp32 operands: d_k = 64 only (the LDS plan of d_k = 128 would exceed 160 KB).
    return a.d_v == 128 ? launch_t<float, 64, 128, 4>(a) : launch_t<float, 64, 64, 4>(a);
}

}  // namespace kda

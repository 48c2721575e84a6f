// KDA chunkwise prefill for gfx950 (CDNA4), bf16 operands: the state advances
// once per 64-token chunk.
//
// The recurrence of "Kimi K3 -- Architecture Notes", section 1.1,
//     S_t = (I - b_t k_t k_t^T) Diag(alpha_t) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t,
// is evaluated chunkwise as section 1.2 describes: the state passes serially
// from chunk to chunk, and the 64 tokens of a chunk are handled together.
// With g_r = sum_{s<=r} log alpha_s (per key channel, from the chunk start),
// G = g_64, and W the chunk's pseudo-values, one chunk from state S is
//
//   P_rs = sum_c q_rc k_sc e^{g_rc - g_sc}   (s <= r)     decayed query-key Gram
//   M_rs = sum_c k_rc k_sc e^{g_rc - g_sc}   (s <  r)     decayed key Gram
//   (I + Diag(b) M) W = Diag(b) (V - (K e^g) S)           unit-lower-triangular system
//   O = (Q e^g) S + P W
//   S <- Diag(e^G) S + (K e^{G-g})^T W
//
// which is the token recurrence regrouped exactly.
//
// Range control (section 1.2 of the notes): with log alpha >= -5 the decay
// over one 16-token tile ("secondary tile") stays within e^-80, which fp32 and
// bf16 represent.  So every Gram factor is taken relative to a tile boundary:
// for the block of row tile i and column tile j <= i, with rho_i the value of g
// before tile i,
//   P_ij = (Q e^{g - rho_i})_i (K e^{rho_i - g})_j^T,
// where the row factor lies in [e^-80, 1] and the column factor in [1, e^80]
// on the diagonal (j = i) and in [0, 1] below it; a column factor below the
// fp32 range then stands for a product that is at most that small.  The
// chunk-referenced operands Q e^g, K e^g and K e^{G-g} are the tile-relative
// ones scaled by per-channel products of tile decays, each <= 1.
//
// Work decomposition: one workgroup of eight waves per (sequence, head, block
// of 64 value columns); the recurrence is independent across value columns.
//   producer waves 0-3 (chunk c + 1): wave i takes tile i; lane = (token r of
//     the tile, 8 consecutive key channels per 32-channel step), which is the
//     operand layout of v_mfma_f32_16x16x32_bf16, so the Gram products of the
//     tile's own diagonal block run from registers.  Per element: the
//     log-decay is prefix-summed over the tile's 16 tokens with DPP row
//     shifts, then e^{g-rho} is one exponential and e^{rho-g} its reciprocal.  The
//     chunk operands and the off-diagonal column operands go to LDS.
//   state waves 4-7 (chunk c): wave w takes 16 value columns; its 128 x 16 (or
//     64 x 16) slab of S, the pseudo-values and the outputs live in MFMA
//     accumulators.  It forms the inverse of one tile's diagonal block
//     (fp32 substitution, on the M and beta the producers left), then
//     T = (K e^g) S and O = (Q e^g) S, solves the block-triangular system by
//     substitution over the four tiles on MFMA
//         W_i = A_i (V_i - T_i - sum_{j<i} M_ij W_j),  A_i = (I + Diag(b_i) M_ii)^{-1} Diag(b_i),
//     adds P W to O and stores it, and applies the state update once.
// Three workgroup barriers per chunk split both roles into matching windows:
//   window 1: producers form the decays (and publish the tile decays);
//             state waves invert, form T and O, decay S.
//   window 2: producers form the operands and the diagonal Gram blocks;
//             state waves solve, add P W, store O.
//   window 3: producers form the off-diagonal Gram blocks;
//             state waves update S.
// Each window only reads what an earlier window wrote, so there are no flags
// and no waits besides the barriers.  Two LDS buffers (chunk parity) hold what
// the producers hand to the state waves.
//
// Global loads run one chunk ahead of their consumer, through buffer
// descriptors whose range ends after the chunk's last valid token: rows past a
// sequence's end read as zero (decay 1, key, query, value and beta 0), and
// output rows past it are not written.
//
// Every accumulator chain uses one MFMA shape (a 16x16x16 bf16 MFMA that
// accumulates directly onto a 16x16x32 result was seen to read stale
// accumulator registers on gfx950).

#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kC = 64;        // chunk length
constexpr int kTiles = 4;     // 16-token tiles per chunk
constexpr int kPW = 4;        // producer waves (one per tile)
constexpr int kSW = 4;        // state waves (16 value columns each)
constexpr int kNW = kPW + kSW;
constexpr int kBV = 16 * kSW; // value columns per workgroup

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x + (x of the lane N places lower in this 16-lane row, or 0 below the row's start)
template <int N>
__device__ __forceinline__ float row_shr_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, true));
}

// Value of lane K of this lane's 16-lane row (DPP row_newbcast; every lane has
// a source, so no old value is needed); folds into the consuming VALU op.
template <int K>
__device__ __forceinline__ float row_bcast_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + K, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_bcast_mov(float v, int k) {   // k is a constant after unrolling
    switch (k) {
        case 0: return row_bcast_mov<0>(v);   case 1: return row_bcast_mov<1>(v);
        case 2: return row_bcast_mov<2>(v);   case 3: return row_bcast_mov<3>(v);
        case 4: return row_bcast_mov<4>(v);   case 5: return row_bcast_mov<5>(v);
        case 6: return row_bcast_mov<6>(v);   case 7: return row_bcast_mov<7>(v);
        case 8: return row_bcast_mov<8>(v);   case 9: return row_bcast_mov<9>(v);
        case 10: return row_bcast_mov<10>(v); case 11: return row_bcast_mov<11>(v);
        case 12: return row_bcast_mov<12>(v); case 13: return row_bcast_mov<13>(v);
        case 14: return row_bcast_mov<14>(v); default: return row_bcast_mov<15>(v);
    }
}

__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
}
__device__ __forceinline__ u32x2 cvt4(f32x4 x) { return u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])}; }
__device__ __forceinline__ u32x4 join(u32x2 a, u32x2 b) { return u32x4{a[0], a[1], b[0], b[1]}; }

template <typename V>
__device__ __forceinline__ V lds_ld(const unsigned char* p) { return *reinterpret_cast<const V*>(p); }
template <typename V>
__device__ __forceinline__ void lds_st(unsigned char* p, V v) { *reinterpret_cast<V*>(p) = v; }

// Blocks of the chunk's 4 x 4 tile grid: (i, j) with j <= i, and j < i.
__host__ __device__ constexpr int tri(int i, int j) { return i * (i + 1) / 2 + j; }
__host__ __device__ constexpr int low(int i, int j) { return i * (i - 1) / 2 + j; }

// ---------------------------------------------------------------------------
// Channel order.  A producer lane (g = lane / 16, token r = lane % 16) holds
// slots j = 0 .. 8 KST - 1, slot j being key channel ch(g, j) = 32 (j / 8) +
// 8 g + j % 8: the 8 channels of K-step j / 8 that an MFMA operand lane of
// group g supplies.  The state waves keep their slab of S in that order too:
// accumulator tile ct, register e of lane (g, v) holds channel
// ch(g, 8 (ct / 2) + 4 (ct % 2) + e), so two accumulator tiles are one K-step
// of the products with the chunk operands.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int slot_channel(int g, int j) { return 32 * (j >> 3) + 8 * g + (j & 7); }
__device__ __forceinline__ int acc_slot(int ct, int e) { return 8 * (ct >> 1) + 4 * (ct & 1) + e; }

// ---------------------------------------------------------------------------
// LDS plan (bf16 operands).  "Fragment" tiles hold one 16-token operand tile
// in the order an MFMA operand reads it: [K-step][lane][16 bytes], so each
// lane reads 16 contiguous bytes.
// ---------------------------------------------------------------------------
template <int DK>
struct Plan {
    static constexpr int KST = DK / 32;                      // K-steps of 32 channels
    static constexpr int FRAG = KST * 64 * 16;               // one 16-token operand tile
    static constexpr int LDK2 = DK + 16;                     // bf16 row stride of K e^{G-g}
    static constexpr int MSTR = 20;                          // fp32 stride of M^T rows
    static constexpr int ASTR = 20;                          // bf16 stride of A rows
    // one buffer (chunk parity)
    static constexpr int K1C = 0;                            // [4] fragment tiles  K e^g
    static constexpr int QC = K1C + kTiles * FRAG;           // [4] fragment tiles  Q e^g
    static constexpr int K2C = QC + kTiles * FRAG;           // [64][LDK2] bf16     K e^{G-g}, row-major
    static constexpr int PF = K2C + kC * LDK2 * 2;           // [10][64] x 8 B   P blocks, lane (g, r): P[r][4g..4g+3]
    static constexpr int MF = PF + 10 * 64 * 8;              // [6][64] x 8 B    -M blocks below the diagonal
    static constexpr int MT = MF + 6 * 64 * 8;               // [4][16][MSTR] fp32  M^T of the diagonal blocks
    static constexpr int AD = MT + kTiles * 16 * MSTR * 4;   // [4][16][ASTR] bf16  A of each tile
    static constexpr int BS = AD + kTiles * 16 * ASTR * 2;   // [64] fp32  beta
    static constexpr int GM = BS + kC * 4;                   // [DK] fp32  chunk decay e^G
    static constexpr int BUF = (GM + DK * 4 + 15) / 16 * 16;
    // producer scratch
    static constexpr int RB = 2 * BUF;                       // [6] fragment tiles  off-diagonal column operands
    static constexpr int GT = RB + 6 * FRAG;                 // [4][DK] fp32  tile decays
    static constexpr int TOTAL = GT + kTiles * DK * 4;
    static_assert(K2C % 16 == 0 && PF % 16 == 0 && MT % 16 == 0 && AD % 16 == 0 && RB % 16 == 0, "alignment");
    static_assert(TOTAL <= 160 * 1024, "LDS plan exceeds 160 KB");
};

// GATED: `decay` holds the decay logits z (bf16) and `beta` the write-strength
// logits; the lower-bounded map of section 1.2 of the notes (Kimi K3 row of its
// table), g = -5 Sigmoid(e^{A_h} z), beta = Sigmoid(logit), is applied on the
// fly.  Otherwise `decay` holds log alpha (fp32) and `beta` beta.
template <int DK, int DV, bool GATED>
__global__ __launch_bounds__(64 * kNW, 1) void chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const void* __restrict__ decay, const float* __restrict__ beta, const float* __restrict__ a_log,
    int64_t total_T, int H, PrefillJob j0, PrefillJob j1) {
    using PL = Plan<DK>;
    using DT = typename std::conditional<GATED, uint16_t, float>::type;
    constexpr int KST = PL::KST;
    constexpr int NSL = 8 * KST;          // channels (slots) per producer lane
    constexpr int SPL = DK / 64;          // factor slots a lane computes for its row (1 or 2)
    constexpr int NCT = DK / 16;          // 16-channel accumulator tiles of the state slab
    constexpr int DW = 8 * (int)sizeof(DT) / 4;   // 32-bit words of 8 decay inputs
    constexpr int NV = DV / kBV;          // value-column workgroups per (sequence, head)
    static_assert(NV == 1 || NV == 2, "value blocking");
    const DT* log_alpha = reinterpret_cast<const DT*>(decay);

    const bool second = (int)blockIdx.x >= j0.blocks;
    const PrefillJob& J = second ? j1 : j0;
    const uint16_t* __restrict__ v = reinterpret_cast<const uint16_t*>(J.v);
    const float* __restrict__ init_state = J.init_state;
    const int32_t* __restrict__ cu_seqlens = J.cu_seqlens;
    uint16_t* __restrict__ o = reinterpret_cast<uint16_t*>(J.o);
    float* __restrict__ final_state = J.final_state;

    // Workgroup -> (unit = sequence * H + head, value block).  With two value
    // blocks, the pair of a unit sits 8 workgroups apart (same XCD), so its
    // second reads of q, k and the decay hit that XCD's L2.  In the jobs of a
    // time split a "sequence" is one segment.
    const int lid = (int)blockIdx.x - (second ? j0.blocks : 0);
    int unit, vblk;
    if constexpr (NV == 2) {
        unit = 8 * (lid >> 4) + (lid & 7);
        vblk = (lid >> 3) & 1;
    } else {
        unit = lid;
        vblk = 0;
    }
    if (unit >= J.units) return;
    const int n = unit / H;
    const int h = unit - n * H;
    const float eA = GATED ? __expf(a_log[h]) : 1.f;    // e^{A_h}, the per-head logit scale

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 4;         // lane group
    const int r = lane & 15;         // producers: token of the tile; state waves: value column

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
    auto chunk_len = [&](int64_t c) { return (int)((len - c * kC) < kC ? (len - c * kC) : kC); };
    // Rows of the [tokens, H] layout from a head's first valid row to the end of
    // its last valid row; beyond the last chunk the range is empty, so loads can
    // be issued unconditionally (they return zero and touch no memory).
    auto valid_rows = [&](int64_t c) {
        return c < nchunks ? (uint32_t)(chunk_len(c) - 1) * (uint32_t)H + 1u : 0u;
    };
    auto row_of = [&](int64_t c) { return (seq0 + (c < nchunks ? c : 0) * kC) * H + h; };

    unsigned char* const scratch = smem + PL::RB;
    float* const sGT = reinterpret_cast<float*>(smem + PL::GT);

    if (wave < kPW) {
        // ===================== producers: wave ti = tile ti ==================
        const int ti = wave;
        const uint32_t tok = 16 * ti + r;                       // token of this lane within the chunk
        const uint32_t rs = (uint32_t)H * DK;                    // elements between consecutive tokens
        uint32_t la_w[KST][DW], qw[KST][4], kw[KST][4];
        float beta_r = 0.f;
        auto load_decay = [&](int64_t c) {
            const Rsrc rr = make_rsrc(log_alpha + row_of(c) * DK, valid_rows(c) * (DK * (uint32_t)sizeof(DT)));
#pragma unroll
            for (int kk = 0; kk < KST; ++kk) {
                const uint32_t el = tok * rs + 32 * kk + 8 * g;
#pragma unroll
                for (int u = 0; u < DW / 4; ++u) {
                    const u32x4 a = buf_ld128(rr, el * (uint32_t)sizeof(DT) + 16 * u);
#pragma unroll
                    for (int e = 0; e < 4; ++e) la_w[kk][4 * u + e] = a[e];
                }
            }
        };
        auto load_qk = [&](int64_t c) {
            const uint32_t nb = valid_rows(c) * (DK * 2u);
            const Rsrc rq = make_rsrc(q + row_of(c) * DK, nb), rk = make_rsrc(k + row_of(c) * DK, nb);
#pragma unroll
            for (int kk = 0; kk < KST; ++kk) {
                const uint32_t off = (tok * rs + 32 * kk + 8 * g) * 2u;
                const u32x4 a = buf_ld128(rq, off), b = buf_ld128(rk, off);
#pragma unroll
                for (int e = 0; e < 4; ++e) { qw[kk][e] = a[e]; kw[kk][e] = b[e]; }
            }
            beta_r = __uint_as_float(buf_ld32(make_rsrc(beta + row_of(c), valid_rows(c) * 4), tok * (uint32_t)H * 4));
        };

        float e1[NSL];                   // 2^{x}: decay from the tile start
        u32x4 QL[KST], KL[KST];          // q e1, k e1 (bf16 row operands of the Gram products)

        // Decays of chunk c: the log-decay prefix-summed over the tile's 16
        // tokens (DPP row shifts), one exponential per element, and the tile's
        // decay per channel to LDS for the other producers.
        auto decays = [&](int64_t c) {
            float x[NSL];
#pragma unroll
            for (int kk = 0; kk < KST; ++kk)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    float lg;     // natural log of the decay
                    if constexpr (GATED) {
                        const uint32_t wd = la_w[kk][j >> 1];
                        const float z = (j & 1) ? bf16_hi(wd) : bf16_lo(wd);
                        lg = -5.f * __builtin_amdgcn_rcpf(1.f + fexp2(-kLog2e * eA * z));
                    } else {
                        lg = __uint_as_float(la_w[kk][j]);
                    }
                    x[8 * kk + j] = lg;
                }
            if constexpr (GATED) {
                // rows past a partial chunk read logits 0, which the map does not send to 0
                if ((int)tok >= chunk_len(c)) {
#pragma unroll
                    for (int s = 0; s < NSL; ++s) x[s] = 0.f;
                }
            }
#pragma unroll
            for (int s = 0; s < NSL; ++s) x[s] = row_shr_add<1>(x[s]);
#pragma unroll
            for (int s = 0; s < NSL; ++s) x[s] = row_shr_add<2>(x[s]);
#pragma unroll
            for (int s = 0; s < NSL; ++s) x[s] = row_shr_add<4>(x[s]);
#pragma unroll
            for (int s = 0; s < NSL; ++s) x[s] = row_shr_add<8>(x[s]);
#pragma unroll
            for (int s = 0; s < NSL; ++s) e1[s] = fexp2(x[s] * kLog2e);
            if (r == 15) {      // the tile's decay per channel
#pragma unroll
                for (int kk = 0; kk < KST; ++kk) {
                    unsigned char* p = reinterpret_cast<unsigned char*>(sGT + ti * DK + 32 * kk + 8 * g);
                    lds_st(p, f32x4{e1[8 * kk], e1[8 * kk + 1], e1[8 * kk + 2], e1[8 * kk + 3]});
                    lds_st(p + 16, f32x4{e1[8 * kk + 4], e1[8 * kk + 5], e1[8 * kk + 6], e1[8 * kk + 7]});
                }
            }
        };

        // Operands of chunk c into buffer c & 1, the column operands of the later
        // tiles' off-diagonal blocks into the scratch area, and the tile's
        // diagonal Gram block.  TI is this wave's tile (specialised, so each
        // wave forms only what its tile needs).
        auto operands = [&](int64_t c, auto tile) {
            constexpr int TI = decltype(tile)::value;
            unsigned char* buf = smem + (c & 1) * PL::BUF;
            // Per-channel products of tile decays for this lane's SPL slots of its
            // row (slot j's values sit in lane j / SPL of the row):
            //   D = prod_{m < TI} (from the chunk start to this tile), F = prod_{m >= TI}
            //   (from this tile's start to the chunk end), G2 = Gamma_TI Gamma_{TI+1},
            //   G3 = Gamma_TI Gamma_{TI+1} Gamma_{TI+2}.
            float fD[SPL], fF[SPL], fG2[SPL], fG3[SPL];
#pragma unroll
            for (int u = 0; u < SPL; ++u) {
                const int ch = slot_channel(g, SPL * r + u);
                float gt[kTiles];
#pragma unroll
                for (int m = 0; m < kTiles; ++m) gt[m] = sGT[m * DK + ch];
                float d = 1.f, f = 1.f;
#pragma unroll
                for (int m = 0; m < kTiles; ++m) {
                    if (m < TI) d *= gt[m];
                    else f *= gt[m];
                }
                fD[u] = d;
                fF[u] = f;
                fG2[u] = TI < 2 ? gt[TI] * gt[TI + 1] : 0.f;
                fG3[u] = TI < 1 ? gt[TI] * gt[TI + 1] * gt[TI + 2] : 0.f;
                if (TI == 0) reinterpret_cast<float*>(buf + PL::GM)[ch] = f;   // e^G of the chunk
            }
            auto bc = [&](const float (&fv)[SPL], int s) { return row_bcast_mov(fv[s % SPL], s / SPL); };
            u32x4 KB[KST];
#pragma unroll
            for (int kk = 0; kk < KST; ++kk) {
                uint32_t ql[4], kl[4], kb[4], qc[4], k1c[4], k2c[4], r1[4], r2[4], r3[4];
#pragma unroll
                for (int jp = 0; jp < 4; ++jp) {
                    float f_ql[2], f_kl[2], f_kb[2], f_qc[2], f_k1[2], f_k2[2], f_r1[2], f_r2[2], f_r3[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int s = 8 * kk + 2 * jp + hh;
                        const float qf = hh ? bf16_hi(qw[kk][jp]) : bf16_lo(qw[kk][jp]);
                        const float kf = hh ? bf16_hi(kw[kk][jp]) : bf16_lo(kw[kk][jp]);
                        const float e = e1[s];
                        f_ql[hh] = qf * e;
                        f_kl[hh] = kf * e;
                        f_kb[hh] = kf * __builtin_amdgcn_rcpf(e);             // k 2^{-x}
                        if constexpr (TI > 0) {
                            const float eD = e * bc(fD, s);                    // 2^{x} D: from the chunk start
                            f_qc[hh] = qf * eD;
                            f_k1[hh] = kf * eD;
                        }
                        if constexpr (TI < kTiles - 1) {
                            f_k2[hh] = f_kb[hh] * bc(fF, s);                   // K 2^{G - g}
                            f_r1[hh] = f_kb[hh] * row_bcast_mov<15>(e);       // column operand of (TI+1, TI)
                        } else {
                            f_k2[hh] = f_kb[hh] * row_bcast_mov<15>(e);       // F = Gamma_3
                        }
                        if constexpr (TI < kTiles - 2) f_r2[hh] = f_kb[hh] * bc(fG2, s);   // of (TI+2, TI)
                        if constexpr (TI < kTiles - 3) f_r3[hh] = f_kb[hh] * bc(fG3, s);   // of (TI+3, TI)
                    }
                    ql[jp] = pack_bf16x2(f_ql[0], f_ql[1]);
                    kl[jp] = pack_bf16x2(f_kl[0], f_kl[1]);
                    kb[jp] = pack_bf16x2(f_kb[0], f_kb[1]);
                    if constexpr (TI > 0) {
                        qc[jp] = pack_bf16x2(f_qc[0], f_qc[1]);
                        k1c[jp] = pack_bf16x2(f_k1[0], f_k1[1]);
                    } else {
                        qc[jp] = ql[jp];
                        k1c[jp] = kl[jp];
                    }
                    k2c[jp] = pack_bf16x2(f_k2[0], f_k2[1]);
                    if constexpr (TI < kTiles - 1) r1[jp] = pack_bf16x2(f_r1[0], f_r1[1]);
                    if constexpr (TI < kTiles - 2) r2[jp] = pack_bf16x2(f_r2[0], f_r2[1]);
                    if constexpr (TI < kTiles - 3) r3[jp] = pack_bf16x2(f_r3[0], f_r3[1]);
                }
                QL[kk] = u32x4{ql[0], ql[1], ql[2], ql[3]};
                KL[kk] = u32x4{kl[0], kl[1], kl[2], kl[3]};
                KB[kk] = u32x4{kb[0], kb[1], kb[2], kb[3]};
                const uint32_t fo = (uint32_t)((TI * KST + kk) * 64 + lane) * 16;
                lds_st(buf + PL::QC + fo, u32x4{qc[0], qc[1], qc[2], qc[3]});
                lds_st(buf + PL::K1C + fo, u32x4{k1c[0], k1c[1], k1c[2], k1c[3]});
                lds_st(buf + PL::K2C + (tok * PL::LDK2 + 32 * kk + 8 * g) * 2, u32x4{k2c[0], k2c[1], k2c[2], k2c[3]});
                const uint32_t ro = (uint32_t)(kk * 64 + lane) * 16;
                if constexpr (TI < kTiles - 1)
                    lds_st(scratch + low(TI + 1, TI) * PL::FRAG + ro, u32x4{r1[0], r1[1], r1[2], r1[3]});
                if constexpr (TI < kTiles - 2)
                    lds_st(scratch + low(TI + 2, TI) * PL::FRAG + ro, u32x4{r2[0], r2[1], r2[2], r2[3]});
                if constexpr (TI < kTiles - 3)
                    lds_st(scratch + low(TI + 3, TI) * PL::FRAG + ro, u32x4{r3[0], r3[1], r3[2], r3[3]});
            }
            // Diagonal block, transposed: D[s][r] = sum_c KB[s][c] X[r][c], so lane
            // (g, r) ends with P[r][4g + e] (and M), the layout the state waves read.
            f32x4 accP = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KST; ++kk) {
                accP = mfma32(KB[kk], QL[kk], accP);
                accM = mfma32(KB[kk], KL[kk], accM);
            }
            f32x4 pv;
            float* sMT = reinterpret_cast<float*>(buf + PL::MT) + TI * 16 * PL::MSTR;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 4 * g + e;
                pv[e] = s <= r ? accP[e] : 0.f;
                // M^T[s][r], columns in (r % 4, r / 4) order (the inverse's read order)
                sMT[s * PL::MSTR + 4 * (r & 3) + (r >> 2)] = s < r ? accM[e] : 0.f;
            }
            lds_st(buf + PL::PF + (tri(TI, TI) * 64 + lane) * 8, cvt4(pv));
            if (g == 0) {
                float b = beta_r;
                if constexpr (GATED)   // beta = Sigmoid(logit); 0 past the end of the sequence
                    b = (int)tok < chunk_len(c) ? __builtin_amdgcn_rcpf(1.f + fexp2(-kLog2e * beta_r)) : 0.f;
                reinterpret_cast<float*>(buf + PL::BS)[tok] = b;
            }
        };

        // Blocks (TI, j), j < TI, of chunk c from the column operands of the
        // earlier tiles (both factors <= 1).
        auto offdiag = [&](int64_t c, auto tile) {
            constexpr int TI = decltype(tile)::value;
            unsigned char* buf = smem + (c & 1) * PL::BUF;
#pragma unroll
            for (int j = 0; j < TI; ++j) {
                f32x4 accP = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KST; ++kk) {
                    const u32x4 rb = lds_ld<u32x4>(scratch + low(TI, j) * PL::FRAG + (kk * 64 + lane) * 16);
                    accP = mfma32(rb, QL[kk], accP);
                    accM = mfma32(rb, KL[kk], accM);
                }
                lds_st(buf + PL::PF + (tri(TI, j) * 64 + lane) * 8, cvt4(accP));
                lds_st(buf + PL::MF + (low(TI, j) * 64 + lane) * 8, cvt4(-accM));
            }
        };
        auto by_tile = [&](auto&& fn, int64_t c) {
            switch (ti) {
                case 0: fn(c, std::integral_constant<int, 0>{}); break;
                case 1: fn(c, std::integral_constant<int, 1>{}); break;
                case 2: fn(c, std::integral_constant<int, 2>{}); break;
                default: fn(c, std::integral_constant<int, 3>{}); break;
            }
        };

        // Two barriers per chunk.  Window 1 of iteration c: the off-diagonal
        // blocks of chunk c (their column operands were written in the window 2
        // before) and the decays of chunk c + 1.  Window 2: the operands of chunk
        // c + 1.  Chunk 0 is made before the loop (two more barriers).
        // Each prefetch is issued in straight-line code once its registers are
        // consumed, never inside a branch: the compiler's in-order memory-count
        // waits then wait for the data they need and not for later prefetches.
        load_decay(0);
        load_qk(0);
        if (nchunks > 0) {
            decays(0);
            load_decay(1);
            __syncthreads();
            by_tile(operands, 0);
            load_qk(1);
            __syncthreads();
            for (int64_t c = 0; c < nchunks; ++c) {
                const bool more = c + 1 < nchunks;
                by_tile(offdiag, c);
                if (more) decays(c + 1);
                load_decay(c + 2);
                __syncthreads();
                if (more) by_tile(operands, c + 1);
                load_qk(c + 2);
                __syncthreads();
            }
        }
    } else {
        // ===================== state waves: 16 value columns each ===============
        // They carry the serial chain of the recurrence: issue priority over the
        // producers on their SIMD.
        __builtin_amdgcn_s_setprio(2);
        const int sw = wave - kPW;
        const int vcol = vblk * kBV + 16 * sw;
        const int v_ = r;                      // this lane's value column (vcol + v_)
        // Slab: Sacc[ct][e] = S[ch(g, acc_slot(ct, e))][vcol + v_].
        f32x4 Sacc[NCT];
        const int64_t sbase = ((int64_t)n * H + h) * DK * DV;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ch = slot_channel(g, acc_slot(ct, e));
                Sacc[ct][e] = J.init_mode == kInitIdentity ? (ch == vcol + v_ ? 1.f : 0.f)
                              : (init_state != nullptr && (J.init_mode == kInitAll || n == 0))
                                  ? init_state[sbase + (int64_t)ch * DV + vcol + v_] : 0.f;
            }
        u32x4 Sop[KST];
        auto pack_state = [&]() {
#pragma unroll
            for (int kk = 0; kk < KST; ++kk) Sop[kk] = join(cvt4(Sacc[2 * kk]), cvt4(Sacc[2 * kk + 1]));
        };
        pack_state();

        // Values: v[16 i + 4 g + e][vcol + v_], raw bf16 words, one chunk ahead.
        uint32_t v_r[kTiles][4];
        auto load_v = [&](int64_t c) {
            const Rsrc rv = v != nullptr
                                ? make_rsrc(v + row_of(c) * DV + vcol, valid_rows(c) * (DV * 2u))
                                : make_rsrc(nullptr, 0u);
            const uint32_t rs = (uint32_t)H * DV;
#pragma unroll
            for (int i = 0; i < kTiles; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) v_r[i][e] = buf_ld16(rv, ((16 * i + 4 * g + e) * rs + v_) * 2u);
        };

        // Inverse of the diagonal block of tile ti:
        //   A = (I + Diag(b) M)^{-1} Diag(b)
        // by right-looking substitution on all 64 lanes: lane = (column j =
        // lane / 4, row residue q = lane % 4), rows r = 4 m + q of column j of
        // X = (I + Diag(b) M)^{-1}:  x_s = [s == j] - b_s sum_{s' < s} M_{s s'} x_{s'}.
        // At step s the lane owning row s forms x_s, a quad broadcast (DPP) hands
        // it to the other three lanes of its column, and every lane adds
        // M_{r s} x_s to its rows; one 16-byte read of M^T row s gives a lane its
        // four M_{r s}.
        auto inverse = [&](unsigned char* buf, int ti) {
            const int j = lane >> 2, qq = lane & 3;
            const float* MT = reinterpret_cast<const float*>(buf + PL::MT) + ti * 16 * PL::MSTR + 4 * qq;
            const float* BS = reinterpret_cast<const float*>(buf + PL::BS) + 16 * ti;
            float bt[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 b4 = *reinterpret_cast<const f32x4*>(BS + 4 * q4);
#pragma unroll
                for (int e = 0; e < 4; ++e) bt[4 * q4 + e] = b4[e];
            }
            f32x4 mr[16];
#pragma unroll
            for (int s2 = 0; s2 < 16; ++s2) mr[s2] = *reinterpret_cast<const f32x4*>(MT + s2 * PL::MSTR);
            float acc[4], xs[4], one[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) { acc[m] = 0.f; xs[m] = 0.f; one[m] = (4 * m + qq == j) ? 1.f : 0.f; }
#pragma unroll
            for (int s2 = 0; s2 < 16; ++s2) {
                const int ms = s2 >> 2, qs = s2 & 3;
                const float cand = fmaf(-bt[s2], acc[ms], one[ms]);   // x_s in the lanes with qq == s % 4
                if (qq == qs) xs[ms] = cand;
                const float xb = quad_bcast(cand, qs);
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (4 * m + 3 > s2) acc[m] = fmaf(mr[s2][m], xb, acc[m]);
            }
            const float bj = bt[j];
            uint16_t* AD = reinterpret_cast<uint16_t*>(buf + PL::AD) + ti * 16 * PL::ASTR;
#pragma unroll
            for (int m = 0; m < 4; ++m) AD[(4 * m + qq) * PL::ASTR + j] = f32_to_bf16(xs[m] * bj);
        };

        f32x4 T[kTiles], O[kTiles];
        // Window 1: the inverse of tile sw, T = (K e^g) S, O^T = S^T (Q e^g)^T,
        // and the decay of S by e^G.
        auto window1 = [&](int64_t c) {
            unsigned char* buf = smem + (c & 1) * PL::BUF;
            inverse(buf, sw);
#pragma unroll
            for (int i = 0; i < kTiles; ++i) {
                f32x4 t = {0.f, 0.f, 0.f, 0.f}, oo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KST; ++kk) {
                    const uint32_t fo = (uint32_t)((i * KST + kk) * 64 + lane) * 16;
                    t = mfma32(lds_ld<u32x4>(buf + PL::K1C + fo), Sop[kk], t);     // rows: tokens 4g + e
                    oo = mfma32(Sop[kk], lds_ld<u32x4>(buf + PL::QC + fo), oo);    // rows: value columns
                }
                T[i] = t;
                O[i] = oo;
            }
            // e^G for the slots of this lane's row, spread over its lanes
            const float* GMp = reinterpret_cast<const float*>(buf + PL::GM);
            float gam[SPL];
#pragma unroll
            for (int u = 0; u < SPL; ++u) gam[u] = GMp[slot_channel(g, SPL * v_ + u)];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = acc_slot(ct, e);
                    Sacc[ct][e] *= row_bcast_mov(gam[s % SPL], s / SPL);
                }
        };

        u32x2 Wb[kTiles];
        // Window 2: the block-triangular solve, P W, and the outputs.
        auto window2 = [&](int64_t c) {
            unsigned char* buf = smem + (c & 1) * PL::BUF;
            auto afrag = [&](int i) { return lds_ld<u32x2>(buf + PL::AD + ((16 * i + r) * PL::ASTR + 4 * g) * 2); };
            auto mfrag = [&](int i, int j) { return lds_ld<u32x2>(buf + PL::MF + (low(i, j) * 64 + lane) * 8); };
            auto pfrag = [&](int i, int j) { return lds_ld<u32x2>(buf + PL::PF + (tri(i, j) * 64 + lane) * 8); };
            f32x4 Z[kTiles];
#pragma unroll
            for (int i = 0; i < kTiles; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) Z[i][e] = bf16_lo(v_r[i][e]) - T[i][e];
            load_v(c + 1);
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            // W_i = A_i (Z_i - sum_{j<i} M_ij W_j); each M_ij W_j is issued as soon
            // as W_j is known.
#pragma unroll
            for (int i = 0; i < kTiles; ++i) {
                Wb[i] = cvt4(mfma16(afrag(i), cvt4(Z[i]), zero));
#pragma unroll
                for (int i2 = i + 1; i2 < kTiles; ++i2) Z[i2] = mfma16(mfrag(i2, i), Wb[i], Z[i2]);
            }
            // O^T += W^T P^T over token-tile pairs (the zero halves keep one shape)
            const u32x2 z2 = {0u, 0u};
            const u32x4 w01 = join(Wb[0], Wb[1]), w23 = join(Wb[2], Wb[3]);
            O[0] = mfma32(w01, join(pfrag(0, 0), z2), O[0]);
            O[1] = mfma32(w01, join(pfrag(1, 0), pfrag(1, 1)), O[1]);
            O[2] = mfma32(w01, join(pfrag(2, 0), pfrag(2, 1)), O[2]);
            O[2] = mfma32(w23, join(pfrag(2, 2), z2), O[2]);
            O[3] = mfma32(w01, join(pfrag(3, 0), pfrag(3, 1)), O[3]);
            O[3] = mfma32(w23, join(pfrag(3, 2), pfrag(3, 3)), O[3]);
            // lane (g, r): token 16 i + r, value columns 4 g .. 4 g + 3
            const Rsrc ro = make_rsrc(o + (row_of(c) - J.o_row0 * H) * DV + vcol, valid_rows(c) * (DV * 2u));
#pragma unroll
            for (int i = 0; i < kTiles; ++i)
                buf_st64(cvt4(O[i]), ro, ((16 * i + r) * (uint32_t)H * DV + 4 * g) * 2u);
        };

        // Window 3: S += (K e^{G-g})^T W.  Lane (g, m) of accumulator tile ct
        // reads row m of K2c^T (channel ch(g', acc_slot(ct, e')) for m = 4 g' +
        // e') at the tokens 4 g .. 4 g + 3 of a tile with ds_read_b64_tr_b16: lane
        // L of its group points at token 4 g + L / 4 and the 4 channels
        // 32 (ct / 2) + 4 (ct % 2) + 8 (L % 4) .. + 3.
        auto window3 = [&](int64_t c) {
            unsigned char* buf = smem + (c & 1) * PL::BUF;
            const int trow = 4 * g + (r >> 2);
            const int tcol = 8 * (r & 3);
            const u32x4 w01 = join(Wb[0], Wb[1]), w23 = join(Wb[2], Wb[3]);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int cb = 32 * (ct >> 1) + 4 * (ct & 1) + tcol;
                u32x2 seg[kTiles];
#pragma unroll
                for (int i = 0; i < kTiles; ++i) {
                    typedef short s16x4t __attribute__((ext_vector_type(4)));
                    const s16x4t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4t*)(buf + PL::K2C +
                                                                    ((16 * i + trow) * PL::LDK2 + cb) * 2));
                    seg[i] = __builtin_bit_cast(u32x2, t);
                }
                Sacc[ct] = mfma32(join(seg[0], seg[1]), w01, Sacc[ct]);
                Sacc[ct] = mfma32(join(seg[2], seg[3]), w23, Sacc[ct]);
            }
            pack_state();
        };

        load_v(0);
        if (nchunks > 0) {
            __syncthreads();                 // chunk 0: decays
            __syncthreads();                 // chunk 0: operands, diagonal blocks
            for (int64_t c = 0; c < nchunks; ++c) {
                window1(c);                  // the producers finish chunk c's off-diagonal blocks meanwhile
                __syncthreads();
                window2(c);
                window3(c);
                __syncthreads();
            }
        }
        if (final_state != nullptr) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    final_state[sbase + (int64_t)slot_channel(g, acc_slot(ct, e)) * DV + vcol + v_] = Sacc[ct][e];
        }
    }
}

// Workgroups of a job: with two value blocks, the pair of a unit sits 8
// workgroups apart (the grid is padded to whole groups of 16).
template <int DV>
int64_t job_blocks(int64_t units) {
    return DV / kBV == 2 ? 16 * ((units + 7) / 8) : units;
}

template <int DK, int DV, bool GATED>
hipError_t launch_jobs(const PrefillArgs& a, PrefillJob j0, PrefillJob j1) {
    using PL = Plan<DK>;
    auto kern = chunk_kernel<DK, DV, GATED>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       PL::TOTAL);
    if (e != hipSuccess) return e;
    j0.blocks = (int32_t)job_blocks<DV>(j0.units);
    j1.blocks = (int32_t)job_blocks<DV>(j1.units);
    const int64_t blocks = (int64_t)j0.blocks + j1.blocks;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kNW), PL::TOTAL, a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, a.log_alpha, a.beta, a.a_log, a.total_T, a.H,
                       j0, j1);
    return hipGetLastError();
}

template <int DK, bool GATED>
hipError_t launch_dk(const PrefillArgs& a, int d_v, const PrefillJob& j0, const PrefillJob& j1) {
    return d_v == 128 ? launch_jobs<DK, 128, GATED>(a, j0, j1) : launch_jobs<DK, 64, GATED>(a, j0, j1);
}

}  // namespace

hipError_t launch_chunk_jobs(const PrefillArgs& a, int d_v, const PrefillJob& j0, const PrefillJob& j1) {
    if (a.gated) return a.d_k == 128 ? launch_dk<128, true>(a, d_v, j0, j1) : launch_dk<64, true>(a, d_v, j0, j1);
    return a.d_k == 128 ? launch_dk<128, false>(a, d_v, j0, j1) : launch_dk<64, false>(a, d_v, j0, j1);
}

}  // namespace kda

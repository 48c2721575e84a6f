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
//   A    = (I + Diag(b) M)^{-1} Diag(b)                  unit-lower-triangular solve
//   W    = A (V - K_Gamma S0)                            pseudo-values, K_Gamma = K * Gamma
//   O    = Q_Gamma S0 + P W                              chunk output, Q_Gamma = Q * Gamma
//   S    = Diag(Gamma_C) S0 + (K * Gamma_C / Gamma)^T W  next chunk's state
//
// which follows from unrolling the recurrence inside the chunk (the delta
// correction of token r sees the decayed state and the corrections of the
// earlier tokens of the chunk; collecting them gives the triangular system).
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
// base 2 (log alpha * log2 e) so that v_exp_f32 is used directly.
//
// Work decomposition: one 256-thread workgroup per (sequence, head, V-block of
// BV value columns); the recurrence is independent across value columns.  The
// workgroup keeps its fp32 state slab [d_k, BV] in MFMA accumulators for the
// whole sequence and walks its chunks in order.  Per chunk:
//   E  elementwise: per-tile log-decay prefix sums, exponentials, scaled
//      operands written to LDS (row-major, the contraction index contiguous);
//   G  the P and M tile products (MFMA);
//   S  the triangular solve in fp32 (diagonal 16x16 blocks by substitution,
//      off-diagonal blocks by fp32 MFMA), A written to LDS;
//   U  U = V - K_Gamma S0 (MFMA), with S0 staged to LDS as an MFMA operand;
//   W  W = A U (MFMA);
//   O  O = Q_Gamma S0 + P W (MFMA), stored; S updated in the accumulators.
//
// Operand precision: bf16 inputs use v_mfma_f32_16x16x32_bf16 with bf16
// operands and fp32 accumulation; fp32 inputs use v_mfma_f32_16x16x4_f32.  The
// state, the decay arithmetic and the solve are fp32 throughout.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kC = 64;        // chunk length
constexpr int kTiles = 4;     // 16-token tiles per chunk
constexpr int kThreads = 256;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// 16x16 MFMA tile products from LDS.  D[m][n] += sum_k A[m*lda + k] * Bt[n*ldb + k]
// (both operands stored with the contraction index contiguous).  Output
// layout (CDNA 16x16 accumulators): lane l, register e holds
// D[4*(l/16) + e][l % 16].
// ---------------------------------------------------------------------------
template <typename OT> struct Mma;

template <> struct Mma<uint16_t> {   // bf16 operands
    static constexpr int KS = 32;
    static __device__ __forceinline__ f32x4 tile(const uint16_t* A, int lda, const uint16_t* Bt, int ldb,
                                                 int K, f32x4 acc) {
        const int lane = threadIdx.x & 63;
        const int r = lane & 15, g = lane >> 4;
        const uint16_t* a = A + r * lda + 8 * g;
        const uint16_t* b = Bt + r * ldb + 8 * g;
        for (int k0 = 0; k0 < K; k0 += KS) {
            const bf16x8 av = *reinterpret_cast<const bf16x8*>(a + k0);
            const bf16x8 bv = *reinterpret_cast<const bf16x8*>(b + k0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
        }
        return acc;
    }
    static __device__ __forceinline__ void put(uint16_t* p, float x) { *p = f32_to_bf16(x); }
    static __device__ __forceinline__ void put4(uint16_t* p, f32x4 x) {
        u32x2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        *reinterpret_cast<u32x2*>(p) = w;
    }
    static __device__ __forceinline__ float get(const uint16_t* p) { return bf16_to_f32(*p); }
};

template <> struct Mma<float> {      // fp32 operands
    static constexpr int KS = 4;
    static __device__ __forceinline__ f32x4 tile(const float* A, int lda, const float* Bt, int ldb,
                                                 int K, f32x4 acc) {
        const int lane = threadIdx.x & 63;
        const int r = lane & 15, g = lane >> 4;
        const float* a = A + r * lda + g;
        const float* b = Bt + r * ldb + g;
        for (int k0 = 0; k0 < K; k0 += KS)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[k0], b[k0], acc, 0, 0, 0);
        return acc;
    }
    static __device__ __forceinline__ void put(float* p, float x) { *p = x; }
    static __device__ __forceinline__ void put4(float* p, f32x4 x) {
        p[0] = x[0]; p[1] = x[1]; p[2] = x[2]; p[3] = x[3];
    }
    static __device__ __forceinline__ float get(const float* p) { return *p; }
};

// fp32 16x16x16 product with element accessors (used by the solve).
template <typename FA, typename FB>
__device__ __forceinline__ f32x4 mma16_f32(FA fa, FB fb, f32x4 acc) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa(r, k0 + g), fb(k0 + g, r), acc, 0, 0, 0);
    return acc;
}

// Index of tile-pair block (i, j), j <= i, among the 10 lower blocks.
__device__ __forceinline__ constexpr int blk(int i, int j) { return i * (i + 1) / 2 + j; }

// ---------------------------------------------------------------------------
// LDS plan.  Phase E/G buffers first; after G the Q/K/K-column region is
// reused for the state operand, the solve's scratch and U^T / W^T.
// ---------------------------------------------------------------------------
template <typename OT, int DK, int BV>
struct Plan {
    static constexpr int ES = sizeof(OT);
    static constexpr int PAD = (ES == 2) ? 8 : 1;   // row padding (elements): conflict-free fragment reads
    static constexpr int LDK = DK + PAD;            // stride of [*, DK] buffers
    static constexpr int LDC = kC + PAD;            // stride of [*, C] buffers
    static constexpr int LDT = kC + 1;              // stride of fp32 [C, C] solve buffer
    // phase E/G
    static constexpr int QE1 = 0;                                  // [C][LDK]  q * e^{g - rho_i}
    static constexpr int KE1 = QE1 + kC * LDK * ES;                // [C][LDK]  k * e^{g - rho_i}
    static constexpr int KCOL = KE1 + kC * LDK * ES;               // 10 x [16][LDK] column operands
    static constexpr int QG = KCOL + 10 * 16 * LDK * ES;           // [C][LDK]  q * e^{g}
    static constexpr int KG = QG + kC * LDK * ES;                  // [C][LDK]  k * e^{g}
    static constexpr int KDT = KG + kC * LDK * ES;                 // [DK][LDC] (k * e^{g_C - g})^T
    static constexpr int PB = KDT + DK * LDC * ES;                 // [C][LDC]  P (lower incl. diagonal)
    static constexpr int MB = PB + kC * LDC * ES;                  // [C][LDC]  M (strictly lower); later A
    static constexpr int BETA = MB + kC * LDC * ES;                // [C] fp32
    static constexpr int SX = BETA + kC * 4;                       // [4][DK] fp32 tile log2-decay totals
    static constexpr int DECAY = SX + kTiles * DK * 4;             // [DK] fp32 e^{g_C}
    static constexpr int TOTAL = DECAY + DK * 4;
    // reuse after phase G (inside [0, QG))
    static constexpr int ST = 0;                                   // [BV][LDK] S0^T (operand)
    static constexpr int TINV = ST + BV * LDK * ES;                // [C][LDT] fp32 (I + bM)^{-1}
    static constexpr int RSCR = TINV + kC * LDT * 4;               // 4 x [16][17] fp32 solve scratch
    static constexpr int UT = TINV;                                // [BV][LDC] U^T (after the solve)
    static constexpr int WT = UT + BV * LDC * ES;                  // [BV][LDC] W^T
    static_assert(RSCR + 4 * 16 * 17 * 4 <= QG, "solve scratch overlaps live buffers");
    static_assert(WT + BV * LDC * ES <= QG, "U/W buffers overlap live buffers");
    static_assert(TOTAL <= 160 * 1024, "LDS plan exceeds 160 KB");
};

template <typename T, int DK, int DV, int BV>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const float* __restrict__ init_state, const int32_t* __restrict__ cu_seqlens,
    int64_t total_T, int H, T* __restrict__ o, float* __restrict__ final_state) {
    using OT = T;
    using MM = Mma<OT>;
    using PL = Plan<OT, DK, BV>;
    constexpr int KS = MM::KS;
    constexpr int CPT = DK / 64;          // channels per thread in phase E
    constexpr int CT_PER_WAVE = DK / 64;  // 16-row channel tiles of S per wave
    constexpr int VT = BV / 16;           // 16-column tiles of S

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    OT* sQE1 = reinterpret_cast<OT*>(smem + PL::QE1);
    OT* sKE1 = reinterpret_cast<OT*>(smem + PL::KE1);
    OT* sKCOL = reinterpret_cast<OT*>(smem + PL::KCOL);
    OT* sQG = reinterpret_cast<OT*>(smem + PL::QG);
    OT* sKG = reinterpret_cast<OT*>(smem + PL::KG);
    OT* sKDT = reinterpret_cast<OT*>(smem + PL::KDT);
    OT* sP = reinterpret_cast<OT*>(smem + PL::PB);
    OT* sM = reinterpret_cast<OT*>(smem + PL::MB);
    OT* sA = sM;
    float* sBeta = reinterpret_cast<float*>(smem + PL::BETA);
    float* sX = reinterpret_cast<float*>(smem + PL::SX);
    float* sDecay = reinterpret_cast<float*>(smem + PL::DECAY);
    OT* sST = reinterpret_cast<OT*>(smem + PL::ST);
    float* sT = reinterpret_cast<float*>(smem + PL::TINV);
    float* sR = reinterpret_cast<float*>(smem + PL::RSCR);
    OT* sUT = reinterpret_cast<OT*>(smem + PL::UT);
    OT* sWT = reinterpret_cast<OT*>(smem + PL::WT);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int vblk = blockIdx.x;
    const int h = blockIdx.y;
    const int n = blockIdx.z;
    const int vbase = vblk * BV;

    // Sequence range, clamped so malformed offsets cannot address out of range.
    int64_t seq0 = 0, seq1 = total_T;
    if (cu_seqlens != nullptr) {
        seq0 = cu_seqlens[n];
        seq1 = cu_seqlens[n + 1];
        seq0 = seq0 < 0 ? 0 : (seq0 > total_T ? total_T : seq0);
        seq1 = seq1 < seq0 ? seq0 : (seq1 > total_T ? total_T : seq1);
    }
    const int64_t len = seq1 - seq0;

    // State slab in accumulators: tile (cl, vt) covers rows 16*(wave*CT_PER_WAVE + cl) .. +15
    // (key channels) and columns vbase + 16*vt .. +15 (value columns).
    f32x4 S[CT_PER_WAVE][VT];
    const int64_t sbase = ((int64_t)n * H + h) * DK * DV;
#pragma unroll
    for (int cl = 0; cl < CT_PER_WAVE; ++cl)
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            const int row0 = 16 * (wave * CT_PER_WAVE + cl) + 4 * lg;
            const int col = vbase + 16 * vt + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[cl][vt][e] = init_state ? init_state[sbase + (int64_t)(row0 + e) * DV + col] : 0.f;
        }


    for (int64_t c0 = 0; c0 < len; c0 += kC) {
        const int L = (int)((len - c0) < kC ? (len - c0) : kC);
        const int64_t tok0 = seq0 + c0;

        // ---------------- phase E: decay prefix sums and scaled operands ----------------
        {
            const int ti = wave;                  // this wave's 16-token tile
            const int cb = lane * CPT;            // first channel of this thread
            float x[16][CPT];
            float qv[16][CPT], kv[16][CPT];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int pos = 16 * ti + r;
                const bool ok = pos < L;
                const int64_t row = (tok0 + pos) * H + h;
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) {
                    const float la = ok ? log_alpha[row * DK + cb + cc] : 0.f;
                    x[r][cc] = (r == 0 ? 0.f : x[r - 1][cc]) + la * kLog2e;
                    qv[r][cc] = ok ? Elem<T>::load(q, row * DK + cb + cc) : 0.f;
                    kv[r][cc] = ok ? Elem<T>::load(k, row * DK + cb + cc) : 0.f;
                }
            }
            if (tid < kC) sBeta[tid] = (tid < L) ? beta[(tok0 + tid) * H + h] : 0.f;
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) sX[ti * DK + cb + cc] = x[15][cc];
            __syncthreads();

            float rho[kTiles + 1][CPT];   // rho[j] = log2-decay before tile j; rho[4] = chunk total
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) {
                rho[0][cc] = 0.f;
#pragma unroll
                for (int j = 0; j < kTiles; ++j) rho[j + 1][cc] = rho[j][cc] + sX[j * DK + cb + cc];
                if (ti == 0) sDecay[cb + cc] = fexp2(rho[kTiles][cc]);
            }
            // Per-channel factors of this tile.
            float sG[CPT], sD[CPT], F[kTiles][CPT];
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) {
                const float X = x[15][cc];
                sG[cc] = fexp2(rho[ti][cc]);                          // e^{rho_i}
                sD[cc] = fexp2(rho[kTiles][cc] - rho[ti + 1][cc]);    // e^{g_C - rho_{i+1}}
#pragma unroll
                for (int ip = 0; ip < kTiles; ++ip)                   // column factor for row tile ip
                    F[ip][cc] = (ip == ti) ? fexp2(-X) : (ip > ti ? fexp2(rho[ip][cc] - rho[ti + 1][cc]) : 0.f);
            }
            float kd[CPT][16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int pos = 16 * ti + r;
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) {
                    const float X = x[15][cc];
                    const float e1 = fexp2(x[r][cc]);
                    const float e2 = fexp2(X - x[r][cc]);
                    const float qe1 = qv[r][cc] * e1, ke1 = kv[r][cc] * e1, ke2 = kv[r][cc] * e2;
                    const int c = cb + cc;
                    MM::put(sQE1 + pos * PL::LDK + c, qe1);
                    MM::put(sKE1 + pos * PL::LDK + c, ke1);
                    MM::put(sQG + pos * PL::LDK + c, qe1 * sG[cc]);
                    MM::put(sKG + pos * PL::LDK + c, ke1 * sG[cc]);
                    kd[cc][r] = ke2 * sD[cc];
#pragma unroll
                    for (int ip = 0; ip < kTiles; ++ip)
                        if (ip >= ti) MM::put(sKCOL + (blk(ip, ti) * 16 + r) * PL::LDK + c, ke2 * F[ip][cc]);
                }
            }
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc)
#pragma unroll
                for (int r = 0; r < 16; r += 4) {
                    f32x4 w4 = {kd[cc][r], kd[cc][r + 1], kd[cc][r + 2], kd[cc][r + 3]};
                    MM::put4(sKDT + (cb + cc) * PL::LDC + 16 * ti + r, w4);
                }
        }
        __syncthreads();

        // ---------------- phase G: P and M tile products ----------------
        // Computed transposed (D[s][r]) so that each lane holds 4 consecutive
        // columns s of one row r of P / M.
        for (int p = wave; p < 32; p += 4) {
            // p in [0,10): P block; [10,20): M block; [20,32): zero upper blocks.
            if (p < 20) {
                const int pb = p < 10 ? p : p - 10;
                int i = 0;
                while (blk(i + 1, 0) <= pb) ++i;
                const int j = pb - blk(i, 0);
                const OT* rowop = (p < 10) ? sQE1 : sKE1;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = MM::tile(sKCOL + blk(i, j) * 16 * PL::LDK, PL::LDK, rowop + 16 * i * PL::LDK, PL::LDK, DK, acc);
                const int r = l16;                      // row within tile i
                OT* dst = (p < 10 ? sP : sM) + (16 * i + r) * PL::LDC + 16 * j + 4 * lg;
                f32x4 val;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 4 * lg + e;           // column within tile j
                    const bool keep = (i > j) || (p < 10 ? (s <= r) : (s < r));
                    val[e] = keep ? acc[e] : 0.f;
                }
                MM::put4(dst, val);
            } else {
                const int zb = p - 20;                  // 12 upper blocks: 6 of P then 6 of M
                const int which = zb / 6, u = zb % 6;   // u -> (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
                const int bi = u < 3 ? 0 : (u < 5 ? 1 : 2);
                const int bj = u < 3 ? u + 1 : (u < 5 ? u - 1 : 3);
                OT* dst = (which == 0 ? sP : sM) + (16 * bi + l16) * PL::LDC + 16 * bj + 4 * lg;
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                MM::put4(dst, z);
            }
        }
        __syncthreads();

        // ---------------- phase S: T = (I + Diag(b) M)^{-1}, A = T Diag(b) ----------------
        {
            // Diagonal blocks: wave w inverts block w by forward substitution, lane = column.
            if (lane < 16) {
                const int base = 16 * wave;
                float t[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float acc = 0.f;
#pragma unroll
                    for (int s = 0; s < r; ++s) acc += MM::get(sM + (base + r) * PL::LDC + base + s) * t[s];
                    t[r] = (r == lane ? 1.f : 0.f) - sBeta[base + r] * acc;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) sT[(base + r) * PL::LDT + base + lane] = t[r];
            }
            __syncthreads();
            // Off-diagonal blocks by diagonals d = i - j:  T_ij = -T_ii Diag(b_i) sum_{k=j}^{i-1} M_ik T_kj.
            for (int d = 1; d < kTiles; ++d) {
                if (wave < kTiles - d) {
                    const int j = wave, i = wave + d;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    for (int kb = j; kb < i; ++kb) {
                        acc = mma16_f32([&](int m, int kk) { return MM::get(sM + (16 * i + m) * PL::LDC + 16 * kb + kk); },
                                        [&](int kk, int nn) { return sT[(16 * kb + kk) * PL::LDT + 16 * j + nn]; }, acc);
                    }
                    float* R = sR + wave * 16 * 17;
#pragma unroll
                    for (int e = 0; e < 4; ++e) R[(4 * lg + e) * 17 + l16] = acc[e] * sBeta[16 * i + 4 * lg + e];
                    // same wave reads R back: wave-level LDS ordering
                    __builtin_amdgcn_s_waitcnt(0xc07f);
                    __builtin_amdgcn_wave_barrier();
                    f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
                    acc2 = mma16_f32([&](int m, int kk) { return sT[(16 * i + m) * PL::LDT + 16 * i + kk]; },
                                     [&](int kk, int nn) { return R[kk * 17 + nn]; }, acc2);
#pragma unroll
                    for (int e = 0; e < 4; ++e) sT[(16 * i + 4 * lg + e) * PL::LDT + 16 * j + l16] = -acc2[e];
                }
                __syncthreads();
            }
            // A[r][s] = T[r][s] b_s (s <= r), zero above the diagonal; written over M.
            for (int idx = tid; idx < kC * kC; idx += kThreads) {
                const int r = idx / kC, s = idx % kC;
                const float val = (s <= r) ? sT[r * PL::LDT + s] * sBeta[s] : 0.f;
                MM::put(sA + r * PL::LDC + s, val);
            }
            // S0^T as an MFMA operand (bf16 or fp32), from the accumulators.
#pragma unroll
            for (int cl = 0; cl < CT_PER_WAVE; ++cl)
#pragma unroll
                for (int vt = 0; vt < VT; ++vt) {
                    const int c = 16 * (wave * CT_PER_WAVE + cl) + 4 * lg;
                    MM::put4(sST + (16 * vt + l16) * PL::LDK + c, S[cl][vt]);
                }
        }
        __syncthreads();

        // ---------------- phase U: U = V - K_Gamma S0, stored as U^T ----------------
        {
            const int rt = wave;
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = MM::tile(sKG + 16 * rt * PL::LDK, PL::LDK, sST + 16 * vt * PL::LDK, PL::LDK, DK, acc);
                // acc[e] = (K_Gamma S0)[16 rt + 4 lg + e][16 vt + l16]
                f32x4 u;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int pos = 16 * rt + 4 * lg + e;
                    const float vv = pos < L ? Elem<T>::load(v, ((tok0 + pos) * H + h) * DV + vbase + 16 * vt + l16) : 0.f;
                    u[e] = vv - acc[e];
                }
                MM::put4(sUT + (16 * vt + l16) * PL::LDC + 16 * rt + 4 * lg, u);
            }
        }
        __syncthreads();

        // ---------------- phase W: W = A U, stored as W^T ----------------
        {
            const int rt = wave;
            constexpr int kUnit = KS > 16 ? KS : 16;
            const int K = ((16 * (rt + 1) + kUnit - 1) / kUnit) * kUnit;   // A is zero beyond the triangle
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = MM::tile(sA + 16 * rt * PL::LDC, PL::LDC, sUT + 16 * vt * PL::LDC, PL::LDC, K, acc);
                MM::put4(sWT + (16 * vt + l16) * PL::LDC + 16 * rt + 4 * lg, acc);
            }
        }
        __syncthreads();

        // ---------------- phase O: O = Q_Gamma S0 + P W;  S <- Diag(Gamma_C) S0 + Kd^T W ----------------
        {
            const int rt = wave;
            constexpr int kUnit = KS > 16 ? KS : 16;
            const int K = ((16 * (rt + 1) + kUnit - 1) / kUnit) * kUnit;
            const int pos = 16 * rt + l16;
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) {
                // D[v][r]: lane holds output row r = 16 rt + l16, columns 16 vt + 4 lg + e.
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = MM::tile(sST + 16 * vt * PL::LDK, PL::LDK, sQG + 16 * rt * PL::LDK, PL::LDK, DK, acc);
                acc = MM::tile(sWT + 16 * vt * PL::LDC, PL::LDC, sP + 16 * rt * PL::LDC, PL::LDC, K, acc);
                if (pos < L) {
                    const int64_t off = ((tok0 + pos) * H + h) * DV + vbase + 16 * vt + 4 * lg;
#pragma unroll
                    for (int e = 0; e < 4; ++e) Elem<T>::store(o, off + e, acc[e]);
                }
            }
#pragma unroll
            for (int cl = 0; cl < CT_PER_WAVE; ++cl) {
                const int ct = wave * CT_PER_WAVE + cl;
                f32x4 dec;
#pragma unroll
                for (int e = 0; e < 4; ++e) dec[e] = sDecay[16 * ct + 4 * lg + e];
#pragma unroll
                for (int vt = 0; vt < VT; ++vt) {
                    f32x4 acc = S[cl][vt] * dec;
                    acc = MM::tile(sKDT + 16 * ct * PL::LDC, PL::LDC, sWT + 16 * vt * PL::LDC, PL::LDC, kC, acc);
                    S[cl][vt] = acc;
                }
            }
        }
        __syncthreads();
    }

    if (final_state != nullptr) {
#pragma unroll
        for (int cl = 0; cl < CT_PER_WAVE; ++cl)
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) {
                const int row0 = 16 * (wave * CT_PER_WAVE + cl) + 4 * lg;
                const int col = vbase + 16 * vt + l16;
#pragma unroll
                for (int e = 0; e < 4; ++e) final_state[sbase + (int64_t)(row0 + e) * DV + col] = S[cl][vt][e];
            }
    }
}

template <typename T, int DK, int DV, int BV>
hipError_t launch_t(const PrefillArgs& a) {
    using PL = Plan<T, DK, BV>;
    auto kern = prefill_kernel<T, DK, DV, BV>;
    static bool attr_set = false;   // per instantiation; the attribute is a property of the function
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, PL::TOTAL);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    dim3 grid(DV / BV, a.H, a.N);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), PL::TOTAL, a.stream,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, a.log_alpha, a.beta, a.init_state,
                       a.cu_seqlens, a.total_T, a.H, (T*)a.o, a.final_state);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a) {
    if (a.bf16) {
        if (a.d_k == 128) return a.d_v == 128 ? launch_t<uint16_t, 128, 128, 64>(a) : launch_t<uint16_t, 128, 64, 64>(a);
        return a.d_v == 128 ? launch_t<uint16_t, 64, 128, 64>(a) : launch_t<uint16_t, 64, 64, 64>(a);
    }
    // fp32 operands: d_k = 64 only (the LDS plan of d_k = 128 would exceed 160 KB).
    return a.d_v == 128 ? launch_t<float, 64, 128, 64>(a) : launch_t<float, 64, 64, 64>(a);
}

}  // namespace kda

// KDA chunkwise prefill for gfx950 (CDNA4) as a pair of workgroups per
// (sequence, head): a producer workgroup and a state workgroup on two CUs of
// one XCD, joined by a ring of chunk images in device memory.
//
// The algebra is the tile recurrence of kda_prefill.hip ("Kimi K3 --
// Architecture Notes", sections 1.1 and 1.2): chunks of 64 tokens cut into
// four 16-token tiles, the state carried from tile to tile,
//   P, M (decayed Grams), A = (I + Diag(b) M)^{-1} Diag(b),
//   W = A (V - (K e1) S),  O = (Q e1) S + P W,  S <- Diag(2^X) S + (K e2)^T W.
// The single-workgroup kernel runs the state-independent half (operands, P,
// M, A) once per value-column workgroup, so a head with 128 value columns
// does it twice, and its four state waves share their SIMDs with producer
// waves.  Here the state-independent half of a head runs once, in its own
// workgroup, and all 128 value columns of the head are carried by one state
// workgroup of eight waves (two per SIMD):
//   producer (role 0): waves 0-3 form chunk c's scaled operands, decays, P and
//       M (wave i = tile i, as in kda_prefill.hip); waves 4-7 form the four
//       16x16 inverses of chunk c - 1 (wave 4 + i = tile i) and copy that
//       chunk's image from LDS into its ring slot.
//   state (role 1): wave w carries value columns 16 w .. 16 w + 15 over all
//       d_k rows of S; it reads chunk c's image from LDS while it loads chunk
//       c + 1's image from the ring into registers, and writes it to the other
//       LDS buffer at the end of the chunk.
// Handshake, per (sequence, head): a "ready" word (the last chunk whose image
// is complete in the ring) and a "free" word (the last chunk the state
// workgroup has taken out of it), both tagged with a per-launch epoch in the
// high 32 bits, so no reset is needed between launches.  The ring data and
// both words are accessed at device scope (sc1): stores complete to the
// device-coherent level before the producer's flag store (vmcnt(0) and a
// workgroup barrier), and the state workgroup issues its ring loads only
// after it has seen the flag.  No cache writeback or invalidation is needed.
// Every wait is bounded; one that runs out is counted in a device word the
// host reads, and the workgroup stops waiting from then on (its outputs are
// then not to be trusted), so no wait can hang the device.
//
// The launch is cooperative, so the two workgroups of a pair are resident
// together; the host uses this kernel only when every workgroup of the grid
// can be resident at once (one per CU), and the single-workgroup kernel
// otherwise.  bf16 operands, d_k = d_v = 128.

#include <atomic>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_prefill_ops.h"

namespace kda {

// Bounded ring waits that ran out on this device; read and reset with the
// flag waits of the single-workgroup kernel (read_wait_giveups).
__device__ uint32_t g_pair_wait_giveups;

namespace {

constexpr int kRing = 3;        // ring slots per (sequence, head)
constexpr int kPairThreads = 512;

// Chunk image (bf16, d_k = 128): the state-independent results one chunk
// hands to the state workgroup, in the layout the state waves read from LDS
// (row paddings as in kda_prefill.hip, against LDS bank conflicts).  A comes
// last so that the part written by the producer waves is one contiguous range.
struct PairPlan {
    static constexpr int DK = 128;
    static constexpr int LDK = DK + 4;       // q e1, k e1 rows
    static constexpr int LDK2 = DK + 16;     // k e2 rows (read transposed)
    static constexpr int LD16 = 16 + 4;      // 16x16 blocks
    static constexpr int MSTR = 20;          // fp32 M^T rows
    static constexpr int QE1 = 0;                                // [64][LDK]  q e1
    static constexpr int KE1 = QE1 + kC * LDK * 2;               // [64][LDK]  k e1
    static constexpr int KE2 = KE1 + kC * LDK * 2;               // [64][LDK2] k e2
    static constexpr int PD = KE2 + kC * LDK2 * 2;               // [4][16][LD16] P per tile
    static constexpr int DEC = PD + kTiles * 16 * LD16 * 2;      // [4][DK] fp32 2^X per tile
    static constexpr int AD = DEC + kTiles * DK * 4;             // [4][16][LD16] A per tile
    static constexpr int IMG = AD + kTiles * 16 * LD16 * 2;      // bytes of one image
    // producer only, per buffer: M^T and beta of each tile
    static constexpr int MS = IMG;
    static constexpr int BS = MS + kTiles * 16 * MSTR * 4;
    static constexpr int PBUF = BS + kTiles * 16 * 4;
    static constexpr int KB = 2 * PBUF;                          // [64][LDK] k 2^{-x} (producer scratch)
    static constexpr int PTOTAL = KB + kC * LDK * 2;
    static constexpr int SPARE = 2 * IMG;                        // state workgroup: two images, then
    static constexpr int STOTAL = SPARE + 64 * 16;               // a spare area for idle lanes' stores
    static constexpr int TOTAL = PTOTAL > STOTAL ? PTOTAL : STOTAL;
    static constexpr int IMG16 = IMG / 16;                       // 16-byte pieces of an image
    static constexpr int REST16 = AD / 16;                       // pieces before A
    static constexpr int A16 = 16 * LD16 * 2 / 16;               // pieces of one tile's A
    static_assert(IMG % 16 == 0 && AD % 16 == 0 && PBUF % 16 == 0 && KB % 16 == 0, "alignment");
    static_assert(REST16 % 4 == 0 && IMG16 % 8 == 0, "copy split");
    static_assert(TOTAL <= 160 * 1024, "LDS plan exceeds 160 KB");
};

constexpr int kFlagStride = 32;   // uint64 words per (sequence, head): ready at 0, free at 16 (own lines)

// Device-scope (sc1) ring accesses: they bypass the CU's vector L1 and are
// coherent across the device, so the handshake needs no cache maintenance.
constexpr int kScDevice = 16;
__device__ __forceinline__ u32x4 ring_ld128(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kScDevice));
}
__device__ __forceinline__ void ring_st128(u32x4 x, Rsrc r, uint32_t off) {
    typedef unsigned int v4u __attribute__((__vector_size__(16)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, x), r, off, 0, kScDevice);
}
__device__ __forceinline__ uint64_t flag_issue(const uint64_t* f) {
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t uniform(uint64_t x) {   // every lane read the same word
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t flag_load(const uint64_t* f) { return uniform(flag_issue(f)); }
__device__ __forceinline__ void flag_store(uint64_t* f, uint64_t x) {
    __hip_atomic_store(f, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool GATED>
__global__ __launch_bounds__(kPairThreads, 1) void prefill_pair_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const void* __restrict__ decay, const float* __restrict__ beta, const float* __restrict__ a_log,
    int64_t total_T, int H, PrefillJob J, unsigned char* __restrict__ ring, uint64_t* __restrict__ flags,
    uint64_t epoch) {
    using T = uint16_t;
    using OT = T;
    using OP = Op<OT>;
    using PP = PairPlan;
    using DT = typename std::conditional<GATED, T, float>::type;
    using Xop = typename OP::Xop;
    constexpr int DK = 128, DV = 128;
    constexpr int KS = OP::KS;
    constexpr int CPL = 8;                // producer: key channels per lane
    constexpr int LPR = DK / CPL;         // producer: lanes per token row
    constexpr int NG = 64 / LPR;          // producer: position groups of a tile
    constexpr int RP = 16 / NG;           // producer: consecutive tile positions per lane
    constexpr int QWN = CPL * (int)sizeof(T) / 4;
    constexpr int NCT = DK / 16;          // 16-row channel tiles of the state
    constexpr int NKS = DK / KS;          // K-steps of the Gram products
    const DT* log_alpha = reinterpret_cast<const DT*>(decay);
    const T* __restrict__ v = reinterpret_cast<const T*>(J.v);
    const float* __restrict__ init_state = J.init_state;
    const int32_t* __restrict__ cu_seqlens = J.cu_seqlens;
    T* __restrict__ o = reinterpret_cast<T*>(J.o);
    float* __restrict__ final_state = J.final_state;

    // Workgroup -> (unit = sequence * H + head, role); the two workgroups of a
    // unit are 8 apart, so that they are dealt to the same XCD.
    const int lid = (int)blockIdx.x;
    const int unit = 8 * (lid >> 4) + (lid & 7);
    const int role = (lid >> 3) & 1;
    if (unit >= J.units) return;
    const int n = unit / H;
    const int h = unit - n * H;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int lg = lane >> 4;

    int64_t seq0 = 0, seq1 = total_T;
    if (cu_seqlens != nullptr) {
        seq0 = cu_seqlens[n];
        seq1 = cu_seqlens[n + 1];
    }
    seq0 = seq0 < 0 ? 0 : (seq0 > total_T ? total_T : seq0);
    seq1 = seq1 < seq0 ? seq0 : (seq1 > total_T ? total_T : seq1);
    const int64_t len = seq1 - seq0;
    const int64_t nchunks = (len + kC - 1) / kC;
    auto chunk_len = [&](int64_t c) { return (int)((len - c * kC) < kC ? (len - c * kC) : kC); };
    auto valid_rows = [&](int64_t c) {
        return c < nchunks ? (uint32_t)(chunk_len(c) - 1) * (uint32_t)H + 1u : 0u;
    };
    auto row_of = [&](int64_t c) { return (seq0 + (c < nchunks ? c : 0) * kC) * H + h; };

    unsigned char* uring = ring + (size_t)unit * kRing * PP::IMG;
    uint64_t* f_ready = flags + (size_t)unit * kFlagStride;
    uint64_t* f_free = f_ready + 16;
    const uint64_t tag = epoch << 32;
    bool broken = false;
    auto wait_flag = [&](const uint64_t* f, uint64_t target) {
        if (broken) return;
        for (int spin = 0; spin < (1 << 20); ++spin) {
            if (flag_load(f) >= target) return;
            __builtin_amdgcn_s_sleep(2);
        }
        broken = true;
        if (lane == 0) atomicAdd(&g_pair_wait_giveups, 1u);
    };

    if (role == 0) {
        // ================= producer =================
        const float eA = GATED ? __expf(a_log[h]) : 1.f;
        if (wave < kTiles) {
            const int ti = wave;
            const int cb = (lane % LPR) * CPL;
            const int pg = lane / LPR;
            const uint32_t p0 = 16 * ti + RP * pg;
            constexpr int LAW = CPL * (int)sizeof(DT) / 4;
            uint32_t la_w[RP][LAW];
            uint32_t qw_r[RP][QWN], kw_r[RP][QWN];
            float beta_r;
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
                                                  (16 * ti + l16) * (uint32_t)H * 4));
            };
            OT* sKB = reinterpret_cast<OT*>(smem + PP::KB);
            // Tile ti of chunk c into buffer c & 1: the scaled operands, 2^X,
            // P (the image), and M^T and beta (for the inverse waves).
            auto si = [&](int64_t c) {
                unsigned char* buf = smem + (c & 1) * PP::PBUF;
                OT* sQE1 = reinterpret_cast<OT*>(buf + PP::QE1);
                OT* sKE1 = reinterpret_cast<OT*>(buf + PP::KE1);
                OT* sKE2 = reinterpret_cast<OT*>(buf + PP::KE2);
                OT* sPD = reinterpret_cast<OT*>(buf + PP::PD);
                float* sDEC = reinterpret_cast<float*>(buf + PP::DEC);
                float* sMS = reinterpret_cast<float*>(buf + PP::MS);
                float* sBS = reinterpret_cast<float*>(buf + PP::BS);
                const int pb = (int)p0;
                const QKRes rq_next = qk_rsrc(c + 1);
                float al[RP][CPL], dec[CPL];
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
                    dec[cc] = t;
                }
                load_la(c + 1);
                __builtin_amdgcn_sched_barrier(0);
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
                level(std::integral_constant<int, 16>{});
                level(std::integral_constant<int, 32>{});
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
                    const int orow = (pb + r) * PP::LDK + cb;
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
                    OP::put8(sKE2 + (pb + r) * PP::LDK2 + cb, ke2[0], ke2[1]);
                    OP::put8(sKB + orow, kb[0], kb[1]);
                    load_qk_row(rq_next, r);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (lane < 16) {
                    if constexpr (GATED)
                        sBS[ti * 16 + lane] = 16 * ti + lane < chunk_len(c)
                                                  ? __builtin_amdgcn_rcpf(1.f + fexp2(-kLog2e * beta_r)) : 0.f;
                    else
                        sBS[ti * 16 + lane] = beta_r;
                }
                load_beta(c + 1);
                wave_lds_sync();
                {
                    const OT* rq = sQE1 + 16 * ti * PP::LDK;
                    const OT* rk = sKE1 + 16 * ti * PP::LDK;
                    const OT* rb = sKB + 16 * ti * PP::LDK;
                    f32x4 accP = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const typename OP::Frag fb = OP::frag(rb, PP::LDK, ks * KS);
                        accP = OP::mma(fb, OP::frag(rq, PP::LDK, ks * KS), accP);
                        accM = OP::mma(fb, OP::frag(rk, PP::LDK, ks * KS), accM);
                    }
                    f32x4 vp;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = 4 * lg + e;
                        vp[e] = s <= l16 ? accP[e] : 0.f;
                        sMS[(ti * 16 + s) * PP::MSTR + 4 * (l16 & 3) + (l16 >> 2)] = s < l16 ? accM[e] : 0.f;
                    }
                    OP::put4(sPD + (ti * 16 + l16) * PP::LD16 + 4 * lg, vp);
                }
            };
            if (nchunks > 0) {
                load_la(0);
                {
                    const QKRes r0 = qk_rsrc(0);
#pragma unroll
                    for (int r = 0; r < RP; ++r) load_qk_row(r0, r);
                    load_beta(0);
                }
                for (int64_t it = 0; it <= nchunks; ++it) {
                    if (it < nchunks) si(it);
                    __syncthreads();
                }
            }
        } else {
            const int ti = wave - kTiles;
            const Rsrc rring = make_rsrc(uring, kRing * PP::IMG);
            // Inverse of tile ti of chunk cc, then the copy of the chunk's image
            // (the producer waves' part, a quarter per wave, and this tile's A)
            // into ring slot cc % kRing once the state workgroup has taken the
            // chunk that used that slot before.
            auto finish = [&](int64_t cc) {
                unsigned char* buf = smem + (cc & 1) * PP::PBUF;
                OT* sAD = reinterpret_cast<OT*>(buf + PP::AD);
                const float* sMS = reinterpret_cast<const float*>(buf + PP::MS);
                const float* sBS = reinterpret_cast<const float*>(buf + PP::BS);
                {
                    // A = (I + Diag(b) M)^{-1} Diag(b): right-looking substitution on
                    // all 64 lanes, lane = (column j = lane / 4, row residue q = lane % 4)
                    // holding rows 4 m + q of column j (as in kda_prefill.hip).
                    const int j = lane >> 2, qq = lane & 3;
                    const float* MT = sMS + ti * 16 * PP::MSTR + 4 * qq;
                    float bt[16];
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const f32x4 b4 = *reinterpret_cast<const f32x4*>(sBS + ti * 16 + 4 * q4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) bt[4 * q4 + e] = b4[e];
                    }
                    f32x4 mr[16];
#pragma unroll
                    for (int s2 = 0; s2 < 16; ++s2) mr[s2] = *reinterpret_cast<const f32x4*>(MT + s2 * PP::MSTR);
                    float acc[4], xs[4], one[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) { acc[m] = 0.f; xs[m] = 0.f; one[m] = (4 * m + qq == j) ? 1.f : 0.f; }
#pragma unroll
                    for (int s2 = 0; s2 < 16; ++s2) {
                        const int ms = s2 >> 2, qs = s2 & 3;
                        const float cand = fmaf(-bt[s2], acc[ms], one[ms]);
                        if (qq == qs) xs[ms] = cand;
                        const float x = quad_bcast(cand, qs);
#pragma unroll
                        for (int m = 0; m < 4; ++m)
                            if (4 * m + 3 > s2) acc[m] = fmaf(mr[s2][m], x, acc[m]);
                    }
                    const float bj = sBS[ti * 16 + j];
#pragma unroll
                    for (int m = 0; m < 4; ++m) OP::put(sAD + (ti * 16 + 4 * m + qq) * PP::LD16 + j, xs[m] * bj);
                }
                wave_lds_sync();
                if (cc >= kRing) wait_flag(f_free, tag | (uint64_t)(cc - kRing + 1));
                const uint32_t slot = (uint32_t)(cc % kRing) * PP::IMG;
                constexpr int PER = PP::REST16 / 4;
#pragma unroll
                for (int jj = 0; jj < (PER + 63) / 64; ++jj) {
                    const int idx = 64 * jj + lane;
                    if (idx < PER) {
                        const int p = ti * PER + idx;
                        ring_st128(*reinterpret_cast<const u32x4*>(buf + 16 * p), rring, slot + 16 * p);
                    }
                }
                if (lane < PP::A16) {
                    const int p = PP::REST16 + ti * PP::A16 + lane;
                    ring_st128(*reinterpret_cast<const u32x4*>(buf + 16 * p), rring, slot + 16 * p);
                }
                __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's ring stores are complete
            };
            if (nchunks > 0) {
                for (int64_t it = 0; it <= nchunks; ++it) {
                    if (it >= 1) finish(it - 1);
                    __syncthreads();
                    if (it >= 1 && tid == 64 * kTiles) flag_store(f_ready, tag | (uint64_t)it);
                }
            }
        }
        return;
    }

    // ================= state workgroup =================
    using Seg = typename OP::Seg;
    const int vcol = 16 * wave;
    const int tro = OP::seg_t_offset(PP::LDK2);
    f32x4 Sacc[NCT];
    const int64_t sbase = ((int64_t)n * H + h) * DK * DV;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            Sacc[ct][e] = init_state != nullptr
                              ? init_state[sbase + (int64_t)(16 * ct + 4 * lg + e) * DV + vcol + l16] : 0.f;
    if (nchunks > 0) {
        uint32_t v_r[kTiles][4];
        auto v_rsrc = [&](int64_t c) {
            return v != nullptr ? make_rsrc(v + row_of(c) * DV + vcol, valid_rows(c) * (DV * (uint32_t)sizeof(T)))
                                : make_rsrc(nullptr, 0u);
        };
        auto load_v_tile = [&](Rsrc rv, int i) {
            const uint32_t rs = (uint32_t)H * DV;
#pragma unroll
            for (int e = 0; e < 4; ++e) v_r[i][e] = buf_ld16(rv, ((16 * i + 4 * lg + e) * rs + l16) * 2);
        };
        // This wave's eighth of an image, pieces wave * SHARE + 64 jj + lane,
        // moved in two halves of HJ rounds (16 registers each).
        constexpr int SHARE = PP::IMG16 / 8;
        constexpr int HJ = (SHARE + 127) / 128;
        u32x4 img_r[HJ];
        auto load_img = [&](int64_t c, int half) {    // an empty range past the last chunk
            const bool ok = c < nchunks;
            const Rsrc rr = make_rsrc(uring + (ok ? (c % kRing) * PP::IMG : 0), ok ? (uint32_t)PP::IMG : 0u);
#pragma unroll
            for (int jj = 0; jj < HJ; ++jj) {
                const int idx = 64 * (HJ * half + jj) + lane;
                const uint32_t off = idx < SHARE ? 16u * (uint32_t)(wave * SHARE + idx) : 0xfffffff0u;
                img_r[jj] = ring_ld128(rr, off);
            }
        };
        // Lanes past the share write a spare area after the two images, so that
        // every store, and hence every load, is unconditional (a load the
        // compiler sinks into a branch is waited for at once).
        auto store_img = [&](int64_t c, int half) {
#pragma unroll
            for (int jj = 0; jj < HJ; ++jj) {
                const int idx = 64 * (HJ * half + jj) + lane;
                const int off = idx < SHARE ? (int)(c & 1) * PP::IMG + 16 * (wave * SHARE + idx) : PP::SPARE + 16 * lane;
                *reinterpret_cast<u32x4*>(smem + off) = img_r[jj];
            }
        };
        // chunk 0's image and values
        wait_flag(f_ready, tag | 1u);
        {
            const Rsrc rv0 = v_rsrc(0);
#pragma unroll
            for (int i = 0; i < kTiles; ++i) load_v_tile(rv0, i);
        }
        load_img(0, 0);
        store_img(0, 0);
        load_img(0, 1);
        store_img(0, 1);
        __syncthreads();
        if (tid == 0) flag_store(f_free, tag | 1u);

        for (int64_t c = 0; c < nchunks; ++c) {
            // Ask early whether chunk c + 1 is ready; the answer is read after
            // tile 0, so that waiting for it waits for no load issued since.
            const uint64_t pre = flag_issue(f_ready);
            __builtin_amdgcn_sched_barrier(0);
            const Rsrc rv_next = v_rsrc(c + 1);
            const unsigned char* buf = smem + (c & 1) * PP::IMG;
            const OT* sQE1 = reinterpret_cast<const OT*>(buf + PP::QE1);
            const OT* sKE1 = reinterpret_cast<const OT*>(buf + PP::KE1);
            const OT* sKE2 = reinterpret_cast<const OT*>(buf + PP::KE2);
            const OT* sPD = reinterpret_cast<const OT*>(buf + PP::PD);
            const OT* sAD = reinterpret_cast<const OT*>(buf + PP::AD);
            const float* sDEC = reinterpret_cast<const float*>(buf + PP::DEC);
            const Rsrc ro = make_rsrc(o + row_of(c) * DV + vcol, valid_rows(c) * (DV * (uint32_t)sizeof(T)));
            constexpr int VPL = NCT / 4;
            struct TileOps { Seg kseg[NCT], qseg[NCT], eseg[NCT], pseg, aseg; float decv[VPL]; };
            auto load_ops = [&](int i, TileOps& t) {
                const OT* krow = sKE1 + (16 * i + l16) * PP::LDK;
                const OT* qrow = sQE1 + (16 * i + l16) * PP::LDK;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) t.kseg[ct] = OP::seg(krow + 16 * ct);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) t.qseg[ct] = OP::seg(qrow + 16 * ct);
                t.pseg = OP::seg(sPD + (16 * i + l16) * PP::LD16);
                t.aseg = OP::seg(sAD + (16 * i + l16) * PP::LD16);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) t.eseg[ct] = OP::seg_t(sKE2 + 16 * i * PP::LDK2 + 16 * ct, tro, PP::LDK2);
                const float* dp = sDEC + i * DK + 16 * ((VPL * l16) >> 2) + 4 * lg + ((VPL * l16) & 3);
#pragma unroll
                for (int u = 0; u < VPL; ++u) t.decv[u] = dp[u];
            };
            TileOps ops[2];
            load_ops(0, ops[0]);
#pragma unroll
            for (int i = 0; i < kTiles; ++i) {
                if (i + 1 < kTiles) load_ops(i + 1, ops[(i + 1) & 1]);
                const TileOps& cur = ops[i & 1];
                Xop Sop[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) Sop[ct] = OP::cvt(Sacc[ct]);
                // U = V_i - (K e1)_i S
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ct = 0; ct < NCT; ct += 2)
                    acc = OP::seg_acc32(cur.kseg[ct], cur.kseg[ct + 1], Sop[ct], Sop[ct + 1], acc);
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = word_elem<T>(v_r[i][e], 0) - acc[e];
                load_v_tile(rv_next, i);
                __builtin_amdgcn_sched_barrier(0);
                // W = A U
                f32x4 w = {0.f, 0.f, 0.f, 0.f};
                w = OP::seg_acc16(cur.aseg, OP::cvt(y), w);
                const Xop Wop = OP::cvt(w);
                // O^T = S^T (Q e1)^T + W^T P^T
                f32x4 oacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ct = 0; ct < NCT; ct += 2)
                    oacc = OP::acc_seg32(Sop[ct], Sop[ct + 1], cur.qseg[ct], cur.qseg[ct + 1], oacc);
                oacc = OP::acc_seg16_k32(Wop, cur.pseg, oacc);
                // S <- Diag(2^X) S + (K e2)^T W
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    f32x4 sd4;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sd4[e] = Sacc[ct][e] * row_bcast(cur.decv[(4 * ct + e) % VPL], (4 * ct + e) / VPL);
                    Sacc[ct] = OP::seg_acc16(cur.eseg[ct], Wop, sd4);
                }
                const uint32_t ooff = ((16 * i + l16) * (uint32_t)H * DV + 4 * lg) * (uint32_t)sizeof(T);
                buf_st64(OP::cvt(oacc), ro, ooff);
                if (i == 0) {
                    // Chunk c + 1's image: wait until it is in the ring, then load
                    // its first half (stored after tile 1, when the second half
                    // is loaded; that one is stored at the end of the chunk).
                    const uint64_t target = tag | (uint64_t)(c + 2);
                    if (c + 1 < nchunks && uniform(pre) < target) wait_flag(f_ready, target);
                    load_img(c + 1, 0);
                    __builtin_amdgcn_sched_barrier(0);
                } else if (i == 1) {
                    store_img(c + 1, 0);
                    load_img(c + 1, 1);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            store_img(c + 1, 1);
            __syncthreads();
            if (c + 1 < nchunks && tid == 0) flag_store(f_free, tag | (uint64_t)(c + 2));
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

// Per (device, stream) ring workspace: launches on one stream run one after
// the other, so they may share it; the epoch in the flags tells launches apart.
struct PairWs {
    unsigned char* ring = nullptr;
    uint64_t* flags = nullptr;
    int64_t units = 0;
    uint64_t epoch = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, PairWs> g_ws;
int g_pair_mode = 1;    // 1: use the pair kernel where it fits; 0: never
std::atomic<int64_t> g_pair_launches{0};

// Workgroups of the grid: the pair of unit u at 16 (u / 8) + u % 8 and + 8.
int64_t pair_blocks(int64_t units) { return 16 * ((units + 7) / 8); }

template <bool GATED>
hipError_t launch_pair_t(const PrefillArgs& a, bool* used) {
    *used = false;
    using PP = PairPlan;
    auto kern = prefill_pair_kernel<GATED>;
    const int64_t units = (int64_t)a.N * a.H;
    const int64_t blocks = pair_blocks(units);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = 0, coop = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev)) != hipSuccess) return e;
    if (!coop || blocks > cus) return hipSuccess;             // not co-resident: the caller runs the other kernel
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(a.stream, &cap)) != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) return hipSuccess;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 PP::TOTAL)) != hipSuccess)
        return e;
    int per_cu = 0;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kPairThreads, PP::TOTAL)) != hipSuccess)
        return e;
    if (blocks > (int64_t)per_cu * cus) return hipSuccess;

    unsigned char* ring;
    uint64_t* flags;
    uint64_t epoch;
    {
        std::lock_guard<std::mutex> lk(g_ws_mu);
        PairWs& ws = g_ws[{dev, a.stream}];
        if (ws.units < units) {
            // Grown to the largest co-resident grid at once, so it is allocated once per stream.
            const int64_t cap = (int64_t)cus / 2;
            if (ws.ring != nullptr) {
                if ((e = hipStreamSynchronize(a.stream)) != hipSuccess) return e;
                (void)hipFree(ws.ring);
                (void)hipFree(ws.flags);
                ws = PairWs{};
            }
            // Without the memory the caller runs the single-workgroup kernel instead.
            if (hipMalloc(&ws.ring, (size_t)cap * kRing * PP::IMG) != hipSuccess ||
                hipMalloc(&ws.flags, (size_t)cap * kFlagStride * sizeof(uint64_t)) != hipSuccess) {
                (void)hipGetLastError();
                if (ws.ring != nullptr) (void)hipFree(ws.ring);
                ws = PairWs{};
                return hipSuccess;
            }
            if ((e = hipMemset(ws.flags, 0, (size_t)cap * kFlagStride * sizeof(uint64_t))) != hipSuccess) return e;
            ws.units = cap;
        }
        ring = ws.ring;
        flags = ws.flags;
        epoch = ++ws.epoch;
    }
    PrefillJob j{a.v, a.init_state, a.cu_seqlens, a.o, a.final_state, 0, 0, 0, (int32_t)units, (int32_t)blocks,
                 kInitAll};
    const uint16_t* qp = static_cast<const uint16_t*>(a.q);
    const uint16_t* kp = static_cast<const uint16_t*>(a.k);
    const void* dp = a.log_alpha;
    const float* bp = a.beta;
    const float* ap = a.a_log;
    int64_t total_T = a.total_T;
    int H = a.H;
    void* args[] = {&qp, &kp, &dp, &bp, &ap, &total_T, &H, &j, &ring, &flags, &epoch};
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3((unsigned)blocks), dim3(kPairThreads),
                                   args, PP::TOTAL, a.stream);
    if (e == hipSuccess) {
        *used = true;
        ++g_pair_launches;
    }
    return e;
}

}  // namespace

hipError_t launch_prefill_pair(const PrefillArgs& a, bool* used) {
    *used = false;
    if (g_pair_mode == 0 || !a.bf16 || a.d_k != 128 || a.d_v != 128 || (int64_t)a.N * a.H == 0) return hipSuccess;
    return a.gated ? launch_pair_t<true>(a, used) : launch_pair_t<false>(a, used);
}

int set_prefill_pair_mode(int mode) {
    const int old = g_pair_mode;
    if (mode == 0 || mode == 1) g_pair_mode = mode;
    return old;
}

int64_t prefill_pair_launches() { return g_pair_launches.load(); }

hipError_t read_pair_wait_giveups(uint32_t* count, bool reset) {
    hipError_t e = hipMemcpyFromSymbol(count, HIP_SYMBOL(g_pair_wait_giveups), sizeof(uint32_t));
    if (e == hipSuccess && reset) {
        const uint32_t zero = 0;
        e = hipMemcpyToSymbol(HIP_SYMBOL(g_pair_wait_giveups), &zero, sizeof(uint32_t));
    }
    return e;
}

}  // namespace kda

// Time split of one long sequence across the GPU (gfx950): the two passes
// after the segment runs.
//
// The recurrence of "Kimi K3 -- Architecture Notes", section 1.1, is affine
// in the state: a run of tokens maps S to Phi S + B, where Phi is the product
// of the step matrices (I - b k k^T) Diag(alpha) and B is the end state from
// a zero start.  One sequence cut into segments p = 0..P-1 of seg_len tokens
// is therefore evaluated as
//   1. every segment at once: from a zero state (segment 0 from the initial
//      state), giving its outputs o0 and its end state B_p; and every segment
//      after the first from the identity with no values, giving Phi_p and the
//      outputs qt_t = Phi_t^T q_t (Phi_t: the product up to token t).  The
//      prefill kernel runs both (kda_prefill.hip);
//   2. the serial scan  S_end,p = Phi_p S_end,p-1 + B_p  (split_scan_kernel);
//   3. the correction  o_t = o0_t + S_end,p-1^T qt_t  for the tokens of
//      segments p >= 1 (split_correct_kernel).
//
// The scan is a chain of small fp32 products (d_k x d_k times d_k x 16 per
// workgroup and step) on v_mfma_f32_16x16x4_f32.  The correction is a
// streaming GEMM: bf16 inputs use v_mfma_f32_16x16x32_bf16 with the state
// split into a bf16 high part and a bf16 remainder (about 16 significant
// bits), fp32 inputs use the fp32 MFMA.

#include "kda_device.h"
#include "kda_internal.h"

#include <mutex>

#include "../../include/kda.h"

namespace kda {
namespace {

// ---------------------------------------------------------------------------
// Scan.  One workgroup (4 waves) per (head, block of 16 value columns).  The
// 16 columns of the running state are kept transposed in LDS, ST[j][m] =
// S[m][c0 + j]; wave w forms row tiles w, w + 4, ... of Phi_p S + B_p.
// MFMA operands: lane (i = l % 16, g = l / 16) supplies Phi[16 ct + i][16 u +
// 4 g + e] and ST[i][16 u + 4 g + e] to the products e = 0..3 of K-block u
// (any assignment of the contraction index to the products is complete, as
// long as both operands use the same one).  The accumulator then holds row
// 16 ct + 4 g + e, column c0 + (l % 16) in register e.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(256) void split_scan_kernel(float* __restrict__ ends, const float* __restrict__ phis,
                                                         float* __restrict__ final_state, int segments, int H) {
    constexpr int NCT = DK / 16;
    constexpr int NB = DV / 16;
    constexpr int LDT = DK + 4;
    __shared__ __attribute__((aligned(16))) float ST[16 * LDT];
    const int h = blockIdx.x / NB;
    const int c0 = 16 * (blockIdx.x % NB);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = lane & 15, g = lane >> 4;
    const size_t slab = (size_t)DK * DV, tslab = (size_t)DK * DK;

    // Start: the end state of segment 0 (the true one).
    {
        const float* src = ends + (size_t)h * slab;
        for (int x = tid; x < DK * 16; x += 256) {
            const int m = x >> 4, j = x & 15;
            ST[j * LDT + m] = src[(size_t)m * DV + c0 + j];
        }
    }
    f32x4 cur[(NCT + 3) / 4];
#pragma unroll
    for (int r = 0; r < (NCT + 3) / 4; ++r) cur[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int p = 1; p < segments; ++p) {
        __syncthreads();
        const float* phi = phis + ((size_t)(p - 1) * H + h) * tslab;
        float* bp = ends + ((size_t)p * H + h) * slab;
#pragma unroll
        for (int r = 0; r < (NCT + 3) / 4; ++r) {
            const int ct = wave + 4 * r;
            if (ct >= NCT) break;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < DK / 16; ++u) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(phi + (size_t)(16 * ct + i) * DK + 16 * u + 4 * g);
                const f32x4 b = *reinterpret_cast<const f32x4*>(ST + i * LDT + 16 * u + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float* dst = bp + (size_t)(16 * ct + 4 * g + e) * DV + c0 + i;
                acc[e] += *dst;
                *dst = acc[e];
            }
            cur[r] = acc;
        }
        __syncthreads();   // every read of ST for step p is done
#pragma unroll
        for (int r = 0; r < (NCT + 3) / 4; ++r) {
            const int ct = wave + 4 * r;
            if (ct >= NCT) break;
            *reinterpret_cast<f32x4*>(ST + i * LDT + 16 * ct + 4 * g) = cur[r];
        }
    }
    if (final_state != nullptr) {
        __syncthreads();
        for (int x = tid; x < DK * 16; x += 256) {
            const int m = x >> 4, j = x & 15;
            final_state[(size_t)h * slab + (size_t)m * DV + c0 + j] = ST[j * LDT + m];
        }
    }
}

// ---------------------------------------------------------------------------
// Correction.  The tokens of segments p >= 1 of every head, in (segment, head,
// token) order, are cut into one contiguous range per workgroup (8 waves), and
// the grid holds two workgroups per CU, so that the device is filled once and
// no partial last round is left.  A range is walked in pieces, one per
// (segment, head) it crosses; a wave takes 16 tokens of each 128-token
// sub-block of a piece.  The state that segment p starts from, S = ends[p - 1],
// is staged transposed in LDS (ST[j][m] = S[m][j]) once per (segment, head): a
// thread takes one column j and 8 (or 4) consecutive rows m, so the global
// reads are coalesced over j and each LDS write is one 16-byte row piece
// (conflict-free at that width).  The
// product is formed as D = ST * QT^T, so a lane (n = l % 16, g = l / 16) ends
// with the correction of token n for the four consecutive value columns
// 16 ct + 4 g + e, which is also the layout of its 8- or 16-byte read-modify-
// write of o.  The o words are loaded beside the qt operands, before the
// products, so both loads are in flight together.
// ---------------------------------------------------------------------------
constexpr int kCorrTok = 128;        // tokens of one sub-block (8 waves x 16)
constexpr int kCorrThreads = 512;

template <typename T, int DK, int DV> struct CorrOps;

template <int DK, int DV> struct CorrOps<uint16_t, DK, DV> {
    static constexpr int LDT = DK + 8;     // bf16 row stride (16-byte aligned rows)
    static constexpr int LDS_BYTES = 2 * DV * LDT * 2;
    typedef u32x2 OW;                      // o words of 4 bf16 outputs
    static __device__ void stage(unsigned char* smem, const float* S, int tid) {
        uint16_t* hi = reinterpret_cast<uint16_t*>(smem);
        uint16_t* lo = hi + DV * LDT;
        const int j = tid % DV;
        for (int m0 = 8 * (tid / DV); m0 < DK; m0 += 8 * (kCorrThreads / DV)) {
            uint32_t wh[4], wl[4];
#pragma unroll
            for (int r = 0; r < 8; r += 2) {
                const float s0 = S[(size_t)(m0 + r) * DV + j], s1 = S[(size_t)(m0 + r + 1) * DV + j];
                const uint32_t h = pack_bf16x2(s0, s1);
                wh[r / 2] = h;
                wl[r / 2] = pack_bf16x2(s0 - bf16_lo(h), s1 - bf16_hi(h));
            }
            *reinterpret_cast<u32x4*>(hi + j * LDT + m0) = u32x4{wh[0], wh[1], wh[2], wh[3]};
            *reinterpret_cast<u32x4*>(lo + j * LDT + m0) = u32x4{wl[0], wl[1], wl[2], wl[3]};
        }
    }
    typedef u32x4 QW[DK / 32];            // qt words of one token (B operands)
    static __device__ void load_q(QW& qw, Rsrc rq, uint32_t qoff) {
        const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) qw[s] = buf_ld128(rq, qoff + 2 * (32 * s + 8 * g));
    }
    static __device__ void product(const unsigned char* smem, const QW& qw, f32x4 (&acc)[DV / 16]) {
        const uint16_t* hi = reinterpret_cast<const uint16_t*>(smem);
        const uint16_t* lo = hi + DV * LDT;
        const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            const bf16x8 b = __builtin_bit_cast(bf16x8, qw[s]);
#pragma unroll
            for (int ct = 0; ct < DV / 16; ++ct) {
                const bf16x8 ah = *reinterpret_cast<const bf16x8*>(hi + (16 * ct + i) * LDT + 32 * s + 8 * g);
                const bf16x8 al = *reinterpret_cast<const bf16x8*>(lo + (16 * ct + i) * LDT + 32 * s + 8 * g);
                acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, acc[ct], 0, 0, 0);
                acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, acc[ct], 0, 0, 0);
            }
        }
    }
    static __device__ OW load_o(Rsrc ro, uint32_t off) { return buf_ld64(ro, off); }
    static __device__ void store_o(Rsrc ro, uint32_t off, OW w, f32x4 c) {
        const f32x4 y = {bf16_lo(w[0]) + c[0], bf16_hi(w[0]) + c[1], bf16_lo(w[1]) + c[2], bf16_hi(w[1]) + c[3]};
        buf_st64(u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])}, ro, off);
    }
};

template <int DK, int DV> struct CorrOps<float, DK, DV> {
    static constexpr int LDT = DK + 4;
    static constexpr int LDS_BYTES = DV * LDT * 4;
    typedef u32x4 OW;
    static __device__ void stage(unsigned char* smem, const float* S, int tid) {
        float* st = reinterpret_cast<float*>(smem);
        const int j = tid % DV;
        for (int m0 = 4 * (tid / DV); m0 < DK; m0 += 4 * (kCorrThreads / DV)) {
            f32x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = S[(size_t)(m0 + r) * DV + j];
            *reinterpret_cast<f32x4*>(st + j * LDT + m0) = x;
        }
    }
    typedef u32x4 QW[DK / 16];
    static __device__ void load_q(QW& qw, Rsrc rq, uint32_t qoff) {
        const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
        for (int u = 0; u < DK / 16; ++u) qw[u] = buf_ld128(rq, qoff + 4 * (16 * u + 4 * g));
    }
    static __device__ void product(const unsigned char* smem, const QW& qw, f32x4 (&acc)[DV / 16]) {
        const float* st = reinterpret_cast<const float*>(smem);
        const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
#pragma unroll
        for (int u = 0; u < DK / 16; ++u) {
#pragma unroll
            for (int ct = 0; ct < DV / 16; ++ct) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(st + (16 * ct + i) * LDT + 16 * u + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], __uint_as_float(qw[u][e]), acc[ct], 0, 0, 0);
            }
        }
    }
    static __device__ OW load_o(Rsrc ro, uint32_t off) { return buf_ld128(ro, off); }
    static __device__ void store_o(Rsrc ro, uint32_t off, OW w, f32x4 c) {
        const f32x4 y = {__uint_as_float(w[0]) + c[0], __uint_as_float(w[1]) + c[1], __uint_as_float(w[2]) + c[2],
                         __uint_as_float(w[3]) + c[3]};
        buf_st128(__builtin_bit_cast(u32x4, y), ro, off);
    }
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kCorrThreads) void split_correct_kernel(const float* __restrict__ ends,
                                                                     const T* __restrict__ qt, T* __restrict__ o,
                                                                     int64_t total_T, int H, int64_t seg_len,
                                                                     int segments, int64_t per_wg, int64_t piece_cap) {
    using CO = CorrOps<T, DK, DV>;
    static_assert(kCorrThreads % DV == 0, "staging");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];   // CO::LDS_BYTES
    // Segments 1 .. P - 2 hold seg_len tokens each, the last one last_len.
    const int64_t last_len = total_T - (int64_t)(segments - 1) * seg_len;
    const int64_t full = (int64_t)(segments - 2) * H * seg_len;
    const int64_t total = full + (int64_t)H * last_len;
    int64_t f = (int64_t)blockIdx.x * per_wg;
    const int64_t f_end = f + per_wg < total ? f + per_wg : total;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = lane & 15, g = lane >> 4;
    int64_t staged = -1;                     // (segment - 1) * H + head of the staged state
    while (f < f_end) {
        int64_t pair, t_in, len;
        if (f < full) {
            pair = f / seg_len;
            t_in = f - pair * seg_len;
            len = seg_len;
        } else {
            const int64_t r = (f - full) / last_len;
            pair = (int64_t)(segments - 2) * H + r;
            t_in = f - full - r * last_len;
            len = last_len;
        }
        const int p = 1 + (int)(pair / H), h = (int)(pair % H);
        int64_t n = len - t_in < f_end - f ? len - t_in : f_end - f;
        n = n < piece_cap ? n : piece_cap;
        if (pair != staged) {
            __syncthreads();                 // the previous piece is done with the staged state
            CO::stage(smem, ends + ((size_t)(p - 1) * H + h) * DK * DV, tid);
            __syncthreads();
            staged = pair;
        }
        const int64_t t_begin = (int64_t)p * seg_len + t_in, t_end = t_begin + n;
        // Row ranges: tokens t_begin .. t_end - 1 of this head.  Rows past t_end
        // read as zero and their stores are dropped.
        const uint32_t rows = (uint32_t)(t_end - t_begin - 1) * (uint32_t)H + 1u;
        const Rsrc rq = make_rsrc(qt + ((t_begin - seg_len) * H + h) * DK, rows * DK * (uint32_t)sizeof(T));
        const Rsrc ro = make_rsrc(o + (t_begin * H + h) * DV, rows * DV * (uint32_t)sizeof(T));
        for (int64_t t0 = 0; t0 < n; t0 += 16 * (kCorrThreads / 64)) {
            const uint32_t tok = (uint32_t)(t0 + 16 * wave + i);   // this lane's token (operand row)
            const uint32_t orow = tok * (uint32_t)H * DV;
            typename CO::QW qw;
            CO::load_q(qw, rq, tok * (uint32_t)H * DK * (uint32_t)sizeof(T));
            typename CO::OW ow[DV / 16];
#pragma unroll
            for (int ct = 0; ct < DV / 16; ++ct) ow[ct] = CO::load_o(ro, (orow + 16 * ct + 4 * g) * (uint32_t)sizeof(T));
            // The staged operands are read again for every sub-block rather than
            // held in registers, which keeps room for more waves per SIMD.
            __asm__ volatile("" ::: "memory");
            f32x4 acc[DV / 16];
#pragma unroll
            for (int ct = 0; ct < DV / 16; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            CO::product(smem, qw, acc);
#pragma unroll
            for (int ct = 0; ct < DV / 16; ++ct)
                CO::store_o(ro, (orow + 16 * ct + 4 * g) * (uint32_t)sizeof(T), ow[ct], acc[ct]);
        }
        f += n;
    }
}

template <int DK, int DV>
hipError_t scan_t(const PrefillArgs& a, const SplitWork& w) {
    const int blocks = a.H * (DV / 16);
    hipLaunchKernelGGL((split_scan_kernel<DK, DV>), dim3(blocks), dim3(256), 0, a.stream, w.ends, w.phis,
                       a.final_state, w.segments, a.H);
    return hipGetLastError();
}

// Workgroups of the correction: two per CU (their LDS fits twice), each with
// a whole number of 128-token sub-blocks, unless there are fewer.
template <typename T, int DK, int DV>
hipError_t correct_t(const PrefillArgs& a, const SplitWork& w) {
    const int64_t last_len = a.total_T - (int64_t)(w.segments - 1) * w.seg_len;
    const int64_t total = (int64_t)(w.segments - 2) * a.H * w.seg_len + (int64_t)a.H * last_len;
    if (w.segments < 2 || total <= 0) return hipSuccess;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int64_t units = (total + kCorrTok - 1) / kCorrTok;              // 128-token sub-blocks
    const int64_t want = 2 * (int64_t)(cus > 0 ? cus : 1);
    const int64_t per_wg = kCorrTok * ((units + want - 1) / want);
    const int64_t blocks = (total + per_wg - 1) / per_wg;
    // Pieces short enough for the 32-bit buffer offsets of one (segment, head):
    // at least 512 tokens, since the host checks 512 H max(d_k, d_v) bytes < 2^32.
    const int64_t row_bytes = (int64_t)a.H * (DK > DV ? DK : DV) * (int64_t)sizeof(T);
    const int64_t piece_cap = kCorrTok * ((((int64_t)1 << 31) / row_bytes) / kCorrTok);
    if (piece_cap < kCorrTok) return hipErrorInvalidValue;
    auto kern = split_correct_kernel<T, DK, DV>;
    constexpr int lds = CorrOps<T, DK, DV>::LDS_BYTES;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kCorrThreads), lds, a.stream,
                       w.ends, (const T*)w.qt, (T*)a.o, a.total_T, a.H, w.seg_len, w.segments, per_wg, piece_cap);
    return hipGetLastError();
}

}  // namespace

// Scratch of the allocation-free split entry point: the segment end states,
// transitions and Phi_t^T q_t rows of one call, in device memory that the code
// object holds (each device that loads the library holds its own copy until the
// process ends).  Host code never uses the array's name as an address: the
// device address is looked up once per device with hipGetSymbolAddress.
constexpr size_t kSplitScratchBytes = KDA_SPLIT_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kSplitScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];
}  // namespace

size_t split_scratch_bytes() { return kSplitScratchBytes; }

hipError_t split_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));    // with this device current
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_split_scan(const PrefillArgs& a, const SplitWork& w) {
    if (a.d_k == 128) return a.d_v == 128 ? scan_t<128, 128>(a, w) : scan_t<128, 64>(a, w);
    return a.d_v == 128 ? scan_t<64, 128>(a, w) : scan_t<64, 64>(a, w);
}

hipError_t launch_split_correct(const PrefillArgs& a, const SplitWork& w) {
    if (a.bf16) {
        if (a.d_k == 128) return a.d_v == 128 ? correct_t<uint16_t, 128, 128>(a, w) : correct_t<uint16_t, 128, 64>(a, w);
        return a.d_v == 128 ? correct_t<uint16_t, 64, 128>(a, w) : correct_t<uint16_t, 64, 64>(a, w);
    }
    if (a.d_k == 128) return a.d_v == 128 ? correct_t<float, 128, 128>(a, w) : correct_t<float, 128, 64>(a, w);
    return a.d_v == 128 ? correct_t<float, 64, 128>(a, w) : correct_t<float, 64, 64>(a, w);
}

}  // namespace kda

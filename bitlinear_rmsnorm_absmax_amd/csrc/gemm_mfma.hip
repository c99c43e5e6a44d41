// Prefill GEMM on int8 MFMA (M >= 64 tokens, MFMA-bound at large M).
//
// Same arithmetic as the skinny kernel (unite.ai BitNet.cpp article, 3.
// BitLinear-Betrieb): int8 MFMA on the 2-bit codes c = w + 1, and
// acc = D - S_m with S_m the sum of the token's int8 activations, accumulated
// from the staged activation chunks while they pass through registers.
// The instruction is v_mfma_i32_32x32x32_i8, which on gfx950 retires twice the
// int8 operations per cycle of the 16x16x64 form.
//
// Tiling: a workgroup of WM x WN waves computes a BM x BN output tile, each
// wave a 64 x 64 sub-tile (2 x 2 MFMA tiles of 32 x 32), walking K in steps
// of BK = 128.
// Each step's activation tile (BM rows x 128 bytes) and packed weight tile
// (BN columns x 8 words) are staged in LDS, double buffered.  Global loads
// run two steps ahead through two register sets (the K loop is unrolled by
// two so the sets keep fixed registers): while step k is multiplied, step k+1
// sits in registers waiting for its LDS buffer and step k+2 is in flight.
// Two waves share each SIMD, so one wave's LDS and memory waits are covered
// by the other's MFMAs.
//
// K-slot assignment: a 32x32x32 MFMA takes 16 K values per lane, lanes
// 0-31 and 32-63 covering two K blocks.  Inside a step, MFMA kk (0..3) of lane
// half h (lane/32) covers packed word 4h + kk, i.e. activation bytes
// [64h + 16kk, +16).  So a lane reads the four weight words of a column it
// needs for the whole step with one 16-byte LDS load.  A weight word is
// unpacked once per wave (shift + mask, four dwords of codes) and feeds the
// wave's two M tiles.
//
// LDS layout: activation rows of 128 bytes whose 16-byte chunks are
// XOR-swizzled with (row & 7) ^ ((row >> 3) & 1), so the 16 rows read by one
// operand fetch cover distinct banks; weight columns of 32 bytes whose two
// 16-byte halves swap for columns with bit 3 set, for the same reason.
// Output layout of a 32x32 tile: lane l holds column l % 32 and, in register
// v, row 8*(v/4) + 4*(l/32) + v%4.
//
// Both operands are re-read by many workgroups (activations by every column
// tile, weights by every row tile), so their loads keep the default cache
// policy and are served from L2 after the first touch.  Blocks are
// renumbered so that each XCD (blocks are dealt round-robin to the 8 XCDs)
// works on a contiguous range of output tiles, which share activation rows in
// that XCD's L2.
//
// Interior tiles (all rows < M, all columns < N, K a multiple of 128) take a
// plain load path; edge tiles clamp addresses and zero-fill what lies outside.
#include "device_common.h"
#include "internal.h"
#include "mfma_epilogue.h"

namespace bl {
namespace {

constexpr int BK = 128;
constexpr int kChunks = BK / 16;  // 16-byte activation chunks per tile row
constexpr int kWords = BK / 16;   // packed words per tile column
constexpr int kXcds = 8;
constexpr int TM = 2, TN = 2;     // 32x32 MFMA tiles per wave (64 x 64)

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// 16-byte half (0, 1) of weight column `col` holding logical words 4h .. 4h+3
__device__ __forceinline__ int bswz(int col, int h) { return h ^ ((col >> 3) & 1); }

template <int WM, int WN>
struct Cfg {
    static constexpr int kThreads = WM * WN * kWave;
    static constexpr int BM = WM * TM * 32;
    static constexpr int BN = WN * TN * 32;
    static constexpr int AP = BM * kChunks / kThreads;  // 16-byte A chunks per thread
    static constexpr int BE = BN * 32 / kThreads;        // weight bytes per thread per step
    static_assert(BM * kChunks % kThreads == 0, "A staging must divide evenly");
    static_assert(BE == 8 || BE == 16, "weight staging is 8 or 16 bytes per thread");
};

typedef unsigned v2u __attribute__((ext_vector_type(2)));

template <int WM, int WN>
struct Stage {
    v4i a[Cfg<WM, WN>::AP];
    v4u b;  // BE bytes used
};

// Every thread issues the same loads every step (no branches around loads),
// so the compiler can count outstanding loads exactly and only waits for the
// register set it is about to store.  Edge tiles clamp addresses into the
// matrix and zero what lies outside with a select.
template <int WM, int WN, bool EDGE>
__device__ __forceinline__ void load_step(Stage<WM, WN>& st, const int8_t* __restrict__ xq,
                                          const uint32_t* __restrict__ wp, int M, int K, int N,
                                          int WR, bool aligned, int m0, int n0, int kt, int tid) {
    using C = Cfg<WM, WN>;
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < C::AP; ++i) {
        const int idx = tid + C::kThreads * i;
        const int row = m0 + idx / kChunks;
        const int kk = k0 + 16 * (idx % kChunks);
        if (!EDGE) {
            st.a[i] = *reinterpret_cast<const v4i*>(xq + (int64_t)row * K + kk);
        } else {
            const bool ok = row < M && kk < K;
            const v4i v = *reinterpret_cast<const v4i*>(xq + (int64_t)min(row, M - 1) * K + min(kk, K - 16));
            st.a[i] = ok ? v : v4i{0, 0, 0, 0};
        }
    }
    // weight bytes [tid*BE, +BE) of the step's BN x 32-byte tile
    const int off = tid * C::BE;
    const int col = n0 + off / 32;
    const int w0 = kt * kWords + (off % 32) / 4;  // first logical word
    constexpr int NW = C::BE / 4;
    if (!EDGE) {
        const uint32_t* p = wp + (int64_t)col * WR + w0;
        if constexpr (NW == 4) {
            st.b = *reinterpret_cast<const v4u*>(p);
        } else {
            const v2u t = *reinterpret_cast<const v2u*>(p);
            st.b = v4u{t.x, t.y, 0u, 0u};
        }
    } else {
        const uint32_t* p = wp + (int64_t)min(col, N - 1) * WR;
        uint32_t t[4] = {0u, 0u, 0u, 0u};
        if (aligned) {
            // whole 8/16-byte group inside the row or wholly past its end
            const int wc = min(w0, WR - NW);
            if constexpr (NW == 4) {
                const v4u v = *reinterpret_cast<const v4u*>(p + wc);
                t[0] = v.x; t[1] = v.y; t[2] = v.z; t[3] = v.w;
            } else {
                const v2u v = *reinterpret_cast<const v2u*>(p + wc);
                t[0] = v.x; t[1] = v.y;
            }
            const bool ok = col < N && w0 < WR;
#pragma unroll
            for (int s = 0; s < NW; ++s) t[s] = ok ? t[s] : 0u;
        } else {
#pragma unroll
            for (int s = 0; s < NW; ++s) {
                const uint32_t v = p[min(w0 + s, WR - 1)];
                t[s] = (col < N && w0 + s < WR) ? v : 0u;
            }
        }
        st.b = v4u{t[0], t[1], t[2], t[3]};
    }
}

template <int WM, int WN>
__device__ __forceinline__ void store_step(const Stage<WM, WN>& st, v4i* As, v4u* Bs, int tid,
                                           int (&s_acc)[Cfg<WM, WN>::AP]) {
    using C = Cfg<WM, WN>;
#pragma unroll
    for (int i = 0; i < C::AP; ++i) {
        const int idx = tid + C::kThreads * i;
        const int r = idx / kChunks;
        As[r * kChunks + ((idx % kChunks) ^ swz(r))] = st.a[i];
        s_acc[i] = byte_sum16(st.a[i], s_acc[i]);
    }
    const int off = tid * C::BE;
    const int col = off / 32;
    const int half = (off % 32) / 16;
    uint32_t* dst = reinterpret_cast<uint32_t*>(Bs + col * 2 + bswz(col, half)) + (off % 16) / 4;
    if constexpr (C::BE == 16)
        *reinterpret_cast<v4u*>(dst) = st.b;
    else
        *reinterpret_cast<v2u*>(dst) = v2u{st.b.x, st.b.y};
}


__device__ __forceinline__ void mma_step(const v4i* As, const v4u* Bs, v16i (&acc)[TM][TN],
                                         int wm, int wn, int l32, int h) {
    // weight words 4h .. 4h+3 of each column: one 16-byte read, four MFMA steps
    v4u wq[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const int col = wn * TN * 32 + 32 * t + l32;
        wq[t] = Bs[col * 2 + bswz(col, h)];
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        v4i bf[TN];
#pragma unroll
        for (int t = 0; t < TN; ++t) bf[t] = unpack_codes(wq[t][kk]);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm * TM * 32 + 32 * i + l32;
            const v4i a = As[r * kChunks + ((4 * h + kk) ^ swz(r))];
#pragma unroll
            for (int t = 0; t < TN; ++t)
                acc[i][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bf[t], acc[i][t], 0, 0, 0);
        }
    }
}

template <int WM, int WN, bool EDGE>
__device__ __forceinline__ void gemm_tile(const int8_t* __restrict__ xq,
                                          const float* __restrict__ gamma, int M, int K,
                                          const uint32_t* __restrict__ wp, int N, float beta,
                                          float* __restrict__ y, int32_t* __restrict__ acc_out,
                                          int m0, int n0, v4i (*As)[Cfg<WM, WN>::BM * kChunks],
                                          v4u (*Bs)[Cfg<WM, WN>::BN * 2]) {
    using C = Cfg<WM, WN>;
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = tid / kWave;
    const int wm = wv / WN, wn = wv % WN;
    const int l32 = lane & 31, h = lane >> 5;
    const int WR = K >> 4;
    const bool aligned = (WR & 3) == 0;
    const int KT = (K + BK - 1) / BK;

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[i][t] = v16i{};
    int s_acc[C::AP];
#pragma unroll
    for (int i = 0; i < C::AP; ++i) s_acc[i] = 0;

    Stage<WM, WN> s0, s1;
    const int last = KT - 1;
    load_step<WM, WN, EDGE>(s0, xq, wp, M, K, N, WR, aligned, m0, n0, 0, tid);
    load_step<WM, WN, EDGE>(s1, xq, wp, M, K, N, WR, aligned, m0, n0, min(1, last), tid);
    store_step<WM, WN>(s0, As[0], Bs[0], tid, s_acc);
    __syncthreads();

    // at the top of step kt: LDS buffer kt&1 holds step kt and the other
    // register set holds step kt+1 (in flight or landed).  Loads past the
    // last step re-read the last step and are never stored.
    for (int kt = 0; kt < KT; kt += 2) {
        // even step kt: LDS buffer 0; s1 holds step kt+1; s0 is free
        load_step<WM, WN, EDGE>(s0, xq, wp, M, K, N, WR, aligned, m0, n0, min(kt + 2, last), tid);
        __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before the MFMAs
        mma_step(As[0], Bs[0], acc, wm, wn, l32, h);
        if (kt + 1 < KT) store_step<WM, WN>(s1, As[1], Bs[1], tid, s_acc);
        __syncthreads();
        if (kt + 1 >= KT) break;
        // odd step kt+1: LDS buffer 1; s0 holds step kt+2; s1 is free
        load_step<WM, WN, EDGE>(s1, xq, wp, M, K, N, WR, aligned, m0, n0, min(kt + 3, last), tid);
        __builtin_amdgcn_sched_barrier(0);
        mma_step(As[1], Bs[1], acc, wm, wn, l32, h);
        if (kt + 2 < KT) store_step<WM, WN>(s0, As[0], Bs[0], tid, s_acc);
        __syncthreads();
    }

    // row sums: the 8 threads staging one tile row are consecutive lanes.
    // The A buffers are free now, so the sums and scales reuse them.
    int* Ssum = reinterpret_cast<int*>(&As[0][0]);
    float* Ssc = reinterpret_cast<float*>(&As[1][0]);
#pragma unroll
    for (int i = 0; i < C::AP; ++i) {
        int sv = s_acc[i];
        sv += __shfl_xor(sv, 1, kWave);
        sv += __shfl_xor(sv, 2, kWave);
        sv += __shfl_xor(sv, 4, kWave);
        const int idx = tid + C::kThreads * i;
        if ((idx % kChunks) == 0) Ssum[idx / kChunks] = sv;
    }
    for (int r = tid; r < C::BM; r += C::kThreads) {
        const int row = m0 + r;
        Ssc[r] = (!EDGE || row < M) ? out_scale(beta, gamma[row]) : 0.f;
    }
    __syncthreads();

    store_tiles<TM, TN>(acc, Ssum, Ssc, wm * TM * 32, wn * TN * 32, m0, n0, M, N, y, acc_out, lane);
}

template <int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_mfma_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ gamma, int M, int K,
    const uint32_t* __restrict__ wp, int N, float beta, float* __restrict__ y,
    int32_t* __restrict__ acc_out, int tiles_n, int tiles_total) {
    using C = Cfg<WM, WN>;
    __shared__ v4i As[2][C::BM * kChunks];
    __shared__ v4u Bs[2][C::BN * 2];

    // XCD-aware renumbering of the linear block id
    int b = blockIdx.x;
    const int full = (tiles_total / kXcds) * kXcds;
    if (b < full) b = (b % kXcds) * (full / kXcds) + b / kXcds;
    const int m0 = (b / tiles_n) * C::BM;
    const int n0 = (b % tiles_n) * C::BN;
    const bool interior = (m0 + C::BM <= M) && (n0 + C::BN <= N) && (K % BK == 0);
    if (interior)
        gemm_tile<WM, WN, false>(xq, gamma, M, K, wp, N, beta, y, acc_out, m0, n0, As, Bs);
    else
        gemm_tile<WM, WN, true>(xq, gamma, M, K, wp, N, beta, y, acc_out, m0, n0, As, Bs);
}

template <int WM, int WN>
hipError_t launch_cfg(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                      int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    using C = Cfg<WM, WN>;
    const int tm = (M + C::BM - 1) / C::BM;
    const int tn = (N + C::BN - 1) / C::BN;
    const int64_t total = (int64_t)tm * tn;
    if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
    gemm_mfma_kernel<WM, WN><<<dim3((unsigned)total), dim3(C::kThreads), 0, s>>>(
        xq, gamma, M, K, wp, N, beta, y, acc, tn, (int)total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma(const int8_t* xq, const float* gamma, int M, int K,
                            const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                            hipStream_t s) {
    if (gemm_dma_supports(M, K, N)) return launch_gemm_dma(xq, gamma, M, K, wp, N, beta, y, acc, s);
    // Large problems: 256 x 128 tiles (8 waves); otherwise 128 x 128 tiles
    // (4 waves) for more workgroups.
    const int64_t big_tiles = (int64_t)((M + 255) / 256) * ((N + 127) / 128);
    if (M >= 256 && big_tiles >= 512) return launch_cfg<4, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    return launch_cfg<2, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

}  // namespace bl

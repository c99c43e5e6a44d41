// Decode product for a few tokens (5 <= M <= 16) on int8 MFMA, activations
// staged in LDS; 2-bit ternary weights, or 1-bit weights (ONEBIT).
//
// Arithmetic as in the other forward kernels (unite.ai BitNet.cpp article, 3.
// BitLinear-Betrieb; datacamp MatMul-free article): v_mfma_i32_16x16x64_i8 on
// the unsigned codes c = w + 1 (2-bit) or c = (w + 1) / 2 (1-bit), giving
// D = sum c q; then acc = D - S (2-bit) or 2 D - S (1-bit) with S the sum of
// the token's int8 activations over K, taken once per workgroup from LDS.
//
// Why LDS: at a handful of tokens the weights are read once from HBM while
// every workgroup needs all M activation rows.  Loading the activation
// operand per lane from global memory (16 rows x 16 bytes per instruction)
// floods the per-CU L1 with scattered requests and stalls the address unit,
// which then also delays the weight stream.  Here each workgroup copies the
// M x K activation block into LDS once, in 1 KB contiguous pieces straight
// from global memory (global_load_lds).
//
// Order (measured with per-wave timestamps: loads of a compute unit return
// in issue order, so copies queued behind weight misses wait for HBM):
//   1. every wave issues its activation copies; a barrier makes sure all
//      copies of the workgroup are queued before any weight load;
//   2. every wave issues the B weight loads of its first batch (unconditional,
//      clamped chunks, so their number is a constant), then waits until at
//      most B * NTW vector-memory operations are outstanding -- exactly its
//      own copies, which are older -- and a second barrier publishes the
//      activations;
//   3. the activation sums S (all threads, from LDS) while the weights are in
//      flight, then the MFMAs, each waiting only for its own weight registers.
// Chunks past a wave's range multiply all-zero codes.
//
// Work split: a workgroup of 8 waves owns CT column tiles of 16; a wave owns
// NTW of them and one of KS = 8 * NTW / CT contiguous K ranges (256-K
// chunks).  Partial sums of the KS waves of a tile meet in LDS.
//
// LDS layout of the activations: row r holds its K bytes as 16-byte pieces,
// piece p stored at slot p ^ (r & 15) of the row, so the 16 rows read by one
// operand fetch fall on different banks.  Requires K % 256 == 0.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kDecWaves = 8;
constexpr int kDecLdsMax = 160 * 1024;
typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base,
                                     16, 0, 0);
#endif
}

// s_waitcnt immediate (gfx9 encoding): vmcnt <= vm, lgkmcnt and expcnt any
constexpr int vm_wait_imm(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | (0xF << 8); }

// Nothing is moved across this point by the compiler, memory or arithmetic.
__device__ __forceinline__ void fence_code() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// ONEBIT: 1-bit weights ([N][K/32], entry 4j + b of a word at bit 8b + j):
// lane (j, g) loads words 8c + 2g, 8c + 2g + 1 of chunk c (the same 64 K
// positions as the 2-bit words 16c + 4g .. +3), and MFMA s takes bits
// 4(s%2) .. +3 of word s/2.
template <int CT, int NTW, int B, bool ONEBIT>
__global__ __launch_bounds__(kDecWaves * kWave) void decode_lds_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ gamma, int M, int K,
    const uint32_t* wp, int N, float beta, float* __restrict__ y, int32_t* __restrict__ acc_out,
    int a_bytes) {
    constexpr int CG = CT / NTW;         // column groups of a workgroup
    constexpr int KS = kDecWaves / CG;   // K ranges per column group
    typedef typename std::conditional<ONEBIT, v2u, v4u>::type wvec;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* As = smem;                                       // activations, a_bytes
    int* red = reinterpret_cast<int*>(smem + a_bytes);     // [8 waves][NTW][4][64]
    int* Ssum = red + kDecWaves * NTW * 4 * kWave;         // [16] activation sums

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int cg = wv % CG, kp = wv / CG;
    const int j = lane & 15, g = lane >> 4;
    const int WR = K >> 4;          // 16-byte pieces per activation row (= 2-bit words per row)
    const int WRW = ONEBIT ? (K >> 5) : WR;  // weight words per row
    const int nchunks = K >> 8;
    const int n_base = blockIdx.x * (16 * CT) + cg * 16 * NTW;

    const int cpw = (nchunks + KS - 1) / KS;
    const int c_begin = kp * cpw;
    const int c_end = min(c_begin + cpw, nchunks);
    const int last = max(min(c_end, nchunks) - 1, 0);

    v4i acc[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[t] = v4i{0, 0, 0, 0};
    // lane (j, g): column j of each tile, packed words 16c + 4g .. +3 of chunk c;
    // columns past N are clamped onto the last one (never stored)
    const uint32_t* wrow[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t)
        wrow[t] = wp + (int64_t)min(n_base + 16 * t + j, N - 1) * WRW + (ONEBIT ? 2 : 4) * g;
    // A-operand row of lane j; rows past M repeat row M-1 (never stored)
    const int arow = min(j, M - 1);
    const char* arow_p = As + arow * K;
    const int axor = arow & 15;

    auto load_batch = [&](int cb, wvec (&bw)[B][NTW]) {
#pragma unroll
        for (int i = 0; i < B; ++i)
#pragma unroll
            for (int t = 0; t < NTW; ++t)
                bw[i][t] = __builtin_nontemporal_load(reinterpret_cast<const wvec*>(
                    wrow[t] + (ONEBIT ? 8 : 16) * min(cb + i, last)));
    };
    auto mul_batch = [&](int cb, const wvec (&bw)[B][NTW]) {
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const bool live = cb + i < c_end;
            const int c = min(cb + i, last);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int p = 16 * c + 4 * g + s;
                const v4i a = *reinterpret_cast<const v4i*>(arow_p + 16 * (p ^ axor));
#pragma unroll
                for (int t = 0; t < NTW; ++t) {
                    v4i b;
                    if constexpr (ONEBIT) {
                        const uint32_t w = live ? bw[i][t][s >> 1] : 0u;
                        const int j0 = 4 * (s & 1);
                        b = v4i{(int)((w >> j0) & 0x01010101u), (int)((w >> (j0 + 1)) & 0x01010101u),
                                (int)((w >> (j0 + 2)) & 0x01010101u), (int)((w >> (j0 + 3)) & 0x01010101u)};
                    } else {
                        b = unpack_codes(live ? bw[i][t][s] : 0u);
                    }
                    acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[t], 0, 0, 0);
                }
            }
        }
    };

    // 1. activation copies of the whole workgroup, queued ahead of any weight load
    {
        const int pieces = M * WR;
        const int ninstr = (pieces + 63) >> 6;
        for (int q = wv; q < ninstr; q += kDecWaves) {
            const int pos = min(q * 64 + lane, pieces - 1);
            const int r = pos / WR, slot = pos - r * WR;
            copy16_to_lds(xq + (int64_t)r * K + 16 * (slot ^ (r & 15)), As + 1024 * q);
        }
    }
    fence_code();
    __builtin_amdgcn_s_barrier();
    fence_code();

    // 2. the first batch of weight loads stays in flight across the barrier
    //    that publishes the activations; 3. activation sums while it lands
    auto publish = [&]() {
        fence_code();
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(B * NTW));  // own copies (older) have landed
        __builtin_amdgcn_s_barrier();
        fence_code();
        // row r = tid / 32, 32 threads per row, whole rows (the slot order
        // inside a row does not change a sum)
        const int r = tid >> 5, part = tid & 31;
        int sum = 0;
        if (r < M)
            for (int q = part; q < WR; q += 32)
                sum = byte_sum16(*reinterpret_cast<const v4i*>(As + r * K + 16 * q), sum);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
        if (part == 0) Ssum[r] = sum;
    };
    if (c_end - c_begin <= B) {
        // one batch
        wvec bw[B][NTW];
        load_batch(c_begin, bw);
        publish();
        mul_batch(c_begin, bw);
    } else {
        // a stream of batches, the next one's loads issued before the current
        // one is multiplied (a wave keeps at most 2 B NTW loads in flight, so
        // load issue does not stall on the compute unit's outstanding-request
        // limit); the loads past the range re-read the last chunk
        wvec b0[B][NTW], b1[B][NTW];
        load_batch(c_begin, b0);
        publish();
        for (int cb = c_begin;;) {
            load_batch(cb + B, b1);
            mul_batch(cb, b0);
            cb += B;
            if (cb >= c_end) break;
            load_batch(cb + B, b0);
            mul_batch(cb, b1);
            cb += B;
            if (cb >= c_end) break;
        }
    }

    // lane (j, g) holds rows 4g + v of column j
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((wv * NTW + t) * 4 + v) * kWave + lane] = acc[t][v];
    __syncthreads();
    if (kp == 0) {
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
            const int col = n_base + 16 * t + j;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 4 * g + v;
                int d = 0;
                for (int k2 = 0; k2 < KS; ++k2)
                    d += red[(((k2 * CG + cg) * NTW + t) * 4 + v) * kWave + lane];
                if (row < M && col < N) {
                    const int a = (ONEBIT ? 2 * d : d) - Ssum[row];
                    const int64_t o = (int64_t)row * N + col;
                    if (y) y[o] = (float)a * out_scale(beta, gamma[row]);
                    if (acc_out) acc_out[o] = a;
                }
            }
        }
    }
}

// LDS bytes: the activation block rounded up to whole 1 KB copies, the
// reduction buffer and the 16 activation sums.
int decode_a_bytes(int M, int K) { return ((M * K + 1023) / 1024) * 1024; }
size_t decode_lds_bytes(int M, int K, int ntw) {
    return (size_t)decode_a_bytes(M, K) + (size_t)kDecWaves * ntw * 4 * kWave * 4 + 16 * 4;
}

template <int CT, int NTW, int B, bool ONEBIT>
hipError_t launch_ctb(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp, int N,
                      float beta, float* y, int32_t* acc, hipStream_t s) {
    static bool attr_set = false;  // per-kernel opt-in to more than 64 KB of dynamic LDS
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&decode_lds_kernel<CT, NTW, B, ONEBIT>),
            hipFuncAttributeMaxDynamicSharedMemorySize, kDecLdsMax);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int blocks = (N + 16 * CT - 1) / (16 * CT);
    decode_lds_kernel<CT, NTW, B, ONEBIT><<<dim3(blocks), dim3(kDecWaves * kWave),
                                            decode_lds_bytes(M, K, NTW), s>>>(
        xq, gamma, M, K, wp, N, beta, y, acc, decode_a_bytes(M, K));
    return hipGetLastError();
}

// Batch: a wave's whole K range in one batch when it has at most 4 chunks,
// else a stream of 2-chunk batches (measured at K = 2560 .. 8192: larger
// batches stall load issue, a 2-chunk stream is 15 % faster at K = 8192).
template <int CT, int NTW, bool ONEBIT>
hipError_t launch_ct(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp, int N,
                     float beta, float* y, int32_t* acc, hipStream_t s) {
    constexpr int KS = kDecWaves * NTW / CT;
    const int cpw = ((K >> 8) + KS - 1) / KS;
    if (cpw <= 4) return launch_ctb<CT, NTW, 4, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    return launch_ctb<CT, NTW, 2, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

template <bool ONEBIT>
hipError_t launch_widths(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                         int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    // widest workgroup that still leaves >= 160 workgroups (measured on
    // N = 2560 .. 28672, K = 2560 .. 8192): fewer, wider groups copy the
    // activation block fewer times, too few leave CUs idle
    const int tiles = (N + 15) / 16;
    if (tiles >= 8 * 160) return launch_ct<8, 2, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    if (tiles >= 4 * 160) return launch_ct<4, 2, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    if (tiles >= 2 * 160) return launch_ct<2, 1, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    return launch_ct<1, 1, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

}  // namespace

bool decode_lds_supports(int M, int K, int N) {
    return M >= 1 && M <= 16 && K >= 256 && K % 256 == 0 && N > 0 &&
           decode_lds_bytes(M, K, 2) <= (size_t)kDecLdsMax;
}

hipError_t launch_decode_lds(const int8_t* xq, const float* gamma, int M, int K,
                             const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                             hipStream_t s) {
    return launch_widths<false>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

hipError_t launch_decode_lds1(const int8_t* xq, const float* gamma, int M, int K,
                              const uint32_t* wp1, int N, float beta, float* y, int32_t* acc,
                              hipStream_t s) {
    return launch_widths<true>(xq, gamma, M, K, wp1, N, beta, y, acc, s);
}

}  // namespace bl

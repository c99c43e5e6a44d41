// Decode product for a few tokens (5 <= M <= 16) on int8 MFMA, activations
// staged in LDS; 2-bit ternary weights, or 1-bit weights (ONEBIT).
//
// Arithmetic as in the skinny kernel (unite.ai BitNet.cpp article, 3.
// BitLinear-Betrieb; datacamp MatMul-free article): v_mfma_i32_16x16x64_i8 on
// the 2-bit codes c = w + 1, acc = D - S_m, S_m from one MFMA per K slot
// against an all-ones operand.
//
// Why LDS: at a handful of tokens the weights are read once from HBM while
// every workgroup needs all M activation rows.  Loading the activation
// operand per lane from global memory (16 rows x 16 bytes per instruction)
// floods the per-CU L1 with scattered requests and stalls the address unit,
// which then also delays the weight stream.  Here each workgroup copies the
// M x K activation block into LDS once, in 1 KB contiguous pieces straight
// from global memory (global_load_lds), and the waves read their operands
// from LDS.  The weight loads of a wave (16 bytes per lane, 16 columns x 64
// contiguous bytes per instruction) are all issued before the copies, so both
// streams are in flight together; one barrier publishes the activations.
//
// Work split: a workgroup of 8 waves owns CT column tiles of 16; a wave owns
// NTW of them and one of KS = 8 * NTW / CT contiguous K ranges (256-K
// chunks).  Partial sums of the KS waves of a tile meet in LDS.
//
// LDS layout of the activations: row r holds its K bytes as 16-byte pieces,
// piece p stored at slot p ^ (r & 15) of the row, so the 16 rows read by one
// operand fetch fall on different banks.  Requires K % 256 == 0.
#include "device_common.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kDecWaves = 8;
constexpr int kDecMaxBatch = 16;   // 256-K chunks whose weight loads a wave keeps in flight
constexpr int kDecLdsMax = 160 * 1024;
typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base,
                                     16, 0, 0);
#endif
}

// ONEBIT: 1-bit weights ([N][K/32], entry 4j + b of a word at bit 8b + j):
// lane (j, g) loads words 8c + 2g, 8c + 2g + 1 of chunk c (the same 64 K
// positions as the 2-bit words 16c + 4g .. +3), MFMA s takes bits 4(s%2) ..
// +3 of word s/2, and acc = 2 D - S.
template <int CT, int NTW, bool ONEBIT>
__global__ __launch_bounds__(kDecWaves * kWave) void decode_lds_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ gamma, int M, int K,
    const uint32_t* __restrict__ wp, int N, float beta, float* __restrict__ y,
    int32_t* __restrict__ acc_out, int a_bytes) {
    constexpr int CG = CT / NTW;         // column groups of a workgroup
    constexpr int KS = kDecWaves / CG;   // K ranges per column group
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* As = smem;                                       // activations, a_bytes
    int* red = reinterpret_cast<int*>(smem + a_bytes);     // [8 waves][NTW][4][64]

    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int cg = wv % CG, kp = wv / CG;
    const int j = lane & 15, g = lane >> 4;
    const int WR = K >> 4;          // 16-byte pieces per activation row (= 2-bit words per row)
    const int WRW = ONEBIT ? (K >> 5) : WR;  // weight words per row
    const int nchunks = K >> 8;
    const int n_base = blockIdx.x * (16 * CT) + cg * 16 * NTW;

    const int cpw = (nchunks + KS - 1) / KS;
    const int c_begin = kp * cpw;
    const int c_end = min(c_begin + cpw, nchunks);

    v4i acc[NTW], accS = v4i{0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[t] = v4i{0, 0, 0, 0};
    const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
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

    auto stage_activations = [&]() {
        const int pieces = M * WR;
        const int ninstr = (pieces + 63) >> 6;
        for (int q = wv; q < ninstr; q += kDecWaves) {
            const int pos = min(q * 64 + lane, pieces - 1);
            const int r = pos / WR, slot = pos - r * WR;
            copy16_to_lds(xq + (int64_t)r * K + 16 * (slot ^ (r & 15)), As + 1024 * q);
        }
    };

    bool staged = false;
    for (int cb = c_begin; cb < c_end; cb += kDecMaxBatch) {
        const int nb = min(kDecMaxBatch, c_end - cb);  // wave-uniform
        v4u bw[kDecMaxBatch][NTW];  // ONEBIT: .x, .y hold the two words
#pragma unroll
        for (int i = 0; i < kDecMaxBatch; ++i)
#pragma unroll
            for (int t = 0; t < NTW; ++t)
                if (i < nb) {
                    if constexpr (ONEBIT) {
                        const v2u w2 = __builtin_nontemporal_load(
                            reinterpret_cast<const v2u*>(wrow[t] + 8 * (cb + i)));
                        bw[i][t] = v4u{w2.x, w2.y, 0u, 0u};
                    } else {
                        bw[i][t] = __builtin_nontemporal_load(
                            reinterpret_cast<const v4u*>(wrow[t] + 16 * (cb + i)));
                    }
                }
        if (!staged) {
            stage_activations();
            __syncthreads();  // also waits for this wave's weight loads
            staged = true;
        }
#pragma unroll
        for (int i = 0; i < kDecMaxBatch; ++i) {
            if (i < nb) {
                const int c = cb + i;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int p = 16 * c + 4 * g + s;
                    const v4i a = *reinterpret_cast<const v4i*>(arow_p + 16 * (p ^ axor));
#pragma unroll
                    for (int t = 0; t < NTW; ++t) {
                        v4i b;
                        if constexpr (ONEBIT) {
                            const uint32_t w = bw[i][t][s >> 1];
                            const int j0 = 4 * (s & 1);
                            b = v4i{(int)((w >> j0) & 0x01010101u), (int)((w >> (j0 + 1)) & 0x01010101u),
                                    (int)((w >> (j0 + 2)) & 0x01010101u), (int)((w >> (j0 + 3)) & 0x01010101u)};
                        } else {
                            b = unpack_codes(bw[i][t][s]);
                        }
                        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[t], 0, 0, 0);
                    }
                    accS = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, ones, accS, 0, 0, 0);
                }
            }
        }
    }
    if (!staged) {  // a wave without chunks still copies its share and joins the barrier
        stage_activations();
        __syncthreads();
    }

    // lane (j, g) holds rows 4g + v of column j
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            red[((wv * NTW + t) * 4 + v) * kWave + lane] = (ONEBIT ? 2 * acc[t][v] : acc[t][v]) - accS[v];
    __syncthreads();
    if (kp == 0) {
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
            const int col = n_base + 16 * t + j;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 4 * g + v;
                int a = 0;
                for (int k2 = 0; k2 < KS; ++k2)
                    a += red[(((k2 * CG + cg) * NTW + t) * 4 + v) * kWave + lane];
                if (row < M && col < N) {
                    const int64_t o = (int64_t)row * N + col;
                    y[o] = (float)a * out_scale(beta, gamma[row]);
                    if (acc_out) acc_out[o] = a;
                }
            }
        }
    }
}

// LDS bytes: the activation block rounded up to whole 1 KB copies, plus the
// reduction buffer.
int decode_a_bytes(int M, int K) { return ((M * K + 1023) / 1024) * 1024; }
size_t decode_lds_bytes(int M, int K, int ntw) {
    return (size_t)decode_a_bytes(M, K) + (size_t)kDecWaves * ntw * 4 * kWave * 4;
}

template <int CT, int NTW, bool ONEBIT>
hipError_t launch_ct(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp, int N,
                     float beta, float* y, int32_t* acc, hipStream_t s) {
    static bool attr_set = false;  // per-kernel opt-in to more than 64 KB of dynamic LDS
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&decode_lds_kernel<CT, NTW, ONEBIT>),
            hipFuncAttributeMaxDynamicSharedMemorySize, kDecLdsMax);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int blocks = (N + 16 * CT - 1) / (16 * CT);
    decode_lds_kernel<CT, NTW, ONEBIT><<<dim3(blocks), dim3(kDecWaves * kWave),
                                         decode_lds_bytes(M, K, NTW), s>>>(
        xq, gamma, M, K, wp, N, beta, y, acc, decode_a_bytes(M, K));
    return hipGetLastError();
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

// 1-bit weights (unite.ai BitNet.cpp article, Mathematische Grundlagen,
// 1. Gewichtsbinarisierung: W_f = Sign(W - alpha), alpha the mean of the
// weights, Sign(v) = +1 for v > 0, else -1).
//
// 1-bit layout: word n*(K/32) + k/32 holds entry e = k mod 32 = 4j + b at bit
// 8b + j as (w + 1) / 2, so (word >> j) & 0x01010101 gives the bits of
// entries 4j .. 4j+3 in byte lanes 0 .. 3: one shift and one mask per four
// weights, the 2-bit layout's unpack at half the bytes.
//
// The product runs v_dot4_i32_i8 on the bits c in {0, 1}: w = 2c - 1, so
// acc = 2 * sum c q - sum q (ternary product of the BitNet.cpp article, 3.
// BitLinear-Betrieb, with the zero code unused).
#include "device_common.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kB1Threads = 256;
typedef unsigned v2u_t __attribute__((ext_vector_type(2)));

__global__ void zero_count_kernel(int* p) { *p = 0; }

// One thread per 1-bit word: 32 entries against alpha64, exact in double.
__global__ __launch_bounds__(kB1Threads) void binarize_pack1_kernel(const float* __restrict__ W,
                                                                   int64_t words,
                                                                   const double* __restrict__ alpha64,
                                                                   uint32_t* __restrict__ packed,
                                                                   int8_t* __restrict__ codes) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= words) return;
    const double a = alpha64[0];
    const v4f* src = reinterpret_cast<const v4f*>(W + 32 * i);
    uint32_t word = 0;
    uint32_t cw[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const v4f v = src[q];
        const float e4[4] = {v.x, v.y, v.z, v.w};
        uint32_t d = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = 4 * q + u;
            const uint32_t bit = ((double)e4[u] > a) ? 1u : 0u;
            word |= bit << (8 * (e & 3) + (e >> 2));
            d |= (bit ? 0x01u : 0xFFu) << (8 * u);  // int8 +1 / -1
        }
        cw[q] = d;
    }
    packed[i] = word;
    v4u* out = reinterpret_cast<v4u*>(codes + 32 * i);
    out[0] = v4u{cw[0], cw[1], cw[2], cw[3]};
    out[1] = v4u{cw[4], cw[5], cw[6], cw[7]};
}

// One thread per 1-bit word of +-1 int8 weights; other values count as bad
// (packed as 0 bits).
__global__ __launch_bounds__(kB1Threads) void pack1_kernel(const int8_t* __restrict__ w, int64_t words,
                                                          uint32_t* __restrict__ packed,
                                                          int* __restrict__ bad_count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int bad = 0;
    if (i < words) {
        const v4u* src = reinterpret_cast<const v4u*>(w + 32 * i);
        const v4u lo = src[0], hi = src[1];
        const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int v = (int)(int8_t)((d[q] >> (8 * u)) & 0xFF);
                const int e = 4 * q + u;
                if (v == 1) word |= 1u << (8 * (e & 3) + (e >> 2));
                else if (v != -1) ++bad;
            }
        packed[i] = word;
    }
    if (bad_count) {
        bad = wave_sum_i(bad);
        if ((threadIdx.x % kWave) == 0 && bad) atomicAdd(bad_count, bad);
    }
}

// Decode product on 1-bit weights (K % 64 == 0).  A wave owns R consecutive weight rows;
// lane l streams the 8-byte units (2 words = 64 weights) l, l+64, ... of each
// row (512 contiguous bytes per wave-wide load) and the 64 activation bytes
// of the same K range per token; MR tokens (rows m0 .. m0+MR-1 of x_q).
template <int MR, int R>
__global__ __launch_bounds__(kB1Threads) void gemv1_kernel(const int8_t* __restrict__ xq,
                                                           const float* __restrict__ gamma, int M,
                                                           int K, const uint32_t* __restrict__ wp,
                                                           int N, float beta, float* __restrict__ y,
                                                           int32_t* __restrict__ acc_out, int m0) {
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int n0 = (blockIdx.x * (kB1Threads / kWave) + wv) * R;
    const int WR = K >> 5;          // words per row
    const int units = WR >> 1;      // 8-byte units per row (K % 64 == 0)
    const uint32_t* wrow = wp + (int64_t)n0 * WR;

    int part[R][MR];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) part[r][m] = 0;
    int spart[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) spart[m] = 0;

    for (int u = lane; u < units; u += kWave) {
        uint32_t w[R][2];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = min(n0 + r, N - 1) - n0;  // rows past N re-read the last one
            const v2u_t v = *reinterpret_cast<const v2u_t*>(wrow + (int64_t)rr * WR + 2 * u);
            w[r][0] = v.x;
            w[r][1] = v.y;
        }
        v4i a[MR][4];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const int row = min(m0 + m, M - 1);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                a[m][s] = *reinterpret_cast<const v4i*>(xq + (int64_t)row * K + 64 * u + 16 * s);
                spart[m] = byte_sum16(a[m][s], spart[m]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // word h covers entries 32h .. 32h+31 of the unit: dword j of
                // its bits pairs with activation bytes 32h + 4j .. +3
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int c = (int)((w[r][h] >> j) & 0x01010101u);
                    const int s = 2 * h + (j >> 2), k = j & 3;
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        const int av = k == 0 ? a[m][s].x : k == 1 ? a[m][s].y : k == 2 ? a[m][s].z : a[m][s].w;
                        part[r][m] = __builtin_amdgcn_sdot4(c, av, part[r][m], false);
                    }
                }
            }
        }
    }

#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const int row = m0 + m;
        const float sc = (row < M) ? out_scale(beta, gamma[row]) : 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int tot = wave_sum_dpp(2 * part[r][m] - spart[m]);
            const int n = n0 + r;
            if (lane == 0 && n < N && row < M) {
                y[(int64_t)row * N + n] = (float)tot * sc;
                if (acc_out) acc_out[(int64_t)row * N + n] = tot;
            }
        }
    }
}

template <int MR>
hipError_t launch_gemv1(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp, int N,
                        float beta, float* y, int32_t* acc, int m0, hipStream_t s) {
    constexpr int R = 4;
    const int rows_per_block = (kB1Threads / kWave) * R;
    const int blocks = (N + rows_per_block - 1) / rows_per_block;
    gemv1_kernel<MR, R><<<dim3(blocks), dim3(kB1Threads), 0, s>>>(xq, gamma, M, K, wp, N, beta, y,
                                                                    acc, m0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_binarize(const float* W, int64_t N, int64_t K, uint32_t* packed1, int8_t* codes,
                           double* alpha64, float* alpha32, double* beta64, float* beta32,
                           hipStream_t s) {
    const int64_t L = N * K;
    // both partial-sum arrays live in the int8 code output (L bytes): alpha's
    // at its start, beta's from the middle; the codes are written last
    double* sa = reinterpret_cast<double*>(codes);
    double* sb = reinterpret_cast<double*>(codes + ((L / 2) & ~(int64_t)15));
    hipError_t e = launch_pairwise_mean(W, L, N, K, false, 256, sa, alpha64, alpha32, s);
    if (e != hipSuccess) return e;
    e = launch_pairwise_mean(W, L, N, K, true, 256, sb, beta64, beta32, s);
    if (e != hipSuccess || L == 0) return e;
    const int64_t words = L / 32;
    binarize_pack1_kernel<<<dim3((unsigned)((words + kB1Threads - 1) / kB1Threads)),
                            dim3(kB1Threads), 0, s>>>(W, words, alpha64, packed1, codes);
    return hipGetLastError();
}

hipError_t launch_pack1(const int8_t* w, int64_t N, int64_t K, uint32_t* packed1, int* bad_count,
                        hipStream_t s) {
    if (bad_count) {
        zero_count_kernel<<<1, 1, 0, s>>>(bad_count);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t words = N * (K / 32);
    if (words == 0) return hipSuccess;
    pack1_kernel<<<dim3((unsigned)((words + kB1Threads - 1) / kB1Threads)), dim3(kB1Threads), 0, s>>>(
        w, words, packed1, bad_count);
    return hipGetLastError();
}

hipError_t launch_forward1(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                           int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    // 5..16 tokens, and 2..4 tokens at K >= 4096 (as for 2-bit weights), with
    // K % 512 == 0 (its 1-bit loads take 512 inputs), and one token on long
    // rows over many row tiles: the LDS-staged MFMA decode kernel in its 1-bit
    // form
    if ((M >= 5 || (M >= 2 && K >= 4096) || (M == 1 && decode_one_token(K, N, true))) &&
        K % 512 == 0 && decode_lds_supports(M, K, N))
        return launch_decode_lds1(xq, gamma, M, K, wp, N, beta, y, acc, s);
    // else groups of up to four tokens on the vector ALUs, each a pass over the weights
    for (int m0 = 0; m0 < M; m0 += 4) {
        const int mr = min(4, M - m0);
        hipError_t e = mr == 1 ? launch_gemv1<1>(xq, gamma, M, K, wp, N, beta, y, acc, m0, s)
                     : mr == 2 ? launch_gemv1<2>(xq, gamma, M, K, wp, N, beta, y, acc, m0, s)
                               : launch_gemv1<4>(xq, gamma, M, K, wp, N, beta, y, acc, m0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace bl

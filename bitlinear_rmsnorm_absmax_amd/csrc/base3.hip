// Base-3 weights at 1.6 bits per weight (unite.ai BitNet.cpp article,
// Ternäres Gewichtssystem / Das Konzept: three states carry about 1.58 bits;
// five ternary codes fit one byte since 3^5 = 243).
//
// Layout: a row is U = ceil(K/80) units of 16 bytes.  Byte b of 32-bit word
// w of unit u holds the weights k = 80u + 20w + 4i + b (i = 0..4) as
// v = sum_i c_k 3^(4-i) with codes c = w + 1, stored as ceil(256 v / 243);
// weights past K are 0 (code 1).
//
// Decode: for the stored byte b, the walk x <- 3x, digit = x >> 8,
// x <- x & 255 yields v's base-3 digits, most significant first.  A word's
// four bytes run as two 16-bit lanes of two registers (bytes 0, 2 and bytes
// 1, 3); 3x never carries across a lane (3 * 255 < 65536), and one
// v_perm_b32 gathers the four digits (byte 1 of each lane) into one dword:
// digit i of bytes 0..3 = codes of weights 20w + 4i .. +3, in K order.  Per
// 20 weights: 3 + 5 * 3 + 4 * 2 = 26 VALU operations.
//
// The product runs v_dot4_i32_i8 on the codes: acc = sum c q - sum q
// (ternary product of the BitNet.cpp article, 3. BitLinear-Betrieb); the
// activation sum of a lane's unit is shared by the R rows of the wave.
#include "device_common.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kB3Threads = 256;

__global__ void zero_count3_kernel(int* p) { *p = 0; }

// One thread per packed word (20 weights) of the [N][U][4] words.
__global__ __launch_bounds__(kB3Threads) void pack3_kernel(const int8_t* __restrict__ w, int64_t N,
                                                          int K, int U,
                                                          uint32_t* __restrict__ packed,
                                                          int* __restrict__ bad_count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t words = N * U * 4;
    int bad = 0;
    if (i < words) {
        const int64_t n = i / (U * 4);
        const int rem = (int)(i - n * U * 4);
        const int k0 = 20 * rem;  // = 80u + 20w
        uint32_t d[5];
#pragma unroll
        for (int q = 0; q < 5; ++q)  // K % 16 == 0: a 4-byte group is all inside or all past K
            d[q] = (k0 + 4 * q < K) ? *reinterpret_cast<const uint32_t*>(w + n * K + k0 + 4 * q) : 0u;
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            int v = 0;
#pragma unroll
            for (int q = 0; q < 5; ++q) {
                int c;
                if (k0 + 4 * q < K) {
                    const int x = (int)(int8_t)((d[q] >> (8 * b)) & 0xFF);
                    if (x < -1 || x > 1) {
                        ++bad;
                        c = 1;
                    } else {
                        c = x + 1;
                    }
                } else {
                    c = 1;
                }
                v = 3 * v + c;
            }
            word |= (uint32_t)((256 * v + 242) / 243) << (8 * b);
        }
        packed[i] = word;
    }
    if (bad_count) {
        bad = wave_sum_i(bad);
        if ((threadIdx.x % kWave) == 0 && bad) atomicAdd(bad_count, bad);
    }
}

// Sum over the 64 lanes of a wave; the result is wave-uniform.
__device__ __forceinline__ int wave_reduce_dpp3(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false);  // row_ror:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Codes of one packed word: c[i] = digit i of bytes 0..3 (weights 4i .. 4i+3).
__device__ __forceinline__ void decode_word(uint32_t w, int c[5]) {
    uint32_t lo = w & 0x00FF00FFu;         // bytes 0 and 2, one per 16-bit lane
    uint32_t hi = (w >> 8) & 0x00FF00FFu;  // bytes 1 and 3
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        lo = (lo << 1) + lo;
        hi = (hi << 1) + hi;
        // {lo.byte1, hi.byte1, lo.byte3, hi.byte3}: the four digits in byte order
        c[i] = (int)__builtin_amdgcn_perm(hi, lo, 0x07030501u);
        if (i < 4) {
            lo &= 0x00FF00FFu;
            hi &= 0x00FF00FFu;
        }
    }
}

// Decode product on base-3 weights.  A wave owns R consecutive weight rows;
// lane l streams the 16-byte units l, l+64, ... of each row and the 80
// activation bytes of the same K range for MR tokens (rows m0 .. m0+MR-1 of
// x_q; activation pieces past K read as zero).
template <int MR, int R>
__global__ __launch_bounds__(kB3Threads) void gemv3_kernel(const int8_t* __restrict__ xq,
                                                           const float* __restrict__ gamma, int M,
                                                           int K, const v4u* __restrict__ wp,
                                                           int N, float beta, float* __restrict__ y,
                                                           int32_t* __restrict__ acc_out, int m0) {
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int n0 = (blockIdx.x * (kB3Threads / kWave) + wv) * R;
    const int U = (K + 79) / 80;

    int part[R][MR];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) part[r][m] = 0;
    int spart[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) spart[m] = 0;

    for (int u = lane; u < U; u += kWave) {
        v4u wq[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(n0 + r, N - 1);  // rows past N re-read the last one
            wq[r] = __builtin_nontemporal_load(wp + (int64_t)row * U + u);
        }
        v4i a[MR][5];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const int row = min(m0 + m, M - 1);
#pragma unroll
            for (int p = 0; p < 5; ++p) {
                const int k = 80 * u + 16 * p;
                a[m][p] = k < K ? *reinterpret_cast<const v4i*>(xq + (int64_t)row * K + k)
                                : v4i{0, 0, 0, 0};
                spart[m] = byte_sum16(a[m][p], spart[m]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t wd[4] = {wq[r].x, wq[r].y, wq[r].z, wq[r].w};
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                int c[5];
                decode_word(wd[w4], c);
#pragma unroll
                for (int i = 0; i < 5; ++i) {
                    const int dw = 5 * w4 + i;  // activation dword of weights 20 w4 + 4i ..
                    const int p = dw >> 2, e = dw & 3;
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        const int av = e == 0 ? a[m][p].x : e == 1 ? a[m][p].y : e == 2 ? a[m][p].z : a[m][p].w;
                        part[r][m] = __builtin_amdgcn_sdot4(c[i], av, part[r][m], false);
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
            const int tot = wave_reduce_dpp3(part[r][m] - spart[m]);
            const int n = n0 + r;
            if (lane == 0 && n < N && row < M) {
                if (y) y[(int64_t)row * N + n] = (float)tot * sc;
                if (acc_out) acc_out[(int64_t)row * N + n] = tot;
            }
        }
    }
}

template <int MR>
hipError_t launch_gemv3(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp, int N,
                        float beta, float* y, int32_t* acc, int m0, hipStream_t s) {
    constexpr int R = 4;
    const int rows_per_block = (kB3Threads / kWave) * R;
    const int blocks = (N + rows_per_block - 1) / rows_per_block;
    gemv3_kernel<MR, R><<<dim3(blocks), dim3(kB3Threads), 0, s>>>(
        xq, gamma, M, K, reinterpret_cast<const v4u*>(wp), N, beta, y, acc, m0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pack3(const int8_t* w, int64_t N, int64_t K, uint32_t* packed3, int* bad_count,
                        hipStream_t s) {
    if (bad_count) {
        zero_count3_kernel<<<1, 1, 0, s>>>(bad_count);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int U = (int)((K + 79) / 80);
    const int64_t words = N * U * 4;
    if (words == 0) return hipSuccess;
    pack3_kernel<<<dim3((unsigned)((words + kB3Threads - 1) / kB3Threads)), dim3(kB3Threads), 0, s>>>(
        w, N, (int)K, U, packed3, bad_count);
    return hipGetLastError();
}

hipError_t launch_forward3(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                           int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    // groups of up to four tokens, each a pass over the weights
    for (int m0 = 0; m0 < M; m0 += 4) {
        const int mr = min(4, M - m0);
        hipError_t e = mr == 1 ? launch_gemv3<1>(xq, gamma, M, K, wp, N, beta, y, acc, m0, s)
                     : mr == 2 ? launch_gemv3<2>(xq, gamma, M, K, wp, N, beta, y, acc, m0, s)
                               : launch_gemv3<4>(xq, gamma, M, K, wp, N, beta, y, acc, m0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace bl

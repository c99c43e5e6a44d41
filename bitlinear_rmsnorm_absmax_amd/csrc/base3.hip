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
            const int tot = wave_sum_dpp(part[r][m] - spart[m]);
            const int n = n0 + r;
            if (lane == 0 && n < N && row < M) {
                if (y) y[(int64_t)row * N + n] = (float)tot * sc;
                if (acc_out) acc_out[(int64_t)row * N + n] = tot;
            }
        }
    }
}

// Up to 16 tokens in one pass over the weights, on int8 MFMA
// (v_mfma_i32_16x16x64_i8, D = sum c q over the codes c = w + 1, then
// acc = D - S as above).
//
// The product is summed over K, so the order in which K positions enter the
// 64-deep MFMA operand is free as long as both operands follow it.  Lane
// (j, g) (j = lane % 16, g = lane / 16) decodes the 16-byte unit 4s + g of
// weight row n0 + j at step s into 80 codes in K order; MFMA t = 0..4 of the
// step takes its codes 16t .. 16t+15, and the activation operand of the same
// lane is the 16 bytes of token j at the same K positions (piece 5u + t of
// the staged row).  Each weight byte is decoded once per token block, and
// the 16 x 64 MACs of an MFMA replace 256 v_dot4 per lane group.
//
// The workgroup (8 waves) stages the M x K activation block in LDS once, as
// rows of 20 * steps 16-byte pieces (pieces past K zero) at an odd pitch in
// pieces (a wave's 16 rows of one piece then fall on distinct banks), and
// takes the per-token sums S from the staged bytes.  It owns CT column tiles
// of 16 rows; the 8 / CT waves of a tile split the steps and meet in LDS.
// Nothing is moved across this point by the compiler, memory or arithmetic.
__device__ __forceinline__ void fence_code3() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

constexpr int kB3Waves = 8;
constexpr int kB3ActMax = 144 * 1024;  // dynamic LDS: the staged activations

int b3_steps(int K) { return ((K + 79) / 80 + 3) / 4; }
size_t b3_act_bytes(int M, int K) { return (size_t)M * (20 * b3_steps(K) + 1) * 16; }

template <int CT, int BATCH>
__global__ __launch_bounds__(kB3Waves * kWave) void gemv3_mfma_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ gamma, int M, int K,
    const v4u* wp, int N, float beta, float* __restrict__ y, int32_t* __restrict__ acc_out) {
    constexpr int KS = kB3Waves / CT;
    constexpr int MR = 16;
    extern __shared__ __attribute__((aligned(16))) int8_t As[];  // [M][pitch][16]
    __shared__ int red[kB3Waves][4][kWave];
    __shared__ int s_wave[kB3Waves][MR];
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int t = wv % CT, ks = wv / CT;
    const int j = lane & 15, g = lane >> 4;
    const int U = (K + 79) / 80;
    const int steps = (U + 3) / 4;
    const int P = 20 * steps;  // staged pieces per row
    const int pitch = P + 1;
    const int spw = (steps + KS - 1) / KS;
    const int s_begin = ks * spw;
    const int s_end = min(s_begin + spw, steps);
    const int n0 = (blockIdx.x * CT + t) * 16;
    // rows past N re-read the last one and units past U the last unit (their
    // activations are zero); neither is stored
    const v4u* wrow = wp + (int64_t)min(n0 + j, N - 1) * U;
    auto load_batch = [&](int sb, v4u (&bw)[BATCH]) {
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
            bw[i] = __builtin_nontemporal_load(wrow + min(4 * min(sb + i, steps - 1) + g, U - 1));
    };

    // stage piece p (k = 16 p) of every token, the token loads of a piece
    // issued together, pieces past K zero (K % 16 == 0); per-token sums from
    // the loaded bytes.  The first pieces are loaded before the first weight
    // batch is issued and stored after it: loads return in issue order, so
    // the staging then waits for its own loads only, and the weights land
    // while the workgroup meets at the barrier.
    int spart[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) spart[m] = 0;
    auto load_pieces = [&](int p, v4i (&v)[MR]) {
        const int k = 16 * p;
#pragma unroll
        for (int m = 0; m < MR; ++m)
            v[m] = (m < M && k < K) ? *reinterpret_cast<const v4i*>(xq + (int64_t)m * K + k) : v4i{0, 0, 0, 0};
    };
    auto store_pieces = [&](int p, const v4i (&v)[MR]) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m < M) {
                *reinterpret_cast<v4i*>(As + ((int64_t)m * pitch + p) * 16) = v[m];
                spart[m] = byte_sum16(v[m], spart[m]);
            }
        }
    };
    v4u b0[BATCH], b1[BATCH];
    {
        v4i v[MR];
        const bool first = tid < P;
        if (first) load_pieces(tid, v);
        fence_code3();
        load_batch(s_begin, b0);
        fence_code3();
        if (first) store_pieces(tid, v);
    }
    for (int p = tid + kB3Waves * kWave; p < P; p += kB3Waves * kWave) {
        v4i v[MR];
        load_pieces(p, v);
        store_pieces(p, v);
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        if (m < M) {
            const int sm = wave_sum_dpp(spart[m]);
            if (lane == 0) s_wave[wv][m] = sm;
        }
    }
    __syncthreads();

    // A-operand row of lane j; rows past M repeat row M-1 (never stored)
    const int8_t* arow = As + (int64_t)min(j, M - 1) * pitch * 16;
    v4i acc = v4i{0, 0, 0, 0};
    auto mul_batch = [&](int sb, const v4u (&bw)[BATCH]) {
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int s = sb + i;
            if (s < s_end) {
                int c[20];
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) {
                    const uint32_t wd = w4 == 0 ? bw[i].x : w4 == 1 ? bw[i].y : w4 == 2 ? bw[i].z : bw[i].w;
                    decode_word(wd, c + 5 * w4);
                }
                const int8_t* ap = arow + 16 * 5 * (4 * s + g);
#pragma unroll
                for (int q = 0; q < 5; ++q) {
                    const v4i a = *reinterpret_cast<const v4i*>(ap + 16 * q);
                    const v4i b = v4i{c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]};
                    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
                }
            }
        }
    };
    // a stream of batches, the next one's loads issued before the current one
    // is multiplied: two batches a trip, loads unconditional (clamped onto
    // the last step, never multiplied) and a scheduling barrier after every
    // step, so that the compiler neither sinks the loads below the multiplies
    // nor waits for all of them at the loop head
    const int nb = max(0, (s_end - s_begin + BATCH - 1) / BATCH);
    int sb = s_begin;
    for (int i = 0; i + 2 <= nb; i += 2, sb += 2 * BATCH) {
        load_batch(sb + BATCH, b1);
        __builtin_amdgcn_sched_barrier(0);
        mul_batch(sb, b0);
        __builtin_amdgcn_sched_barrier(0);
        load_batch(sb + 2 * BATCH, b0);
        __builtin_amdgcn_sched_barrier(0);
        mul_batch(sb + BATCH, b1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (nb & 1) mul_batch(sb, b0);  // its loads were issued by the last trip (or before the loop)

    // lane (j, g) holds tokens 4g + v of column j
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wv][v][lane] = acc[v];
    __syncthreads();
    if (ks == 0) {
        const int col = n0 + j;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = 4 * g + v;
            if (row >= M || col >= N) continue;
            int d = 0;
#pragma unroll
            for (int k2 = 0; k2 < KS; ++k2) d += red[t + CT * k2][v][lane];
            int srow = 0;
#pragma unroll
            for (int w = 0; w < kB3Waves; ++w) srow += s_wave[w][row];
            const int a = d - srow;
            if (y) y[(int64_t)row * N + col] = (float)a * out_scale(beta, gamma[row]);
            if (acc_out) acc_out[(int64_t)row * N + col] = a;
        }
    }
}

template <int CT, int BATCH>
hipError_t launch_b3(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp, int N,
                     float beta, float* y, int32_t* acc, hipStream_t s) {
    static DynLdsOptIn opt_in;
    const hipError_t e =
        opt_in.ensure(reinterpret_cast<const void*>(&gemv3_mfma_kernel<CT, BATCH>), kB3ActMax);
    if (e != hipSuccess) return e;
    const int blocks = (N + 16 * CT - 1) / (16 * CT);
    gemv3_mfma_kernel<CT, BATCH><<<dim3(blocks), dim3(kB3Waves * kWave), b3_act_bytes(M, K), s>>>(
        xq, gamma, M, K, reinterpret_cast<const v4u*>(wp), N, beta, y, acc);
    return hipGetLastError();
}

// The widest CT <= 4 that still leaves >= 160 workgroups (or CT = 1):
// measured at K = 4096 N = 11008, 172 workgroups of 4 tiles beat 344 of 2 by
// 20 % and 86 of 8 by 30 %; at K = 8192 N = 28672, 448 of 4 beat 224 of 8 by
// 6 % (two waves a tile split its steps).  A wave's
// steps in one batch when it has at most 4, else a stream of 2-step batches.
template <int CT>
hipError_t launch_b3_ct(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp, int N,
                        float beta, float* y, int32_t* acc, hipStream_t s) {
    constexpr int KS = kB3Waves / CT;
    const int spw = (b3_steps(K) + KS - 1) / KS;
    if (spw <= 4) return launch_b3<CT, 4>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    return launch_b3<CT, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

hipError_t launch_gemv3_mfma(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                             int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    const int64_t tiles = (N + 15) / 16;
    if ((tiles + 3) / 4 >= 160) return launch_b3_ct<4>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    if ((tiles + 1) / 2 >= 160) return launch_b3_ct<2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    return launch_b3_ct<1>(xq, gamma, M, K, wp, N, beta, y, acc, s);
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
    // 2..16 tokens whose activation block fits in LDS: one pass on MFMA (one
    // token: the vector kernel below, 7 % faster at K = 4096 N = 11008)
    if (M >= 2 && M <= 16 && b3_act_bytes(M, K) <= (size_t)kB3ActMax)
        return launch_gemv3_mfma(xq, gamma, M, K, wp, N, beta, y, acc, s);
    // else groups of up to four tokens, each a pass over the weights
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

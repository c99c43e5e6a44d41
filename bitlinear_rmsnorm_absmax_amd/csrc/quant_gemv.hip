// Fused per-token absmax quantisation (optionally after RMSNorm) and
// one-token ternary product: the BitLinear forward as one launch
// (datacamp MatMul-free article, Kerncomponenten: RMS norm, then absmax
// quantisation, then the ternary product; unite.ai BitNet.cpp article,
// 2. Aktivierungsquantisierung and 3. BitLinear-Betrieb).
//
// Every workgroup quantises the whole token itself (the row is K fp32 or bf16
// values, read from L2 after the first workgroup) into an LDS copy of the
// codes, then runs the VALU product of gemv_valu.hip on its R rows per wave
// with the activations from LDS.  The quantisation runs on the workgroup's
// first kQuantThreads threads (the quantiser's own layout); a workgroup of
// WAVES waves multiplies WAVES * R rows, so wider workgroups repeat the
// quantisation fewer times:
//   1. the quantiser threads issue the loads of the row's first chunks, then
//      (after a barrier) each wave queues the loads of its first weight units,
//      so the weight stream is in flight during the quantisation;
//   2. absmax (and the float64 sum of squares) over the row in the chunking
//      and reduction order of quant_rows_kernel: the codes and gamma are
//      bit-identical to bitlinear_quant_act's;
//   3. codes to LDS (workgroup 0 also writes x_q and gamma), their sum S
//      reduced once for the workgroup;
//   4. acc = sum c q - S with v_dot4_i32_i8 on the 2-bit codes c = w + 1,
//      y = fl32(acc) * fl32(beta * gamma) / 128.
// Requires K % 64 == 0 (whole 16-byte weight units), K <= kFusedMaxK and
// N <= kFusedMaxN.
#include "device_common.h"
#include "internal.h"
#include "quant_rows.h"

namespace bl {
namespace {

constexpr int kQWaves = kQuantThreads / kWave;  // waves that quantise
constexpr int kFgRows = 4;                       // weight rows per wave

template <Src S, bool RMS, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void quant_gemv_kernel(
    RowSrc src, int K, const float* __restrict__ gain, float eps, const uint32_t* __restrict__ wp,
    int N, float beta, float* __restrict__ y, int32_t* __restrict__ acc_out,
    int8_t* __restrict__ q_out, float* __restrict__ gamma_out) {
    constexpr int R = kFgRows;
    __shared__ __attribute__((aligned(16))) int8_t sq[kFusedMaxK];
    __shared__ int s_sum[kQWaves];
    static_assert(WAVES >= kQWaves, "the quantiser's threads are part of the workgroup");

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int n0 = (blockIdx.x * WAVES + wv) * R;
    const bool quantiser = tid < kQuantThreads;
    const int WR = K >> 4;       // packed words per row
    const int units = WR >> 2;   // 16-byte units per row (K % 64 == 0)
    const uint32_t* wrow = wp + (int64_t)n0 * WR;

    // weight unit u of the wave's rows; rows past N and units past the row
    // read as zero codes.  The loads are unconditional (clamped onto the last
    // row / unit, then zeroed), so the compiler counts them exactly and waits
    // for the row chunks issued before them without waiting for them.
    auto load_unit = [&](int u, uint32_t (&w)[R][4]) {
        const int uc = min(u, units - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t rc = (int64_t)min(n0 + r, N - 1) - n0;
            const v4u v = __builtin_nontemporal_load(
                reinterpret_cast<const v4u*>(wrow + rc * WR + 4 * uc));
            const bool ok = u < units && n0 + r < N;
            w[r][0] = ok ? v.x : 0u; w[r][1] = ok ? v.y : 0u;
            w[r][2] = ok ? v.z : 0u; w[r][3] = ok ? v.w : 0u;
        }
    };
    // absmax (+ sum of squares) exactly as the quantiser's pass over row 0.
    // The row's first chunks (and their gains) are loaded before any weight
    // load is issued: a compute unit returns loads in issue order, so the
    // quantisation then runs while the weights stream in, instead of after.
    const int nchunk = K / 16;
    float cache[kQuantCache][16];
    float gcache[RMS ? kQuantCache : 1][16];
    auto load_gain = [&](int c, float g16[16]) {
        const float4* pg = reinterpret_cast<const float4*>(gain + (int64_t)c * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 g = pg[i];
            g16[4 * i] = g.x; g16[4 * i + 1] = g.y; g16[4 * i + 2] = g.z; g16[4 * i + 3] = g.w;
        }
    };
    if (quantiser) {
#pragma unroll
        for (int i = 0; i < kQuantCache; ++i) {
            const int c = tid + i * kQuantThreads;
            if (c < nchunk) {
                load_chunk<S>(src, 0, K, c, cache[i]);
                if constexpr (RMS) load_gain(c, gcache[i]);
            }
        }
    }
    __syncthreads();  // every wave's weight loads queue behind the row's
    uint32_t wcur[R][4];
    load_unit(lane, wcur);

    float amax = 0.0f;
    double ss = 0.0;
    auto process = [&](float v[16], const float g16[16]) {
        if constexpr (RMS) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float xv = v[e];
                ss += (double)xv * (double)xv;
                v[e] = g16[e] * xv;
            }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
    };
    if (quantiser) {
#pragma unroll
        for (int i = 0; i < kQuantCache; ++i) {
            const int c = tid + i * kQuantThreads;
            if (c < nchunk) process(cache[i], gcache[RMS ? i : 0]);
        }
        for (int c = tid + kQuantCache * kQuantThreads; c < nchunk; c += kQuantThreads) {
            float v[16], g16[16];
            load_chunk<S>(src, 0, K, c, v);
            if constexpr (RMS) load_gain(c, g16);
            process(v, g16);
        }
    }
    block_reduce<kQWaves>(amax, ss, RMS);
    float gamma = amax;
    if constexpr (RMS) {
        const double r = 1.0 / sqrt(ss / (double)K + (double)eps);
        gamma = (float)(r * (double)amax);
    }

    // codes into LDS (and to x_q from workgroup 0); their sum for the offset
    int csum = 0;
    auto put_codes = [&](int c, const float v[16]) {
        uint32_t d[4] = {0u, 0u, 0u, 0u};
        if (amax != 0.0f) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int q0 = quant_code(v[4 * j], amax), q1 = quant_code(v[4 * j + 1], amax);
                const int q2 = quant_code(v[4 * j + 2], amax), q3 = quant_code(v[4 * j + 3], amax);
                csum += q0 + q1 + q2 + q3;
                d[j] = pack4(q0, q1, q2, q3);
            }
        }
        const v4u dv = v4u{d[0], d[1], d[2], d[3]};
        *reinterpret_cast<v4u*>(sq + 16 * c) = dv;
        if (blockIdx.x == 0) *reinterpret_cast<v4u*>(q_out + 16 * (int64_t)c) = dv;
    };
    if (quantiser) {
#pragma unroll
        for (int i = 0; i < kQuantCache; ++i) {
            const int c = tid + i * kQuantThreads;
            if (c < nchunk) put_codes(c, cache[i]);
        }
        for (int c = tid + kQuantCache * kQuantThreads; c < nchunk; c += kQuantThreads) {
            float v[16];
            load_chunk<S>(src, 0, K, c, v);
            if constexpr (RMS) {
                const float4* pg = reinterpret_cast<const float4*>(gain + (int64_t)c * 16);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 g = pg[i];
                    v[4 * i + 0] *= g.x; v[4 * i + 1] *= g.y; v[4 * i + 2] *= g.z; v[4 * i + 3] *= g.w;
                }
            }
            put_codes(c, v);
        }
        csum = wave_sum_i(csum);
        if (lane == 0) s_sum[wv] = csum;
    }
    if (blockIdx.x == 0 && tid == 0) gamma_out[0] = gamma;
    __syncthreads();  // codes and partial sums visible to every wave
    int S_tot = 0;
#pragma unroll
    for (int i = 0; i < kQWaves; ++i) S_tot += s_sum[i];

    // product: lane streams units lane, lane + 64, ... of its R rows
    int part[R];
#pragma unroll
    for (int r = 0; r < R; ++r) part[r] = 0;
    for (int ub = lane; ub < units; ub += kWave) {
        uint32_t wnext[R][4];
        if (ub + kWave < units) load_unit(ub + kWave, wnext);
        v4i a[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) a[s] = *reinterpret_cast<const v4i*>(sq + 16 * (4 * ub + s));
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const v4i c = unpack_codes(wcur[r][s]);
                int d = part[r];
                d = __builtin_amdgcn_sdot4(c.x, a[s].x, d, false);
                d = __builtin_amdgcn_sdot4(c.y, a[s].y, d, false);
                d = __builtin_amdgcn_sdot4(c.z, a[s].z, d, false);
                d = __builtin_amdgcn_sdot4(c.w, a[s].w, d, false);
                part[r] = d;
            }
        }
        if (ub + kWave < units) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) wcur[r][s] = wnext[r][s];
        }
    }

    const float sc = out_scale(beta, gamma);
    int av = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int tot = wave_sum_dpp(part[r]) - S_tot;
        if (lane == r) av = tot;
    }
    const int n = n0 + lane;
    if (lane < R && n < N) {
        if (y) y[n] = (float)av * sc;
        if (acc_out) acc_out[n] = av;
    }
}

template <Src S, bool RMS, int WAVES>
hipError_t launch_fg(const void* x, int K, const float* gain, float eps, const uint32_t* wp, int N,
                     float beta, float* y, int32_t* acc, int8_t* q_out, float* gamma_out,
                     hipStream_t s) {
    const int rows_per_block = WAVES * kFgRows;
    const int blocks = (N + rows_per_block - 1) / rows_per_block;
    RowSrc src{x, nullptr};
    quant_gemv_kernel<S, RMS, WAVES><<<dim3(blocks), dim3(WAVES * kWave), 0, s>>>(
        src, K, gain, eps, wp, N, beta, y, acc, q_out, gamma_out);
    return hipGetLastError();
}

template <Src S, bool RMS>
hipError_t launch_fg_w(int waves, const void* x, int K, const float* gain, float eps,
                       const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                       int8_t* q_out, float* gamma_out, hipStream_t s) {
    if (waves >= 16) return launch_fg<S, RMS, 16>(x, K, gain, eps, wp, N, beta, y, acc, q_out, gamma_out, s);
    if (waves >= 8) return launch_fg<S, RMS, 8>(x, K, gain, eps, wp, N, beta, y, acc, q_out, gamma_out, s);
    return launch_fg<S, RMS, 4>(x, K, gain, eps, wp, N, beta, y, acc, q_out, gamma_out, s);
}

// Narrowest workgroup (4, 8 or 16 waves of 4 rows) that leaves at most 256
// workgroups.  Measured, one token, cold weights, against the two calls:
// K = N = 2048 4.2 vs 5.4 us (4 waves); K = 2560, N = 6912 5.2 vs 6.2 us (8);
// K = 6912, N = 2560 7.6 vs 7.8 us (4); K = 4096, N = 11008 7.5 vs 7.8 us
// (16).  Past 16384 rows even 16-wave groups number more than 256, each
// repeating the quantisation, and the two calls win (K = 8192, N = 28672:
// 18.4 vs 21.8 us), so quant_gemv_supports() excludes them.
int fg_waves(int N) {
    if ((N + 15) / 16 <= 256) return 4;
    if ((N + 31) / 32 <= 256) return 8;
    return 16;
}

}  // namespace


hipError_t launch_quant_gemv(const void* x, bool bf16, int K, const float* gain, float eps,
                             const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                             int8_t* q_out, float* gamma_out, hipStream_t s) {
    if (!quant_gemv_supports(1, K, N)) return hipErrorInvalidValue;
    const int w = fg_waves(N);
    if (bf16) {
        if (gain) return launch_fg_w<Src::BF16, true>(w, x, K, gain, eps, wp, N, beta, y, acc, q_out, gamma_out, s);
        return launch_fg_w<Src::BF16, false>(w, x, K, gain, eps, wp, N, beta, y, acc, q_out, gamma_out, s);
    }
    if (gain) return launch_fg_w<Src::F32, true>(w, x, K, gain, eps, wp, N, beta, y, acc, q_out, gamma_out, s);
    return launch_fg_w<Src::F32, false>(w, x, K, gain, eps, wp, N, beta, y, acc, q_out, gamma_out, s);
}

}  // namespace bl

// Per-token absmax int8 quantisation kernels (unite.ai BitNet.cpp article,
// Mathematische Grundlagen, 2. Aktivierungsquantisierung), the fused
// RMSNorm + quantisation variant (datacamp MatMul-free article,
// Kerncomponenten: RMS norm before quantisation), and the GLU glue
// h = SiLU(gate) * up followed by the same quantisation (datacamp article,
// MatMul-vrije GLU).
//
// One workgroup of 256 threads per token row (512 for the SiLU rows longer
// than 4096 elements).  A row is split into 16-element
// chunks (K % 16 == 0) dealt round-robin to the threads, so each load and
// each 16-byte code store is contiguous across the wave.  The first
// kQuantCache chunks of every thread stay in registers between the absmax
// pass and the quantisation pass, so rows up to 256 * 16 * kQuantCache
// elements are read from HBM exactly once; longer rows re-read the remainder
// (L2-resident by then).
#include "device_common.h"
#include "internal.h"
#include "quant_rows.h"

namespace bl {
namespace {

__device__ __forceinline__ void store_codes(int8_t* q, int64_t row, int K, int c,
                                            const float v[16], float gamma) {
    uint32_t d[4];
    if (gamma == 0.0f) {
        d[0] = d[1] = d[2] = d[3] = 0u;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            d[j] = pack4(quant_code(v[4 * j], gamma), quant_code(v[4 * j + 1], gamma),
                         quant_code(v[4 * j + 2], gamma), quant_code(v[4 * j + 3], gamma));
    }
    uint4* p = reinterpret_cast<uint4*>(q + row * (int64_t)K + (int64_t)c * 16);
    *p = make_uint4(d[0], d[1], d[2], d[3]);
}

// Plain fp32 rows (no RMSNorm): the row as 16-byte pieces of 4 entries dealt
// round-robin to THREADS threads, so every wave load reads 1 KB contiguous and
// every code store writes 256 B; the first NV pieces of a thread stay in
// registers between the absmax pass and the quantisation (the rest is re-read
// from L2).  The absmax is a max, exact in any order, and each code is the
// same per-entry function, so gamma and the codes are bit-identical to
// quant_rows_kernel's.  THREADS grows as the rows get fewer (about 512 K
// threads in all).  Back-to-back, against quant_rows_kernel: M = 512,
// K = 8192 8.3 -> 6.6 us; K = 6912 7.9 -> 6.1 us; M = 64, K = 8192 4.9 ->
// 3.9 us; M = 2048, K = 4096 (256 threads) 12.7 -> 10.0 us.  (bf16 rows
// measured no faster this way and keep quant_rows_kernel.)
template <int THREADS, int NV>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4, 8)))
void quant_f32_kernel(const float* __restrict__ x, int K, int8_t* __restrict__ q,
                      float* __restrict__ gamma_out) {
    const int64_t row = blockIdx.x;
    const int nvec = K / 4;
    const v4f* src = reinterpret_cast<const v4f*>(x + row * (int64_t)K);
    v4f cache[NV];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = threadIdx.x + i * THREADS;
        cache[i] = idx < nvec ? __builtin_nontemporal_load(src + idx) : v4f{0.f, 0.f, 0.f, 0.f};
    }
    auto vmax = [&](const v4f& t) {
        amax = fmaxf(amax, fabsf(t.x));
        amax = fmaxf(amax, fabsf(t.y));
        amax = fmaxf(amax, fabsf(t.z));
        amax = fmaxf(amax, fabsf(t.w));
    };
#pragma unroll
    for (int i = 0; i < NV; ++i) vmax(cache[i]);
    for (int idx = threadIdx.x + NV * THREADS; idx < nvec; idx += THREADS)
        vmax(__builtin_nontemporal_load(src + idx));
    double ss = 0.0;
    block_reduce<THREADS / kWave>(amax, ss, false);
    if (threadIdx.x == 0) gamma_out[row] = amax;
    auto store = [&](int idx, const v4f& t) {
        const uint32_t c = amax == 0.0f ? 0u
                                        : pack4(quant_code(t.x, amax), quant_code(t.y, amax),
                                                quant_code(t.z, amax), quant_code(t.w, amax));
        *reinterpret_cast<uint32_t*>(q + row * (int64_t)K + 4 * (int64_t)idx) = c;
    };
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = threadIdx.x + i * THREADS;
        if (idx < nvec) store(idx, cache[i]);
    }
    for (int idx = threadIdx.x + NV * THREADS; idx < nvec; idx += THREADS)
        store(idx, __builtin_nontemporal_load(src + idx));
}

// RMS: gain applied before the absmax (u = g * x), sum of x^2 in float64.
// H_OUT: also write the fp32 values being quantised (the SiLU*up product).
// THREADS: kQuantThreads, or wider for rows without RMSNorm (their only
// reduction is a max, exact in any order, so gamma and the codes do not
// depend on how the chunks are dealt).  Plain fp32 / bf16 rows are held to
// 64 VGPRs (8 waves a SIMD), so 2048 rows of 256 threads run in one round
// (bf16, K = 4096: 68 -> 56 VGPRs, 7.05 -> 6.88 us).
template <Src S, bool RMS, bool H_OUT, int THREADS = kQuantThreads>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu((S == Src::F32 || S == Src::BF16) && !RMS ? 8 : 1))) void quant_rows_kernel(
    RowSrc src, int K, const float* __restrict__ gain, float eps, float* __restrict__ h_out,
    int8_t* __restrict__ q, float* __restrict__ gamma_out) {
    const int64_t row = blockIdx.x;
    const int nchunk = K / 16;
    float cache[kQuantCache][16];
    float amax = 0.0f;
    double ss = 0.0;

    auto prepare = [&](int c, float v[16]) {
        load_chunk<S>(src, row, K, c, v);
        if constexpr (RMS) {
            const float4* pg = reinterpret_cast<const float4*>(gain + (int64_t)c * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float4 g = pg[i];
                float gg[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float xv = v[4 * i + j];
                    ss += (double)xv * (double)xv;
                    v[4 * i + j] = gg[j] * xv;
                }
            }
        }
        if constexpr (H_OUT) {
            float4* ph = reinterpret_cast<float4*>(h_out + row * (int64_t)K + (int64_t)c * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ph[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
    };

#pragma unroll
    for (int i = 0; i < kQuantCache; ++i) {
        int c = threadIdx.x + i * THREADS;
        if (c < nchunk) prepare(c, cache[i]);
    }
    for (int c = threadIdx.x + kQuantCache * THREADS; c < nchunk; c += THREADS) {
        float v[16];
        prepare(c, v);
    }
    block_reduce<THREADS / kWave>(amax, ss, RMS);

    float gamma = amax;
    if constexpr (RMS) {
        double r = 1.0 / sqrt(ss / (double)K + (double)eps);
        gamma = (float)(r * (double)amax);
    }
    if (threadIdx.x == 0) gamma_out[row] = gamma;

#pragma unroll
    for (int i = 0; i < kQuantCache; ++i) {
        int c = threadIdx.x + i * THREADS;
        if (c < nchunk) store_codes(q, row, K, c, cache[i], amax);
    }
    for (int c = threadIdx.x + kQuantCache * THREADS; c < nchunk; c += THREADS) {
        float v[16];
        load_chunk<S>(src, row, K, c, v);
        if constexpr (RMS) {
            const float4* pg = reinterpret_cast<const float4*>(gain + (int64_t)c * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float4 g = pg[i];
                v[4 * i + 0] *= g.x; v[4 * i + 1] *= g.y; v[4 * i + 2] *= g.z; v[4 * i + 3] *= g.w;
            }
        }
        store_codes(q, row, K, c, v, amax);
    }
}

// Few long rows: P workgroups per row (grid P x M).  Every workgroup reads
// the whole row with the chunk dealing and reduction order of
// quant_rows_kernel (256 threads, chunk c to thread c mod 256, the same
// block_reduce), so its absmax -- and with RMS its float64 sum of squares --
// are bit-identical to that kernel's; then it quantises only its own run of
// chunks, re-read from L2.  The row is read P times (from L2 after the first
// touch) instead of one compute unit working through it alone: one token at
// K = 8192 takes one workgroup 6.9 us.
template <Src S, bool RMS>
__global__ __launch_bounds__(kQuantThreads) void quant_split_kernel(
    RowSrc src, int K, const float* __restrict__ gain, float eps, int8_t* __restrict__ q,
    float* __restrict__ gamma_out) {
    const int64_t row = blockIdx.y;
    const int P = gridDim.x, p = blockIdx.x;
    const int nchunk = K / 16;
    float amax = 0.0f;
    double ss = 0.0;
    for (int c = threadIdx.x; c < nchunk; c += kQuantThreads) {
        float v[16];
        load_chunk<S>(src, row, K, c, v);
        if constexpr (RMS) {
            const float4* pg = reinterpret_cast<const float4*>(gain + (int64_t)c * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float4 g = pg[i];
                float gg[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float xv = v[4 * i + j];
                    ss += (double)xv * (double)xv;
                    v[4 * i + j] = gg[j] * xv;
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
    block_reduce(amax, ss, RMS);
    if (p == 0 && threadIdx.x == 0) {
        float gamma = amax;
        if constexpr (RMS) gamma = (float)((1.0 / sqrt(ss / (double)K + (double)eps)) * (double)amax);
        gamma_out[row] = gamma;
    }
    const int per = (nchunk + P - 1) / P;
    const int c0 = p * per, c1 = min(nchunk, c0 + per);
    for (int c = c0 + (int)threadIdx.x; c < c1; c += kQuantThreads) {
        float v[16];
        load_chunk<S>(src, row, K, c, v);
        if constexpr (RMS) {
            const float4* pg = reinterpret_cast<const float4*>(gain + (int64_t)c * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float4 g = pg[i];
                v[4 * i + 0] *= g.x; v[4 * i + 1] *= g.y; v[4 * i + 2] *= g.z; v[4 * i + 3] *= g.w;
            }
        }
        store_codes(q, row, K, c, v, amax);
    }
}

// Group quantisation (unite.ai BitNet.cpp article, Gruppenquantisierung und
// -normalisierung): row `row` split into G runs of K/G inputs, each run
// quantised with its own absmax scale.  One workgroup per (row, run): an
// absmax pass and a quantisation pass over the run's 16-element chunks (the
// second pass re-reads the run, L2-resident by then).  RMS: the whole row's
// sum of squares first (same chunk order and reduction as quant_rows_kernel,
// so r is the ungrouped r), gamma = fl32(r * max |u|) per run.  Outputs are
// group-major: q + (g*M + row)*K/G, gamma_out[g*M + row].
template <Src S, bool RMS>
__global__ __launch_bounds__(kQuantThreads) void quant_groups_kernel(
    RowSrc src, int K, int G, int M, const float* __restrict__ gain, float eps,
    int8_t* __restrict__ q, float* __restrict__ gamma_out) {
    const int64_t row = blockIdx.x;
    const int g = blockIdx.y;
    const int KG = K / G, nch = KG / 16;
    auto load_u = [&](int c, float v[16]) {  // chunk c of the row, gain applied
        load_chunk<S>(src, row, K, c, v);
        if constexpr (RMS) {
            const float4* pg = reinterpret_cast<const float4*>(gain + (int64_t)c * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float4 g4 = pg[i];
                v[4 * i + 0] *= g4.x; v[4 * i + 1] *= g4.y; v[4 * i + 2] *= g4.z; v[4 * i + 3] *= g4.w;
            }
        }
    };
    double r = 1.0;
    if constexpr (RMS) {
        float unused = 0.0f;
        double ss = 0.0;
        for (int c = threadIdx.x; c < K / 16; c += kQuantThreads) {
            float v[16];
            load_chunk<S>(src, row, K, c, v);
#pragma unroll
            for (int e = 0; e < 16; ++e) ss += (double)v[e] * (double)v[e];
        }
        block_reduce(unused, ss, true);
        r = 1.0 / sqrt(ss / (double)K + (double)eps);
        __syncthreads();  // the reduction scratch is reused below
    }
    float amax = 0.0f;
    double unused = 0.0;
    for (int c = threadIdx.x; c < nch; c += kQuantThreads) {
        float v[16];
        load_u(g * nch + c, v);
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
    block_reduce(amax, unused, false);
    if (threadIdx.x == 0) gamma_out[(int64_t)g * M + row] = RMS ? (float)(r * (double)amax) : amax;
    int8_t* qg = q + (int64_t)g * M * KG;
    for (int c = threadIdx.x; c < nch; c += kQuantThreads) {
        float v[16];
        load_u(g * nch + c, v);
        store_codes(qg, row, KG, c, v, amax);
    }
}

// Rows with K == 0: gamma = 0 and nothing else to write.
__global__ void zero_gamma_kernel(float* gamma, int64_t M) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < M) gamma[i] = 0.0f;
}

}  // namespace

hipError_t launch_quant_act(const void* x, int bf16, int64_t M, int64_t K, const float* gain,
                            float eps, int8_t* q, float* gamma, hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (K == 0) {
        zero_gamma_kernel<<<dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s>>>(gamma, M);
        return hipGetLastError();
    }
    RowSrc src{x, nullptr};
    dim3 grid((unsigned)M), block(kQuantThreads);
    const int k = (int)K;
    const int P = quant_split_ways(M, K);
    if (P > 1) {
        dim3 sgrid((unsigned)P, (unsigned)M);
        if (bf16) {
            if (gain)
                quant_split_kernel<Src::BF16, true><<<sgrid, block, 0, s>>>(src, k, gain, eps, q, gamma);
            else
                quant_split_kernel<Src::BF16, false><<<sgrid, block, 0, s>>>(src, k, nullptr, 0.f, q, gamma);
        } else {
            if (gain)
                quant_split_kernel<Src::F32, true><<<sgrid, block, 0, s>>>(src, k, gain, eps, q, gamma);
            else
                quant_split_kernel<Src::F32, false><<<sgrid, block, 0, s>>>(src, k, nullptr, 0.f, q, gamma);
        }
        return hipGetLastError();
    }
    if (bf16) {
        if (gain)
            quant_rows_kernel<Src::BF16, true, false><<<grid, block, 0, s>>>(src, k, gain, eps, nullptr, q, gamma);
        else
            quant_rows_kernel<Src::BF16, false, false><<<grid, block, 0, s>>>(src, k, nullptr, 0.f, nullptr, q, gamma);
    } else {
        const float* xf = static_cast<const float*>(x);
        if (gain)
            quant_rows_kernel<Src::F32, true, false><<<grid, block, 0, s>>>(src, k, gain, eps, nullptr, q, gamma);
        else if (M <= 512)
            quant_f32_kernel<1024, 2><<<grid, dim3(1024), 0, s>>>(xf, k, q, gamma);
        else if (M <= 1024)
            quant_f32_kernel<512, 4><<<grid, dim3(512), 0, s>>>(xf, k, q, gamma);
        else
            quant_f32_kernel<256, 8><<<grid, dim3(256), 0, s>>>(xf, k, q, gamma);
    }
    return hipGetLastError();
}

hipError_t launch_quant_act_grouped(const void* x, int bf16, int64_t M, int64_t K, int64_t G,
                                    const float* gain, float eps, int8_t* q, float* gamma,
                                    hipStream_t s) {
    if (M == 0) return hipSuccess;
    RowSrc src{x, nullptr};
    dim3 grid((unsigned)M, (unsigned)G), block(kQuantThreads);
    const int k = (int)K, g = (int)G, m = (int)M;
    if (bf16) {
        if (gain)
            quant_groups_kernel<Src::BF16, true><<<grid, block, 0, s>>>(src, k, g, m, gain, eps, q, gamma);
        else
            quant_groups_kernel<Src::BF16, false><<<grid, block, 0, s>>>(src, k, g, m, nullptr, 0.f, q, gamma);
    } else {
        if (gain)
            quant_groups_kernel<Src::F32, true><<<grid, block, 0, s>>>(src, k, g, m, gain, eps, q, gamma);
        else
            quant_groups_kernel<Src::F32, false><<<grid, block, 0, s>>>(src, k, g, m, nullptr, 0.f, q, gamma);
    }
    return hipGetLastError();
}

hipError_t launch_silu_mul_quant(const float* gate, const float* up, int64_t M, int64_t F,
                                 float* h, int8_t* h_q, float* gamma, hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (F == 0) {
        zero_gamma_kernel<<<dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s>>>(gamma, M);
        return hipGetLastError();
    }
    RowSrc src{gate, up};
    dim3 grid((unsigned)M), block(kQuantThreads);
    if (F / 16 > kQuantThreads) {
        // wider rows: one 16-element chunk per thread up to 8192 elements (the
        // float64 SiLU is the bulk of the work; more waves hide its latency)
        if (h)
            quant_rows_kernel<Src::SILU_MUL, false, true, 2 * kQuantThreads>
                <<<grid, dim3(2 * kQuantThreads), 0, s>>>(src, (int)F, nullptr, 0.f, h, h_q, gamma);
        else
            quant_rows_kernel<Src::SILU_MUL, false, false, 2 * kQuantThreads>
                <<<grid, dim3(2 * kQuantThreads), 0, s>>>(src, (int)F, nullptr, 0.f, nullptr, h_q, gamma);
        return hipGetLastError();
    }
    if (h)
        quant_rows_kernel<Src::SILU_MUL, false, true><<<grid, block, 0, s>>>(src, (int)F, nullptr, 0.f, h, h_q, gamma);
    else
        quant_rows_kernel<Src::SILU_MUL, false, false><<<grid, block, 0, s>>>(src, (int)F, nullptr, 0.f, nullptr, h_q, gamma);
    return hipGetLastError();
}

hipError_t launch_silu_mul_quant_acc(const int32_t* acc_gu, const float* gamma_in, int64_t M,
                                     int64_t F, float beta_gate, float beta_up, float* h,
                                     int8_t* h_q, float* gamma, hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (F == 0) {
        zero_gamma_kernel<<<dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s>>>(gamma, M);
        return hipGetLastError();
    }
    RowSrc src{acc_gu, nullptr, gamma_in, beta_gate, beta_up};
    dim3 grid((unsigned)M), block(kQuantThreads);
    if (F / 16 > kQuantThreads) {
        // wider rows: one 16-element chunk per thread up to 8192 elements (the
        // float64 SiLU is the bulk of the work; more waves hide its latency)
        if (h)
            quant_rows_kernel<Src::SILU_ACC, false, true, 2 * kQuantThreads>
                <<<grid, dim3(2 * kQuantThreads), 0, s>>>(src, (int)F, nullptr, 0.f, h, h_q, gamma);
        else
            quant_rows_kernel<Src::SILU_ACC, false, false, 2 * kQuantThreads>
                <<<grid, dim3(2 * kQuantThreads), 0, s>>>(src, (int)F, nullptr, 0.f, nullptr, h_q, gamma);
        return hipGetLastError();
    }
    if (h)
        quant_rows_kernel<Src::SILU_ACC, false, true><<<grid, block, 0, s>>>(src, (int)F, nullptr, 0.f, h, h_q, gamma);
    else
        quant_rows_kernel<Src::SILU_ACC, false, false><<<grid, block, 0, s>>>(src, (int)F, nullptr, 0.f, nullptr, h_q, gamma);
    return hipGetLastError();
}

}  // namespace bl

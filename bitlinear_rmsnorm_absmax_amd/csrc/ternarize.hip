// Absmean ternarisation of fp32 weights, then packing (datacamp article,
// section "MatMul vervangen door ternaire bewerkingen": the weight matrix is
// scaled by its mean absolute value and every entry rounded to the nearest of
// -1, 0, 1).
//
// beta64 = S / (N*K), S the pairwise sum in double of |W| over the row-major
// entries (a run splits after the largest power of two below its length);
// code = +1 if W > beta64/2, -1 if W < -beta64/2, else 0, compared exactly in
// double (round-half-even of W/beta64 clipped to [-1, 1]; ties go to 0).
//
// The pairwise tree over L entries is the complete binary tree over the
// entries padded with +0 to a power of two (a +0 leaf changes no sum), so it
// is evaluated bottom-up in aligned groups of 64:
//   1. leaf pass: each aligned group of 64 entries -> one double; a wave loads
//      1 KB runs coalesced (lane l holds entries 4l..4l+3 of each 256-entry
//      run), adds its four in pairs, then 16 lanes finish the group with an
//      xor butterfly (fp addition is commutative, so the butterfly is the
//      same tree);
//   2. level passes: groups of 64 partial sums -> one, until at most 64 are
//      left; one wave reduces those and divides by N*K;
//   3. codes + packing: one thread per packed word (code w+1 of entry 4j+b at
//      bit 8b + 2j, the layout of bitlinear_pack_weights).
// The partial sums live in the packed output buffer (about N*K/8 bytes of
// its N*K/4), ping-ponging between two regions; step 3 overwrites them.
// launch_pairwise_mean is also the mean of the weight binarisation (signed
// entries, 256-entry leaf groups: the same tree, a quarter of the scratch).
#include "device_common.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kTernBlock = 256;

__device__ __forceinline__ double xor_pair_sum(double v, int mask) {
    return v + __shfl_xor(v, mask, kWave);
}

// Pass 1: group g = entries [G g, G g + G) of the flat matrix (zero past L),
// G = 64 (16 lanes per group) or 256 (the whole wave); ABS: |W| else W.
template <int G, bool ABS>
__global__ __launch_bounds__(kTernBlock) void group_sums_leaf_kernel(const float* __restrict__ W,
                                                                     int64_t L, int64_t groups,
                                                                     double* __restrict__ out) {
    constexpr int kLanes = G / 4;  // lanes per group
    const int lane = threadIdx.x % kWave;
    const int64_t wave = ((int64_t)blockIdx.x * kTernBlock + threadIdx.x) / kWave;
    const int64_t base = wave * 1024;  // 1024 / G groups per wave
    if (base >= L) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t e = base + 256 * i + 4 * lane;  // entries e .. e+3, group e / G
        v4f v = v4f{0.f, 0.f, 0.f, 0.f};
        if (e < L) v = *reinterpret_cast<const v4f*>(W + e);  // L % 16 == 0: all four or none
        double s;
        if constexpr (ABS)
            s = (fabs((double)v.x) + fabs((double)v.y)) + (fabs((double)v.z) + fabs((double)v.w));
        else
            s = ((double)v.x + (double)v.y) + ((double)v.z + (double)v.w);
#pragma unroll
        for (int m = 1; m < kLanes; m <<= 1) s = xor_pair_sum(s, m);
        const int64_t g = e / G;
        if ((lane % kLanes) == 0 && g < groups) out[g] = s;
    }
}

// Level pass: out[g] = pairwise sum of in[64g .. 64g + 64) (zero past n).
__global__ __launch_bounds__(kTernBlock) void group_sums_kernel(const double* __restrict__ in,
                                                                int64_t n, int64_t groups,
                                                                double* __restrict__ out) {
    const int lane = threadIdx.x % kWave;
    const int64_t g = ((int64_t)blockIdx.x * kTernBlock + threadIdx.x) / kWave;
    if (g >= groups) return;
    const int64_t i = 64 * g + lane;
    double s = i < n ? in[i] : 0.0;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) s = xor_pair_sum(s, m);
    if (lane == 0) out[g] = s;
}

// Last level (n <= 64 partial sums, zero past n) on one wave, then the mean.
__global__ __launch_bounds__(kWave) void finish_kernel(const double* __restrict__ in, int64_t n,
                                                       int64_t N, int64_t K,
                                                       double* __restrict__ beta64,
                                                       float* __restrict__ beta32) {
    const int lane = threadIdx.x;
    double s = lane < n ? in[lane] : 0.0;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) s = xor_pair_sum(s, m);
    if (lane == 0) {
        const double b = (N > 0 && K > 0) ? s / ((double)N * (double)K) : 0.0;
        beta64[0] = b;
        beta32[0] = (float)b;
    }
}

__global__ __launch_bounds__(kTernBlock) void ternarize_pack_kernel(const float* __restrict__ W,
                                                                    int64_t words,
                                                                    const double* __restrict__ beta64,
                                                                    uint32_t* __restrict__ packed,
                                                                    int8_t* __restrict__ codes) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= words) return;
    const double b = beta64[0];
    const double half = 0.5 * b;
    const v4f* src = reinterpret_cast<const v4f*>(W + 16 * i);
    uint32_t word = 0;
    int c[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const v4f v = src[q];
        const float e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const double d = (double)e4[u];
            const int code = (b > 0.0 && d > half) ? 1 : (b > 0.0 && d < -half) ? -1 : 0;
            const int e = 4 * q + u;
            c[e] = code;
            word |= (uint32_t)(code + 1) << (8 * (e & 3) + 2 * (e >> 2));
        }
    }
    packed[i] = word;
    if (codes) {
        v4i out;
        out.x = (int)pack4(c[0], c[1], c[2], c[3]);
        out.y = (int)pack4(c[4], c[5], c[6], c[7]);
        out.z = (int)pack4(c[8], c[9], c[10], c[11]);
        out.w = (int)pack4(c[12], c[13], c[14], c[15]);
        *reinterpret_cast<v4i*>(codes + 16 * i) = out;
    }
}

int64_t waves_to_blocks(int64_t waves) { return (waves * kWave + kTernBlock - 1) / kTernBlock; }

}  // namespace

hipError_t launch_pairwise_mean(const float* W, int64_t L, int64_t N, int64_t K, bool abs_values,
                                int group, double* scratch, double* mean64, float* mean32,
                                hipStream_t s) {
    if (L == 0) {
        finish_kernel<<<dim3(1), dim3(kWave), 0, s>>>(nullptr, 0, 0, 0, mean64, mean32);
        return hipGetLastError();
    }
    int64_t n = (L + group - 1) / group;  // group sums after the leaf pass
    // region A: n doubles at `scratch`; region B (at most n/64 + 1 doubles)
    // right after; level passes run only while n > 64
    double* a = scratch;
    double* b = a + n;
    const dim3 leaf_grid((unsigned)waves_to_blocks((L + 1023) / 1024));
    if (group == 64) {
        if (abs_values) group_sums_leaf_kernel<64, true><<<leaf_grid, dim3(kTernBlock), 0, s>>>(W, L, n, a);
        else group_sums_leaf_kernel<64, false><<<leaf_grid, dim3(kTernBlock), 0, s>>>(W, L, n, a);
    } else {
        if (abs_values) group_sums_leaf_kernel<256, true><<<leaf_grid, dim3(kTernBlock), 0, s>>>(W, L, n, a);
        else group_sums_leaf_kernel<256, false><<<leaf_grid, dim3(kTernBlock), 0, s>>>(W, L, n, a);
    }
    double* src = a;
    double* dst = b;
    while (n > 64) {
        const int64_t groups = (n + 63) / 64;
        group_sums_kernel<<<dim3((unsigned)waves_to_blocks(groups)), dim3(kTernBlock), 0, s>>>(
            src, n, groups, dst);
        n = groups;
        double* t = src;
        src = dst;
        dst = t;
    }
    finish_kernel<<<dim3(1), dim3(kWave), 0, s>>>(src, n, N, K, mean64, mean32);
    return hipGetLastError();
}


hipError_t launch_ternarize(const float* W, int64_t N, int64_t K, uint32_t* packed, int8_t* codes,
                            float* beta32, double* beta64, hipStream_t s) {
    const int64_t L = N * K;
    // the partial sums (about L/8 bytes) live in the packed buffer (L/4 bytes)
    hipError_t e = launch_pairwise_mean(W, L, N, K, true, 64, reinterpret_cast<double*>(packed),
                                        beta64, beta32, s);
    if (e != hipSuccess || L == 0) return e;
    const int64_t words = L / 16;
    ternarize_pack_kernel<<<dim3((unsigned)((words + kTernBlock - 1) / kTernBlock)),
                            dim3(kTernBlock), 0, s>>>(W, words, beta64, packed, codes);
    return hipGetLastError();
}

}  // namespace bl

// Group-scale epilogue of the grouped BitLinear product (unite.ai BitNet.cpp
// article, Gruppenquantisierung und -normalisierung, with 3. BitLinear-Betrieb
// per group): y[m][n] = sum over g of fl32(acc[g][m][n]) * s[g][m],
// s[g][m] = fl32(beta[g] * gamma[g][m]) / 128, added in group order
// g = 0 .. G-1 in fp32.  The per-group integer products come from the
// ungrouped forward kernels (acc-only mode) on the group-major operands.
#include "device_common.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kGsThreads = 256;

// Four consecutive outputs of one row per thread (N % 4 == 0, acc and y
// 16-byte aligned), else one.
template <int V>
__global__ __launch_bounds__(kGsThreads) void group_sum_kernel(const int32_t* __restrict__ acc,
                                                               const float* __restrict__ gamma,
                                                               const float* __restrict__ beta,
                                                               int64_t M, int64_t N, int G,
                                                               float* __restrict__ y) {
    const int64_t MN = M * N;
    const int64_t i = ((int64_t)blockIdx.x * kGsThreads + threadIdx.x) * V;
    if (i >= MN) return;
    const int64_t m = i / N;
    float s[V];
    for (int g = 0; g < G; ++g) {  // the first term starts the sum
        const float sc = out_scale(beta[g], gamma[(int64_t)g * M + m]);
        const int32_t* a = acc + (int64_t)g * MN + i;
        float t[V];
        if constexpr (V == 4) {
            const v4i a4 = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(a));
            t[0] = (float)a4.x * sc; t[1] = (float)a4.y * sc;
            t[2] = (float)a4.z * sc; t[3] = (float)a4.w * sc;
        } else {
            t[0] = (float)a[0] * sc;
        }
#pragma unroll
        for (int v = 0; v < V; ++v) s[v] = g == 0 ? t[v] : s[v] + t[v];
    }
    if constexpr (V == 4)
        *reinterpret_cast<v4f*>(y + i) = v4f{s[0], s[1], s[2], s[3]};
    else
        y[i] = s[0];
}

}  // namespace

hipError_t launch_group_sum(const int32_t* acc, const float* gamma, const float* beta, int64_t M,
                            int64_t N, int64_t G, float* y, hipStream_t s) {
    const int64_t MN = M * N;
    if (MN == 0) return hipSuccess;
    const bool vec = N % 4 == 0 && reinterpret_cast<uintptr_t>(acc) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(y) % 16 == 0;
    if (vec) {
        const int64_t threads = MN / 4;
        group_sum_kernel<4><<<dim3((unsigned)((threads + kGsThreads - 1) / kGsThreads)),
                              dim3(kGsThreads), 0, s>>>(acc, gamma, beta, M, N, (int)G, y);
    } else {
        group_sum_kernel<1><<<dim3((unsigned)((MN + kGsThreads - 1) / kGsThreads)),
                              dim3(kGsThreads), 0, s>>>(acc, gamma, beta, M, N, (int)G, y);
    }
    return hipGetLastError();
}

}  // namespace bl

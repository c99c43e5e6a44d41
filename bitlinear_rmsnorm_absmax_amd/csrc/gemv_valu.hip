// Decode GEMV on the vector ALUs (M <= 4 tokens, HBM-bound).
//
// Ternary product (unite.ai BitNet.cpp article, 3. BitLinear-Betrieb;
// datacamp MatMul-free article: products by -1, 0, +1 become negate, skip,
// keep) with v_dot4_i32_i8 on the 2-bit codes c = w + 1: a code byte of 0, 1
// or 2 turns each 4-wide dot product into a sum of selected and doubled
// activations, and acc = sum c*q - sum q corrects the +1 offset once per
// lane (the activation sum of a lane's K slice is shared by every row).
//
// A wave owns R consecutive weight rows.  Lane l streams the 16-byte units
// (4 packed words = 64 weights) u = l, l+64, ... of each row, so one wave-wide
// load covers 1 KB of a row contiguously; the loads of all R rows are issued
// before the first dot product.  The activation unit of the lane
// (64 int8 per token) is loaded once per unit and reused by the R rows.  The
// R x M lane partials are reduced across the wave with DPP row operations
// (quad permutes and row rotations inside each 16-lane row) followed by four
// v_readlane reads; the rescale is fused into the store.
#include "device_common.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kGvThreads = 256;
constexpr int kGvWaves = kGvThreads / kWave;

// KS > 1 (few rows): the KS waves of a group share its R rows, wave ks taking
// the units ks*64 + lane, (ks + KS)*64 + lane, ...; their exact int32 partial
// sums meet in LDS and the group's first wave stores.
template <int MR, int R, int U, int KS>
__global__ __launch_bounds__(kGvThreads) void gemv_valu_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ gamma, int M, int K,
    const uint32_t* __restrict__ wp, int N, float beta, float* __restrict__ y,
    int32_t* __restrict__ acc_out) {
    static_assert(kGvWaves % KS == 0, "K slices divide the workgroup");
    __shared__ int s_part[KS > 1 ? kGvWaves : 1][R][MR];
    const int lane = threadIdx.x % kWave;
    // wave index made scalar so row addressing stays on the SALU
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int ks = wv % KS;
    const int n0 = (blockIdx.x * (kGvWaves / KS) + wv / KS) * R;  // waves past N load and store nothing
    const int WR = K >> 4;
    const int units = (WR + 3) >> 2;
    const bool aligned = (WR & 3) == 0;
    const bool full = aligned && n0 + R <= N;
    const uint32_t* wrow = wp + (int64_t)n0 * WR;  // first weight row of the wave

    int part[R][MR];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) part[r][m] = 0;
    int spart[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) spart[m] = 0;

    // U units per lane are loaded together (all U*R weight loads in flight
    // before the first dot product); longer rows loop over such batches
    for (int ub = lane + ks * kWave; ub < units; ub += U * KS * kWave) {
        uint32_t w[U][R][4];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int wb = 4 * (ub + i * KS * kWave);
            const bool live = ub + i * KS * kWave < units;
            if (full && live) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const v4u v = __builtin_nontemporal_load(
                        reinterpret_cast<const v4u*>(wrow + (uint32_t)(r * WR + wb)));
                    w[i][r][0] = v.x; w[i][r][1] = v.y; w[i][r][2] = v.z; w[i][r][3] = v.w;
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) w[i][r][s] = 0u;
                    if (live && n0 + r < N) {
                        const uint32_t* p = wrow + (uint32_t)(r * WR + wb);
                        if (aligned) {
                            const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
                            w[i][r][0] = v.x; w[i][r][1] = v.y; w[i][r][2] = v.z; w[i][r][3] = v.w;
                        } else {
#pragma unroll
                            for (int s = 0; s < 4; ++s) w[i][r][s] = (wb + s < WR) ? p[s] : 0u;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int wb = 4 * (ub + i * KS * kWave);
            const bool live = ub + i * KS * kWave < units;
            v4i a[MR][4];
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (live && m < M && wb + s < WR)
                        a[m][s] = *reinterpret_cast<const v4i*>(xq + (int64_t)m * K + 16 * (wb + s));
                    else
                        a[m][s] = v4i{0, 0, 0, 0};
                    spart[m] = byte_sum16(a[m][s], spart[m]);
                }
#pragma unroll
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const v4i c = unpack_codes(w[i][r][s]);
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        int d = part[r][m];
                        d = __builtin_amdgcn_sdot4(c.x, a[m][s].x, d, false);
                        d = __builtin_amdgcn_sdot4(c.y, a[m][s].y, d, false);
                        d = __builtin_amdgcn_sdot4(c.z, a[m][s].z, d, false);
                        d = __builtin_amdgcn_sdot4(c.w, a[m][s].w, d, false);
                        part[r][m] = d;
                    }
                }
            }
        }
    }

    // lane r (< R) collects row n0 + r for every token
    float yv[MR];
    int av[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        yv[m] = 0.f;
        av[m] = 0;
    }
    int tots[R][MR];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) tots[r][m] = wave_sum_dpp(part[r][m] - spart[m]);
    if constexpr (KS > 1) {
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < MR; ++m) s_part[wv][r][m] = tots[r][m];
        }
        __syncthreads();
        if (ks != 0) return;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                int t = 0;
#pragma unroll
                for (int k2 = 0; k2 < KS; ++k2) t += s_part[wv + k2][r][m];
                tots[r][m] = t;
            }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const float sc = (m < M) ? out_scale(beta, gamma[m]) : 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int tot = tots[r][m];
            if (lane == r) {
                av[m] = tot;
                yv[m] = (float)tot * sc;
            }
        }
    }
    const int n = n0 + lane;
    if (lane < R && n < N) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m < M) {
                if (y) y[(int64_t)m * N + n] = yv[m];
                if (acc_out) acc_out[(int64_t)m * N + n] = av[m];
            }
        }
    }
}

template <int MR, int R, int KS>
hipError_t launch_gvk(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                      int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    const int rows_per_block = kGvWaves / KS * R;
    const int blocks = (N + rows_per_block - 1) / rows_per_block;
    // one unit per lane in flight per row (batching two units per lane measured
    // slower at K = 8192: fewer waves fit and each waits longer)
    gemv_valu_kernel<MR, R, 1, KS><<<dim3(blocks), dim3(kGvThreads), 0, s>>>(xq, gamma, M, K, wp, N,
                                                                             beta, y, acc);
    return hipGetLastError();
}

// K slices per row group: up to 4 while the waves stay within 4096 and every
// slice gets units (a row longer than (KS - 1) * 64 units).  Measured at one
// token, K = 6912, N = 2560 (640 row groups of 4): 4.45 -> 4.03 us with 2.
template <int MR, int R>
hipError_t launch_gv(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                     int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    const int64_t groups = (N + R - 1) / R;
    const int units = ((K >> 4) + 3) >> 2;
    if (groups * 4 <= 4096 && units > 3 * kWave)
        return launch_gvk<MR, R, 4>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    if (groups * 2 <= 4096 && units > kWave)
        return launch_gvk<MR, R, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    return launch_gvk<MR, R, 1>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

}  // namespace

hipError_t launch_gemv_valu(const int8_t* xq, const float* gamma, int M, int K,
                            const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                            hipStream_t s) {
    if (M <= 1) return launch_gv<1, 4>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    if (M <= 2) return launch_gv<2, 4>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    return launch_gv<4, 4>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

}  // namespace bl

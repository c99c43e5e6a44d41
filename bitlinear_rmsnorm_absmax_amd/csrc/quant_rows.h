// Row-source loading and block reductions of the per-token quantisers, shared
// by the quantisation kernels and the fused quantise + one-token product, so
// both read a row in the same 16-element chunks, dealt to the same threads,
// and reduce absmax and the float64 sum of squares in the same order (the
// fused kernel's gamma is then bit-identical to the quantiser's).
#pragma once

#include "device_common.h"

namespace bl {

constexpr int kQuantThreads = 256;
constexpr int kQuantCache = 2;

// F32 / BF16: activations x.  SILU_MUL: h = SiLU(gate) * up from fp32 gate
// and up.  SILU_ACC: the same h from the int32 accumulators of one product
// with stacked gate and up weights, each half rescaled as the product would
// rescale it, fl32(acc) * fl32(beta * gamma_m) / 128.
enum class Src { F32, BF16, SILU_MUL, SILU_ACC };

struct RowSrc {
    const void* a;  // x (fp32 / bf16), gate (fp32) or the [M][2F] accumulators (int32)
    const float* b; // up (SILU_MUL only)
    const float* gamma = nullptr;  // SILU_ACC: per-row scale of the product's input
    float beta_a = 0.f;            // SILU_ACC: beta of the gate half
    float beta_b = 0.f;            // SILU_ACC: beta of the up half
};

// Load chunk c (16 elements) of row `row` (length K) as fp32.
template <Src S>
__device__ __forceinline__ void load_chunk(const RowSrc& src, int64_t row, int K, int c,
                                           float v[16]) {
    const int64_t base = row * (int64_t)K + (int64_t)c * 16;
    if constexpr (S == Src::F32) {
        const v4f* p = reinterpret_cast<const v4f*>(static_cast<const float*>(src.a) + base);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v4f t = __builtin_nontemporal_load(p + i);
            v[4 * i + 0] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
        }
    } else if constexpr (S == Src::BF16) {
        const v4u* p = reinterpret_cast<const v4u*>(static_cast<const uint16_t*>(src.a) + base);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            v4u t = __builtin_nontemporal_load(p + i);
            uint32_t d[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j + 0] = __uint_as_float(d[j] << 16);          // exact widening
                v[8 * i + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
            }
        }
    } else if constexpr (S == Src::SILU_ACC) {
        // row stride 2K: the gate half, then the up half of the stacked product
        const int64_t abase = row * 2 * (int64_t)K + (int64_t)c * 16;
        const int32_t* pa = static_cast<const int32_t*>(src.a);
        const float g = src.gamma[row];
        const float sg = out_scale(src.beta_a, g), su = out_scale(src.beta_b, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v4i ag = *reinterpret_cast<const v4i*>(pa + abase + 4 * i);
            const v4i au = *reinterpret_cast<const v4i*>(pa + abase + K + 4 * i);
            const int gi[4] = {ag.x, ag.y, ag.z, ag.w};
            const int ui[4] = {au.x, au.y, au.z, au.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float gate = (float)gi[j] * sg;
                const float up = (float)ui[j] * su;
                const double z = (double)gate;
                const double sl = z / (1.0 + exp(-z));
                v[4 * i + j] = (float)(sl * (double)up);
            }
        }
    } else {
        const float4* pg = reinterpret_cast<const float4*>(static_cast<const float*>(src.a) + base);
        const float4* pu = reinterpret_cast<const float4*>(src.b + base);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 g = pg[i];
            float4 u = pu[i];
            float gg[4] = {g.x, g.y, g.z, g.w};
            float uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // silu(z) * up in float64, rounded once to fp32
                double z = (double)gg[j];
                double sl = z / (1.0 + exp(-z));
                v[4 * i + j] = (float)(sl * (double)uu[j]);
            }
        }
    }
}

// Block-wide reductions: max of a float and sum of a double over the first NW
// waves of the block (kQuantThreads threads by default); every thread of the
// block calls it and gets the result.  Each participating wave reduces with
// an xor butterfly, then the wave results are combined in wave order.
template <int NW = kQuantThreads / kWave>
__device__ __forceinline__ void block_reduce(float& amax, double& ss, bool with_ss) {
    __shared__ float s_max[NW];
    __shared__ double s_ss[NW];
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    if (wv < NW) {
        amax = wave_max(amax);
        if (with_ss) ss = wave_sum_d(ss);
        if (lane == 0) {
            s_max[wv] = amax;
            s_ss[wv] = ss;
        }
    }
    __syncthreads();
    amax = s_max[0];
    ss = s_ss[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
        amax = fmaxf(amax, s_max[i]);
        ss += s_ss[i];
    }
}

}  // namespace bl

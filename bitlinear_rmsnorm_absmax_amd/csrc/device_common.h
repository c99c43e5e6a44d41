// Device helpers shared by the kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Per-token absmax code: the entry divided by gamma (one correctly rounded
// fp32 division), scaled by Qb = 128 (exact), rounded to nearest-even and
// clipped to [-127, 127].  gamma > 0 here; a zero token is handled by the
// caller.
__device__ __forceinline__ int quant_code(float x, float gamma) {
    float t = __fdiv_rn(x, gamma) * 128.0f;
    float r = __builtin_rintf(t);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// Four codes -> one dword of int8 lanes (byte b = code of element b).
__device__ __forceinline__ uint32_t pack4(int c0, int c1, int c2, int c3) {
    return (uint32_t)(c0 & 0xFF) | ((uint32_t)(c1 & 0xFF) << 8) | ((uint32_t)(c2 & 0xFF) << 16) |
           ((uint32_t)(c3 & 0xFF) << 24);
}

// Output scale of a token: fl32(beta * gamma) / 128 (the division is exact).
__device__ __forceinline__ float out_scale(float beta, float gamma) {
    return (beta * gamma) * 0.0078125f;
}

// Codes of packed word `w`: dword j holds the 2-bit codes (0, 1, 2) of
// weights 4j .. 4j+3 in its four bytes.
__device__ __forceinline__ v4i unpack_codes(uint32_t w) {
    v4i r;
    r.x = (int)(w & 0x03030303u);
    r.y = (int)((w >> 2) & 0x03030303u);
    r.z = (int)((w >> 4) & 0x03030303u);
    r.w = (int)((w >> 6) & 0x03030303u);
    return r;
}

// Sum of the 16 signed bytes of a v4i.
__device__ __forceinline__ int byte_sum16(v4i a, int acc) {
    acc = __builtin_amdgcn_sdot4(a.x, 0x01010101, acc, false);
    acc = __builtin_amdgcn_sdot4(a.y, 0x01010101, acc, false);
    acc = __builtin_amdgcn_sdot4(a.z, 0x01010101, acc, false);
    acc = __builtin_amdgcn_sdot4(a.w, 0x01010101, acc, false);
    return acc;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

}  // namespace bl

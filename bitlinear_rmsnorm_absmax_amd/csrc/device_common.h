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

// Signed weights w = c - 1 (-1, 0, +1) of packed word `w`, same byte order as
// unpack_codes: each masked code byte (0, 1, 2) selects byte c of the table
// 0x000100FF (v_perm_b32), giving 0xFF, 0x00 or 0x01.  A product on these
// needs no activation-sum correction.
__device__ __forceinline__ v4i unpack_signed(uint32_t w) {
    constexpr uint32_t kTable = 0x000100FFu;
    v4i r;
    r.x = (int)__builtin_amdgcn_perm(0u, kTable, w & 0x03030303u);
    r.y = (int)__builtin_amdgcn_perm(0u, kTable, (w >> 2) & 0x03030303u);
    r.z = (int)__builtin_amdgcn_perm(0u, kTable, (w >> 4) & 0x03030303u);
    r.w = (int)__builtin_amdgcn_perm(0u, kTable, (w >> 6) & 0x03030303u);
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

// Sum of an int over the 64 lanes of a wave with DPP row operations (quad
// permutes, then rotations by 4 and 8 inside each row of 16 lanes) and the
// four row results read back with v_readlane; the result is wave-uniform.
__device__ __forceinline__ int wave_sum_dpp(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false);  // row_ror:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Maximum of a non-negative float over the 64 lanes of a wave, with the DPP
// pattern of wave_sum_dpp (fmaxf: a NaN loses to a number, as in fmaxf
// chains); the result is wave-uniform.
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Copy 16 bytes per lane from global memory straight into LDS at
// lds_wave_base + 16 * lane (global_load_lds_dwordx4; the base is
// wave-uniform and goes to M0).  The builtin exists only in the device pass;
// the host pass compiles kernels to launch stubs and must not see it.
__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base,
                                     16, 0, 0);
#endif
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

}  // namespace bl

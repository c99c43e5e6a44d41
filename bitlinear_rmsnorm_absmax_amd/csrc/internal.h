// Internal declarations shared by the host dispatch (api.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// Every launcher validates nothing (api.cpp does) and returns the launch
// status (hipGetLastError after the launch).

hipError_t launch_quant_act(const void* x, int bf16, int64_t M, int64_t K, const float* gain,
                            float eps, int8_t* q, float* gamma, hipStream_t s);

hipError_t launch_silu_mul_quant(const float* gate, const float* up, int64_t M, int64_t F,
                                 float* h, int8_t* h_q, float* gamma, hipStream_t s);

hipError_t launch_pack(const int8_t* w, int64_t N, int64_t K, uint32_t* packed, int32_t* bad,
                       hipStream_t s);

// y (and acc when non-NULL) = 0 for K == 0.
hipError_t launch_fill_zero(float* y, int32_t* acc, int64_t count, hipStream_t s);

// Path 1: VALU dot4 GEMV, M <= 8.
hipError_t launch_gemv_valu(const int8_t* xq, const float* gamma, int M, int K,
                            const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                            hipStream_t s);

// Path 2: skinny int8 MFMA (M padded to 16-row tiles), M <= 64.
hipError_t launch_skinny_mfma(const int8_t* xq, const float* gamma, int M, int K,
                              const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                              hipStream_t s);

// Decode product with the activation block staged in LDS (5 <= M <= 16,
// K % 256 == 0); decode_lds_supports() tells whether a shape fits.
bool decode_lds_supports(int M, int K, int N);
hipError_t launch_decode_lds(const int8_t* xq, const float* gamma, int M, int K,
                             const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                             hipStream_t s);

// Path 3: LDS-tiled int8 MFMA GEMM.  The LDS-ring variant needs K % 128 == 0.
bool gemm_dma_supports(int M, int K, int N);

// Absmean ternarisation + packing (three stream-ordered launches; the packed
// buffer holds the per-row sums in between, so K >= 32).
hipError_t launch_ternarize(const float* W, int64_t N, int64_t K, uint32_t* packed, int8_t* codes,
                            float* beta32, double* beta64, hipStream_t s);
hipError_t launch_gemm_dma(const int8_t* xq, const float* gamma, int M, int K,
                           const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                           hipStream_t s);
hipError_t launch_gemm_mfma(const int8_t* xq, const float* gamma, int M, int K,
                            const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                            hipStream_t s);

}  // namespace bl

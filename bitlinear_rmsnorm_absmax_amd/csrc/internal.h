// Internal declarations shared by the host dispatch (api.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

namespace bl {

// Opt-in of one kernel to more than 64 KB of dynamic LDS, made once per
// device (the attribute belongs to the calling thread's current device, the
// device of the launch's stream in the usual setup).  The dynamic maximum
// set is `bytes`, at most the compute unit's 160 KB less the kernel's static
// LDS (hipFuncGetAttributes): the two together may not exceed it.  One
// object per kernel (a function-local static of its launcher); concurrent
// first calls may both set the attribute, which is idempotent.
class DynLdsOptIn {
  public:
    hipError_t ensure(const void* kernel, int bytes) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < kMaxDevices && done_[dev].load(std::memory_order_acquire)) return hipSuccess;
        hipFuncAttributes attr{};
        e = hipFuncGetAttributes(&attr, kernel);
        if (e != hipSuccess) return e;
        const int cap = 160 * 1024 - (int)attr.sharedSizeBytes;
        e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                bytes < cap ? bytes : cap);
        if (e == hipSuccess && dev >= 0 && dev < kMaxDevices) done_[dev].store(true, std::memory_order_release);
        return e;
    }

  private:
    static constexpr int kMaxDevices = 64;
    std::atomic<bool> done_[kMaxDevices] = {};
};

// Every launcher validates nothing (api.cpp does) and returns the launch
// status (hipGetLastError after the launch).

hipError_t launch_quant_act(const void* x, int bf16, int64_t M, int64_t K, const float* gain,
                            float eps, int8_t* q, float* gamma, hipStream_t s);
// Workgroups per row launch_quant_act uses (1: one workgroup per row).
int quant_split_ways(int64_t M, int64_t K);

// Fused quantisation + one-token product (quant_gemv.hip): M == 1,
// K % 64 == 0, K <= kFusedMaxK (the codes are staged in LDS), N <= kFusedMaxN.
constexpr int kFusedMaxK = 16384;
constexpr int kFusedMaxN = 16384;
bool quant_gemv_supports(int M, int K, int N);
hipError_t launch_quant_gemv(const void* x, bool bf16, int K, const float* gain, float eps,
                             const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                             int8_t* q_out, float* gamma_out, hipStream_t s);

hipError_t launch_silu_mul_quant(const float* gate, const float* up, int64_t M, int64_t F,
                                 float* h, int8_t* h_q, float* gamma, hipStream_t s);
// The same from the int32 accumulators [M][2F] of one product with stacked
// gate and up weights (gate half, then up half of each row).
hipError_t launch_silu_mul_quant_acc(const int32_t* acc_gu, const float* gamma_in, int64_t M,
                                     int64_t F, float beta_gate, float beta_up, float* h,
                                     int8_t* h_q, float* gamma, hipStream_t s);

hipError_t launch_pack(const int8_t* w, int64_t N, int64_t K, uint32_t* packed, int32_t* bad,
                       hipStream_t s);

// y (and acc when non-NULL) = 0 for K == 0.
hipError_t launch_fill_zero(float* y, int32_t* acc, int64_t count, hipStream_t s);

// Path 1: VALU dot4 GEMV, M <= 4 (the ABI's limit; one pass over the weights).
// Forward launchers: y == nullptr stores only the accumulators (acc).
hipError_t launch_gemv_valu(const int8_t* xq, const float* gamma, int M, int K,
                            const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                            hipStream_t s);

// Path 2: skinny int8 MFMA (M padded to 16-row tiles), M <= 64.
hipError_t launch_skinny_mfma(const int8_t* xq, const float* gamma, int M, int K,
                              const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                              hipStream_t s);

// Decode product with the activation block staged in LDS (M <= 16,
// K % 256 == 0); decode_lds_supports() tells whether a shape fits.  Its
// shape rules (shapes.cpp): eight waves a workgroup, at most 160 KB of LDS.
constexpr int kDecWaves = 8;
constexpr int kDecLdsMax = 160 * 1024;
int decode_a_bytes(int M, int K);
size_t decode_lds_bytes(int M, int K, int ntw, int G = 1);
int grouped_width(int tiles, int G, int nchunks);
bool decode_lds_supports(int M, int K, int N);
// One token quantised inside the decode kernel (fp32 or bf16 row, optional
// RMSNorm gain) and multiplied, when decode_one_token(K, N): x_q and gamma
// are written, bit-identical to bitlinear_quant_act's.
hipError_t launch_quant_decode1(const void* x, bool bf16, int K, const float* gain, float eps,
                                const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                                int8_t* x_q, float* gamma, hipStream_t s);
// Whether one token runs on the decode kernel instead of the VALU GEMV
// (2-bit or 1-bit weights).
bool decode_one_token(int K, int N, bool onebit = false);
hipError_t launch_decode_lds(const int8_t* xq, const float* gamma, int M, int K,
                             const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                             hipStream_t s);
// Same kernel on 1-bit weights [N][K/32].
// Grouped decode product in one launch (group-major x_q [G][M][K/G],
// gamma [G][M], packed weights [G][N][K/G/16], beta [G] on the device; acc
// [G][M][N] and y written), when decode_lds_grouped_supports() holds.
bool decode_lds_grouped_supports(int M, int K, int G, int N);
hipError_t launch_decode_lds_grouped(const int8_t* xq, const float* gamma, int M, int K, int G,
                                     const uint32_t* wp, int N, const float* beta_g, float* y,
                                     int32_t* acc, hipStream_t s);
hipError_t launch_decode_lds1(const int8_t* xq, const float* gamma, int M, int K,
                              const uint32_t* wp1, int N, float beta, float* y, int32_t* acc,
                              hipStream_t s);

// Path 3: LDS-tiled int8 MFMA GEMM.  The LDS-ring variant needs K % 128 == 0.
bool gemm_dma_supports(int M, int K, int N);

// Pairwise double mean of |W| (abs_values) or W over L = N*K entries, leaf
// groups of `group` (64 or 256) entries; scratch of pairwise_scratch_bytes().
hipError_t launch_pairwise_mean(const float* W, int64_t L, int64_t N, int64_t K, bool abs_values,
                                int group, double* scratch, double* mean64, float* mean32,
                                hipStream_t s);
size_t pairwise_scratch_bytes(int64_t L, int group);

// 1-bit weights: binarisation Sign(W - alpha) + packing (the partial sums live
// in the int8 code output), packing of +-1 weights, and the decode product
// (groups of up to four tokens per pass over the weights; K % 64 == 0).
hipError_t launch_binarize(const float* W, int64_t N, int64_t K, uint32_t* packed1, int8_t* codes,
                           double* alpha64, float* alpha32, double* beta64, float* beta32,
                           hipStream_t s);
hipError_t launch_pack1(const int8_t* w, int64_t N, int64_t K, uint32_t* packed1, int* bad_count,
                        hipStream_t s);
hipError_t launch_forward1(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                           int N, float beta, float* y, int32_t* acc, hipStream_t s);

// Absmean ternarisation + packing (stream-ordered launches; the packed buffer
// holds the partial sums in between, so K >= 32).
hipError_t launch_ternarize(const float* W, int64_t N, int64_t K, uint32_t* packed, int8_t* codes,
                            float* beta32, double* beta64, hipStream_t s);
// Group quantisation: q [G][M][K/G], gamma [G][M] (K/G % 16 == 0).
hipError_t launch_quant_act_grouped(const void* x, int bf16, int64_t M, int64_t K, int64_t G,
                                    const float* gain, float eps, int8_t* q, float* gamma,
                                    hipStream_t s);
// y = sum over g of fl32(acc[g]) * fl32(beta[g] * gamma[g][m]) / 128 (beta on the device).
hipError_t launch_group_sum(const int32_t* acc, const float* gamma, const float* beta, int64_t M,
                            int64_t N, int64_t G, float* y, hipStream_t s);
// Base-3 weights (1.6 bits): packing [N][ceil(K/80)][16 bytes] and the
// decode product: 2..16 tokens on int8 MFMA with the activation block staged
// in LDS (gemv3_mfma_kernel), one token -- and blocks too large for LDS, in
// passes of up to four tokens -- on the vector ALUs (gemv3_kernel).
hipError_t launch_pack3(const int8_t* w, int64_t N, int64_t K, uint32_t* packed3, int* bad_count,
                        hipStream_t s);
hipError_t launch_forward3(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                           int N, float beta, float* y, int32_t* acc, hipStream_t s);
hipError_t launch_gemm_dma(const int8_t* xq, const float* gamma, int M, int K,
                           const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                           hipStream_t s);
hipError_t launch_gemm_mfma(const int8_t* xq, const float* gamma, int M, int K,
                            const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                            hipStream_t s);

// Measurement floors (floor.hip): an empty kernel, and a read-only pass over
// `bytes` (a multiple of 16) at p (16-byte aligned).
hipError_t launch_floor_empty(hipStream_t s);
hipError_t launch_floor_stream_read(const void* p, int64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_floor_mfma(const int8_t* xq, int M, int K, const uint32_t* wp, int N,
                             uint32_t* sink, hipStream_t s);

}  // namespace bl

/*
 * CPU oracle for the ternary BitLinear layer: TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct loops that restate the published formulas.
 * Only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library; the product path never does.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * Sources (cited by title and section):
 *   [U] "Microsofts Inference Framework bringt 1-Bit große Sprachmodelle auf
 *       lokale Geräte" (unite.ai), section "Mathematische Grundlagen":
 *       2. Aktivierungsquantisierung and 3. BitLinear-Betrieb; section
 *       "Ternäres Gewichtssystem / Das Konzept".
 *   [D] "MatMul-free language models" (datacamp.com, Dutch), sections
 *       "MatMul vervangen door ternaire bewerkingen" (also the absmean
 *       ternarisation) and "Kerncomponenten: MLGRU EN GLU".
 *
 * Parity status: every function below is pinned by the CPU tests except the
 * float64 SiLU evaluation, whose transcendental is checked only through
 * identities and limits (parity unpinned beyond those).
 */
#ifndef BITLINEAR_ORACLE_H
#define BITLINEAR_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* bf16 bit patterns -> fp32 by exact widening. */
void oracle_bf16_to_f32(const uint16_t* in, int64_t n, float* out);

/* Per-token absmax int8 quantisation, [U] 2. Aktivierungsquantisierung.
 * x fp32 [M][K] -> q int8 [M][K], gamma fp32 [M]. */
void oracle_quant_act(const float* x, int64_t M, int64_t K, int8_t* q, float* gamma);

/* RMSNorm ([D] RMS norm before quantisation) followed by the quantiser above.
 * g fp32 [K] is the gain; eps the fp32 epsilon. */
void oracle_rmsnorm_quant_act(const float* x, const float* g, float eps, int64_t M,
                              int64_t K, int8_t* q, float* gamma);

/* Group quantisation ([U] Gruppenquantisierung und -normalisierung): the K
 * inputs split into G equal runs, each run of each token quantised with its
 * own absmax scale.  gain NULL = no RMSNorm.  q int8 [G][M][K/G],
 * gamma fp32 [G][M] (group-major).  K % G == 0. */
void oracle_quant_act_grouped(const float* x, const float* gain, float eps, int64_t M,
                              int64_t K, int64_t G, int8_t* q, float* gamma);

/* Literal RMSNorm-then-quantise evaluated in float64 (informational). */
void oracle_rmsnorm_quant_act_literal(const float* x, const float* g, float eps,
                                      int64_t M, int64_t K, int8_t* q, double* gamma);

/* 2-bit code packing of ternary weights w int8 [N][K] -> uint32 [N][K/16].
 * Returns the number of entries outside {-1,0,+1}. */
int64_t oracle_pack(const int8_t* w, int64_t N, int64_t K, uint32_t* packed);

/* Inverse of oracle_pack (code 3 unpacks to 2, an out-of-range marker). */
void oracle_unpack(const uint32_t* packed, int64_t N, int64_t K, int8_t* w);

/* acc[m][n] = sum_k w[n][k] * q[m][k]  ([U] 3. BitLinear-Betrieb, [D] ternary
 * accumulation).  Returns 0, or 1 if a result does not fit int32. */
int oracle_accumulate(const int8_t* q, int64_t M, int64_t K, const int8_t* w,
                      int64_t N, int32_t* acc);

/* y[m][n] = acc[m][n] * beta * gamma[m] / 128, float64 then rounded to fp32. */
void oracle_rescale(const int32_t* acc, const float* gamma, int64_t M, int64_t N,
                    float beta, float* y);

/* h[i] = silu(gate[i]) * up[i] in float64 ([D] MatMul-vrije GLU). */
void oracle_silu_mul(const float* gate, const float* up, int64_t n, double* h);

/* Absmean ternarisation ([D] MatMul vervangen door ternaire bewerkingen: the
 * weight matrix is scaled by its mean absolute value and every entry rounded
 * to the nearest of -1, 0, 1).  beta64 = S / (N*K) with S the pairwise sum in
 * double of |W| over the row-major entries (a run splits after the largest
 * power of two below its length).  Entry code: +1 if W > beta64/2, -1 if
 * W < -beta64/2, else 0, compared exactly in double, which is
 * round-half-even of W/beta64 clipped to [-1, 1] (a tie |W| = beta/2 rounds
 * to 0).  beta64 = 0 gives all zeros.  Returns beta64. */
double oracle_ternarize(const float* W, int64_t N, int64_t K, int8_t* w);

/* Weight binarisation ([U] Mathematische Grundlagen, 1. Gewichtsbinarisierung:
 * W_f = Sign(W - alpha) with alpha the mean of the weights and Sign(v) = +1 for
 * v > 0, else -1).  alpha64 = pairwise double sum of W (row-major, as in
 * oracle_ternarize) / (N*K); code = +1 if W > alpha64 (exact comparison in
 * double), else -1, so W == alpha64 gives -1.  Returns alpha64. */
double oracle_binarize(const float* W, int64_t N, int64_t K, int8_t* w);

/* 1-bit packing of +-1 weights: word n*(K/32) + k/32 holds entry e = k mod 32
 * = 4j + b (j = e / 4, b = e mod 4) at bit 8b + j as (w + 1) / 2, so
 * (word >> j) & 0x01010101 gives the bits of entries 4j .. 4j+3 in bytes
 * 0 .. 3.  K % 32 == 0.  Returns the number of entries not in {-1, +1}
 * (packed as 0 bits). */
int64_t oracle_pack1(const int8_t* w, int64_t N, int64_t K, uint32_t* packed);
void oracle_unpack1(const uint32_t* packed, int64_t N, int64_t K, int8_t* w);

/* Number of OpenMP threads the accumulate loop runs on. */
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

/* Base-3 packing, 1.6 bits per weight ([U] Ternäres Gewichtssystem: about
 * 1.58 bits carry three states; 3^5 = 243 fits a byte).  Ternary w int8
 * [N][K] -> bytes [N][ceil(K/80)][16]: byte b of word w of unit u holds the
 * weights k = 80u + 20w + 4i + b, i = 0..4, as v = sum (w_k + 1) 3^(4-i),
 * stored as ceil(256 v / 243); weights past K are 0.  Returns the number of
 * entries outside {-1, 0, 1} (packed as 0). */
int64_t oracle_pack3(const int8_t* w, int64_t N, int64_t K, uint8_t* packed);

/* Inverse of oracle_pack3: v = floor(243 b / 256), then base-3 digits. */
void oracle_unpack3(const uint8_t* packed, int64_t N, int64_t K, int8_t* w);

#ifdef __cplusplus
}
#endif
#endif

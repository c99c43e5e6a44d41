/*
 * bitlinear.h -- C ABI of the MI355X (gfx950) ternary BitLinear library.
 *
 * The layer (following "Microsofts Inference Framework bringt 1-Bit große
 * Sprachmodelle auf lokale Geräte" (unite.ai), Mathematische Grundlagen,
 * 2. Aktivierungsquantisierung and 3. BitLinear-Betrieb, and "MatMul-free
 * language models" (datacamp.com), MatMul vervangen door ternaire
 * bewerkingen / Kerncomponenten: MLGRU EN GLU):
 *
 *   gamma_m = max_k |x_mk|                       (per token)
 *   q_mk    = clamp(rne(fl32(x_mk / gamma_m) * 128), -127, 127), 0 if gamma_m = 0
 *   acc_mn  = sum_k w_nk * q_mk                  (w in {-1, 0, +1}, exact int32)
 *   y_mn    = fl32(acc_mn) * (fl32(beta * gamma_m) / 128)
 *
 * Conventions shared by every entry point:
 *  - Every pointer argument is a DEVICE pointer (memory from hipMalloc or a
 *    torch CUDA/HIP tensor) unless stated otherwise.  Matrices are row-major
 *    and contiguous.  The caller owns all memory; the library never
 *    allocates, frees or retains it.
 *  - All calls are asynchronous on `stream` (0 = the null stream).  The
 *    returned status covers argument validation, which runs on the host
 *    before anything is launched (nothing is written on a validation error),
 *    and the launch itself.  A fault inside a kernel surfaces at the caller's
 *    next synchronisation, as usual in HIP.
 *  - Sizes are int64_t; M, N, K may be 0 (empty work).  N (weight rows) is
 *    at most 2^30.  K, the reduction
 *    length, must be a multiple of 16 and at most 131072, so |acc| <= 127*K
 *    < 2^24 and fl32(acc) is exact.
 *  - Pointers to int8 / packed data and to the activations x must be 16-byte
 *    aligned; float / int32 vectors must be 4-byte aligned.
 *  - No C++ exception crosses the boundary.  On a non-OK status,
 *    bitlinear_last_error() returns a message (thread-local).
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Packed-weight layout version; bumps whenever the layout below changes. */
#define BITLINEAR_ABI_VERSION 1
#define BITLINEAR_MAX_K 131072

typedef enum {
    BITLINEAR_OK = 0,
    BITLINEAR_ERR_NULL = 1,   /* a required pointer is NULL                       */
    BITLINEAR_ERR_SHAPE = 2,  /* negative size, K % 16 != 0, K > BITLINEAR_MAX_K   */
    BITLINEAR_ERR_ALIGN = 3,  /* a pointer violates the alignment rule above        */
    BITLINEAR_ERR_DTYPE = 4,  /* unknown bitlinear_dtype_t                          */
    BITLINEAR_ERR_HIP = 5,    /* the HIP runtime reported an error at launch        */
    BITLINEAR_ERR_VALUE = 6   /* an argument value outside its domain (path id,
                                 non-finite beta, negative or non-finite eps)       */
} bitlinear_status_t;

typedef enum { BITLINEAR_F32 = 0, BITLINEAR_BF16 = 1 } bitlinear_dtype_t;

/* Forward kernel choice for bitlinear_forward_path. */
typedef enum {
    BITLINEAR_PATH_AUTO = 0,    /* pick by M (what bitlinear_forward does)          */
    BITLINEAR_PATH_GEMV = 1,    /* VALU dot4 GEMV, lanes reduced with DPP; M <= 4   */
    BITLINEAR_PATH_SKINNY = 2,  /* int8 MFMA with M padded to 16-row tiles; M <= 64 */
    BITLINEAR_PATH_GEMM = 3     /* LDS-tiled int8 MFMA GEMM; any M                  */
} bitlinear_path_t;

/*
 * Per-token absmax int8 activation quantisation (unite.ai article,
 * Mathematische Grundlagen, 2. Aktivierungsquantisierung; Qb = 2^(8-1) = 128,
 * gamma = infinity norm of the token, codes clipped to [-127, 127], rounding
 * to nearest with ties to even), optionally after RMSNorm (datacamp article,
 * Kerncomponenten: the RMS norm that normalises activations before they are
 * quantised).
 *
 *   x        [M][K] activations, fp32 or bf16 (x_dtype); bf16 is widened exactly.
 *   rms_gain NULL: no normalisation.  Else fp32 [K] gain g of
 *            RMSNorm(x) = g * x / sqrt(mean(x^2) + rms_eps).  The quantiser
 *            divides by the absmax of its input, so the RMS factor cancels
 *            from the codes: q is computed from u = fl32(g * x) and gamma_m =
 *            fl32(r_m * max|u|) with r_m = 1/sqrt(mean_k x_mk^2 + eps)
 *            evaluated in float64.
 *   rms_eps  >= 0 and finite (ignored without rms_gain).
 *   x_q      out [M][K] int8 codes.
 *   gamma    out [M] fp32 per-token scale (0 for an all-zero token).
 * Preconditions: finite inputs.
 */
bitlinear_status_t bitlinear_quant_act(const void* x, bitlinear_dtype_t x_dtype, int64_t M,
                                       int64_t K, const float* rms_gain, float rms_eps,
                                       int8_t* x_q, float* gamma, hipStream_t stream);

/*
 * Packs ternary weights (unite.ai article, Ternäres Gewichtssystem / Das
 * Konzept: each weight is one of -1, 0, +1) at 2 bits each.
 *
 *   w        [N][K] int8, entries in {-1, 0, +1}.
 *   w_packed out [N][K/16] uint32.  code = w + 1 (-1 -> 0, 0 -> 1, +1 -> 2);
 *            weight k of row n sits in word n*(K/16) + k/16 at bit
 *            8*b + 2*j where e = k % 16 = 4*j + b.  So (word >> 2j) & 0x03030303
 *            holds the codes of weights 4j .. 4j+3 in bytes 0..3.  An entry
 *            outside {-1, 0, +1} is stored as code 3 and counted.
 *   bad_count optional device int32: set to the number of entries outside
 *            {-1, 0, +1} (no host synchronisation).  NULL to skip.
 */
bitlinear_status_t bitlinear_pack_weights(const int8_t* w, int64_t N, int64_t K,
                                          uint32_t* w_packed, int32_t* bad_count,
                                          hipStream_t stream);

/*
 * BitLinear forward on quantised activations (unite.ai article, 3.
 * BitLinear-Betrieb: ternary weights times quantised activations, rescaled by
 * beta * gamma / Qb; datacamp article: the products become additions,
 * subtractions and skips).
 *
 *   x_q, gamma  outputs of bitlinear_quant_act ([M][K] int8, [M] fp32).
 *   w_packed    [N][K/16] from bitlinear_pack_weights (16-byte aligned).
 *   beta        per-tensor fp32 weight scale (finite).
 *   y           out [M][N] fp32; may be NULL when acc is given (then only the
 *               accumulators are written, e.g. for bitlinear_silu_mul_quant_acc).
 *   acc         optional out [M][N] int32 accumulators; NULL to skip.
 * The result does not depend on which kernel runs (bit-identical acc and y).
 */
bitlinear_status_t bitlinear_forward(const int8_t* x_q, const float* gamma, int64_t M, int64_t K,
                                     const uint32_t* w_packed, int64_t N, float beta, float* y,
                                     int32_t* acc, hipStream_t stream);

/*
 * The whole BitLinear forward from unquantised activations: bitlinear_quant_act
 * followed by bitlinear_forward (datacamp article, Kerncomponenten: RMS norm,
 * absmax quantisation, ternary product; unite.ai article, 2.
 * Aktivierungsquantisierung and 3. BitLinear-Betrieb).  Arguments as in those
 * two calls; x_q and gamma are outputs here and are written in every case.
 * One token runs as one kernel in which each workgroup quantises the token
 * into LDS and multiplies its weight rows: on the MFMA decode kernel when
 * K >= 4096, K % 512 == 0 and N / 64 >= 150 (long rows over many row tiles),
 * else on the vector ALUs when K % 64 == 0, K <= 16384 and N <= 16384;
 * otherwise the two calls run in order on `stream`.  x_q, gamma, y and acc are
 * bit-identical to those of the two calls; y may be NULL when acc is given.
 */
bitlinear_status_t bitlinear_quant_forward(const void* x, bitlinear_dtype_t x_dtype, int64_t M,
                                           int64_t K, const float* rms_gain, float rms_eps,
                                           const uint32_t* w_packed, int64_t N, float beta,
                                           int8_t* x_q, float* gamma, float* y, int32_t* acc,
                                           hipStream_t stream);

/* 1 if bitlinear_quant_forward runs this shape as one kernel, else 0 (the two
 * calls).  Host-only, no HIP call. */
int bitlinear_quant_forward_one_launch(int64_t M, int64_t K, int64_t N);

/* bitlinear_forward with an explicit kernel (bitlinear_path_t).  A path that
 * cannot take this M (GEMV: M > 4, SKINNY: M > 64) returns BITLINEAR_ERR_VALUE. */
bitlinear_status_t bitlinear_forward_path(const int8_t* x_q, const float* gamma, int64_t M,
                                          int64_t K, const uint32_t* w_packed, int64_t N,
                                          float beta, float* y, int32_t* acc, int path,
                                          hipStream_t stream);

/*
 * GLU glue of the MatMul-free channel mixer (datacamp article, Kerncomponenten:
 * one projection passes through SiLU and multiplies the other elementwise;
 * the product feeds the next BitLinear layer), followed by the per-token
 * absmax quantisation of bitlinear_quant_act.
 *
 *   gate, up  [M][F] fp32 (outputs of the gate and up projections).
 *   h         optional out [M][F] fp32: h = silu(gate) * up, evaluated in
 *             float64 (silu(z) = z / (1 + e^-z)) and rounded once to fp32.
 *             NULL to skip.
 *   h_q       out [M][F] int8 codes of h; gamma_h out [M] fp32.
 * F follows the rules of K (multiple of 16, at most 131072).
 */
bitlinear_status_t bitlinear_silu_mul_quant(const float* gate, const float* up, int64_t M,
                                            int64_t F, float* h, int8_t* h_q, float* gamma_h,
                                            hipStream_t stream);

/*
 * The same GLU glue when the gate and up projections are one product with the
 * two weight matrices stacked along N ([W_gate; W_up], 2F rows, one packed
 * buffer) and that product wrote only its accumulators (bitlinear_forward with
 * y = NULL): one launch and one weight stream for both projections.
 *
 *   acc_gu     [M][2F] int32: row m holds the F gate accumulators, then the F
 *              up accumulators.
 *   gamma      [M] fp32 scale of the product's input (from bitlinear_quant_act).
 *   beta_gate, beta_up  per-tensor scales of the two weight matrices (finite).
 * gate and up are rescaled exactly as bitlinear_forward rescales,
 * fl32(acc) * fl32(beta * gamma_m) / 128, then h, h_q and gamma_h follow
 * bitlinear_silu_mul_quant: the outputs are bit-identical to running the two
 * projections separately and bitlinear_silu_mul_quant on their outputs.
 */
bitlinear_status_t bitlinear_silu_mul_quant_acc(const int32_t* acc_gu, const float* gamma,
                                                int64_t M, int64_t F, float beta_gate,
                                                float beta_up, float* h, int8_t* h_q,
                                                float* gamma_h, hipStream_t stream);

/*
 * bitlinear_ternarize -- absmean ternarisation of full-precision weights,
 * then packing (datacamp article "MatMul-free language models", section
 * "MatMul vervangen door ternaire bewerkingen": the weight matrix is scaled
 * by its mean absolute value and every entry rounded to the nearest of -1, 0,
 * 1).  The step before bitlinear_pack_weights for weights that are not yet
 * ternary.
 *
 *   beta64 = S / (N*K), S = pairwise sum in double of |W| over the
 *            row-major entries (a run of entries splits after the largest
 *            power of two below its length)
 *   code   = +1 if W > beta64/2, -1 if W < -beta64/2, else 0 (compared
 *            exactly in double: round-half-even of W/beta64 clipped to
 *            [-1, 1]; |W| = beta64/2 gives 0; beta64 = 0 gives all zeros)
 *
 * W          device fp32 [N][K] row-major, 16-byte aligned, finite.
 * w_packed   device uint32 [N][K/16] out, the codes packed as by
 *            bitlinear_pack_weights.  While the call runs it also holds the
 *            partial sums (about N*K/8 bytes), hence K >= 32.
 * w_ternary  device int8 [N][K] out (the codes), 16-byte aligned; may be NULL.
 * beta       device fp32 [1] out: fl32(beta64), the scale bitlinear_forward takes.
 * beta64     device double [1] out: the mean itself.
 * N, K       N >= 0; K == 0 or (K >= 32 and K % 16 == 0), K <= BITLINEAR_MAX_K;
 *            N*K == 0 writes beta = beta64 = 0 and nothing else.
 * Cost: W is read twice (sum, then codes).  3 + ceil(log64(N*K/4096))
 * launches on `stream`; none allocates.
 */
bitlinear_status_t bitlinear_ternarize(const float* W, int64_t N, int64_t K, uint32_t* w_packed,
                                       int8_t* w_ternary, float* beta, double* beta64,
                                       hipStream_t stream);

/*
 * 1-bit weights (unite.ai article "Microsofts Inference Framework bringt 1-Bit
 * große Sprachmodelle auf lokale Geräte", section "Mathematische Grundlagen",
 * 1. Gewichtsbinarisierung: W_f = Sign(W - alpha), alpha the mean of the
 * weights, Sign(v) = +1 for v > 0 and -1 otherwise).
 *
 * 1-bit packed layout: uint32 [N][K/32]; word n*(K/32) + k/32 holds entry
 * e = k mod 32 = 4j + b at bit 8b + j as (w + 1) / 2 (so +1 -> 1, -1 -> 0).
 * The +-1 codes are also valid ternary codes: bitlinear_pack_weights turns
 * them into the 2-bit layout for bitlinear_forward (the path for many tokens).
 */

/*
 * bitlinear_binarize -- alpha64 = pairwise double sum of W over the row-major
 * entries (as in bitlinear_ternarize) / (N*K); code = +1 if W > alpha64
 * (exact comparison in double), else -1 (W == alpha64 gives -1).  Also the
 * scale beta64 = mean |W| (the absmean of bitlinear_ternarize).
 *
 * W          device fp32 [N][K] row-major, 16-byte aligned, finite.
 * w_packed1  device uint32 [N][K/32] out (1-bit layout), 4-byte aligned.
 * w_codes    device int8 [N][K] out, the +-1 codes, 16-byte aligned.  While
 *            the call runs it also holds the partial sums of both means.
 * alpha, beta      device fp32 [1] out: fl32(alpha64), fl32(beta64).
 * alpha64, beta64  device double [1] out.
 * N, K       N >= 0; K % 32 == 0, K <= BITLINEAR_MAX_K; N*K == 0 writes the
 *            four scalars as 0 and nothing else.
 */
bitlinear_status_t bitlinear_binarize(const float* W, int64_t N, int64_t K, uint32_t* w_packed1,
                                      int8_t* w_codes, float* alpha, double* alpha64, float* beta,
                                      double* beta64, hipStream_t stream);

/*
 * bitlinear_pack_weights1 -- +-1 int8 weights [N][K] (device, 16-byte aligned,
 * K % 32 == 0) -> the 1-bit layout [N][K/32].  bad_count (optional device
 * int32) receives the number of entries that are not +-1 (packed as -1).
 */
bitlinear_status_t bitlinear_pack_weights1(const int8_t* w, int64_t N, int64_t K,
                                           uint32_t* w_packed1, int32_t* bad_count,
                                           hipStream_t stream);

/*
 * bitlinear_forward1 -- bitlinear_forward on 1-bit weights: acc_mn =
 * sum_k w_nk q_mk with w in {-1, +1}, y = fl32(acc) * (fl32(beta * gamma_m)/128).
 * Arguments as for bitlinear_forward; w_packed1 is [N][K/32] in the 1-bit
 * layout (8-byte aligned) and K % 64 == 0.  A decode product: 5..16 tokens
 * (K % 256 == 0, activations fitting in LDS) run on int8 MFMA, other counts
 * on the vector ALUs with one pass over the weights per four tokens; for many
 * tokens pack the codes for bitlinear_forward.
 */
bitlinear_status_t bitlinear_forward1(const int8_t* x_q, const float* gamma, int64_t M, int64_t K,
                                      const uint32_t* w_packed1, int64_t N, float beta, float* y,
                                      int32_t* acc, hipStream_t stream);

/*
 * Group quantisation (unite.ai article, section "Gruppenquantisierung und
 * -normalisierung": weights and activations are divided into G groups and
 * the quantisation parameters are estimated per group instead of for the
 * whole matrix, so the groups need no communication).  Groups split the K
 * inputs into G equal runs of KG = K/G: token m's run g has its own absmax
 * scale gamma[g][m], weight group g (input columns g*KG .. (g+1)*KG) its own
 * scale beta[g], each group is a BitLinear product of its own, and the layer
 * output is the sum of the G group outputs.  All grouped operands are
 * group-major, so group g of each is one contiguous block (the layout a
 * per-group shard would hold).
 */

/* Activations of the grouped layer: the quantiser of bitlinear_quant_act per
 * run.  x [M][K] fp32/bf16 as for bitlinear_quant_act; x_q out int8
 * [G][M][KG] (16-byte aligned); gamma out fp32 [G][M].  With rms_gain the
 * RMSNorm factor r is the token's whole-row factor and gamma[g][m] =
 * fl32(r * max over the run of |gain * x|).  Requires G >= 1, K % G == 0,
 * KG % 16 == 0.  K == 0 writes gamma = 0.  One launch. */
bitlinear_status_t bitlinear_quant_act_grouped(const void* x, bitlinear_dtype_t x_dtype, int64_t M,
                                               int64_t K, int64_t G, const float* rms_gain,
                                               float rms_eps, int8_t* x_q, float* gamma,
                                               hipStream_t stream);

/* Grouped product:
 *   acc[g][m][n] = sum over k < KG of w_g[n][k] * x_q[g][m][k]  (exact int32)
 *   y[m][n]      = sum over g (in order g = 0 .. G-1, fp32) of
 *                  fl32(acc[g][m][n]) * (fl32(beta[g] * gamma[g][m]) / 128)
 * x_q [G][M][KG] int8 and gamma [G][M] from bitlinear_quant_act_grouped.
 * w_packed uint32 [G][N][KG/16]: group g's ternary block packed as by
 * bitlinear_pack_weights (packing a group-major int8 [G][N][KG] tensor as
 * G*N rows of KG gives this layout).  beta: DEVICE fp32 [G] (finite; as
 * written by bitlinear_ternarize_grouped).  y out fp32 [M][N].  acc out int32
 * [G][M][N] (the group products).
 * Requires G >= 1, K % G == 0, KG % 64 == 0; other limits as for
 * bitlinear_forward with K = KG.
 * Decode shapes (M <= 16, G in {2, 4, 8}, KG % 256 == 0, the activations
 * fitting in LDS): one launch of the LDS decode kernel with the group terms
 * added in its epilogue; acc may be NULL there.  Otherwise each group runs
 * the kernel bitlinear_forward picks for (M, KG, N) in accumulator-only mode
 * into acc, then one launch adds the groups (G + 1 launches); acc is then
 * required (NULL returns BITLINEAR_ERR_NULL).  None allocates. */
bitlinear_status_t bitlinear_forward_grouped(const int8_t* x_q, const float* gamma, int64_t M,
                                             int64_t K, int64_t G, const uint32_t* w_packed,
                                             int64_t N, const float* beta, float* y, int32_t* acc,
                                             hipStream_t stream);

/* 1 if bitlinear_forward_grouped takes the one-launch path for this shape
 * (acc may then be NULL), else 0.  Host-only, no HIP call. */
int bitlinear_forward_grouped_one_launch(int64_t M, int64_t K, int64_t G, int64_t N);

/* Absmean ternarisation per weight group (the rule of bitlinear_ternarize
 * applied to each group's N x KG block).  W_grouped: fp32 [G][N][KG], group g
 * = input columns g*KG .. (g+1)*KG of the [N][K] weight matrix, contiguous.
 * w_packed out uint32 [G][N][KG/16] (the layout bitlinear_forward_grouped
 * takes); w_ternary optional out int8 [G][N][KG]; beta out fp32 [G]; beta64
 * out double [G].  Requires G >= 1, K % G == 0, KG % 64 == 0.  3 or more
 * launches per group on `stream`; none allocates. */
bitlinear_status_t bitlinear_ternarize_grouped(const float* W_grouped, int64_t N, int64_t K,
                                               int64_t G, uint32_t* w_packed, int8_t* w_ternary,
                                               float* beta, double* beta64, hipStream_t stream);

/*
 * Base-3 weights at 1.6 bits per weight (unite.ai article, section
 * "Ternäres Gewichtssystem / Das Konzept": three states carry about 1.58
 * bits; five ternary codes fit one byte since 3^5 = 243 <= 256), 20 % fewer
 * weight bytes than the 2-bit layout.
 *
 * Layout: a row is U = ceil(K/80) units of 16 bytes, row n at byte 16*U*n.
 * Byte b of little-endian 32-bit word w of unit u holds the weights
 * k = 80u + 20w + 4i + b, i = 0..4, as v = sum (w_k + 1) * 3^(4-i), stored
 * as the byte ceil(256 v / 243) (so v = floor(243 b / 256)); weights past K
 * are 0.
 */

/* Ternary int8 [N][K] -> base-3 bytes [N][16*ceil(K/80)] (16-byte aligned).
 * bad_count as for bitlinear_pack_weights (entries outside {-1,0,1} pack as
 * 0).  K % 16 == 0.  One launch (two with bad_count). */
bitlinear_status_t bitlinear_pack_weights3(const int8_t* w, int64_t N, int64_t K,
                                           uint32_t* w_packed3, int32_t* bad_count,
                                           hipStream_t stream);

/* bitlinear_forward on base-3 weights: the same acc, y and argument rules,
 * with w_packed3 the bitlinear_pack_weights3 layout (16-byte aligned).  A
 * decode product: 2..16 tokens whose activation block fits in LDS run in one
 * pass over the weights on int8 MFMA (the base-3 bytes decoded to codes in
 * registers); one token, and larger blocks in passes of up to four tokens,
 * on the vector ALUs.  For many tokens use the 2-bit layout. */
bitlinear_status_t bitlinear_forward3(const int8_t* x_q, const float* gamma, int64_t M, int64_t K,
                                      const uint32_t* w_packed3, int64_t N, float beta, float* y,
                                      int32_t* acc, hipStream_t stream);

/*
 * Measurement floors.  Not steps of the layer: the references a roofline
 * report needs next to the layer's kernels on the same device -- the duration
 * of a launch that does nothing, of a read-only pass over the same number of
 * bytes a product streams (the weight matrix), with the coalesced 16-byte
 * loads the decode kernels issue, and of the int8 multiplies of a product
 * with no memory work around them.
 *
 * bitlinear_floor_empty: launches one empty workgroup on `stream`.
 * bitlinear_floor_stream_read: reads `bytes` (>= 0, a multiple of 16) at p
 *   (device, 16-byte aligned) once.  sink: device uint32 [1]; stored only if
 *   the xor of all the 32-bit words read equals 0x9E3779B9 (it keeps the
 *   loads from being optimised away), so its content carries no meaning.
 */
bitlinear_status_t bitlinear_floor_empty(hipStream_t stream);
bitlinear_status_t bitlinear_floor_stream_read(const void* p, int64_t bytes, uint32_t* sink,
                                               hipStream_t stream);

/*
 * bitlinear_floor_mfma: the v_mfma_i32_32x32x32_i8 work of a product at
 *   (M, K, N) on the GEMM's 128 x 256 tiles -- one workgroup of four waves per
 *   tile, two workgroups per CU, 32 MFMAs per wave for each 128 inputs of K --
 *   with operands loaded once from the product's own inputs (x_q [M][K] int8
 *   and w_packed [N][K/16] in the layout of bitlinear_pack_weights, both
 *   device, 16-byte aligned: each wave's activation rows and signed weights of
 *   the first 128 inputs) and then multiplied from registers only.  Its
 *   duration is what those multiplies take on this device with that data and
 *   nothing else to wait for.  M in [0, 65535 * 128], N in [0, 2^30],
 *   K in [0, 131072] a multiple of 128, at most 2^31 - 1 tiles of 128 x 256;
 *   M, N or K = 0 launches nothing.
 *   sink: device uint32 [1], stored only if the xor of all accumulators equals
 *   0x9E3779B9, so its content carries no meaning.
 */
bitlinear_status_t bitlinear_floor_mfma(const int8_t* x_q, int64_t M, int64_t K,
                                        const uint32_t* w_packed, int64_t N, uint32_t* sink,
                                        hipStream_t stream);

/* Text of the last non-OK status on this thread ("" if none). */
const char* bitlinear_last_error(void);

/* BITLINEAR_ABI_VERSION of the loaded library. */
int bitlinear_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BITLINEAR_H */

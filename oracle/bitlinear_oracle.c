/*
 * CPU oracle for the ternary BitLinear layer: TEST INFRASTRUCTURE ONLY.
 * See bitlinear_oracle.h for the sources and the scope.  Built with
 * gcc -O2 -ffp-contract=off -fno-fast-math so every float operation below is
 * one IEEE operation in the precision its operands have.
 */
#include "bitlinear_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Qb = 2^(b-1) for b = 8 bit activations ([U] 2. Aktivierungsquantisierung). */
#define ORACLE_QB 128.0f
/* Largest code kept by the clip: the bounds -Qb+eps .. Qb-eps with a small
 * eps leave the integers -127 .. 127. */
#define ORACLE_QMAX 127.0f

void oracle_bf16_to_f32(const uint16_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t bits = ((uint32_t)in[i]) << 16;
        memcpy(&out[i], &bits, sizeof bits);
    }
}

/* Round to the nearest integer, ties to the even neighbour, written out so it
 * does not depend on the floating-point environment.  |t| <= 128 here, so
 * t - floor(t) is exact. */
static float round_half_even(float t) {
    float f = floorf(t);
    float frac = t - f;
    if (frac > 0.5f) return f + 1.0f;
    if (frac < 0.5f) return f;
    return (fmodf(f, 2.0f) == 0.0f) ? f : f + 1.0f;
}

static double round_half_even_d(double t) {
    double f = floor(t);
    double frac = t - f;
    if (frac > 0.5) return f + 1.0;
    if (frac < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* One token: gamma = ||x||_inf; each entry is divided by gamma, scaled by Qb,
 * rounded and clipped to [-127, 127].  gamma = 0 quantises to zeros. */
static float quant_row(const float* x, int64_t K, int8_t* q) {
    float gamma = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float a = fabsf(x[k]);
        if (a > gamma) gamma = a;
    }
    for (int64_t k = 0; k < K; ++k) {
        if (gamma == 0.0f) {
            q[k] = 0;
            continue;
        }
        float ratio = x[k] / gamma;   /* one correctly rounded fp32 division */
        float t = ratio * ORACLE_QB;  /* exact: Qb is a power of two */
        float r = round_half_even(t);
        if (r > ORACLE_QMAX) r = ORACLE_QMAX;
        if (r < -ORACLE_QMAX) r = -ORACLE_QMAX;
        q[k] = (int8_t)r;
    }
    return gamma;
}

void oracle_quant_act(const float* x, int64_t M, int64_t K, int8_t* q, float* gamma) {
    for (int64_t m = 0; m < M; ++m) gamma[m] = quant_row(x + m * K, K, q + m * K);
}

/* RMSNorm: x * g / sqrt(mean(x^2) + eps) ([D], figure list: RMS norm before
 * quantisation).  The quantiser divides by the absmax of its input, so the
 * common factor r = 1/sqrt(mean(x^2)+eps) cancels from the codes: they are the
 * codes of u = g*x (fp32), and r survives only in gamma = r * max|u|, with r
 * and that product evaluated in float64 and rounded once to fp32. */
void oracle_rmsnorm_quant_act(const float* x, const float* g, float eps, int64_t M,
                              int64_t K, int8_t* q, float* gamma) {
    float* u = (float*)malloc((size_t)(K > 0 ? K : 1) * sizeof(float));
    for (int64_t m = 0; m < M; ++m) {
        const float* xm = x + m * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) ss += (double)xm[k] * (double)xm[k];
        double mean = K > 0 ? ss / (double)K : 0.0;
        double r = 1.0 / sqrt(mean + (double)eps);
        for (int64_t k = 0; k < K; ++k) u[k] = g[k] * xm[k];
        float absmax_u = quant_row(u, K, q + m * K);
        gamma[m] = (float)(r * (double)absmax_u);
    }
    free(u);
}

/* Group quantisation ([U] Gruppenquantisierung und -normalisierung: weights
 * and activations are divided into G groups and the quantisation parameters
 * are computed per group instead of for the whole matrix).  Groups split the
 * K inputs into G equal runs; token m's run g gets its own absmax scale
 * gamma[g][m] and codes q[g][m][0 .. K/G).  With a gain (RMSNorm), r is the
 * token's whole-row factor and gamma[g][m] = fl32(r * max over the run of
 * |u|), u = fl32(gain * x), as in the ungrouped variant.  Outputs are
 * group-major: q [G][M][K/G], gamma [G][M]. */
void oracle_quant_act_grouped(const float* x, const float* gain, float eps, int64_t M,
                              int64_t K, int64_t G, int8_t* q, float* gamma) {
    const int64_t KG = K / G;
    float* u = (float*)malloc((size_t)(KG > 0 ? KG : 1) * sizeof(float));
    for (int64_t m = 0; m < M; ++m) {
        const float* xm = x + m * K;
        double r = 1.0;
        if (gain) {
            double ss = 0.0;
            for (int64_t k = 0; k < K; ++k) ss += (double)xm[k] * (double)xm[k];
            r = 1.0 / sqrt((K > 0 ? ss / (double)K : 0.0) + (double)eps);
        }
        for (int64_t g = 0; g < G; ++g) {
            for (int64_t k = 0; k < KG; ++k) {
                const float xv = xm[g * KG + k];
                u[k] = gain ? gain[g * KG + k] * xv : xv;
            }
            const float absmax = quant_row(u, KG, q + (g * M + m) * KG);
            gamma[g * M + m] = gain ? (float)(r * (double)absmax) : absmax;
        }
    }
    free(u);
}

/* The same two steps evaluated literally in float64: normalise, then quantise
 * the normalised vector.  Codes may differ from the fp32 contract only where
 * the scaled value sits within rounding distance of a half-integer. */
void oracle_rmsnorm_quant_act_literal(const float* x, const float* g, float eps,
                                      int64_t M, int64_t K, int8_t* q, double* gamma) {
    double* y = (double*)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    for (int64_t m = 0; m < M; ++m) {
        const float* xm = x + m * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) ss += (double)xm[k] * (double)xm[k];
        double r = 1.0 / sqrt((K > 0 ? ss / (double)K : 0.0) + (double)eps);
        double gm = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            y[k] = (double)xm[k] * r * (double)g[k];
            if (fabs(y[k]) > gm) gm = fabs(y[k]);
        }
        gamma[m] = gm;
        for (int64_t k = 0; k < K; ++k) {
            double t = gm == 0.0 ? 0.0 : y[k] / gm * 128.0;
            double rq = round_half_even_d(t);
            if (rq > 127.0) rq = 127.0;
            if (rq < -127.0) rq = -127.0;
            q[m * K + k] = (int8_t)rq;
        }
    }
    free(y);
}

/* Storage of ternary weights ([U] Das Konzept: three states per weight, just
 * over one bit of information) as 2-bit codes: code = w + 1, so -1 -> 0,
 * 0 -> 1, +1 -> 2; 3 marks an entry that was not ternary.  Sixteen
 * consecutive weights of a row form one little-endian uint32 word; the weight
 * at position e = 4j + b inside the group sits at bit 8b + 2j. */
int64_t oracle_pack(const int8_t* w, int64_t N, int64_t K, uint32_t* packed) {
    int64_t bad = 0;
    int64_t words = K / 16;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t c = 0; c < words; ++c) {
            uint32_t word = 0;
            for (int e = 0; e < 16; ++e) {
                int v = w[n * K + c * 16 + e];
                uint32_t code;
                if (v == -1) code = 0;
                else if (v == 0) code = 1;
                else if (v == 1) code = 2;
                else { code = 3; ++bad; }
                int j = e / 4, b = e % 4;
                word |= code << (8 * b + 2 * j);
            }
            packed[n * words + c] = word;
        }
    }
    return bad;
}

void oracle_unpack(const uint32_t* packed, int64_t N, int64_t K, int8_t* w) {
    int64_t words = K / 16;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t c = 0; c < words; ++c)
            for (int e = 0; e < 16; ++e) {
                int j = e / 4, b = e % 4;
                int code = (int)((packed[n * words + c] >> (8 * b + 2 * j)) & 3u);
                w[n * K + c * 16 + e] = (int8_t)(code - 1);
            }
}

/* Ternary accumulation: multiplying by -1 negates, by 0 gives nothing, by +1
 * passes the value through ([D] MatMul vervangen door ternaire bewerkingen),
 * so each output is a signed sum of the quantised activations. */
int oracle_accumulate(const int8_t* q, int64_t M, int64_t K, const int8_t* w,
                      int64_t N, int32_t* acc) {
    int overflow = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : overflow)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const int8_t* qm = q + m * K;
            const int8_t* wn = w + n * K;
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) {
                if (wn[k] == 1) s += qm[k];
                else if (wn[k] == -1) s -= qm[k];
            }
            if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
            acc[m * N + n] = (int32_t)s;
        }
    }
    return overflow;
}

/* Output scale beta * gamma / Qb ([U] 3. BitLinear-Betrieb). */
void oracle_rescale(const int32_t* acc, const float* gamma, int64_t M, int64_t N,
                    float beta, float* y) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double v = (double)acc[m * N + n] * (double)beta * (double)gamma[m] / 128.0;
            y[m * N + n] = (float)v;
        }
}

/* GLU channel mixer glue ([D] Kerncomponenten: MLGRU EN GLU): one projection
 * goes through SiLU(z) = z / (1 + e^-z) and is multiplied elementwise by the
 * other. */
void oracle_silu_mul(const float* gate, const float* up, int64_t n, double* h) {
    for (int64_t i = 0; i < n; ++i) {
        double z = (double)gate[i];
        h[i] = z / (1.0 + exp(-z)) * (double)up[i];
    }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the parallel loops started from the calling thread (timing
 * of the baseline on one core); n <= 0 is ignored. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Pairwise sum of |x[a..b)| in double: a run of one entry is its value; a
 * longer run splits after the largest power of two below its length. */
static double pairwise_abs(const float* x, int64_t a, int64_t b) {
    const int64_t n = b - a;
    if (n == 1) return fabs((double)x[a]);
    int64_t p = 1;
    while (p * 2 < n) p *= 2;
    return pairwise_abs(x, a, a + p) + pairwise_abs(x, a + p, b);
}

/* [D] absmean ternarisation: the mean absolute value (pairwise double sum of
 * the row-major entries, divided by N*K); then each entry against half of it. */
double oracle_ternarize(const float* W, int64_t N, int64_t K, int8_t* w) {
    const int64_t total_n = N * K;
    const double beta = total_n > 0 ? pairwise_abs(W, 0, total_n) / ((double)N * (double)K) : 0.0;
    const double half = beta * 0.5;
    for (int64_t i = 0; i < total_n; ++i) {
        const double v = (double)W[i];
        w[i] = (int8_t)((v > half && beta > 0.0) ? 1 : (v < -half && beta > 0.0) ? -1 : 0);
    }
    return beta;
}

/* Pairwise sum of x[a..b) in double, split as in pairwise_abs. */
static double pairwise_signed(const float* x, int64_t a, int64_t b) {
    const int64_t n = b - a;
    if (n == 1) return (double)x[a];
    int64_t p = 1;
    while (p * 2 < n) p *= 2;
    return pairwise_signed(x, a, a + p) + pairwise_signed(x, a + p, b);
}

/* [U] 1. Gewichtsbinarisierung: centre on the mean, then the sign (+1 only
 * for a strictly positive difference). */
double oracle_binarize(const float* W, int64_t N, int64_t K, int8_t* w) {
    const int64_t total_n = N * K;
    const double alpha = total_n > 0 ? pairwise_signed(W, 0, total_n) / ((double)N * (double)K) : 0.0;
    for (int64_t i = 0; i < total_n; ++i) w[i] = (int8_t)(((double)W[i] > alpha) ? 1 : -1);
    return alpha;
}

int64_t oracle_pack1(const int8_t* w, int64_t N, int64_t K, uint32_t* packed) {
    int64_t bad = 0;
    const int64_t words = K / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t q = 0; q < words; ++q) {
            uint32_t word = 0;
            for (int e = 0; e < 32; ++e) {
                const int8_t v = w[n * K + 32 * q + e];
                uint32_t bit = 0;
                if (v == 1) bit = 1;
                else if (v != -1) ++bad;
                const int j = e / 4, b = e % 4;
                word |= bit << (8 * b + j);
            }
            packed[n * words + q] = word;
        }
    return bad;
}

void oracle_unpack1(const uint32_t* packed, int64_t N, int64_t K, int8_t* w) {
    const int64_t words = K / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t q = 0; q < words; ++q) {
            const uint32_t word = packed[n * words + q];
            for (int e = 0; e < 32; ++e) {
                const int j = e / 4, b = e % 4;
                w[n * K + 32 * q + e] = (int8_t)(((word >> (8 * b + j)) & 1u) ? 1 : -1);
            }
        }
}

/* Base-3 packing at 1.6 bits per weight ([U] Ternäres Gewichtssystem: three
 * states need a little more than one bit, about 1.58; five ternary codes
 * fit one byte since 3^5 = 243 <= 256).  Layout: a row is U = ceil(K/80)
 * units of 16 bytes; byte b of 32-bit word w of unit u holds the five
 * weights k = 80u + 20w + 4i + b (i = 0..4) as v = sum_i (w_k + 1) * 3^(4-i),
 * stored as the byte ceil(256 v / 243); weights past K are 0.  The stored
 * byte decodes as v = floor(243 b / 256) and then by base-3 digits. */
static const int pow3[5] = {81, 27, 9, 3, 1};

int64_t oracle_pack3(const int8_t* w, int64_t N, int64_t K, uint8_t* packed) {
    const int64_t U = (K + 79) / 80;
    int64_t bad = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t u = 0; u < U; ++u) {
            for (int wd = 0; wd < 4; ++wd) {
                for (int b = 0; b < 4; ++b) {
                    int v = 0;
                    for (int i = 0; i < 5; ++i) {
                        const int64_t k = 80 * u + 20 * wd + 4 * i + b;
                        int c = 1;
                        if (k < K) {
                            const int x = w[n * K + k];
                            if (x < -1 || x > 1) ++bad;
                            else c = x + 1;
                        }
                        v += c * pow3[i];
                    }
                    packed[(n * U + u) * 16 + 4 * wd + b] = (uint8_t)((256 * v + 242) / 243);
                }
            }
        }
    }
    return bad;
}

void oracle_unpack3(const uint8_t* packed, int64_t N, int64_t K, int8_t* w) {
    const int64_t U = (K + 79) / 80;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t u = 0; u < U; ++u) {
            for (int wd = 0; wd < 4; ++wd) {
                for (int b = 0; b < 4; ++b) {
                    int v = (243 * (int)packed[(n * U + u) * 16 + 4 * wd + b]) / 256;
                    for (int i = 0; i < 5; ++i) {
                        const int c = v / pow3[i];
                        v -= c * pow3[i];
                        const int64_t k = 80 * u + 20 * wd + 4 * i + b;
                        if (k < K) w[n * K + k] = (int8_t)(c - 1);
                    }
                }
            }
        }
    }
}

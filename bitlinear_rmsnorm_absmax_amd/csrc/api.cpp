// C ABI of the ternary BitLinear library: argument validation, kernel choice
// by M, launches on the caller's stream.  Validation touches no HIP API, so
// every error path returns before the runtime is involved.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/bitlinear.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

bitlinear_status_t fail(bitlinear_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

bitlinear_status_t ok() {
    g_err[0] = '\0';
    return BITLINEAR_OK;
}

bitlinear_status_t from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(BITLINEAR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Largest M handled by one grid dimension of the GEMM (65535 row tiles of 128).
constexpr int64_t kMaxM = 65535LL * 128;
// Largest N (and weight-row count of the packing calls).  The launchers and
// kernels take N as int and round it up to their tile widths (at most a few
// hundred columns) or add a tile offset to a row index, so N stays 2^30 below
// INT_MAX; 2^30 rows are 4 GiB of packed weights even at K = 16.
constexpr int64_t kMaxN = 1LL << 30;

bitlinear_status_t check_k(const char* fn, const char* name, int64_t K) {
    if (K < 0 || K % 16 != 0 || K > BITLINEAR_MAX_K)
        return fail(BITLINEAR_ERR_SHAPE, "%s: %s=%lld must be in [0, %d] and a multiple of 16", fn,
                    name, (long long)K, BITLINEAR_MAX_K);
    return BITLINEAR_OK;
}

bitlinear_status_t check_rows(const char* fn, const char* name, int64_t v, int64_t max) {
    if (v < 0 || v > max)
        return fail(BITLINEAR_ERR_SHAPE, "%s: %s=%lld out of range [0, %lld]", fn, name,
                    (long long)v, (long long)max);
    return BITLINEAR_OK;
}

#define BL_TRY(expr)                                  \
    do {                                              \
        bitlinear_status_t st_ = (expr);              \
        if (st_ != BITLINEAR_OK) return st_;          \
    } while (0)

bitlinear_status_t need(const char* fn, const char* name, const void* p, bool required,
                        size_t align) {
    if (!required) return BITLINEAR_OK;
    if (!p) return fail(BITLINEAR_ERR_NULL, "%s: %s is NULL", fn, name);
    if (!aligned(p, align))
        return fail(BITLINEAR_ERR_ALIGN, "%s: %s is not %zu-byte aligned", fn, name, align);
    return BITLINEAR_OK;
}

// Kernel choice by M (or the forced path); y == nullptr stores only acc.
hipError_t launch_forward_kernel(const int8_t* x_q, const float* gamma, int64_t M, int64_t K,
                                 const uint32_t* w_packed, int64_t N, float beta, float* y,
                                 int32_t* acc, int path, hipStream_t stream) {
    if (path == BITLINEAR_PATH_AUTO) {
        // 17..32 tokens over at least 128 column tiles of 128 (N >= 16257) run
        // the GEMM's 64-row tiles: K = 8192, N = 28672 at 17..32 tokens 28-30 us
        // against 49-75 us on the skinny kernel; with fewer column tiles the
        // skinny kernel keeps more CUs busy (K = 6912, N = 2560: 10-12 vs 21 us)
        // one token: the VALU GEMV, or the decode kernel (in the skinny path)
        // on long rows over many row tiles
        const bool wide_n = (N + 127) / 128 >= 128 && K % 256 == 0;
        path = (M == 1) ? (bl::decode_one_token((int)K, (int)N) ? BITLINEAR_PATH_SKINNY : BITLINEAR_PATH_GEMV)
             : (M <= 16 || (M <= 32 && !wide_n)) ? BITLINEAR_PATH_SKINNY
                                                  : BITLINEAR_PATH_GEMM;
    }
    const int m = (int)M, n = (int)N, k = (int)K;
    switch (path) {
        case BITLINEAR_PATH_GEMV:
            return bl::launch_gemv_valu(x_q, gamma, m, k, w_packed, n, beta, y, acc, stream);
        case BITLINEAR_PATH_SKINNY:
            return bl::launch_skinny_mfma(x_q, gamma, m, k, w_packed, n, beta, y, acc, stream);
        default:
            return bl::launch_gemm_mfma(x_q, gamma, m, k, w_packed, n, beta, y, acc, stream);
    }
}

// Group count G: K split into G equal runs whose length is a multiple of `unit`.
bitlinear_status_t check_groups(const char* fn, int64_t K, int64_t G, int64_t unit) {
    if (G < 1 || G > BITLINEAR_MAX_K)
        return fail(BITLINEAR_ERR_SHAPE, "%s: G=%lld must be in [1, %d]", fn, (long long)G,
                    BITLINEAR_MAX_K);
    if (K % G != 0 || (K / G) % unit != 0)
        return fail(BITLINEAR_ERR_SHAPE, "%s: K=%lld must be G=%lld runs of a multiple of %lld", fn,
                    (long long)K, (long long)G, (long long)unit);
    return BITLINEAR_OK;
}

bitlinear_status_t forward_impl(const char* fn, const int8_t* x_q, const float* gamma,
                                int64_t M, int64_t K, const uint32_t* w_packed, int64_t N,
                                float beta, float* y, int32_t* acc, int path,
                                hipStream_t stream) {
    BL_TRY(check_rows(fn, "M", M, kMaxM));
    BL_TRY(check_rows(fn, "N", N, kMaxN));
    BL_TRY(check_k(fn, "K", K));
    if (path < BITLINEAR_PATH_AUTO || path > BITLINEAR_PATH_GEMM)
        return fail(BITLINEAR_ERR_VALUE, "%s: unknown path %d", fn, path);
    if (!std::isfinite(beta)) return fail(BITLINEAR_ERR_VALUE, "%s: beta is not finite", fn);
    const bool any_out = M > 0 && N > 0;
    const bool any_in = any_out && K > 0;
    BL_TRY(need(fn, "x_q", x_q, any_in, 16));
    BL_TRY(need(fn, "gamma", gamma, any_in, 4));
    BL_TRY(need(fn, "w_packed", w_packed, any_in, 16));
    BL_TRY(need(fn, "y", y, any_out && !acc, 4));
    if (y && !aligned(y, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: y is not 4-byte aligned", fn);
    if (acc && !aligned(acc, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: acc is not 4-byte aligned", fn);
    if (path == BITLINEAR_PATH_GEMV && M > 4)
        return fail(BITLINEAR_ERR_VALUE, "%s: the GEMV path takes M <= 4 (M=%lld)", fn, (long long)M);
    if (path == BITLINEAR_PATH_SKINNY && M > 64)
        return fail(BITLINEAR_ERR_VALUE, "%s: the skinny path takes M <= 64 (M=%lld)", fn, (long long)M);
    if (!any_out) return ok();
    if (K == 0) return from_hip(bl::launch_fill_zero(y, acc, M * N, stream), fn);

    return from_hip(launch_forward_kernel(x_q, gamma, M, K, w_packed, N, beta, y, acc, path, stream),
                    fn);
}

}  // namespace

extern "C" {

bitlinear_status_t bitlinear_quant_act(const void* x, bitlinear_dtype_t x_dtype, int64_t M,
                                       int64_t K, const float* rms_gain, float rms_eps,
                                       int8_t* x_q, float* gamma, hipStream_t stream) {
    const char* fn = "bitlinear_quant_act";
    BL_TRY(check_rows(fn, "M", M, (1LL << 31) - 1));
    BL_TRY(check_k(fn, "K", K));
    if (x_dtype != BITLINEAR_F32 && x_dtype != BITLINEAR_BF16)
        return fail(BITLINEAR_ERR_DTYPE, "%s: unknown dtype %d", fn, (int)x_dtype);
    if (rms_gain && !(std::isfinite(rms_eps) && rms_eps >= 0.0f))
        return fail(BITLINEAR_ERR_VALUE, "%s: rms_eps must be finite and >= 0", fn);
    const bool any = M > 0 && K > 0;
    BL_TRY(need(fn, "x", x, any, 16));
    BL_TRY(need(fn, "x_q", x_q, any, 16));
    BL_TRY(need(fn, "gamma", gamma, M > 0, 4));
    if (rms_gain && !aligned(rms_gain, 16))
        return fail(BITLINEAR_ERR_ALIGN, "%s: rms_gain is not 16-byte aligned", fn);
    if (M == 0) return ok();
    return from_hip(bl::launch_quant_act(x, x_dtype == BITLINEAR_BF16, M, K, rms_gain, rms_eps,
                                         x_q, gamma, stream),
                    fn);
}

bitlinear_status_t bitlinear_pack_weights(const int8_t* w, int64_t N, int64_t K,
                                          uint32_t* w_packed, int32_t* bad_count,
                                          hipStream_t stream) {
    const char* fn = "bitlinear_pack_weights";
    BL_TRY(check_rows(fn, "N", N, kMaxN));
    BL_TRY(check_k(fn, "K", K));
    const bool any = N > 0 && K > 0;
    BL_TRY(need(fn, "w", w, any, 16));
    BL_TRY(need(fn, "w_packed", w_packed, any, 16));
    if (bad_count && !aligned(bad_count, 4))
        return fail(BITLINEAR_ERR_ALIGN, "%s: bad_count is not 4-byte aligned", fn);
    if (!any && !bad_count) return ok();
    return from_hip(bl::launch_pack(w, N, K, w_packed, bad_count, stream), fn);
}

bitlinear_status_t bitlinear_forward(const int8_t* x_q, const float* gamma, int64_t M, int64_t K,
                                     const uint32_t* w_packed, int64_t N, float beta, float* y,
                                     int32_t* acc, hipStream_t stream) {
    return forward_impl("bitlinear_forward", x_q, gamma, M, K, w_packed, N, beta, y, acc,
                        BITLINEAR_PATH_AUTO, stream);
}

bitlinear_status_t bitlinear_forward_path(const int8_t* x_q, const float* gamma, int64_t M,
                                          int64_t K, const uint32_t* w_packed, int64_t N,
                                          float beta, float* y, int32_t* acc, int path,
                                          hipStream_t stream) {
    return forward_impl("bitlinear_forward_path", x_q, gamma, M, K, w_packed, N, beta, y, acc,
                        path, stream);
}

bitlinear_status_t bitlinear_quant_forward(const void* x, bitlinear_dtype_t x_dtype, int64_t M,
                                           int64_t K, const float* rms_gain, float rms_eps,
                                           const uint32_t* w_packed, int64_t N, float beta,
                                           int8_t* x_q, float* gamma, float* y, int32_t* acc,
                                           hipStream_t stream) {
    const char* fn = "bitlinear_quant_forward";
    BL_TRY(check_rows(fn, "M", M, kMaxM));
    BL_TRY(check_rows(fn, "N", N, kMaxN));
    BL_TRY(check_k(fn, "K", K));
    if (x_dtype != BITLINEAR_F32 && x_dtype != BITLINEAR_BF16)
        return fail(BITLINEAR_ERR_DTYPE, "%s: unknown dtype %d", fn, (int)x_dtype);
    if (rms_gain && !(std::isfinite(rms_eps) && rms_eps >= 0.0f))
        return fail(BITLINEAR_ERR_VALUE, "%s: rms_eps must be finite and >= 0", fn);
    if (!std::isfinite(beta)) return fail(BITLINEAR_ERR_VALUE, "%s: beta is not finite", fn);
    const bool any_q = M > 0 && K > 0;
    const bool any_out = M > 0 && N > 0;
    BL_TRY(need(fn, "x", x, any_q, 16));
    BL_TRY(need(fn, "x_q", x_q, any_q, 16));
    BL_TRY(need(fn, "gamma", gamma, M > 0, 4));
    if (rms_gain && !aligned(rms_gain, 16))
        return fail(BITLINEAR_ERR_ALIGN, "%s: rms_gain is not 16-byte aligned", fn);
    BL_TRY(need(fn, "w_packed", w_packed, any_out && K > 0, 16));
    BL_TRY(need(fn, "y", y, any_out && !acc, 4));
    if (y && !aligned(y, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: y is not 4-byte aligned", fn);
    if (acc && !aligned(acc, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: acc is not 4-byte aligned", fn);
    if (M == 0) return ok();
    // one token on long rows over many row tiles: quantised inside the
    // two-part decode kernel; smaller one-token shapes: the VALU fused kernel
    if (M == 1 && bl::decode_one_token((int)K, (int)N))
        return from_hip(bl::launch_quant_decode1(x, x_dtype == BITLINEAR_BF16, (int)K, rms_gain, rms_eps,
                                                 w_packed, (int)N, beta, y, acc, x_q, gamma, stream),
                        fn);
    if (bl::quant_gemv_supports((int)M, (int)K, (int)N))
        return from_hip(bl::launch_quant_gemv(x, x_dtype == BITLINEAR_BF16, (int)K, rms_gain,
                                              rms_eps, w_packed, (int)N, beta, y, acc, x_q, gamma,
                                              stream),
                        fn);
    hipError_t e = bl::launch_quant_act(x, x_dtype == BITLINEAR_BF16, M, K, rms_gain, rms_eps, x_q,
                                        gamma, stream);
    if (e != hipSuccess || !any_out) return from_hip(e, fn);
    if (K == 0) return from_hip(bl::launch_fill_zero(y, acc, M * N, stream), fn);
    return from_hip(launch_forward_kernel(x_q, gamma, M, K, w_packed, N, beta, y, acc,
                                          BITLINEAR_PATH_AUTO, stream),
                    fn);
}

bitlinear_status_t bitlinear_silu_mul_quant(const float* gate, const float* up, int64_t M,
                                            int64_t F, float* h, int8_t* h_q, float* gamma_h,
                                            hipStream_t stream) {
    const char* fn = "bitlinear_silu_mul_quant";
    BL_TRY(check_rows(fn, "M", M, (1LL << 31) - 1));
    BL_TRY(check_k(fn, "F", F));
    const bool any = M > 0 && F > 0;
    BL_TRY(need(fn, "gate", gate, any, 16));
    BL_TRY(need(fn, "up", up, any, 16));
    BL_TRY(need(fn, "h_q", h_q, any, 16));
    BL_TRY(need(fn, "gamma_h", gamma_h, M > 0, 4));
    if (h && !aligned(h, 16)) return fail(BITLINEAR_ERR_ALIGN, "%s: h is not 16-byte aligned", fn);
    if (M == 0) return ok();
    return from_hip(bl::launch_silu_mul_quant(gate, up, M, F, h, h_q, gamma_h, stream), fn);
}

bitlinear_status_t bitlinear_silu_mul_quant_acc(const int32_t* acc_gu, const float* gamma,
                                                int64_t M, int64_t F, float beta_gate,
                                                float beta_up, float* h, int8_t* h_q,
                                                float* gamma_h, hipStream_t stream) {
    const char* fn = "bitlinear_silu_mul_quant_acc";
    BL_TRY(check_rows(fn, "M", M, (1LL << 31) - 1));
    BL_TRY(check_k(fn, "F", F));
    if (!std::isfinite(beta_gate) || !std::isfinite(beta_up))
        return fail(BITLINEAR_ERR_VALUE, "%s: beta_gate and beta_up must be finite", fn);
    const bool any = M > 0 && F > 0;
    BL_TRY(need(fn, "acc_gu", acc_gu, any, 16));
    BL_TRY(need(fn, "gamma", gamma, any, 4));
    BL_TRY(need(fn, "h_q", h_q, any, 16));
    BL_TRY(need(fn, "gamma_h", gamma_h, M > 0, 4));
    if (h && !aligned(h, 16)) return fail(BITLINEAR_ERR_ALIGN, "%s: h is not 16-byte aligned", fn);
    if (M == 0) return ok();
    return from_hip(bl::launch_silu_mul_quant_acc(acc_gu, gamma, M, F, beta_gate, beta_up, h, h_q,
                                                  gamma_h, stream),
                    fn);
}

bitlinear_status_t bitlinear_ternarize(const float* W, int64_t N, int64_t K, uint32_t* w_packed,
                                       int8_t* w_ternary, float* beta, double* beta64,
                                       hipStream_t stream) {
    const char* fn = "bitlinear_ternarize";
    BL_TRY(check_rows(fn, "N", N, kMaxN));
    BL_TRY(check_k(fn, "K", K));
    if (K != 0 && K < 32)
        return fail(BITLINEAR_ERR_SHAPE, "%s: K=%lld must be 0 or >= 32", fn, (long long)K);
    const bool any = N > 0 && K > 0;
    if (any && N * (K / 16) > (1LL << 40))
        return fail(BITLINEAR_ERR_SHAPE, "%s: N*K/16 exceeds 2^40", fn);
    BL_TRY(need(fn, "W", W, any, 16));
    BL_TRY(need(fn, "w_packed", w_packed, any, 16));
    BL_TRY(need(fn, "beta", beta, true, 4));
    BL_TRY(need(fn, "beta64", beta64, true, 8));
    if (w_ternary && !aligned(w_ternary, 16))
        return fail(BITLINEAR_ERR_ALIGN, "%s: w_ternary is not 16-byte aligned", fn);
    return from_hip(bl::launch_ternarize(W, any ? N : 0, any ? K : 0, w_packed, w_ternary, beta,
                                         beta64, stream),
                    fn);
}

bitlinear_status_t bitlinear_binarize(const float* W, int64_t N, int64_t K, uint32_t* w_packed1,
                                      int8_t* w_codes, float* alpha, double* alpha64, float* beta,
                                      double* beta64, hipStream_t stream) {
    const char* fn = "bitlinear_binarize";
    BL_TRY(check_rows(fn, "N", N, kMaxN));
    if (K < 0 || K % 32 != 0 || K > BITLINEAR_MAX_K)
        return fail(BITLINEAR_ERR_SHAPE, "%s: K=%lld must be in [0, %d] and a multiple of 32", fn,
                    (long long)K, BITLINEAR_MAX_K);
    const bool any = N > 0 && K > 0;
    if (any && N * (K / 32) > (1LL << 40))
        return fail(BITLINEAR_ERR_SHAPE, "%s: N*K/32 exceeds 2^40", fn);
    BL_TRY(need(fn, "W", W, any, 16));
    BL_TRY(need(fn, "w_packed1", w_packed1, any, 4));
    BL_TRY(need(fn, "w_codes", w_codes, any, 16));
    BL_TRY(need(fn, "alpha", alpha, true, 4));
    BL_TRY(need(fn, "alpha64", alpha64, true, 8));
    BL_TRY(need(fn, "beta", beta, true, 4));
    BL_TRY(need(fn, "beta64", beta64, true, 8));
    if (any) {  // both partial-sum arrays must fit their halves of the code buffer
        const int64_t L = N * K;
        if ((int64_t)bl::pairwise_scratch_bytes(L, 256) > ((L / 2) & ~(int64_t)15))
            return fail(BITLINEAR_ERR_SHAPE, "%s: N*K=%lld too small for the scratch", fn,
                        (long long)L);
    }
    return from_hip(bl::launch_binarize(W, any ? N : 0, any ? K : 0, w_packed1, w_codes, alpha64,
                                        alpha, beta64, beta, stream),
                    fn);
}

bitlinear_status_t bitlinear_pack_weights1(const int8_t* w, int64_t N, int64_t K,
                                           uint32_t* w_packed1, int32_t* bad_count,
                                           hipStream_t stream) {
    const char* fn = "bitlinear_pack_weights1";
    BL_TRY(check_rows(fn, "N", N, kMaxN));
    if (K < 0 || K % 32 != 0 || K > BITLINEAR_MAX_K)
        return fail(BITLINEAR_ERR_SHAPE, "%s: K=%lld must be in [0, %d] and a multiple of 32", fn,
                    (long long)K, BITLINEAR_MAX_K);
    const bool any = N > 0 && K > 0;
    BL_TRY(need(fn, "w", w, any, 16));
    BL_TRY(need(fn, "w_packed1", w_packed1, any, 4));
    if (bad_count && !aligned(bad_count, 4))
        return fail(BITLINEAR_ERR_ALIGN, "%s: bad_count is not 4-byte aligned", fn);
    if (!any && !bad_count) return ok();
    return from_hip(bl::launch_pack1(w, any ? N : 0, any ? K : 0, w_packed1, bad_count, stream), fn);
}

bitlinear_status_t bitlinear_forward1(const int8_t* x_q, const float* gamma, int64_t M, int64_t K,
                                      const uint32_t* w_packed1, int64_t N, float beta, float* y,
                                      int32_t* acc, hipStream_t stream) {
    const char* fn = "bitlinear_forward1";
    BL_TRY(check_rows(fn, "M", M, (1LL << 31) - 1));
    BL_TRY(check_rows(fn, "N", N, kMaxN));
    if (K < 0 || K % 64 != 0 || K > BITLINEAR_MAX_K)
        return fail(BITLINEAR_ERR_SHAPE, "%s: K=%lld must be in [0, %d] and a multiple of 64", fn,
                    (long long)K, BITLINEAR_MAX_K);
    if (!std::isfinite(beta)) return fail(BITLINEAR_ERR_VALUE, "%s: beta is not finite", fn);
    const bool any_out = M > 0 && N > 0;
    const bool any_in = any_out && K > 0;
    BL_TRY(need(fn, "x_q", x_q, any_in, 16));
    BL_TRY(need(fn, "gamma", gamma, any_in, 4));
    BL_TRY(need(fn, "w_packed1", w_packed1, any_in, 8));
    BL_TRY(need(fn, "y", y, any_out, 4));
    if (acc && !aligned(acc, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: acc is not 4-byte aligned", fn);
    if (!any_out) return ok();
    if (K == 0) return from_hip(bl::launch_fill_zero(y, acc, M * N, stream), fn);
    return from_hip(bl::launch_forward1(x_q, gamma, (int)M, (int)K, w_packed1, (int)N, beta, y, acc,
                                        stream),
                    fn);
}

bitlinear_status_t bitlinear_quant_act_grouped(const void* x, bitlinear_dtype_t x_dtype, int64_t M,
                                               int64_t K, int64_t G, const float* rms_gain,
                                               float rms_eps, int8_t* x_q, float* gamma,
                                               hipStream_t stream) {
    const char* fn = "bitlinear_quant_act_grouped";
    BL_TRY(check_rows(fn, "M", M, (1LL << 31) - 1));
    BL_TRY(check_k(fn, "K", K));
    BL_TRY(check_groups(fn, K, G, 16));
    if (x_dtype != BITLINEAR_F32 && x_dtype != BITLINEAR_BF16)
        return fail(BITLINEAR_ERR_DTYPE, "%s: unknown dtype %d", fn, (int)x_dtype);
    if (rms_gain && !(std::isfinite(rms_eps) && rms_eps >= 0.0f))
        return fail(BITLINEAR_ERR_VALUE, "%s: rms_eps must be finite and >= 0", fn);
    const bool any = M > 0 && K > 0;
    BL_TRY(need(fn, "x", x, any, 16));
    BL_TRY(need(fn, "x_q", x_q, any, 16));
    BL_TRY(need(fn, "gamma", gamma, M > 0, 4));
    if (rms_gain && !aligned(rms_gain, 16))
        return fail(BITLINEAR_ERR_ALIGN, "%s: rms_gain is not 16-byte aligned", fn);
    if (M == 0) return ok();
    if (K == 0)  // every run is empty: gamma = 0
        return from_hip(bl::launch_quant_act(x, 0, M * G, 0, nullptr, 0.f, x_q, gamma, stream), fn);
    return from_hip(bl::launch_quant_act_grouped(x, x_dtype == BITLINEAR_BF16, M, K, G, rms_gain,
                                                 rms_eps, x_q, gamma, stream),
                    fn);
}

bitlinear_status_t bitlinear_forward_grouped(const int8_t* x_q, const float* gamma, int64_t M,
                                             int64_t K, int64_t G, const uint32_t* w_packed,
                                             int64_t N, const float* beta, float* y, int32_t* acc,
                                             hipStream_t stream) {
    const char* fn = "bitlinear_forward_grouped";
    BL_TRY(check_rows(fn, "M", M, kMaxM));
    BL_TRY(check_rows(fn, "N", N, kMaxN));
    BL_TRY(check_k(fn, "K", K));
    BL_TRY(check_groups(fn, K, G, 64));
    const bool any_out = M > 0 && N > 0;
    const bool any_in = any_out && K > 0;
    BL_TRY(need(fn, "x_q", x_q, any_in, 16));
    BL_TRY(need(fn, "gamma", gamma, any_in, 4));
    BL_TRY(need(fn, "w_packed", w_packed, any_in, 16));
    BL_TRY(need(fn, "beta", beta, any_in, 4));
    BL_TRY(need(fn, "y", y, any_out, 4));
    if (acc && !aligned(acc, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: acc is not 4-byte aligned", fn);
    if (!any_out) return ok();
    if (K == 0) {
        hipError_t e = bl::launch_fill_zero(y, nullptr, M * N, stream);
        if (e == hipSuccess && acc)
            e = bl::launch_fill_zero(reinterpret_cast<float*>(acc), nullptr, G * M * N, stream);
        return from_hip(e, fn);
    }
    if (bl::decode_lds_grouped_supports((int)M, (int)K, (int)G, (int)N))  // one launch
        return from_hip(bl::launch_decode_lds_grouped(x_q, gamma, (int)M, (int)K, (int)G, w_packed,
                                                      (int)N, beta, y, acc, stream),
                        fn);
    if (!acc)
        return fail(BITLINEAR_ERR_NULL,
                    "%s: acc is NULL; it may be NULL only on the one-launch path (G in {2, 4, 8}, "
                    "M <= 16, K/G %% 256 == 0)", fn);
    const int64_t KG = K / G;
    for (int64_t g = 0; g < G; ++g) {
        const hipError_t e = launch_forward_kernel(x_q + g * M * KG, gamma + g * M, M, KG,
                                                   w_packed + g * N * (KG / 16), N, 1.0f, nullptr,
                                                   acc + g * M * N, BITLINEAR_PATH_AUTO, stream);
        if (e != hipSuccess) return from_hip(e, fn);
    }
    return from_hip(bl::launch_group_sum(acc, gamma, beta, M, N, G, y, stream), fn);
}

int bitlinear_quant_forward_one_launch(int64_t M, int64_t K, int64_t N) {
    if (M != 1 || K < 1 || K > BITLINEAR_MAX_K || N < 1 || N > kMaxN) return 0;
    return (bl::decode_one_token((int)K, (int)N) || bl::quant_gemv_supports((int)M, (int)K, (int)N)) ? 1 : 0;
}

int bitlinear_forward_grouped_one_launch(int64_t M, int64_t K, int64_t G, int64_t N) {
    if (M < 1 || M > 16 || N < 1 || N > kMaxN || K < 256 || K > BITLINEAR_MAX_K || G < 2 || G > 8)
        return 0;
    return bl::decode_lds_grouped_supports((int)M, (int)K, (int)G, (int)N) ? 1 : 0;
}

bitlinear_status_t bitlinear_ternarize_grouped(const float* W_grouped, int64_t N, int64_t K,
                                               int64_t G, uint32_t* w_packed, int8_t* w_ternary,
                                               float* beta, double* beta64, hipStream_t stream) {
    const char* fn = "bitlinear_ternarize_grouped";
    BL_TRY(check_rows(fn, "N", N, kMaxN));
    BL_TRY(check_k(fn, "K", K));
    BL_TRY(check_groups(fn, K, G, 64));
    const bool any = N > 0 && K > 0;
    if (any && N * (K / 16) > (1LL << 40))
        return fail(BITLINEAR_ERR_SHAPE, "%s: N*K/16 exceeds 2^40", fn);
    BL_TRY(need(fn, "W_grouped", W_grouped, any, 16));
    BL_TRY(need(fn, "w_packed", w_packed, any, 16));
    BL_TRY(need(fn, "beta", beta, true, 4));
    BL_TRY(need(fn, "beta64", beta64, true, 8));
    if (w_ternary && !aligned(w_ternary, 16))
        return fail(BITLINEAR_ERR_ALIGN, "%s: w_ternary is not 16-byte aligned", fn);
    const int64_t KG = K / G;
    for (int64_t g = 0; g < G; ++g) {
        const hipError_t e = bl::launch_ternarize(
            any ? W_grouped + g * N * KG : nullptr, any ? N : 0, any ? KG : 0,
            any ? w_packed + g * N * (KG / 16) : nullptr,
            (any && w_ternary) ? w_ternary + g * N * KG : nullptr, beta + g, beta64 + g, stream);
        if (e != hipSuccess) return from_hip(e, fn);
    }
    return ok();
}

bitlinear_status_t bitlinear_pack_weights3(const int8_t* w, int64_t N, int64_t K,
                                           uint32_t* w_packed3, int32_t* bad_count,
                                           hipStream_t stream) {
    const char* fn = "bitlinear_pack_weights3";
    BL_TRY(check_rows(fn, "N", N, kMaxN));
    BL_TRY(check_k(fn, "K", K));
    const bool any = N > 0 && K > 0;
    BL_TRY(need(fn, "w", w, any, 16));
    BL_TRY(need(fn, "w_packed3", w_packed3, any, 16));
    if (bad_count && !aligned(bad_count, 4))
        return fail(BITLINEAR_ERR_ALIGN, "%s: bad_count is not 4-byte aligned", fn);
    if (!any && !bad_count) return ok();
    return from_hip(bl::launch_pack3(w, any ? N : 0, any ? K : 0, w_packed3, bad_count, stream), fn);
}

bitlinear_status_t bitlinear_forward3(const int8_t* x_q, const float* gamma, int64_t M, int64_t K,
                                      const uint32_t* w_packed3, int64_t N, float beta, float* y,
                                      int32_t* acc, hipStream_t stream) {
    const char* fn = "bitlinear_forward3";
    BL_TRY(check_rows(fn, "M", M, (1LL << 31) - 1));
    BL_TRY(check_rows(fn, "N", N, kMaxN));
    BL_TRY(check_k(fn, "K", K));
    if (!std::isfinite(beta)) return fail(BITLINEAR_ERR_VALUE, "%s: beta is not finite", fn);
    const bool any_out = M > 0 && N > 0;
    const bool any_in = any_out && K > 0;
    BL_TRY(need(fn, "x_q", x_q, any_in, 16));
    BL_TRY(need(fn, "gamma", gamma, any_in, 4));
    BL_TRY(need(fn, "w_packed3", w_packed3, any_in, 16));
    BL_TRY(need(fn, "y", y, any_out, 4));
    if (acc && !aligned(acc, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: acc is not 4-byte aligned", fn);
    if (!any_out) return ok();
    if (K == 0) return from_hip(bl::launch_fill_zero(y, acc, M * N, stream), fn);
    return from_hip(bl::launch_forward3(x_q, gamma, (int)M, (int)K, w_packed3, (int)N, beta, y, acc,
                                        stream),
                    fn);
}

bitlinear_status_t bitlinear_floor_empty(hipStream_t stream) {
    return from_hip(bl::launch_floor_empty(stream), "bitlinear_floor_empty");
}

bitlinear_status_t bitlinear_floor_stream_read(const void* p, int64_t bytes, uint32_t* sink,
                                               hipStream_t stream) {
    const char* fn = "bitlinear_floor_stream_read";
    if (bytes < 0 || bytes % 16 != 0)
        return fail(BITLINEAR_ERR_SHAPE, "%s: bytes=%lld must be >= 0 and a multiple of 16", fn,
                    (long long)bytes);
    BL_TRY(need(fn, "p", p, bytes > 0, 16));
    BL_TRY(need(fn, "sink", sink, bytes > 0, 4));
    if (bytes == 0) return ok();
    return from_hip(bl::launch_floor_stream_read(p, bytes, sink, stream), fn);
}

bitlinear_status_t bitlinear_floor_mfma(const int8_t* x_q, int64_t M, int64_t K,
                                        const uint32_t* w_packed, int64_t N, uint32_t* sink,
                                        hipStream_t stream) {
    const char* fn = "bitlinear_floor_mfma";
    BL_TRY(check_rows(fn, "M", M, kMaxM));
    BL_TRY(check_k(fn, "K", K));
    BL_TRY(check_rows(fn, "N", N, kMaxN));
    if (K % 128 != 0)
        return fail(BITLINEAR_ERR_SHAPE, "%s: K=%lld must be a multiple of 128", fn, (long long)K);
    if (((M + 127) / 128) * ((N + 255) / 256) > 0x7FFFFFFF)
        return fail(BITLINEAR_ERR_SHAPE, "%s: M=%lld, N=%lld need more than 2^31-1 tiles of 128 x 256", fn,
                    (long long)M, (long long)N);
    const bool any = M > 0 && N > 0 && K > 0;
    BL_TRY(need(fn, "x_q", x_q, any, 16));
    BL_TRY(need(fn, "w_packed", w_packed, any, 16));
    BL_TRY(need(fn, "sink", sink, any, 4));
    if (!any) return ok();
    return from_hip(bl::launch_floor_mfma(x_q, (int)M, (int)K, w_packed, (int)N, sink, stream), fn);
}

const char* bitlinear_last_error(void) { return g_err; }

int bitlinear_abi_version(void) { return BITLINEAR_ABI_VERSION; }

}  // extern "C"

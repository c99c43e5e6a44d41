// Skinny ternary product on int8 MFMA (M <= 64 tokens, HBM-bound).
//
// The ternary product (unite.ai BitNet.cpp article, 3. BitLinear-Betrieb;
// datacamp MatMul-free article: multiplying by -1, 0, +1 is negate, drop,
// keep) is run as v_mfma_i32_16x16x64_i8 on the 2-bit codes c = w + 1 in
// {0, 1, 2}: sum_k c_nk q_mk = acc_mn + S_m with S_m = sum_k q_mk, so
// acc = D - S.  One packed uint32 word holds 16 consecutive weights of one
// output column and unpacks with one shift and one mask per dword into the
// 16 int8 K-slots that a lane supplies to the B operand; the A operand of the
// same lane takes the 16 activation bytes of the same K positions, so the two
// operands agree slot for slot whatever order the instruction sums them in.
//
// Work split: a workgroup (4 or 8 waves) owns 16*NT output columns.  Its
// waves split K into contiguous ranges of 256-wide chunks; per chunk a lane
// streams one 16-byte load per N-tile (four packed words = 64 weights), so the
// 64 lanes of a wave read 16 columns x 64 contiguous bytes.  A wave issues the
// loads of kBatch chunks before its first MFMA, so several KB per wave are in
// flight at once.  Activations (M <= 64 rows, padded to 16-row tiles) come
// from L2.  S_m comes from one extra MFMA per K-slot against an all-ones B
// operand, which lands it in the accumulator layout at no VALU cost.  Partial
// sums of the waves meet in LDS; the rescale y = fl32(acc) *
// fl32(beta*gamma)/128 is fused into the store.
#include "device_common.h"
#include "internal.h"

namespace bl {
namespace {

// K-chunks (256 K each) whose loads a wave issues together before multiplying:
// four for one 16-row activation tile, fewer as the activation registers grow.
template <int MT>
constexpr int batch_chunks() { return MT == 1 ? 4 : (MT == 2 ? 2 : 1); }

template <int MT, int NT, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void skinny_mfma_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ gamma, int M, int K,
    const uint32_t* __restrict__ wp, int N, float beta, float* __restrict__ y,
    int32_t* __restrict__ acc_out, int chunks_per_wave) {
    __shared__ int red[WAVES][MT * NT][4][kWave];

    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int j = lane & 15;  // A row / B column within a 16-tile
    const int g = lane >> 4;  // K block of the lane inside one MFMA
    const int WR = K >> 4;    // packed words per weight row
    const int nchunks = (WR + 15) >> 4;
    const bool aligned = (WR & 3) == 0;
    const int n_base = blockIdx.x * (16 * NT);
    const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
    constexpr int kBatch = batch_chunks<MT>();

    v4i acc[MT][NT];
    v4i accS[MT];  // sum of the activation codes of each row (every column)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        accS[mt] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[mt][t] = v4i{0, 0, 0, 0};
    }

    const int c_begin = wv * chunks_per_wave;
    const int c_end = min(c_begin + chunks_per_wave, nchunks);
    for (int c0 = c_begin; c0 < c_end; c0 += kBatch) {
        uint32_t bw[kBatch][NT][4];
        v4i a[kBatch][MT][4];
        // issue every load of the batch first
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int c = c0 + i;
            const int wb = c * 16 + 4 * g;  // first packed word of this lane in chunk c
            const bool live = c < c_end;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int n = n_base + 16 * t + j;
#pragma unroll
                for (int s = 0; s < 4; ++s) bw[i][t][s] = 0u;
                if (live && n < N) {
                    const uint32_t* p = wp + (int64_t)n * WR + wb;
                    if (aligned && wb + 4 <= WR) {
                        v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
                        bw[i][t][0] = v.x; bw[i][t][1] = v.y; bw[i][t][2] = v.z; bw[i][t][3] = v.w;
                    } else {
#pragma unroll
                        for (int s = 0; s < 4; ++s) bw[i][t][s] = (wb + s < WR) ? p[s] : 0u;
                    }
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = 16 * mt + j;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (live && row < M && wb + s < WR)
                        a[i][mt][s] = *reinterpret_cast<const v4i*>(xq + (int64_t)row * K + 16 * (wb + s));
                    else
                        a[i][mt][s] = v4i{0, 0, 0, 0};
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const v4i b = unpack_codes(bw[i][t][s]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[mt][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i][mt][s], b, acc[mt][t], 0, 0, 0);
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    accS[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i][mt][s], ones, accS[mt], 0, 0, 0);
            }
        }
    }

    // lane (j, g) holds output rows 4g + v of column j; accS holds the row sums
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int t = 0; t < NT; ++t) red[wv][mt * NT + t][v][lane] = acc[mt][t][v] - accS[mt][v];
    __syncthreads();

    for (int p = wv; p < MT * NT; p += WAVES) {
        const int mt = p / NT, t = p % NT;
        const int col = n_base + 16 * t + j;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = 16 * mt + 4 * g + v;
            int a = 0;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) a += red[w][p][v][lane];
            if (row < M && col < N) {
                const int64_t o = (int64_t)row * N + col;
                if (y) y[o] = (float)a * out_scale(beta, gamma[row]);
                if (acc_out) acc_out[o] = a;
            }
        }
    }
}

template <int MT, int NT, int WAVES>
hipError_t launch_mt_nt(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                        int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    const int WR = K / 16;
    const int nchunks = (WR + 15) / 16;
    const int cpw = (nchunks + WAVES - 1) / WAVES;
    const int blocks = (N + 16 * NT - 1) / (16 * NT);
    skinny_mfma_kernel<MT, NT, WAVES><<<dim3(blocks), dim3(WAVES * kWave), 0, s>>>(
        xq, gamma, M, K, wp, N, beta, y, acc, cpw);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                     int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    // measured on K = 4096 / 8192 decode shapes: up to 4 tokens, 4 waves split
    // K and a wave owns one column tile; 5..16 tokens, 2 waves split K and a
    // wave owns two column tiles (the activation rows are then re-read from L2
    // half as often per weight byte)
    if (MT == 1 && M > 4) return launch_mt_nt<MT, 2, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    return launch_mt_nt<MT, 1, 4>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

}  // namespace

hipError_t launch_skinny_mfma(const int8_t* xq, const float* gamma, int M, int K,
                              const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                              hipStream_t s) {
    // 5..16 tokens, and 2..4 tokens at K >= 4096: the LDS-staged kernel
    // (measured on N x K = 11008 x 4096, 28672 x 8192, 6912 x 2560 and
    // 2560 x 2560: at K = 8192 it takes 16 us for 2..4 tokens against 18..23 us
    // here, at K = 4096, N = 11008 6.1-6.6 us against 6.5-7.3 us; at K = 2560
    // this kernel is as fast or faster below 5 tokens)
    // (one token too on long rows over many row tiles, decode_one_token)
    if ((M >= 5 || (M >= 2 && K >= 4096) || (M == 1 && decode_one_token(K, N))) &&
        decode_lds_supports(M, K, N))
        return launch_decode_lds(xq, gamma, M, K, wp, N, beta, y, acc, s);
    switch ((M + 15) / 16) {
        case 1: return launch_mt<1>(xq, gamma, M, K, wp, N, beta, y, acc, s);
        case 2: return launch_mt<2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
        case 3: return launch_mt<3>(xq, gamma, M, K, wp, N, beta, y, acc, s);
        default: return launch_mt<4>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    }
}

}  // namespace bl

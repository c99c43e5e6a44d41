// Prefill GEMM on int8 MFMA (M >= 64 tokens, MFMA-bound at large M).
//
// Same arithmetic as the skinny kernel (unite.ai BitNet.cpp article, 3.
// BitLinear-Betrieb): v_mfma_i32_16x16x64_i8 on the 2-bit codes c = w + 1,
// and acc = D - S_m with S_m the sum of the token's int8 activations.
//
// Tiling: a workgroup of 4 waves computes a BM x BN = 128 x 128 output tile
// (each wave 64 x 64 = 4 x 4 MFMA tiles) and walks K in steps of BK = 128.
// Per step it stages the activation tile (128 rows x 128 bytes) and the packed
// weight tile (128 columns x 8 words = 32 bytes) in LDS, double-buffered: the
// global loads of step k+1 are in flight while step k is multiplied.  A lane's
// B operand is one packed word (16 consecutive weights of one column),
// unpacked in registers by shift+mask and reused by the wave's four M tiles;
// its A operand is 16 activation bytes of the same K positions read from LDS.
// The activation tile is stored with its 16-byte chunks XOR-swizzled by row so
// that the 16 rows read by one MFMA operand fetch land in distinct LDS banks.
// S_m is accumulated from the staged activation chunks while they pass
// through registers.  The epilogue subtracts S_m and applies the rescale
// y = fl32(acc) * fl32(beta*gamma_m)/128 on the way out.
#include "device_common.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kGmThreads = 256;
constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kChunksPerRow = BK / 16;        // 16-byte activation chunks per tile row
constexpr int kWordsPerCol = BK / 16;         // packed words per tile column
constexpr int kBStride = kWordsPerCol + 1;    // padded LDS row of the weight tile

__device__ __forceinline__ int swz(int row) { return (row >> 1) & (kChunksPerRow - 1); }

__global__ __launch_bounds__(kGmThreads) void gemm_mfma_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ gamma, int M, int K,
    const uint32_t* __restrict__ wp, int N, float beta, float* __restrict__ y,
    int32_t* __restrict__ acc_out) {
    __shared__ v4i As[2][BM][kChunksPerRow];
    __shared__ uint32_t Bs[2][BN][kBStride];
    __shared__ int Ssum[BM];
    __shared__ float Ssc[BM];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = tid / kWave;
    const int wm = wv >> 1, wn = wv & 1;
    const int j = lane & 15, g = lane >> 4;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int WR = K >> 4;
    const bool aligned = (WR & 3) == 0;
    const int KT = (K + BK - 1) / BK;

    // global -> register staging assignment
    const int a_ch = tid & (kChunksPerRow - 1);   // chunk within a tile row
    const int a_r0 = tid / kChunksPerRow;         // rows a_r0 + 32*i
    const int b_col = tid >> 1;
    const int b_half = tid & 1;

    v4i ga[4];
    uint32_t gb[4];
    int s_acc[4] = {0, 0, 0, 0};

    auto load_tile = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + a_r0 + 32 * i;
            const int kk = k0 + 16 * a_ch;
            if (row < M && kk < K)
                ga[i] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4i*>(xq + (int64_t)row * K + kk));
            else
                ga[i] = v4i{0, 0, 0, 0};
        }
        const int col = n0 + b_col;
        const int wb = kt * kWordsPerCol + 4 * b_half;
        if (col < N) {
            const uint32_t* p = wp + (int64_t)col * WR + wb;
            if (aligned && wb + 4 <= WR) {
                v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
                gb[0] = v.x; gb[1] = v.y; gb[2] = v.z; gb[3] = v.w;
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) gb[s] = (wb + s < WR) ? p[s] : 0u;
            }
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) gb[s] = 0u;
        }
    };

    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = a_r0 + 32 * i;
            As[buf][r][a_ch ^ swz(r)] = ga[i];
            s_acc[i] = byte_sum16(ga[i], s_acc[i]);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) Bs[buf][b_col][4 * b_half + s] = gb[s];
    };

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][t] = v4i{0, 0, 0, 0};

    if (KT > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) load_tile(kt + 1);
#pragma unroll
        for (int kk = 0; kk < BK / 64; ++kk) {
            v4i bf[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                bf[t] = unpack_codes(Bs[buf][wn * 64 + 16 * t + j][kk * 4 + g]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 64 + 16 * i + j;
                const v4i af = As[buf][r][(kk * 4 + g) ^ swz(r)];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[i][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[t], acc[i][t], 0, 0, 0);
            }
        }
        if (kt + 1 < KT) store_tile(buf ^ 1);
        __syncthreads();
    }

    // row sums: the 8 threads sharing a tile row are consecutive lanes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int sv = s_acc[i];
        sv += __shfl_xor(sv, 1, kWave);
        sv += __shfl_xor(sv, 2, kWave);
        sv += __shfl_xor(sv, 4, kWave);
        if (a_ch == 0) Ssum[a_r0 + 32 * i] = sv;
    }
    if (tid < BM) {
        const int row = m0 + tid;
        Ssc[tid] = (row < M) ? out_scale(beta, gamma[row]) : 0.f;
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int rl = wm * 64 + 16 * i + 4 * g + v;
            const int row = m0 + rl;
            const int sm = Ssum[rl];
            const float sc = Ssc[rl];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int col = n0 + wn * 64 + 16 * t + j;
                if (row < M && col < N) {
                    const int a = acc[i][t][v] - sm;
                    const int64_t o = (int64_t)row * N + col;
                    y[o] = (float)a * sc;
                    if (acc_out) acc_out[o] = a;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_mfma(const int8_t* xq, const float* gamma, int M, int K,
                            const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                            hipStream_t s) {
    dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
    gemm_mfma_kernel<<<grid, dim3(kGmThreads), 0, s>>>(xq, gamma, M, K, wp, N, beta, y, acc);
    return hipGetLastError();
}

}  // namespace bl

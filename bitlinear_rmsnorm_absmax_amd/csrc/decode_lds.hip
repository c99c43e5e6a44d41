// Decode product for a few tokens (5 <= M <= 16) on int8 MFMA, activations
// staged in LDS; 2-bit ternary weights, or 1-bit weights (ONEBIT).
//
// Arithmetic as in the other forward kernels (unite.ai BitNet.cpp article, 3.
// BitLinear-Betrieb; datacamp MatMul-free article): v_mfma_i32_16x16x64_i8 on
// the unsigned codes c = w + 1 (2-bit) or c = (w + 1) / 2 (1-bit), giving
// D = sum c q; then acc = D - S (2-bit) or 2 D - S (1-bit) with S the sum of
// the token's int8 activations over K, taken once per workgroup from LDS.
//
// Why LDS: at a handful of tokens the weights are read once from HBM while
// every workgroup needs all M activation rows.  Loading the activation
// operand per lane from global memory (16 rows x 16 bytes per instruction)
// floods the per-CU L1 with scattered requests and stalls the address unit,
// which then also delays the weight stream.  Here each workgroup copies the
// M x K activation block into LDS once, in 1 KB contiguous pieces straight
// from global memory (global_load_lds).
//
// Order (measured with per-wave timestamps: loads of a compute unit return
// in issue order, so copies queued behind weight misses wait for HBM):
//   1. every wave issues its activation copies; a barrier makes sure all
//      copies of the workgroup are queued before any weight load;
//   2. every wave issues the B weight loads of its first batch (unconditional,
//      clamped chunks, so their number is a constant), then waits until at
//      most B * NTW vector-memory operations are outstanding -- exactly its
//      own copies, which are older -- and a second barrier publishes the
//      activations;
//   3. the activation sums S (all threads, from LDS) while the weights are in
//      flight, then the MFMAs, each waiting only for its own weight registers.
// Chunks past a wave's range multiply all-zero codes.
//
// Work split: a workgroup of 8 waves owns CT column tiles of 16; a wave owns
// NTW of them and one of KS = 8 * NTW / CT contiguous K ranges (256-K
// chunks).  Partial sums of the KS waves of a tile meet in LDS.
//
// LDS layout of the activations: row r holds its K bytes as 16-byte pieces,
// piece p stored at slot p ^ (r & 15) of the row, so the 16 rows read by one
// operand fetch fall on different banks.  Requires K % 256 == 0.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace bl {
namespace {

constexpr int kDecWaves = 8;
constexpr int kDecLdsMax = 160 * 1024;
typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base,
                                     16, 0, 0);
#endif
}

// s_waitcnt immediate (gfx9 encoding): vmcnt <= vm, lgkmcnt and expcnt any
constexpr int vm_wait_imm(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | (0xF << 8); }

// Nothing is moved across this point by the compiler, memory or arithmetic.
__device__ __forceinline__ void fence_code() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// ONEBIT: 1-bit weights ([N][K/32], entry 4j + b of a word at bit 8b + j):
// lane (j, g) loads words 8c + 2g, 8c + 2g + 1 of chunk c (the same 64 K
// positions as the 2-bit words 16c + 4g .. +3), and MFMA s takes bits
// 4(s%2) .. +3 of word s/2.
template <int CT, int NTW, int B, bool ONEBIT, int G>
__global__ __launch_bounds__(kDecWaves * kWave) void decode_lds_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ gamma, int M, int K,
    const uint32_t* wp, int N, float beta, float* __restrict__ y, int32_t* __restrict__ acc_out,
    int a_bytes, const float* __restrict__ beta_g) {
    constexpr int CG = CT / NTW;         // column groups of a workgroup
    constexpr int KS = kDecWaves / CG;   // K ranges per column group
    static_assert(KS % G == 0, "every wave's K range lies inside one group");
    typedef typename std::conditional<ONEBIT, v2u, v4u>::type wvec;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* As = smem;                                       // activations, a_bytes
    int* red = reinterpret_cast<int*>(smem + a_bytes);     // [8 waves][NTW][4][64]
    int* Ssum = red + kDecWaves * NTW * 4 * kWave;         // [G][16] activation sums
    float* Ssc = reinterpret_cast<float*>(Ssum + 16 * G);  // [G][16] output scales

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int cg = wv % CG, kp = wv / CG;
    const int j = lane & 15, g = lane >> 4;
    const int WR = K >> 4;          // 16-byte pieces per activation row (= 2-bit words per row)
    const int nchunks = K >> 8;
    const int n_base = blockIdx.x * (16 * CT) + cg * 16 * NTW;

    const int cpw = (nchunks + KS - 1) / KS;
    const int c_begin = kp * cpw;
    const int c_end = min(c_begin + cpw, nchunks);
    const int last = max(min(c_end, nchunks) - 1, 0);
    // groups (G > 1): group-major operands, KG = K / G inputs per group; the
    // launcher makes every wave's chunk range lie inside one group, gw
    const int KG = K / G, cpg = nchunks / G;
    const int gw = G > 1 ? c_begin / cpg : 0;
    const int WRWG = ONEBIT ? (KG >> 5) : (KG >> 4);  // weight words per row of a group

    v4i acc[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[t] = v4i{0, 0, 0, 0};
    // lane (j, g): column j of each tile, packed words 16c + 4g .. +3 of chunk c;
    // columns past N are clamped onto the last one (never stored)
    const uint32_t* wrow[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t)
        wrow[t] = wp + ((int64_t)gw * N + min(n_base + 16 * t + j, N - 1)) * WRWG + (ONEBIT ? 2 : 4) * g;
    // A-operand row of lane j; rows past M repeat row M-1 (never stored)
    const int arow = min(j, M - 1);
    const char* arow_p = As + arow * K;
    const int axor = arow & 15;

    auto load_batch = [&](int cb, wvec (&bw)[B][NTW]) {
#pragma unroll
        for (int i = 0; i < B; ++i)
#pragma unroll
            for (int t = 0; t < NTW; ++t)
                bw[i][t] = __builtin_nontemporal_load(reinterpret_cast<const wvec*>(
                    wrow[t] + (ONEBIT ? 8 : 16) * (min(cb + i, last) - gw * cpg)));
    };
    auto mul_batch = [&](int cb, const wvec (&bw)[B][NTW]) {
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const bool live = cb + i < c_end;
            const int c = min(cb + i, last);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int p = 16 * c + 4 * g + s;
                const v4i a = *reinterpret_cast<const v4i*>(arow_p + 16 * (p ^ axor));
#pragma unroll
                for (int t = 0; t < NTW; ++t) {
                    v4i b;
                    if constexpr (ONEBIT) {
                        const uint32_t w = live ? bw[i][t][s >> 1] : 0u;
                        const int j0 = 4 * (s & 1);
                        b = v4i{(int)((w >> j0) & 0x01010101u), (int)((w >> (j0 + 1)) & 0x01010101u),
                                (int)((w >> (j0 + 2)) & 0x01010101u), (int)((w >> (j0 + 3)) & 0x01010101u)};
                    } else {
                        b = unpack_codes(live ? bw[i][t][s] : 0u);
                    }
                    acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[t], 0, 0, 0);
                }
            }
        }
    };

    // 1. activation copies of the whole workgroup, queued ahead of any weight load
    {
        // row = pos / WR and group = k / KG by multiply-high with a reciprocal
        // taken once: floor(x / d) = umulhi(x, floor((2^32 - 1) / d) + 1),
        // exact for x * d < 2^32 (here pos * WR < 2^30 and (k/256) * (KG/256)
        // < 2^18); the reciprocal of d = 1 does not fit 32 bits, so a group
        // of 256 inputs takes k >> 8 directly
        const int pieces = M * WR;
        const int ninstr = (pieces + 63) >> 6;
        const uint32_t wr_inv = 0xFFFFFFFFu / (uint32_t)WR + 1u;  // WR >= 16
        const uint32_t kg_inv = (G > 1 && KG > 256) ? 0xFFFFFFFFu / (uint32_t)(KG >> 8) + 1u : 0u;
        for (int q = wv; q < ninstr; q += kDecWaves) {
            const int pos = min(q * 64 + lane, pieces - 1);
            const int r = (int)__umulhi((uint32_t)pos, wr_inv), slot = pos - r * WR;
            const int k = 16 * (slot ^ (r & 15));  // input index of the piece
            const int kg = G == 1 ? 0 : KG == 256 ? (k >> 8) : (int)__umulhi((uint32_t)(k >> 8), kg_inv);
            copy16_to_lds(xq + ((int64_t)kg * M + r) * KG + (k - kg * KG), As + 1024 * q);
        }
    }
    fence_code();
    __builtin_amdgcn_s_barrier();
    fence_code();

    // 2. the first batch of weight loads stays in flight across the barrier
    //    that publishes the activations; 3. activation sums while it lands
    auto publish = [&]() {
        fence_code();
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(B * NTW));  // own copies (older) have landed
        __builtin_amdgcn_s_barrier();
        fence_code();
        // row r = tid / 32, 32 threads per row, per group (the slot order
        // inside a row does not change a sum; group gg holds slots
        // gg*KG/16 .. (gg+1)*KG/16 since KG is a multiple of 256)
        // output scales fl32(beta_g * gamma[g][m]) / 128 of every (group, row)
        if (tid < 16 * G) {
            const int gi = tid >> 4, ri = tid & 15;
            Ssc[tid] = ri < M ? out_scale(beta_g ? beta_g[gi] : beta, gamma[(int64_t)gi * M + ri]) : 0.0f;
        }
        // 32 / G lanes per (row, group): lane `sub` of group gg takes the
        // group's pieces sub, sub + 32/G, ...
        constexpr int L = 32 / G;
        const int r = tid >> 5, gg = (tid & 31) / L, sub = tid & (L - 1);
        const int pg = KG >> 4;  // pieces per group
        int sum = 0;
        if (r < M)
            for (int q = gg * pg + sub; q < (gg + 1) * pg; q += L)
                sum = byte_sum16(*reinterpret_cast<const v4i*>(As + r * K + 16 * q), sum);
#pragma unroll
        for (int o = L / 2; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
        if (sub == 0) Ssum[gg * 16 + r] = sum;
    };
    if (c_end - c_begin <= B) {
        // one batch
        wvec bw[B][NTW];
        load_batch(c_begin, bw);
        publish();
        mul_batch(c_begin, bw);
    } else {
        // a stream of batches, the next one's loads issued before the current
        // one is multiplied (a wave keeps at most 2 B NTW loads in flight, so
        // load issue does not stall on the compute unit's outstanding-request
        // limit); the loads past the range re-read the last chunk
        wvec b0[B][NTW], b1[B][NTW];
        load_batch(c_begin, b0);
        publish();
        for (int cb = c_begin;;) {
            load_batch(cb + B, b1);
            mul_batch(cb, b0);
            cb += B;
            if (cb >= c_end) break;
            load_batch(cb + B, b0);
            mul_batch(cb, b1);
            cb += B;
            if (cb >= c_end) break;
        }
    }

    // lane (j, g) holds rows 4g + v of column j
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((wv * NTW + t) * 4 + v) * kWave + lane] = acc[t][v];
    __syncthreads();
    if (kp == 0) {
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
            const int col = n_base + 16 * t + j;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 4 * g + v;
                if (row >= M || col >= N) continue;
                // group gi = K parts gi*KPG .. (gi+1)*KPG; y adds the group
                // terms in group order (G == 1: the one term)
                constexpr int KPG = KS / G;
                float yv = 0.0f;
#pragma unroll
                for (int gi = 0; gi < G; ++gi) {
                    int d = 0;
#pragma unroll
                    for (int k2 = gi * KPG; k2 < (gi + 1) * KPG; ++k2)
                        d += red[(((k2 * CG + cg) * NTW + t) * 4 + v) * kWave + lane];
                    const int a = (ONEBIT ? 2 * d : d) - Ssum[gi * 16 + row];
                    const float term = (float)a * Ssc[gi * 16 + row];
                    yv = gi == 0 ? term : yv + term;
                    if (acc_out) acc_out[((int64_t)gi * M + row) * N + col] = a;
                }
                if (y) y[(int64_t)row * N + col] = yv;
            }
        }
    }
}

// LDS bytes: the activation block rounded up to whole 1 KB copies, the
// reduction buffer, and 16 activation sums and 16 output scales per group.
int decode_a_bytes(int M, int K) { return ((M * K + 1023) / 1024) * 1024; }
size_t decode_lds_bytes(int M, int K, int ntw, int G = 1) {
    return (size_t)decode_a_bytes(M, K) + (size_t)kDecWaves * ntw * 4 * kWave * 4 + 2 * 16 * 4 * (size_t)G;
}

template <int CT, int NTW, int B, bool ONEBIT, int G>
hipError_t launch_ctb(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp, int N,
                      float beta, float* y, int32_t* acc, hipStream_t s, const float* beta_g) {
    static DynLdsOptIn opt_in;
    const hipError_t e = opt_in.ensure(
        reinterpret_cast<const void*>(&decode_lds_kernel<CT, NTW, B, ONEBIT, G>), kDecLdsMax);
    if (e != hipSuccess) return e;
    const int blocks = (N + 16 * CT - 1) / (16 * CT);
    decode_lds_kernel<CT, NTW, B, ONEBIT, G><<<dim3(blocks), dim3(kDecWaves * kWave),
                                               decode_lds_bytes(M, K, NTW, G), s>>>(
        xq, gamma, M, K, wp, N, beta, y, acc, decode_a_bytes(M, K), beta_g);
    return hipGetLastError();
}

// Batch: a wave's whole K range in one batch when it has at most 4 chunks,
// else a stream of 2-chunk batches (measured at K = 2560 .. 8192: larger
// batches stall load issue, a 2-chunk stream is 15 % faster at K = 8192).
template <int CT, int NTW, bool ONEBIT, int G = 1>
hipError_t launch_ct(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp, int N,
                     float beta, float* y, int32_t* acc, hipStream_t s,
                     const float* beta_g = nullptr) {
    constexpr int KS = kDecWaves * NTW / CT;
    const int cpw = ((K >> 8) + KS - 1) / KS;
    if (cpw <= 4) return launch_ctb<CT, NTW, 4, ONEBIT, G>(xq, gamma, M, K, wp, N, beta, y, acc, s, beta_g);
    return launch_ctb<CT, NTW, 2, ONEBIT, G>(xq, gamma, M, K, wp, N, beta, y, acc, s, beta_g);
}

// Grouped launch of one width: G as a template argument (2, 4 or 8, at most
// the width's K parts).
template <int CT, int NTW>
hipError_t launch_ct_groups(const int8_t* xq, const float* gamma, int M, int K, int G,
                            const uint32_t* wp, int N, const float* beta_g, float* y, int32_t* acc,
                            hipStream_t s) {
    constexpr int KS = kDecWaves * NTW / CT;
    if (G == 2) return launch_ct<CT, NTW, false, 2>(xq, gamma, M, K, wp, N, 0.f, y, acc, s, beta_g);
    if constexpr (KS >= 4)
        if (G == 4) return launch_ct<CT, NTW, false, 4>(xq, gamma, M, K, wp, N, 0.f, y, acc, s, beta_g);
    if constexpr (KS >= 8)
        if (G == 8) return launch_ct<CT, NTW, false, 8>(xq, gamma, M, K, wp, N, 0.f, y, acc, s, beta_g);
    return hipErrorInvalidValue;
}

// K parts of the widths below, widest first: <8,2> 2, <4,2> 4, <2,1> 4, <1,1> 8.
// Grouped launches need KS % G == 0 and (K/256) % KS == 0 so that every wave's
// K range lies inside one group.
int grouped_width(int tiles, int G, int nchunks) {
    const int ct[4] = {8, 4, 2, 1}, ks[4] = {2, 4, 4, 8}, min_tiles[4] = {8 * 200, 4 * 200, 2 * 200, 0};
    int pick = -1;
    for (int i = 3; i >= 0; --i)  // the widest fitting config that still leaves >= 200 workgroups
        if (ks[i] % G == 0 && nchunks % ks[i] == 0 && (pick < 0 || tiles >= min_tiles[i])) pick = i;
    return pick < 0 ? -1 : ct[pick];
}

template <bool ONEBIT>
hipError_t launch_widths(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                         int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    // widest workgroup that still leaves >= 200 workgroups: fewer, wider
    // groups copy the activation block fewer times, too few leave CUs idle.
    // Measured on N = 2560 .. 28672, K = 2560 .. 8192, 2 to 16 tokens: at
    // K = 4096, N = 11008 (688 tiles) 344 workgroups of 2 tiles beat 172 of 4
    // up to 8 tokens (M = 4: 6.5 vs 7.2 us; M = 8: 6.7 vs 7.2 us) and tie at
    // 16; at K = 8192, N = 28672 224 groups of 8 tiles beat 448 of 4.
    const int tiles = (N + 15) / 16;
    if (tiles >= 8 * 200) return launch_ct<8, 2, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    if (tiles >= 4 * 200) return launch_ct<4, 2, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    if (tiles >= 2 * 200) return launch_ct<2, 1, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    return launch_ct<1, 1, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

}  // namespace

bool decode_lds_supports(int M, int K, int N) {
    return M >= 1 && M <= 16 && K >= 256 && K % 256 == 0 && N > 0 &&
           decode_lds_bytes(M, K, 2) <= (size_t)kDecLdsMax;
}

bool decode_lds_grouped_supports(int M, int K, int G, int N) {
    if ((G != 2 && G != 4 && G != 8) || M < 1 || M > 16 || N <= 0 || K % 256 != 0 || K % G != 0 || (K / G) % 256 != 0)
        return false;
    return grouped_width((N + 15) / 16, G, K >> 8) > 0 &&
           decode_lds_bytes(M, K, 2, G) <= (size_t)kDecLdsMax;
}

hipError_t launch_decode_lds_grouped(const int8_t* xq, const float* gamma, int M, int K, int G,
                                     const uint32_t* wp, int N, const float* beta_g, float* y,
                                     int32_t* acc, hipStream_t s) {
    if (G != 2 && G != 4 && G != 8) return hipErrorInvalidValue;
    switch (grouped_width((N + 15) / 16, G, K >> 8)) {
        case 8: return launch_ct_groups<8, 2>(xq, gamma, M, K, G, wp, N, beta_g, y, acc, s);
        case 4: return launch_ct_groups<4, 2>(xq, gamma, M, K, G, wp, N, beta_g, y, acc, s);
        case 2: return launch_ct_groups<2, 1>(xq, gamma, M, K, G, wp, N, beta_g, y, acc, s);
        case 1: return launch_ct_groups<1, 1>(xq, gamma, M, K, G, wp, N, beta_g, y, acc, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_lds(const int8_t* xq, const float* gamma, int M, int K,
                             const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                             hipStream_t s) {
    return launch_widths<false>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

hipError_t launch_decode_lds1(const int8_t* xq, const float* gamma, int M, int K,
                              const uint32_t* wp1, int N, float beta, float* y, int32_t* acc,
                              hipStream_t s) {
    return launch_widths<true>(xq, gamma, M, K, wp1, N, beta, y, acc, s);
}

}  // namespace bl

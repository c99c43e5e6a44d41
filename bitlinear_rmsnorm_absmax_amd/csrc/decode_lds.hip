// Decode product for a few tokens (M <= 16) on int8 MFMA, activations
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
// Work split: a workgroup of 8 waves owns CT column tiles of 16 / H rows; a
// wave owns NTW of them and one of KS = 8 * NTW / CT contiguous K ranges
// (256 H-input units).  Partial sums of the KS waves of a tile meet in LDS.
//
// LDS layout of the activations: row r holds its K bytes as 16-byte pieces,
// piece p stored at slot p ^ (r & 15) of the row, so the 16 rows read by one
// operand fetch fall on different banks.  Requires K % 256 == 0.
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "quant_rows.h"

namespace bl {
namespace {

typedef unsigned v2u __attribute__((ext_vector_type(2)));

// One token quantised inside the kernel (FQ != 0): the fp32 or bf16 row, the
// optional RMSNorm gain and epsilon, and where workgroup 0 writes the codes
// and gamma.
struct FusedRow {
    const void* x = nullptr;
    const float* gain = nullptr;
    float eps = 0.0f;
    int8_t* q_out = nullptr;
    float* gamma_out = nullptr;
};

// s_waitcnt immediate (gfx9 encoding): vmcnt <= vm, lgkmcnt and expcnt any
constexpr int vm_wait_imm(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | (0xF << 8); }

// Nothing is moved across this point by the compiler, memory or arithmetic.
__device__ __forceinline__ void fence_code() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// ONEBIT: 1-bit weights ([N][K/32], entry 4j + b of a word at bit 8b + j),
// K % 512 == 0: the unit of a load is 512 inputs (16 words a row) instead of
// 256, so that a lane still loads 16 bytes: lane (j, g) loads words
// 16u + 4g .. +3 of unit u (K positions 512u + 128g .. +127), and MFMA
// s = 0..7 of the unit takes bits 4(s%2) .. +3 of word s/2, the 16 inputs at
// 512u + 128g + 16s, with the activation piece 32u + 8g + s.  (Loads of 8
// bytes, one 256-input chunk each, ran 8 tokens at K = 8192, N = 28672 in
// 15.6 us, no faster than the 2-bit weights at twice the bytes.)
//
// H > 1 (one group, M <= 16 / H; 1-bit weights H = 2): an MFMA tile holds
// RT = 16 / H weight rows, each over H K parts, so that a load instruction
// reads RT rows x 64 H contiguous bytes (8 x 128 B or 4 x 256 B, which stream
// at 5.9-6.0 TB/s where 16 rows x 64 B with the rows spread over neighbouring
// lanes reach 4.7).  A row i = h + H m holds token m over K part h, B column
// j = h + H r holds tile row r over part h, and lane (j, g) loads the 16-byte
// piece h + H g of each 64 H-byte unit of its row (the row of a lane pair or
// quad is contiguous in memory); both operands take the K positions of that
// piece (activation pieces 4 (h + H g) + s, 1-bit: 8 (h + H g) + s).  D[h + H m][h' + H r] is the product
// of token m and row r over part h when h == h' (the other blocks mix parts
// and are not used); token m's sum over row r is the sum of the H diagonal
// blocks, which the epilogue adds from the partials in LDS.
// TG > 1 (H == 2): TG groups of 8 tokens, each with its own MFMA and A rows,
// share every unpacked weight fragment (M <= 8 TG), so 9..16 tokens keep the
// 8 x 128 B loads.  With one K range per tile (KS == 1) the two diagonal
// blocks are added in registers (lane 2r + 16 q' and its odd neighbour) and no
// LDS reduction buffer is allocated.
// FQ != 0 (one token, two K parts): the token arrives unquantised (FQ = 1
// fp32, 2 bf16; FRMS: RMSNorm first) and every workgroup quantises it into
// its LDS row, in the chunk order and reduction order of the quantiser
// (quant_rows.h, the first 256 threads), so gamma and the codes are
// bit-identical to bitlinear_quant_act's; workgroup 0 also writes them out.
// The row's first chunks are loaded before the weights (loads of a compute
// unit return in issue order) and quantised while the first weights land.
template <int CT, int NTW, int B, bool ONEBIT, int G, int H = 1, int TG = 1, int FQ = 0,
          bool FRMS = false>
__global__ __launch_bounds__(kDecWaves * kWave) void decode_lds_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ gamma, int M, int K,
    const uint32_t* wp, int N, float beta, float* __restrict__ y, int32_t* __restrict__ acc_out,
    int a_bytes, const float* __restrict__ beta_g, FusedRow fr) {
    constexpr int CG = CT / NTW;         // column groups of a workgroup
    constexpr int KS = kDecWaves / CG;   // K ranges per column group
    static_assert(KS % G == 0, "every wave's K range lies inside one group");
    static_assert(H == 1 || ((H == 2 || H == 4 || H == 8 || H == 16) && G == 1 && (!ONEBIT || H == 2)),
                  "K parts: one group (1-bit weights: two parts)");
    static_assert(TG == 1 || (H == 2 && KS == 1), "token groups: two K parts, one K range");
    static_assert(FQ == 0 || (H == 2 && TG == 1 && KS == 1 && !ONEBIT), "fused quantisation: one token");
    constexpr bool kRegEpi = H == 2 && KS == 1;  // diagonal blocks added in registers
    constexpr int kRedNtw = kRegEpi ? 0 : NTW;   // LDS reduction buffer: [8 waves][kRedNtw][4][64]
    typedef v4u wvec;
    constexpr int kHLog = H == 16 ? 4 : H == 8 ? 3 : H == 4 ? 2 : H == 2 ? 1 : 0;
    constexpr int RT = 16 / H;                            // weight rows of a tile
    constexpr int kUnitLog = (ONEBIT ? 9 : 8) + kHLog;    // inputs per load unit: 512 H (1-bit) or 256 H
    constexpr int kUnitWords = 16 * H;                    // packed words of a row per unit
    constexpr int kSteps = ONEBIT ? 8 : 4;                // MFMAs per unit
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* As = smem;                                       // activations, a_bytes
    int* red = reinterpret_cast<int*>(smem + a_bytes);     // [8 waves][kRedNtw][4][64]
    int* Ssum = red + kDecWaves * kRedNtw * 4 * kWave;     // [G][16] activation sums
    float* Ssc = reinterpret_cast<float*>(Ssum + 16 * G);  // [G][16] output scales

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int cg = wv % CG, kp = wv / CG;
    const int j = lane & 15, g = lane >> 4;
    const int h = j & (H - 1), jr = j >> kHLog;  // K part and tile row (token) of lane j
    const int WR = K >> 4;          // 16-byte pieces per activation row (= 2-bit words per row)
    const int nchunks = K >> kUnitLog;  // load units
    const int n_base = blockIdx.x * (RT * CT) + cg * RT * NTW;

    const int cpw = (nchunks + KS - 1) / KS;
    const int c_begin = kp * cpw;
    const int c_end = min(c_begin + cpw, nchunks);
    const int last = max(min(c_end, nchunks) - 1, 0);
    // groups (G > 1): group-major operands, KG = K / G inputs per group; the
    // launcher makes every wave's chunk range lie inside one group, gw
    const int KG = K / G, cpg = nchunks / G;
    const int gw = G > 1 ? c_begin / cpg : 0;
    const int WRWG = ONEBIT ? (KG >> 5) : (KG >> 4);  // weight words per row of a group

    v4i acc[TG][NTW];
#pragma unroll
    for (int q = 0; q < TG; ++q)
#pragma unroll
        for (int t = 0; t < NTW; ++t) acc[q][t] = v4i{0, 0, 0, 0};
    // lane (j, g): row jr of each tile, packed words 16 H c + 4 (h + H g) .. +3
    // of unit c (H == 1: column j, words 16c + 4g); rows past N are clamped
    // onto the last one (never stored)
    const uint32_t* wrow[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t)
        wrow[t] = wp + ((int64_t)gw * N + min(n_base + RT * t + jr, N - 1)) * WRWG + 4 * (h + H * g);
    // A-operand token of lane j in each token group; tokens past M repeat
    // token M-1 (never stored)
    const char* arow_p[TG];
    int axor[TG];
#pragma unroll
    for (int q = 0; q < TG; ++q) {
        const int arow = min(RT * q + jr, M - 1);
        arow_p[q] = As + arow * K;
        axor[q] = arow & 15;
    }

    auto load_batch = [&](int cb, wvec (&bw)[B][NTW]) {
#pragma unroll
        for (int i = 0; i < B; ++i)
#pragma unroll
            for (int t = 0; t < NTW; ++t)
                bw[i][t] = __builtin_nontemporal_load(reinterpret_cast<const wvec*>(
                    wrow[t] + kUnitWords * (min(cb + i, last) - gw * cpg)));
    };
    auto mul_batch = [&](int cb, const wvec (&bw)[B][NTW]) {
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const bool live = cb + i < c_end;
            const int c = min(cb + i, last);
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
                const int p = ONEBIT ? 32 * H * c + 8 * (h + H * g) + s : 16 * H * c + 4 * (h + H * g) + s;
                v4i a[TG];
#pragma unroll
                for (int q = 0; q < TG; ++q)
                    a[q] = *reinterpret_cast<const v4i*>(arow_p[q] + 16 * (p ^ axor[q]));
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
#pragma unroll
                    for (int q = 0; q < TG; ++q)
                        acc[q][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[q], b, acc[q][t], 0, 0, 0);
                }
            }
        }
    };

    // the output scale's inputs of (group, row) tid, loaded before anything
    // else and used only at publish: issued after the weight loads, their
    // first use would wait for all of those
    float g_mine = 0.0f, b_mine = beta;
    if (FQ == 0 && tid < 16 * G) {
        const int gi = tid >> 4, ri = tid & 15;
        if (ri < M) g_mine = gamma[(int64_t)gi * M + ri];
        if (beta_g) b_mine = beta_g[gi];
    }

    // 1. activation copies of the whole workgroup, queued ahead of any weight
    //    load (fused quantisation: the first chunks of the token's row)
    constexpr Src kQS = FQ == 2 ? Src::BF16 : Src::F32;
    const RowSrc qsrc{fr.x, nullptr};
    const bool quantiser = FQ != 0 && tid < kQuantThreads;
    const int qchunks = K / 16;
    // raw 16-byte vectors of the cached chunks (4 of fp32, 2 of bf16): the
    // widening to fp32 waits for the load, so it is left to the absmax pass,
    // after the weight loads have been issued
    constexpr int kRawVec = FQ == 2 ? 2 : 4;
    v4u qraw[FQ ? kQuantCache : 1][kRawVec];
    float gcache[FRMS ? kQuantCache : 1][16];
    auto raw_chunk = [&](int c, v4u (&r)[kRawVec]) {
        const v4u* p = reinterpret_cast<const v4u*>(static_cast<const char*>(fr.x) +
                                                    (int64_t)c * 16 * (FQ == 2 ? 2 : 4));
#pragma unroll
        for (int i = 0; i < kRawVec; ++i) r[i] = __builtin_nontemporal_load(p + i);
    };
    auto widen = [&](const v4u (&r)[kRawVec], float v[16]) {
#pragma unroll
        for (int i = 0; i < kRawVec; ++i) {
            const uint32_t d[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                if constexpr (FQ == 2) {
                    v[8 * i + 2 * jj] = __uint_as_float(d[jj] << 16);  // exact widening
                    v[8 * i + 2 * jj + 1] = __uint_as_float(d[jj] & 0xFFFF0000u);
                } else {
                    v[4 * i + jj] = __uint_as_float(d[jj]);
                }
            }
        }
    };
    auto load_gain = [&](int c, float g16[16]) {
        const float4* pg = reinterpret_cast<const float4*>(fr.gain + (int64_t)c * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 gv = pg[i];
            g16[4 * i] = gv.x; g16[4 * i + 1] = gv.y; g16[4 * i + 2] = gv.z; g16[4 * i + 3] = gv.w;
        }
    };
    // plain rows (no RMSNorm: the absmax is a max, exact in any order): all
    // threads take the row as 16-byte pieces dealt round-robin, so every wave
    // load reads 1 KB contiguous; the first kPlainVec pieces of a thread stay
    // in registers
    constexpr int kPlainVec = 4;
    constexpr int kEpv = FQ == 2 ? 8 : 4;  // entries per 16-byte piece
    const int npiece = K / kEpv;
    const v4u* xrow = reinterpret_cast<const v4u*>(fr.x);
    v4u praw[FQ != 0 && !FRMS ? kPlainVec : 1];
    if constexpr (FQ != 0 && !FRMS) {
#pragma unroll
        for (int i = 0; i < kPlainVec; ++i) {
            const int idx = min(tid + i * kDecWaves * kWave, npiece - 1);
            praw[i] = __builtin_nontemporal_load(xrow + idx);
        }
    } else if constexpr (FQ != 0) {
        if (quantiser) {
#pragma unroll
            for (int i = 0; i < kQuantCache; ++i) {
                const int c = tid + i * kQuantThreads;
                if (c < qchunks) {
                    raw_chunk(c, qraw[i]);
                    if constexpr (FRMS) load_gain(c, gcache[i]);
                }
            }
        }
    } else {
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
    __shared__ int s_qsum[kDecWaves];
    __shared__ float s_qmax[kDecWaves];
    // plain rows: absmax over the pieces, codes of each piece into the LDS
    // row (4 or 8 bytes at its entries' offset), their sum
    auto publish_plain = [&]() {
        float amax = 0.0f;
        auto pmax = [&](const v4u& t) {
            const uint32_t d[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                if constexpr (FQ == 2) {
                    amax = fmaxf(amax, fabsf(__uint_as_float(d[jj] << 16)));
                    amax = fmaxf(amax, fabsf(__uint_as_float(d[jj] & 0xFFFF0000u)));
                } else {
                    amax = fmaxf(amax, fabsf(__uint_as_float(d[jj])));
                }
            }
        };
        constexpr int T = kDecWaves * kWave;
#pragma unroll
        for (int i = 0; i < kPlainVec; ++i)
            if (tid + i * T < npiece) pmax(praw[i]);
        for (int idx = tid + kPlainVec * T; idx < npiece; idx += T) pmax(__builtin_nontemporal_load(xrow + idx));
        // wave maxima with DPP, then across the waves (a max: any order)
        amax = wave_max_dpp(amax);
        if (lane == 0) s_qmax[wv] = amax;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kDecWaves; ++i) amax = fmaxf(amax, s_qmax[i]);
        int csum = 0;
        auto put = [&](int idx, const v4u& t) {
            const uint32_t d[4] = {t.x, t.y, t.z, t.w};
            uint32_t c[2] = {0u, 0u};
            if (amax != 0.0f) {
                if constexpr (FQ == 2) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int q0 = quant_code(__uint_as_float(d[2 * h2] << 16), amax);
                        const int q1 = quant_code(__uint_as_float(d[2 * h2] & 0xFFFF0000u), amax);
                        const int q2 = quant_code(__uint_as_float(d[2 * h2 + 1] << 16), amax);
                        const int q3 = quant_code(__uint_as_float(d[2 * h2 + 1] & 0xFFFF0000u), amax);
                        csum += q0 + q1 + q2 + q3;
                        c[h2] = pack4(q0, q1, q2, q3);
                    }
                } else {
                    const int q0 = quant_code(__uint_as_float(d[0]), amax), q1 = quant_code(__uint_as_float(d[1]), amax);
                    const int q2 = quant_code(__uint_as_float(d[2]), amax), q3 = quant_code(__uint_as_float(d[3]), amax);
                    csum += q0 + q1 + q2 + q3;
                    c[0] = pack4(q0, q1, q2, q3);
                }
            }
            if constexpr (FQ == 2) {
                *reinterpret_cast<v2u*>(As + 8 * idx) = v2u{c[0], c[1]};
                if (blockIdx.x == 0) *reinterpret_cast<v2u*>(fr.q_out + 8 * (int64_t)idx) = v2u{c[0], c[1]};
            } else {
                *reinterpret_cast<uint32_t*>(As + 4 * idx) = c[0];
                if (blockIdx.x == 0) *reinterpret_cast<uint32_t*>(fr.q_out + 4 * (int64_t)idx) = c[0];
            }
        };
#pragma unroll
        for (int i = 0; i < kPlainVec; ++i)
            if (tid + i * T < npiece) put(tid + i * T, praw[i]);
        for (int idx = tid + kPlainVec * T; idx < npiece; idx += T) put(idx, __builtin_nontemporal_load(xrow + idx));
        csum = wave_sum_dpp(csum);
        if (lane == 0) s_qsum[wv] = csum;
        if (blockIdx.x == 0 && tid == 0) fr.gamma_out[0] = amax;
        __syncthreads();  // the codes and the partial sums are visible
        if (tid < 16) {
            int S = 0;
#pragma unroll
            for (int i = 0; i < kDecWaves; ++i) S += s_qsum[i];
            Ssum[tid] = tid == 0 ? S : 0;
            Ssc[tid] = tid == 0 ? out_scale(beta, amax) : 0.0f;
        }
    };
    // fused quantisation: absmax (and the float64 sum of squares) over the
    // row as the quantiser takes it, codes into the LDS row (slot = piece:
    // row 0 is not swizzled), their sum, and the output scale
    auto publish_fused = [&]() {
        float amax = 0.0f;
        double ss = 0.0;
        auto process = [&](float v[16], const float g16[16]) {
            if constexpr (FRMS) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float xv = v[e];
                    ss += (double)xv * (double)xv;
                    v[e] = g16[e] * xv;
                }
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
        };
        float qcache[kQuantCache][16];
        if (quantiser) {
#pragma unroll
            for (int i = 0; i < kQuantCache; ++i) {
                const int c = tid + i * kQuantThreads;
                if (c < qchunks) {
                    widen(qraw[i], qcache[i]);
                    process(qcache[i], gcache[FRMS ? i : 0]);
                }
            }
            for (int c = tid + kQuantCache * kQuantThreads; c < qchunks; c += kQuantThreads) {
                float v[16], g16[16];
                load_chunk<kQS>(qsrc, 0, K, c, v);
                if constexpr (FRMS) load_gain(c, g16);
                process(v, g16);
            }
        }
        block_reduce<kQuantThreads / kWave>(amax, ss, FRMS);
        float gq = amax;
        if constexpr (FRMS) gq = (float)((1.0 / sqrt(ss / (double)K + (double)fr.eps)) * (double)amax);
        int csum = 0;
        auto put_codes = [&](int c, const float v[16]) {
            uint32_t d[4] = {0u, 0u, 0u, 0u};
            if (amax != 0.0f) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int q0 = quant_code(v[4 * jj], amax), q1 = quant_code(v[4 * jj + 1], amax);
                    const int q2 = quant_code(v[4 * jj + 2], amax), q3 = quant_code(v[4 * jj + 3], amax);
                    csum += q0 + q1 + q2 + q3;
                    d[jj] = pack4(q0, q1, q2, q3);
                }
            }
            const v4u dv = v4u{d[0], d[1], d[2], d[3]};
            *reinterpret_cast<v4u*>(As + 16 * c) = dv;
            if (blockIdx.x == 0) *reinterpret_cast<v4u*>(fr.q_out + 16 * (int64_t)c) = dv;
        };
        if (quantiser) {
#pragma unroll
            for (int i = 0; i < kQuantCache; ++i) {
                const int c = tid + i * kQuantThreads;
                if (c < qchunks) put_codes(c, qcache[i]);
            }
            for (int c = tid + kQuantCache * kQuantThreads; c < qchunks; c += kQuantThreads) {
                float v[16];
                load_chunk<kQS>(qsrc, 0, K, c, v);
                if constexpr (FRMS) {
                    float g16[16];
                    load_gain(c, g16);
#pragma unroll
                    for (int e = 0; e < 16; ++e) v[e] *= g16[e];
                }
                put_codes(c, v);
            }
            csum = wave_sum_i(csum);
            if (lane == 0) s_qsum[wv] = csum;
        }
        if (blockIdx.x == 0 && tid == 0) fr.gamma_out[0] = gq;
        __syncthreads();  // the codes and the partial sums are visible
        if (tid < 16) {
            int S = 0;
#pragma unroll
            for (int i = 0; i < kQuantThreads / kWave; ++i) S += s_qsum[i];
            Ssum[tid] = tid == 0 ? S : 0;
            Ssc[tid] = tid == 0 ? out_scale(beta, gq) : 0.0f;
        }
    };
    auto publish = [&]() {
        if constexpr (FQ != 0 && !FRMS) {
            publish_plain();
            return;
        } else if constexpr (FQ != 0) {
            publish_fused();
            return;
        }
        fence_code();
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(B * NTW));  // own copies (older) have landed
        __builtin_amdgcn_s_barrier();
        fence_code();
        // row r = tid / 32, 32 threads per row, per group (the slot order
        // inside a row does not change a sum; group gg holds slots
        // gg*KG/16 .. (gg+1)*KG/16 since KG is a multiple of 256)
        // output scales fl32(beta_g * gamma[g][m]) / 128 of every (group, row)
        if (tid < 16 * G) Ssc[tid] = (tid & 15) < M ? out_scale(b_mine, g_mine) : 0.0f;
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
    // a stream of batches, the next one's loads issued before the current one
    // is multiplied (a wave keeps at most 2 B NTW loads in flight, so load
    // issue does not stall on the compute unit's outstanding-request limit);
    // loads past the range re-read the last chunk.  Two batches a trip with
    // no exit in between, and a scheduling barrier after every step:
    // otherwise the compiler sinks a batch's loads below the multiplies and
    // rotates the loop so that it waits for all loads (vmcnt(0)) at its head,
    // and no load is in flight while a batch is multiplied.  One batch is the
    // same code with no trip: a separate branch for it got a vmcnt(0) before
    // its weight loads, which then waited for the activation copies.
    wvec b0[B][NTW], b1[B][NTW];
    const int nb = max((c_end - c_begin + B - 1) / B, 0);  // batches of this wave
    load_batch(c_begin, b0);
    publish();
    int cb = c_begin;
    for (int i = 0; i + 2 <= nb; i += 2, cb += 2 * B) {
        load_batch(cb + B, b1);
        __builtin_amdgcn_sched_barrier(0);
        mul_batch(cb, b0);
        __builtin_amdgcn_sched_barrier(0);
        load_batch(cb + 2 * B, b0);
        __builtin_amdgcn_sched_barrier(0);
        mul_batch(cb + B, b1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (nb & 1) mul_batch(cb, b0);  // its loads were issued by the last trip (or before the loop)

    if constexpr (kRegEpi) {
        // lane l holds D[4 (l / 16) + v][l % 16]: the block entries of token
        // m = 2 g' + b of group q and tile row r sit at register 2b of lane
        // 2r + 16 g' (part 0) and register 2b + 1 of the next lane (part 1)
        __syncthreads();  // Ssum and Ssc are written (every wave passed publish)
        const int r = jr;  // = (lane & 15) >> 1
#pragma unroll
        for (int q = 0; q < TG; ++q)
#pragma unroll
            for (int t = 0; t < NTW; ++t) {
                const int o1 = __shfl_xor(acc[q][t][1], 1, kWave);
                const int o3 = __shfl_xor(acc[q][t][3], 1, kWave);
                const int col = n_base + RT * t + r;
                if (h != 0 || col >= N) continue;
#pragma unroll
                for (int b2 = 0; b2 < 2; ++b2) {
                    const int m = RT * q + 2 * g + b2;
                    if (m >= M) continue;
                    const int d = acc[q][t][2 * b2] + (b2 ? o3 : o1);
                    const int a = (ONEBIT ? 2 * d : d) - Ssum[m];
                    if (acc_out) acc_out[(int64_t)m * N + col] = a;
                    if (y) y[(int64_t)m * N + col] = (float)a * Ssc[m];
                }
            }
        return;
    }
    // lane (j, g) holds rows 4g + v of column j
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((wv * kRedNtw + t) * 4 + v) * kWave + lane] = acc[0][t][v];
    __syncthreads();
    if constexpr (H > 1) {
        // output (token m, tile row r) of tile t: the diagonal blocks
        // D[h + H m][h + H r], h < H, held by lane (h + H r) + 16 ((h + H m) / 4)
        // at register (h + H m) % 4 of every K range's partial
        if (kp == 0 && lane < RT * RT) {
            const int m = lane / RT, r = lane % RT;
#pragma unroll
            for (int t = 0; t < NTW; ++t) {
                const int col = n_base + RT * t + r;
                if (m >= M || col >= N) continue;
                int d = 0;
#pragma unroll
                for (int hh = 0; hh < H; ++hh) {
                    const int i = hh + H * m, src = hh + H * r + 16 * (i >> 2), v = i & 3;
#pragma unroll
                    for (int k2 = 0; k2 < KS; ++k2) d += red[(((k2 * CG + cg) * kRedNtw + t) * 4 + v) * kWave + src];
                }
                const int a = (ONEBIT ? 2 * d : d) - Ssum[m];
                if (acc_out) acc_out[(int64_t)m * N + col] = a;
                if (y) y[(int64_t)m * N + col] = (float)a * Ssc[m];
            }
        }
    } else if (kp == 0) {
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
                        d += red[(((k2 * CG + cg) * kRedNtw + t) * 4 + v) * kWave + lane];
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


template <int CT, int NTW, int B, bool ONEBIT, int G, int H = 1, int TG = 1, int FQ = 0, bool FRMS = false>
hipError_t launch_ctb(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp, int N,
                      float beta, float* y, int32_t* acc, hipStream_t s, const float* beta_g,
                      FusedRow fr = {}) {
    static DynLdsOptIn opt_in;
    const hipError_t e = opt_in.ensure(
        reinterpret_cast<const void*>(&decode_lds_kernel<CT, NTW, B, ONEBIT, G, H, TG, FQ, FRMS>),
        kDecLdsMax);
    if (e != hipSuccess) return e;
    constexpr int rows = 16 / H * CT;  // weight rows of a workgroup
    constexpr int red_ntw = (H == 2 && kDecWaves * NTW / CT == 1) ? 0 : NTW;  // no LDS reduction
    const size_t lds = decode_lds_bytes(M, K, red_ntw, G);
    if (M > 16 / H * TG || lds > (size_t)kDecLdsMax) return hipErrorInvalidValue;
    const int blocks = (N + rows - 1) / rows;
    decode_lds_kernel<CT, NTW, B, ONEBIT, G, H, TG, FQ, FRMS>
        <<<dim3(blocks), dim3(kDecWaves * kWave), lds, s>>>(xq, gamma, M, K, wp, N, beta, y, acc,
                                                            decode_a_bytes(M, K), beta_g, fr);
    return hipGetLastError();
}

// Batch: a wave's whole K range in one batch when it has at most 4 load units,
// else a stream of 2-unit batches (measured at K = 2560 .. 8192: larger
// batches stall load issue, a 2-chunk stream is 15 % faster at K = 8192).
template <int CT, int NTW, bool ONEBIT, int G = 1, int H = 1, int TG = 1, int FQ = 0, bool FRMS = false>
hipError_t launch_ct(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp, int N,
                     float beta, float* y, int32_t* acc, hipStream_t s,
                     const float* beta_g = nullptr, FusedRow fr = {}) {
    constexpr int KS = kDecWaves * NTW / CT;
    constexpr int unit_log = (ONEBIT ? 9 : 8) + (H == 16 ? 4 : H == 8 ? 3 : H == 4 ? 2 : H == 2 ? 1 : 0);
    const int cpw = ((K >> unit_log) + KS - 1) / KS;  // load units a wave
    // one batch no larger than the wave's units (a larger one re-reads the
    // last unit and multiplies zero codes for the rest)
    if (cpw <= 1) return launch_ctb<CT, NTW, 1, ONEBIT, G, H, TG, FQ, FRMS>(xq, gamma, M, K, wp, N, beta, y, acc, s, beta_g, fr);
    if (cpw <= 2) return launch_ctb<CT, NTW, 2, ONEBIT, G, H, TG, FQ, FRMS>(xq, gamma, M, K, wp, N, beta, y, acc, s, beta_g, fr);
    if (cpw <= 4) return launch_ctb<CT, NTW, 4, ONEBIT, G, H, TG, FQ, FRMS>(xq, gamma, M, K, wp, N, beta, y, acc, s, beta_g, fr);
    return launch_ctb<CT, NTW, 2, ONEBIT, G, H, TG, FQ, FRMS>(xq, gamma, M, K, wp, N, beta, y, acc, s, beta_g, fr);
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

// Shape routing of the ungrouped decode product (2-bit or 1-bit weights).
template <bool ONEBIT>
hipError_t launch_route(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp, int N,
                        float beta, float* y, int32_t* acc, hipStream_t s) {
    // up to 8 tokens (K a multiple of the two-part unit: 512 inputs, 1024 for
    // 1-bit weights): two K parts per tile, 8 rows x 128 B a load, one tile a
    // wave over the whole K.  Widest workgroup that leaves >= 200 workgroups
    // of 128 rows or >= 150 of 64 rows, else 32 rows (measured, bit-identical
    // to one part: 8 tokens at K = 8192, N = 28672 15.9 -> 12.0-12.5 us, 1-bit
    // 10.8 -> 9.9 us; 2..8 tokens at K = 4096, N = 11008 5.7-6.3 -> 4.8-5.1 us,
    // 1-bit 5.0-5.2 -> 4.7-4.8 us; 5 tokens at K = 2560, N = 6912 5.6 -> 4.1 us)
    constexpr int kPart = ONEBIT ? 1024 : 512;
    if (M <= 8 && K % kPart == 0) {
        if (N / 128 >= 200) return launch_ct<16, 2, ONEBIT, 1, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
        if (N / 64 >= 150) return launch_ct<8, 1, ONEBIT, 1, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
        return launch_ct<4, 1, ONEBIT, 1, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    }
    // 9..16 tokens on 2-bit weights (K % 512 == 0, many row tiles): two K
    // parts and two token groups sharing every weight fragment, one K range
    // per tile (a workgroup holds up to 128 KB of activations, so one per
    // compute unit: 128-row workgroups once there are >= 200 of them, which
    // then fill the chip in one round; else 64 rows).  Bit-identical, 16
    // tokens at K = 8192, N = 28672 15.7 -> 14.4 us; at K = 4096, N = 11008
    // 6.9 -> 6.0 us; 9..12 tokens there 6.3-6.4 -> 5.6-5.8 us; K = 5120,
    // N = 13824 7.8 -> 6.9 us (with fewer row tiles, e.g. N = 4000 or 6912, it
    // is no faster; on 1-bit weights it is slower: 16 tokens at K = 8192,
    // N = 28672 13.0 against 11.2 us)
    if (!ONEBIT && K % kPart == 0 && N / 64 >= 150) {
        if (N / 128 >= 200) return launch_ct<16, 2, false, 1, 2, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
        return launch_ct<8, 1, false, 1, 2, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    }
    // else one 16-row tile a wave, the widest workgroup that still leaves
    // >= 200 workgroups (fewer, wider groups copy the activation block fewer
    // times, too few leave CUs idle).  Against two tiles a wave: 16 tokens at
    // K = 8192, N = 28672 16.6 -> 15.8 us, at K = 4096, N = 11008 6.9 -> 6.7 us;
    // 1-bit 11.4 -> 11.2 us and 6.0 -> 5.3 us
    const int tiles = (N + 15) / 16;
    if (tiles >= 8 * 200) return launch_ct<8, 1, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    if (tiles >= 4 * 200) return launch_ct<4, 1, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    if (tiles >= 2 * 200) return launch_ct<2, 1, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    return launch_ct<1, 1, ONEBIT>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

}  // namespace

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
    return launch_route<false>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

namespace {
template <int FQ, bool FRMS>
hipError_t launch_quant_decode_t(int K, const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                                 hipStream_t s, FusedRow fr) {
    // the two-part one-token routes of launch_route (x_q and gamma come from
    // the kernel itself: their pointers are the outputs)
    if (N / 128 >= 200)
        return launch_ct<16, 2, false, 1, 2, 1, FQ, FRMS>(fr.q_out, fr.gamma_out, 1, K, wp, N, beta, y, acc, s,
                                                          nullptr, fr);
    return launch_ct<8, 1, false, 1, 2, 1, FQ, FRMS>(fr.q_out, fr.gamma_out, 1, K, wp, N, beta, y, acc, s,
                                                     nullptr, fr);
}
}  // namespace

hipError_t launch_quant_decode1(const void* x, bool bf16, int K, const float* gain, float eps,
                                const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                                int8_t* x_q, float* gamma, hipStream_t s) {
    const FusedRow fr{x, gain, eps, x_q, gamma};
    if (bf16)
        return gain ? launch_quant_decode_t<2, true>(K, wp, N, beta, y, acc, s, fr)
                    : launch_quant_decode_t<2, false>(K, wp, N, beta, y, acc, s, fr);
    return gain ? launch_quant_decode_t<1, true>(K, wp, N, beta, y, acc, s, fr)
                : launch_quant_decode_t<1, false>(K, wp, N, beta, y, acc, s, fr);
}

hipError_t launch_decode_lds1(const int8_t* xq, const float* gamma, int M, int K,
                              const uint32_t* wp1, int N, float beta, float* y, int32_t* acc,
                              hipStream_t s) {
    return launch_route<true>(xq, gamma, M, K, wp1, N, beta, y, acc, s);
}

}  // namespace bl

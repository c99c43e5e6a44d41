// Prefill GEMM on int8 MFMA with an LDS ring fed by direct global->LDS loads
// (K a multiple of 128).
//
// Arithmetic (unite.ai BitNet.cpp article, 3. BitLinear-Betrieb):
// v_mfma_i32_32x32x32_i8; the ring kernel multiplies the signed weights
// w = c - 1 (unpack_signed), so acc = D directly, while the pipelined kernel
// multiplies the 2-bit codes c = w + 1 and removes acc = D - S_m with S_m the
// sum of the token's int8 activations.  Both are exact integer sums.
//
// Pipeline: the activation tile (BM rows x 128 bytes) and packed weight tile
// (BN columns x 8 words) of each K step are copied straight from global
// memory into one of STAGES LDS buffers with global_load_lds_dwordx4, so the
// copies occupy no registers and
// STAGES-1 steps are in flight while one is multiplied.  Every wave issues the
// same number of copies each step and waits for its own copies with an
// explicit vmcnt; the barrier that follows makes the whole step visible and
// also tells every wave that the buffer about to be refilled has been read.
// Past the last step the copies re-read the last step into the free buffer,
// so the counts stay uniform.  Each lane's 16-byte copy lands at
// M0 + 16 * lane, so the global address of a lane is chosen to put the right
// chunk at its swizzled LDS position.
//
// Layout and operand mapping follow gemm_mfma.hip: activation rows of 128
// bytes with chunk c stored at c ^ ((row & 7) ^ ((row >> 3) & 1)); weight
// columns of 32 bytes with halves swapped when bit 3 of the column is set;
// MFMA kk (0..3) of lane half h covers packed word 4h + kk.  In the pipelined
// kernel S_m is summed from the activation fragments the waves already hold,
// the K range split between the WN waves that share a row.
#include "device_common.h"
#include "internal.h"
#include "mfma_epilogue.h"

namespace bl {
namespace {

constexpr int BK = 128;

constexpr int kXcds = 8;

// Block -> output tile.  The hardware deals consecutive workgroups to the eight
// XCDs in turn; renumbering puts each XCD's workgroups on consecutive tiles,
// and the tiles run row tiles fastest, so the row tiles of one column range --
// all the workgroups that read those packed weight columns -- share one XCD's
// L2.  Measured against columns fastest (the tiles of one row range per XCD,
// each weight column then fetched by several XCDs), bit-identical output:
// M = 512, K = 8192, N = 28672 142.8 -> 140.1 us; M = 2048, K = 4096,
// N = 11008 125.6 -> 123.1 us; M = 64 31.6 -> 31.4 us.  Returns m0, sets n0.
__device__ __forceinline__ int tile_origin(int blk, int tiles_n, int tiles_total, int BM, int BN,
                                           int& n0) {
    int b = blk;
    const int full = (tiles_total / kXcds) * kXcds;
    if (b < full) b = (b % kXcds) * (full / kXcds) + b / kXcds;
    const int tiles_m = tiles_total / tiles_n;
    n0 = (b / tiles_m) * BN;
    return (b % tiles_m) * BM;
}

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int bswz(int col, int h) { return h ^ ((col >> 3) & 1); }


// s_waitcnt immediate (gfx9 encoding): vmcnt <= vm, lgkmcnt <= lgkm, expcnt any
constexpr int waitcnt_imm(int vm, int lgkm) {
    return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 0xF) << 8);
}

template <int WM, int WN, int TM, int TN, int STAGES>
struct DCfg {
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = kWaves * kWave;
    static constexpr int BM = WM * TM * 32;
    static constexpr int BN = WN * TN * 32;
    static constexpr int kABytes = BM * BK;        // activation bytes per stage
    static constexpr int kBBytes = BN * 32;        // packed weight bytes per stage
    static constexpr int kStageBytes = kABytes + kBBytes;
    static constexpr int kAInstr = kABytes / 1024 / kWaves;  // 16-byte copies per wave per step
    static constexpr int kBInstr = kBBytes / 1024 / kWaves;  // 16-byte copies per wave per step
    static constexpr int kPerStep = kAInstr + kBInstr;
    static_assert(kABytes % (1024 * kWaves) == 0, "activation copies divide the waves");
    static_assert(kBBytes % (1024 * kWaves) == 0, "weight copies divide the waves");
};

// KSP > 1 splits K inside the workgroup: KSP groups of WM x WN waves, each
// with its own LDS ring, run the same loop (so every wave meets the same
// barriers) over their own K / KSP inputs; the groups' accumulators are added
// through LDS before the epilogue.  For few tiles on a long K: the sequential
// K steps of a tile drop by KSP and the compute unit holds KSP times the waves.
template <int WM, int WN, int TM, int TN, int STAGES, int KSP>
__global__ __launch_bounds__(KSP * WM * WN * 64)
__attribute__((amdgpu_waves_per_eu(KSP * WM * WN > 8 ? 3 : 2, KSP * WM * WN > 8 ? 3 : 2)))
void gemm_dma_kernel(const int8_t* __restrict__ xq, const float* __restrict__ gamma, int M,
                     int K, const uint32_t* __restrict__ wp, int N, float beta,
                     float* __restrict__ y, int32_t* __restrict__ acc_out, int tiles_n,
                     int tiles_total) {
    using C = DCfg<WM, WN, TM, TN, STAGES>;
    __shared__ __attribute__((aligned(16))) char lds[KSP * STAGES * C::kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv_all = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int kgrp = wv_all / C::kWaves;   // K group
    const int wv = wv_all % C::kWaves;     // wave within its group
    const int wm = wv / WN, wn = wv % WN;
    char* ring = lds + kgrp * STAGES * C::kStageBytes;
    const int l32 = lane & 31, h = lane >> 5;

    int n0;
    const int m0 = tile_origin(blockIdx.x, tiles_n, tiles_total, C::BM, C::BN, n0);
    const int WR = K >> 4;
    const int KT = K / BK / KSP;  // K steps of each group (K % (BK * KSP) == 0)

    // per-lane source offsets of this wave's copies at step 0 (32-bit, from
    // the block's first row / column); rows and columns past the matrix are
    // clamped onto its last row / column (their products are never stored)
    const int8_t* abase = xq + (int64_t)m0 * K + (int64_t)kgrp * KT * BK;
    const uint32_t* bbase = wp + (int64_t)n0 * WR + (int64_t)kgrp * KT * (BK / 16);
    uint32_t aoff[C::kAInstr];
#pragma unroll
    for (int i = 0; i < C::kAInstr; ++i) {
        const int q = wv * C::kAInstr + i;
        const int row = 8 * q + lane / 8;
        const int lchunk = (lane % 8) ^ swz(row);
        aoff[i] = (uint32_t)(min(m0 + row, M - 1) - m0) * (uint32_t)K + 16u * lchunk;
    }
    uint32_t boff[C::kBInstr];
#pragma unroll
    for (int i = 0; i < C::kBInstr; ++i) {
        const int q = wv * C::kBInstr + i;
        const int col = 32 * q + lane / 2;
        const int lhalf = (lane % 2) ^ ((col >> 3) & 1);
        boff[i] = (uint32_t)(min(n0 + col, N - 1) - n0) * (uint32_t)WR + 4u * lhalf;
    }

    auto issue = [&](int kt, int buf) {
        char* stage = ring + buf * C::kStageBytes;
        const int8_t* a_step = abase + (int64_t)kt * BK;
        const uint32_t* b_step = bbase + (int64_t)kt * (BK / 16);
#pragma unroll
        for (int i = 0; i < C::kAInstr; ++i)
            copy16_to_lds(a_step + aoff[i], stage + 1024 * (wv * C::kAInstr + i));
#pragma unroll
        for (int i = 0; i < C::kBInstr; ++i)
            copy16_to_lds(b_step + boff[i], stage + C::kABytes + 1024 * (wv * C::kBInstr + i));
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[i][t] = v16i{};

#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p) issue(min(p, KT - 1), p);

    for (int kt = 0; kt < KT; ++kt) {
        // this wave's copies of step kt are done (later steps may be in flight)
        __builtin_amdgcn_s_waitcnt(waitcnt_imm((STAGES - 2) * C::kPerStep, 0));
        __builtin_amdgcn_s_barrier();
        issue(min(kt + STAGES - 1, KT - 1), (kt + STAGES - 1) % STAGES);

        const char* stage = ring + (kt % STAGES) * C::kStageBytes;
        const v4i* As = reinterpret_cast<const v4i*>(stage);
        const v4u* Bs = reinterpret_cast<const v4u*>(stage + C::kABytes);
        // all LDS operand reads of the step first, so their latency overlaps
        // the unpacking and the first MFMAs
        v4u wq[TN];
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            const int col = wn * TN * 32 + 32 * t + l32;
            wq[t] = Bs[col * 2 + bswz(col, h)];
        }
        v4i af[4][TM];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * TM * 32 + 32 * i + l32;
                af[kk][i] = As[r * 8 + ((4 * h + kk) ^ swz(r))];
            }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            // signed weights: measured against the codes with in-loop row sums,
            // bit-identical, M = 64, K = 8192, N = 28672 32.0 -> 30.2 us; M = 96,
            // K = 4096, N = 11008 17.3 -> 16.3 us; M = 512, K = 6912, N = 2560
            // 24.5 -> 23.7 us (the pipelined kernel below loses 2-5 % with them)
            v4i bf[TN];
#pragma unroll
            for (int t = 0; t < TN; ++t) bf[t] = unpack_signed(wq[t][kk]);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int t = 0; t < TN; ++t)
                    acc[i][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[kk][i], bf[t], acc[i][t], 0, 0, 0);
            }
        }
    }
    // every copy (including the re-reads past the end) has landed before the
    // LDS is reused below or released
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __syncthreads();

    // KSP > 1: the accumulators of groups 1.. go through LDS (lane-major, one
    // int per lane and register) to group 0, whose waves own the epilogue
    constexpr int kAccInts = C::kWaves * TM * TN * 16 * kWave;  // one group's accumulators
    int* red = reinterpret_cast<int*>(lds);
    int* S = reinterpret_cast<int*>(lds) + (KSP > 1 ? kAccInts : 0);  // [BM], all 0 (no offset)
    float* Ssc = reinterpret_cast<float*>(S + C::BM);
    static_assert((int64_t)((KSP > 1 ? kAccInts : 0) + 2 * C::BM) * 4 <=
                      (int64_t)KSP * STAGES * C::kStageBytes,
                  "the accumulator exchange and the row tables fit the rings");
    if constexpr (KSP > 1) {
        for (int g = 1; g < KSP; ++g) {
            if (kgrp == g) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int t = 0; t < TN; ++t)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            red[((wv * TM * TN + i * TN + t) * 16 + v) * kWave + lane] = acc[i][t][v];
            }
            __syncthreads();
            if (kgrp == 0) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int t = 0; t < TN; ++t)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            acc[i][t][v] += red[((wv * TM * TN + i * TN + t) * 16 + v) * kWave + lane];
            }
            __syncthreads();
        }
    }
    epilogue_tables(nullptr, 0, C::BM, m0, M, gamma, beta, S, Ssc, tid, KSP * C::kThreads);
    __syncthreads();
    if (kgrp == 0)
        store_tiles<TM, TN>(acc, S, Ssc, wm * TM * 32, wn * TN * 32, m0, n0, M, N, y, acc_out, lane);
}


// Biased byte sum of 16 int8 values: sum (q + 128) + acc.  v_sad_u8 against 0
// adds the four unsigned bytes; flipping the sign bit first maps q to q + 128.
// It runs on the vector ALU (v_dot4 would share the matrix pipe with the MFMAs).
__device__ __forceinline__ unsigned biased_sum16(v4i a, unsigned acc) {
    acc = __builtin_amdgcn_sad_u8((unsigned)a.x ^ 0x80808080u, 0u, acc);
    acc = __builtin_amdgcn_sad_u8((unsigned)a.y ^ 0x80808080u, 0u, acc);
    acc = __builtin_amdgcn_sad_u8((unsigned)a.z ^ 0x80808080u, 0u, acc);
    acc = __builtin_amdgcn_sad_u8((unsigned)a.w ^ 0x80808080u, 0u, acc);
    return acc;
}

// Software-pipelined variant of the ring loop above (same LDS layout, copies
// and three-stage ring):
//   - the A fragments of the next 32-wide K slice are read while the MFMAs of
//     the current one run, and the packed weight words of the next K step are
//     read right after the step's barrier, which sits between the two halves of
//     the last slice's MFMAs, so the barrier and the first reads of a step
//     overlap MFMA work;
//   - wave wn takes the four K slices of a step in the order wn, wn + 1, ...
//     (mod 4), so its share of the row sums (the slices kk with kk % WN == wn)
//     falls on fixed unrolled positions and the loop has no branch on it; the
//     weight words are then read one 32-bit word per slice;
//   - the row sums use biased_sum16, the bias is removed once at the end.
// Measured with a 1 x 4 wave layout (each wave 128 rows x 64 columns, so each
// packed word is unpacked once per workgroup), A/B in one session:
// M = 512, K = 8192, N = 28672 125 -> 116 us; M = 2048, K = 4096, N = 11008
// 101 -> 96 us.
template <int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_pipe_kernel(const int8_t* __restrict__ xq, const float* __restrict__ gamma, int M,
                      int K, const uint32_t* __restrict__ wp, int N, float beta,
                      float* __restrict__ y, int32_t* __restrict__ acc_out, int tiles_n,
                      int tiles_total) {
    constexpr int STAGES = 3;
    using C = DCfg<WM, WN, TM, TN, STAGES>;
    static_assert(4 % WN == 0, "the K slices of a step divide between the waves of a row");
    __shared__ __attribute__((aligned(16))) char lds[STAGES * C::kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wv / WN, wn = wv % WN;
    const int l32 = lane & 31, h = lane >> 5;

    int n0;
    const int m0 = tile_origin(blockIdx.x, tiles_n, tiles_total, C::BM, C::BN, n0);
    const int WR = K >> 4;
    const int KT = K / BK;

    // per-lane source offsets as in gemm_dma_kernel (rows / columns past the
    // matrix clamped onto its last row / column)
    const int8_t* abase = xq + (int64_t)m0 * K;
    const uint32_t* bbase = wp + (int64_t)n0 * WR;
    uint32_t aoff[C::kAInstr];
#pragma unroll
    for (int i = 0; i < C::kAInstr; ++i) {
        const int q = wv * C::kAInstr + i;
        const int row = 8 * q + lane / 8;
        const int lchunk = (lane % 8) ^ swz(row);
        aoff[i] = (uint32_t)(min(m0 + row, M - 1) - m0) * (uint32_t)K + 16u * lchunk;
    }
    uint32_t boff[C::kBInstr];
#pragma unroll
    for (int i = 0; i < C::kBInstr; ++i) {
        const int q = wv * C::kBInstr + i;
        const int col = 32 * q + lane / 2;
        const int lhalf = (lane % 2) ^ ((col >> 3) & 1);
        boff[i] = (uint32_t)(min(n0 + col, N - 1) - n0) * (uint32_t)WR + 4u * lhalf;
    }
    auto issue = [&](int kt, int buf) {
        char* stage = lds + buf * C::kStageBytes;
        const int8_t* a_step = abase + (int64_t)kt * BK;
        const uint32_t* b_step = bbase + (int64_t)kt * (BK / 16);
#pragma unroll
        for (int i = 0; i < C::kAInstr; ++i)
            copy16_to_lds(a_step + aoff[i], stage + 1024 * (wv * C::kAInstr + i));
#pragma unroll
        for (int i = 0; i < C::kBInstr; ++i)
            copy16_to_lds(b_step + boff[i], stage + C::kABytes + 1024 * (wv * C::kBInstr + i));
    };
    // packed words of K slice (kk + wn) % 4 for this lane's columns
    auto read_words = [&](int buf, uint32_t (&wq)[TN][4]) {
        const uint32_t* Bs = reinterpret_cast<const uint32_t*>(lds + buf * C::kStageBytes + C::kABytes);
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            const int col = wn * TN * 32 + 32 * t + l32;
            const uint32_t* p = Bs + (col * 2 + bswz(col, h)) * 4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) wq[t][kk] = p[(kk + wn) & 3];
        }
    };
    auto read_frags = [&](int buf, int kk, v4i (&af)[TM]) {
        const v4i* As = reinterpret_cast<const v4i*>(lds + buf * C::kStageBytes);
        const int ke = (kk + wn) & 3;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm * TM * 32 + 32 * i + l32;
            af[i] = As[r * 8 + ((4 * h + ke) ^ swz(r))];
        }
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[i][t] = v16i{};
    unsigned s_biased[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) s_biased[i] = 0u;

    // steps 0 and 1 in flight; step 0 landed everywhere; step 2 queued
    issue(0, 0);
    issue(min(1, KT - 1), 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(C::kPerStep, 0));
    __builtin_amdgcn_s_barrier();
    issue(min(2, KT - 1), 2);
    uint32_t wq[TN][4], wqn[TN][4];
    v4i a[2][TM];
    read_words(0, wq);
    read_frags(0, 0, a[0]);

    int buf = 0;
    for (int kt = 0; kt < KT; ++kt) {
        const bool more = kt + 1 < KT;  // uniform
        const int nbuf = buf == STAGES - 1 ? 0 : buf + 1;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (kk < 3) read_frags(buf, kk + 1, a[(kk + 1) & 1]);
            v4i bf[TN];
#pragma unroll
            for (int t = 0; t < TN; ++t) bf[t] = unpack_codes(wq[t][kk]);
            if (kk % WN == 0) {
#pragma unroll
                for (int i = 0; i < TM; ++i) s_biased[i] = biased_sum16(a[kk & 1][i], s_biased[i]);
            }
            if (kk < 3) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int t = 0; t < TN; ++t)
                        acc[i][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[kk & 1][i], bf[t], acc[i][t], 0, 0, 0);
            } else {
#pragma unroll
                for (int i = 0; i < TM / 2; ++i)
#pragma unroll
                    for (int t = 0; t < TN; ++t)
                        acc[i][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[1][i], bf[t], acc[i][t], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (more) {
                    // this wave's copies of step kt+1 have landed and its reads
                    // of this buffer are done; after the barrier every wave's
                    // are, so step kt+1 can be read and this buffer refilled
                    // (with step kt+3, or the last step again past the end)
                    __builtin_amdgcn_s_waitcnt(waitcnt_imm(C::kPerStep, 0));
                    __builtin_amdgcn_s_barrier();
                    issue(min(kt + 3, KT - 1), buf);
                    read_words(nbuf, wqn);
                    read_frags(nbuf, 0, a[0]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = TM / 2; i < TM; ++i)
#pragma unroll
                    for (int t = 0; t < TN; ++t)
                        acc[i][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[1][i], bf[t], acc[i][t], 0, 0, 0);
            }
        }
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) wq[t][kk] = wqn[t][kk];
        buf = nbuf;
    }
    // every copy (including the re-reads past the end) has landed before the
    // LDS is reused below or released
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __syncthreads();

    int* Sp = reinterpret_cast<int*>(lds);  // [WN][BM] partial row sums
    int* S = Sp + WN * C::BM;               // [BM]
    float* Ssc = reinterpret_cast<float*>(S + C::BM);
    // each lane summed 16 bytes for 4 / WN slices of each of the KT steps
    const unsigned bias = 2048u * (unsigned)KT * (unsigned)(4 / WN);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int sp = (int)(s_biased[i] - bias);
        const int sv = sp + __shfl_xor(sp, 32, kWave);
        if (h == 0) Sp[wn * C::BM + wm * TM * 32 + 32 * i + l32] = sv;
    }
    __syncthreads();
    epilogue_tables(Sp, WN, C::BM, m0, M, gamma, beta, S, Ssc, tid, C::kThreads);
    __syncthreads();
    store_tiles<TM, TN>(acc, S, Ssc, wm * TM * 32, wn * TN * 32, m0, n0, M, N, y, acc_out, lane);
}

template <int WM, int WN, int TM, int TN, int STAGES, int KSP = 1>
hipError_t launch_dcfg(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                       int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    using C = DCfg<WM, WN, TM, TN, STAGES>;
    if (K % (BK * KSP) != 0) return hipErrorInvalidValue;
    const int tm = (M + C::BM - 1) / C::BM;
    const int tn = (N + C::BN - 1) / C::BN;
    const int64_t total = (int64_t)tm * tn;
    if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
    gemm_dma_kernel<WM, WN, TM, TN, STAGES, KSP>
        <<<dim3((unsigned)total), dim3(KSP * C::kThreads), 0, s>>>(xq, gamma, M, K, wp, N, beta, y,
                                                                   acc, tn, (int)total);
    return hipGetLastError();
}


template <int WM, int WN, int TM, int TN>
hipError_t launch_pipe(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                       int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    using C = DCfg<WM, WN, TM, TN, 3>;
    if (K % BK != 0) return hipErrorInvalidValue;
    const int tm = (M + C::BM - 1) / C::BM;
    const int tn = (N + C::BN - 1) / C::BN;
    const int64_t total = (int64_t)tm * tn;
    if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
    gemm_pipe_kernel<WM, WN, TM, TN><<<dim3((unsigned)total), dim3(C::kThreads), 0, s>>>(
        xq, gamma, M, K, wp, N, beta, y, acc, tn, (int)total);
    return hipGetLastError();
}

}  // namespace

bool gemm_dma_supports(int M, int K, int N) { return K % BK == 0 && K > 0 && M > 0 && N > 0; }

hipError_t launch_gemm_dma(const int8_t* xq, const float* gamma, int M, int K,
                           const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                           hipStream_t s) {
    // 128 x 256 tiles with a 3-stage ring (72 KB of LDS, two workgroups per
    // CU) once there is at least one such tile per CU, on the pipelined loop
    // with four waves side by side; else 128 x 128 tiles for more workgroups.
    // Measured on the M = 512 .. 2048 prefill shapes: the third stage gains
    // 7-10 % over two, and at M = 512, N = 28672 the wide tiles win even with
    // fewer tiles than workgroup slots.
    const int64_t wide_tiles = (int64_t)((M + 127) / 128) * ((N + 255) / 256);
    if (M >= 256 && wide_tiles >= 256)
        return launch_pipe<1, 4, 4, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    // at most one 64 x 128 tile per CU on a K of whole 256-steps: 64 x 128
    // tiles, two K groups per workgroup (8 waves).  Small M wastes no padded
    // rows and few-tile shapes spread over more CUs.  Measured against the
    // 128 x 128 route below: M = 64, K = 8192, N = 28672 47 -> 31 us; M = 96,
    // K = 4096, N = 11008 25 -> 17 us; M = 512, K = 6912, N = 2560 35 -> 24 us;
    // M = 512, K = 2560, N = 2560 18 -> 13 us; with more than 256 such tiles it
    // loses (M = 200, K = 4096, N = 11008 27 -> 31 us).
    const int64_t tiles64 = (int64_t)((M + 63) / 64) * ((N + 127) / 128);
    // long K in a multiple of 3 steps: three K groups (12 waves, 3 a SIMD)
    // shorten each tile's sequence of steps further (M = 512, K = 6912,
    // N = 2560: 22.8 -> 22.2 us)
    if (tiles64 <= 256 && K >= 36 * BK && K % (3 * BK) == 0)
        return launch_dcfg<2, 2, 1, 2, 3, 3>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    if (tiles64 <= 256 && K % (2 * BK) == 0)
        return launch_dcfg<2, 2, 1, 2, 3, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    // else 128 x 128 tiles on the pipelined loop (2 x 2 waves of 64 x 64).
    // Measured against the ring loop on the same tiles, with or without two K
    // groups per workgroup: equal or up to 6 % faster (M = 512, K = 2560,
    // N = 6912 20.9 -> 19.9 us; M = 1024, K = 4096, N = 11008 67.7 -> 64.8 us).
    return launch_pipe<2, 2, 2, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

}  // namespace bl

// Prefill GEMM on int8 MFMA with an LDS ring fed by direct global->LDS loads
// (K a multiple of 128).
//
// Arithmetic (unite.ai BitNet.cpp article, 3. BitLinear-Betrieb):
// v_mfma_i32_32x32x32_i8 on the int8 activations and the signed weights
// w = c - 1 unpacked from the 2-bit codes (unpack_signed), so the MFMA sums
// are the accumulators themselves (exact integer sums).
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
// MFMA kk (0..3) of lane half h covers packed word 4h + kk.
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

template <int WM, int WN, int TM, int TN, int STAGES>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_dma_kernel(const int8_t* __restrict__ xq, const float* __restrict__ gamma, int M,
                     int K, const uint32_t* __restrict__ wp, int N, float beta,
                     float* __restrict__ y, int32_t* __restrict__ acc_out, int tiles_n,
                     int tiles_total) {
    using C = DCfg<WM, WN, TM, TN, STAGES>;
    __shared__ __attribute__((aligned(16))) char lds[STAGES * C::kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wv / WN, wn = wv % WN;
    char* ring = lds;
    const int l32 = lane & 31, h = lane >> 5;

    int n0;
    const int m0 = tile_origin(blockIdx.x, tiles_n, tiles_total, C::BM, C::BN, n0);
    const int WR = K >> 4;
    const int KT = K / BK;  // K steps (K % BK == 0)

    // per-lane source offsets of this wave's copies at step 0 (32-bit, from
    // the block's first row / column); rows and columns past the matrix are
    // clamped onto its last row / column (their products are never stored)
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
            // 24.5 -> 23.7 us
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

    int* S = reinterpret_cast<int*>(lds);  // [BM], all 0 (no offset)
    float* Ssc = reinterpret_cast<float*>(S + C::BM);
    static_assert((int64_t)2 * C::BM * 4 <= (int64_t)STAGES * C::kStageBytes, "the row tables fit the ring");
    epilogue_tables(nullptr, 0, C::BM, m0, M, gamma, beta, S, Ssc, tid, C::kThreads);
    __syncthreads();
    store_tiles<TM, TN>(acc, S, Ssc, wm * TM * 32, wn * TN * 32, m0, n0, M, N, y, acc_out, lane);
}


// 64-row tiles with two K groups that share each weight copy.  A stage holds
// 2P consecutive 128-input steps: group g multiplies steps P g .. P g + P-1 of
// it.  The stage holds both groups' activation steps (64 rows x 128 bytes
// each, laid out as above) and all 2P steps of the tile's 128 weight columns
// as 64 P contiguous bytes a column, so one weight copy instruction reads
// 16 / P columns x 64 P bytes where the ring above reads 32 columns x 32 bytes.
// The 4P 16-byte pieces of column c (piece j = 2 s + h: step s of the stage,
// packed words 4h .. 4h+3) sit at positions j ^ ((c >> (3 - P)) & (4P - 1)),
// so the 16 neighbouring columns of a ds_read_b128 phase fall on different
// banks.  Eight waves (two groups of four side by side, 64 rows x 32 columns
// each) issue 3P copies a stage each: 2P activation copies and P weight
// copies.  P = 1, measured against the two-group ring (one step a stage,
// 32 columns x 32 bytes a weight copy) with weights streamed from HBM (copies
// rotated over 512 MB), bit-identical: M = 64, K = 8192, N = 28672 26.8 ->
// 24.5 us; M = 32 26.8 -> 24.5 us; M = 64, K = 4096, N = 11008 12.9 ->
// 11.8 us; M = 96 14.4 -> 13.4 us.
template <int STAGES, int P>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_pair_kernel(const int8_t* __restrict__ xq, const float* __restrict__ gamma, int M, int K,
                      const uint32_t* __restrict__ wp, int N, float beta, float* __restrict__ y,
                      int32_t* __restrict__ acc_out, int tiles_n, int tiles_total) {
    static_assert(P == 1 || P == 2, "one or two steps a group per stage");
    constexpr int BM = 64, BN = 128, TM = 2, TN = 1;
    constexpr int kABytes = BM * BK;             // one activation step
    constexpr int kColBytes = 64 * P;            // weight bytes of a column per stage
    constexpr int kStageBytes = 2 * P * kABytes + BN * kColBytes;
    constexpr int kPerStep = 3 * P;              // copies of a wave per stage
    constexpr int kColsPerCopy = 16 / P;
    constexpr int kSwzShift = 3 - P, kSwzMask = 4 * P - 1;
    __shared__ __attribute__((aligned(16))) char lds[STAGES * kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);  // 0..7
    const int kgrp = wv / 4, wn = wv % 4;
    const int l32 = lane & 31, h = lane >> 5;

    int n0;
    const int m0 = tile_origin(blockIdx.x, tiles_n, tiles_total, BM, BN, n0);
    const int WR = K >> 4;
    const int KP = K / (2 * P * BK);  // stages of K (K % (256 P) == 0)

    // activation copies q = 2P wv .. 2P wv + 2P-1 of 16P: step q / 8 of the
    // stage, rows 8 (q % 8) .. +7; weight copies P wv .. P wv + P-1 of 8P:
    // columns (16 / P) q .. +(16 / P - 1).  Rows and columns past the matrix
    // are clamped (their products are never stored).
    uint32_t aoff[2 * P];
#pragma unroll
    for (int i = 0; i < 2 * P; ++i) {
        const int q = 2 * P * wv + i;
        const int row = 8 * (q % 8) + lane / 8;
        const int lchunk = (lane % 8) ^ swz(row);
        aoff[i] = (uint32_t)(min(m0 + row, M - 1) - m0) * (uint32_t)K + (uint32_t)((q / 8) * BK) +
                  16u * lchunk;
    }
    uint32_t boff[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int c = kColsPerCopy * (P * wv + i) + lane / (4 * P);
        const int j = (lane % (4 * P)) ^ ((c >> kSwzShift) & kSwzMask);
        boff[i] = (uint32_t)(min(n0 + c, N - 1) - n0) * (uint32_t)WR + 4u * j;
    }
    const int8_t* abase = xq + (int64_t)m0 * K;
    const uint32_t* bbase = wp + (int64_t)n0 * WR;

    auto issue = [&](int kp, int buf) {
        char* stage = lds + buf * kStageBytes;
        const int8_t* a_step = abase + (int64_t)kp * (2 * P * BK);
#pragma unroll
        for (int i = 0; i < 2 * P; ++i) {
            const int q = 2 * P * wv + i;
            copy16_to_lds(a_step + aoff[i], stage + (q / 8) * kABytes + 1024 * (q % 8));
        }
        const uint32_t* b_step = bbase + (int64_t)kp * (16 * P);
#pragma unroll
        for (int i = 0; i < P; ++i)
            copy16_to_lds(b_step + boff[i], stage + 2 * P * kABytes + 1024 * (P * wv + i));
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[i][0] = v16i{};

#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p) issue(min(p, KP - 1), p);

    for (int kp = 0; kp < KP; ++kp) {
        // this wave's copies of stage kp are done (later stages may be in flight)
        __builtin_amdgcn_s_waitcnt(waitcnt_imm((STAGES - 2) * kPerStep, 0));
        __builtin_amdgcn_s_barrier();
        issue(min(kp + STAGES - 1, KP - 1), (kp + STAGES - 1) % STAGES);

        const char* stage = lds + (kp % STAGES) * kStageBytes;
        const v4u* Bs = reinterpret_cast<const v4u*>(stage + 2 * P * kABytes);
        const int col = wn * 32 + l32;
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const int st = P * kgrp + u;  // step of the stage
            const v4i* As = reinterpret_cast<const v4i*>(stage + st * kABytes);
            const v4u wq = Bs[col * (4 * P) + ((2 * st + h) ^ ((col >> kSwzShift) & kSwzMask))];
            v4i af[4][TM];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int r = 32 * i + l32;
                    af[kk][i] = As[r * 8 + ((4 * h + kk) ^ swz(r))];
                }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const v4i bf = unpack_signed(wq[kk]);
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    acc[i][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[kk][i], bf, acc[i][0], 0, 0, 0);
            }
        }
    }
    // every copy (including the re-reads past the end) has landed before the
    // LDS is reused below or released
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __syncthreads();

    // group 1's accumulators go through LDS (lane-major) to group 0, whose
    // waves own the epilogue
    constexpr int kAccInts = 4 * TM * TN * 16 * kWave;
    int* red = reinterpret_cast<int*>(lds);
    int* S = red + kAccInts;  // [BM], all 0 (no offset)
    float* Ssc = reinterpret_cast<float*>(S + BM);
    static_assert((kAccInts + 2 * BM) * 4 <= STAGES * kStageBytes, "the exchange fits the ring");
    if (kgrp == 1) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) red[((wn * TM + i) * 16 + v) * kWave + lane] = acc[i][0][v];
    }
    __syncthreads();
    if (kgrp == 0) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][0][v] += red[((wn * TM + i) * 16 + v) * kWave + lane];
    }
    __syncthreads();
    epilogue_tables(nullptr, 0, BM, m0, M, gamma, beta, S, Ssc, tid, 512);
    __syncthreads();
    if (kgrp == 0) store_tiles<TM, TN>(acc, S, Ssc, 0, wn * 32, m0, n0, M, N, y, acc_out, lane);
}

template <int STAGES, int P>
hipError_t launch_pair(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                       int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    if (K % (2 * P * BK) != 0) return hipErrorInvalidValue;
    const int64_t total = (int64_t)((M + 63) / 64) * ((N + 127) / 128);
    if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int tn = (N + 127) / 128;
    gemm_pair_kernel<STAGES, P><<<dim3((unsigned)total), dim3(512), 0, s>>>(xq, gamma, M, K, wp, N, beta,
                                                                            y, acc, tn, (int)total);
    return hipGetLastError();
}


template <int WM, int WN, int TM, int TN, int STAGES>
hipError_t launch_dcfg(const int8_t* xq, const float* gamma, int M, int K, const uint32_t* wp,
                       int N, float beta, float* y, int32_t* acc, hipStream_t s) {
    using C = DCfg<WM, WN, TM, TN, STAGES>;
    if (K % BK != 0) return hipErrorInvalidValue;
    const int tm = (M + C::BM - 1) / C::BM;
    const int tn = (N + C::BN - 1) / C::BN;
    const int64_t total = (int64_t)tm * tn;
    if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
    gemm_dma_kernel<WM, WN, TM, TN, STAGES>
        <<<dim3((unsigned)total), dim3(C::kThreads), 0, s>>>(xq, gamma, M, K, wp, N, beta, y, acc, tn,
                                                             (int)total);
    return hipGetLastError();
}


}  // namespace

bool gemm_dma_supports(int M, int K, int N) { return K % BK == 0 && K > 0 && M > 0 && N > 0; }

hipError_t launch_gemm_dma(const int8_t* xq, const float* gamma, int M, int K,
                           const uint32_t* wp, int N, float beta, float* y, int32_t* acc,
                           hipStream_t s) {
    // 128 x 256 tiles (four waves side by side, each 128 rows x 64 columns, so
    // each packed word is unpacked once per workgroup; 72 KB of LDS, two
    // workgroups per CU) once there is at least one such tile per CU; at
    // M = 512, N = 28672 they win even with fewer tiles than workgroup slots.
    // Until the signed weights a software-pipelined form of this loop (A
    // fragments of the next K slice read during the current MFMAs, the step's
    // barrier between two halves of the last slice, row sums on v_sad_u8) was
    // the faster one; with them the plain ring is faster, bit-identical,
    // interleaved A/B: M = 512, K = 8192, N = 28672 120.3 -> 117.5 us;
    // M = 2048, K = 4096, N = 11008 110.2 -> 102.9 us; M = 1024 61.4 -> 60.0 us;
    // the 128 x 128 route below at M = 512, K = 2560, N = 13824 30.4 -> 29.2 us.
    const int64_t wide_tiles = (int64_t)((M + 127) / 128) * ((N + 255) / 256);
    if (M >= 256 && wide_tiles >= 256)
        return launch_dcfg<1, 4, 4, 2, 3>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    // at most one 64 x 128 tile per CU on a K of whole 256-steps: 64 x 128
    // tiles, two K groups per workgroup (8 waves).  Small M wastes no padded
    // rows and few-tile shapes spread over more CUs.  Measured against the
    // 128 x 128 route below: M = 64, K = 8192, N = 28672 47 -> 31 us; M = 96,
    // K = 4096, N = 11008 25 -> 17 us; M = 512, K = 6912, N = 2560 35 -> 24 us;
    // M = 512, K = 2560, N = 2560 18 -> 13 us; with more than 256 such tiles it
    // loses (M = 200, K = 4096, N = 11008 27 -> 31 us).  Each group's four
    // waves sit side by side (64 rows x 32 columns each, so every unpacked
    // weight word feeds two MFMAs); against 2 x 2 waves of 32 x 64, interleaved
    // A/B, bit-identical: M = 64, K = 8192, N = 28672 30.9 -> 28.6 us; M = 32
    // 29.1 -> 28.0 us; M = 512, K = 2560, N = 2560 11.3 -> 10.6 us; M = 96,
    // K = 4096, N = 11008 15.3 both.
    const int64_t tiles64 = (int64_t)((M + 63) / 64) * ((N + 127) / 128);
    // the two groups sharing each weight copy (gemm_pair_kernel): with
    // K % 512 == 0 up to K = 8192 two steps a group per stage (8 columns x
    // 128 bytes a copy) in two 48 KB stages, against one step in three or
    // four stages, weights streamed from HBM, bit-identical: M = 64, K = 8192,
    // N = 28672 22.9-24.4 -> 22.6-22.8 us; M = 32 23.0-24.6 -> 22.5-22.7 us;
    // M = 96, K = 4096, N = 11008 13.4-13.9 -> 12.9-13.1 us; M = 512,
    // K = 2560, N = 2560 9.0-9.3 -> 8.8 us; M = 200, K = 8192, N = 4096
    // 19.2-19.7 -> 18.9-19.1 us (M = 64, K = 4096 11.8-12.0 -> 12.1-12.2 us).
    // Longer K over fewer tiles keeps one step a group in four stages
    // (M = 64, K = 9216, N = 11008 21.2-21.5 against 21.9-22.1 us; K = 12288,
    // N = 8192 26.6-26.7 against 28.2 us).  Both replaced a route with three
    // K groups of separate rings for K >= 4608 in a multiple of 384, which
    // they beat on its shapes: M = 512, K = 6912, N = 2560 17.8-18.4 ->
    // 16.9-17.3 us; M = 300, N = 1536 18.1-18.2 -> 17.6-17.7 us; M = 100,
    // K = 4608, N = 1000 14.0-14.2 -> 13.3 us; M = 64, K = 9216, N = 11008
    // 23.9-24.4 -> 21.2-21.5 us.
    if (tiles64 <= 256 && K % (4 * BK) == 0 && K <= 64 * BK)
        return launch_pair<2, 2>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    if (tiles64 <= 256 && K % (2 * BK) == 0)
        return launch_pair<4, 1>(xq, gamma, M, K, wp, N, beta, y, acc, s);
    // else 128 x 128 tiles (2 x 2 waves of 64 x 64)
    return launch_dcfg<2, 2, 2, 2, 3>(xq, gamma, M, K, wp, N, beta, y, acc, s);
}

}  // namespace bl

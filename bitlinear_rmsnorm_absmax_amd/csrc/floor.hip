// Measurement aids for the roofline report: the floors a kernel of the
// library is compared with.  An empty kernel gives the launch floor; a
// read-only pass over a buffer, with the 16-byte-per-lane coalesced loads the
// decode kernels use, gives the time the same bytes take to stream from HBM;
// a register-only int8 MFMA loop with the grid, waves and operand data of the
// 128 x 256-tile GEMM gives the time its multiplies take with no memory work.
#include "device_common.h"
#include "internal.h"
#include "mfma_epilogue.h"

namespace bl {
namespace {

constexpr int kFloorThreads = 256;
constexpr int kFloorUnroll = 4;

__global__ __launch_bounds__(kFloorThreads) void floor_empty_kernel() {}

// Thread t of the grid reads the 16-byte pieces t, t + S, t + 2S, ... (S = the
// grid's thread count), four loads in flight, and folds them with xor.  The
// fold is stored only when it equals a fixed odd constant, so the loads stay
// live and the kernel writes nothing in practice.
__global__ __launch_bounds__(kFloorThreads) void floor_stream_read_kernel(
    const v4u* __restrict__ p, int64_t pieces, uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kFloorThreads;
    int64_t i = (int64_t)blockIdx.x * kFloorThreads + threadIdx.x;
    uint32_t fold = 0;
    for (; i + (kFloorUnroll - 1) * stride < pieces; i += kFloorUnroll * stride) {
        v4u v[kFloorUnroll];
#pragma unroll
        for (int u = 0; u < kFloorUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < kFloorUnroll; ++u) fold ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < pieces; i += stride) {
        const v4u v = p[i];
        fold ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (fold == 0x9E3779B9u) sink[0] = fold;
}

// One workgroup per 128 x 256 output tile, four waves of 128 rows x 64
// columns, two workgroups per CU: the shape of the GEMM's widest tiles.  Each
// wave loads the operands of its first K step as the GEMM's MFMAs take them
// (activation chunk 4h + kk of each of its rows, signed weights of packed word
// 4h + kk of each of its columns) and then issues the GEMM's 32 MFMAs a step
// for `steps` steps on those registers, so the multiplies see the call's own
// data, in the same order, with nothing else to wait for.  The xor of the
// accumulators is stored only when it equals a fixed odd constant.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void floor_mfma_kernel(const int8_t* __restrict__ xq, const uint32_t* __restrict__ wp, int M, int K,
                       int N, int tiles_m, int steps, uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const int l32 = lane & 31, h = lane >> 5;
    const int m0 = (int)(blockIdx.x % (unsigned)tiles_m) * 128;
    const int n0 = (int)(blockIdx.x / (unsigned)tiles_m) * 256 + wv * 64;
    v4i af[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = min(m0 + 32 * i + l32, M - 1);
        const v4i* row = reinterpret_cast<const v4i*>(xq + (int64_t)r * K);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) af[kk][i] = row[4 * h + kk];
    }
    v4i bf[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int c = min(n0 + 32 * t + l32, N - 1);
        const v4u w = *reinterpret_cast<const v4u*>(wp + (int64_t)c * (K >> 4) + 4 * h);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) bf[t][kk] = unpack_signed(w[kk]);
    }
    v16i acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[i][t] = v16i{};
    for (int st = 0; st < steps; ++st) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    acc[i][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[kk][i], bf[t][kk], acc[i][t], 0, 0, 0);
    }
    uint32_t fold = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) fold ^= (uint32_t)acc[i][t][v];
    if (fold == 0x9E3779B9u) sink[0] = fold;
}

}  // namespace

hipError_t launch_floor_mfma(const int8_t* xq, int M, int K, const uint32_t* wp, int N,
                             uint32_t* sink, hipStream_t s) {
    const int64_t tm = (M + 127) / 128, tn = ((int64_t)N + 255) / 256;
    if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
    floor_mfma_kernel<<<dim3((unsigned)(tm * tn)), dim3(256), 0, s>>>(xq, wp, M, K, N, (int)tm, K / 128,
                                                                      sink);
    return hipGetLastError();
}

hipError_t launch_floor_empty(hipStream_t s) {
    floor_empty_kernel<<<dim3(1), dim3(64), 0, s>>>();
    return hipGetLastError();
}

hipError_t launch_floor_stream_read(const void* p, int64_t bytes, uint32_t* sink, hipStream_t s) {
    const int64_t pieces = bytes / 16;
    // one pass of four pieces per thread where that takes at most 8192
    // workgroups (58.7 MB: 3584 workgroups), a grid-stride loop beyond
    const int64_t per_block = (int64_t)kFloorThreads * kFloorUnroll;
    const int blocks = (int)std::min<int64_t>(std::max<int64_t>((pieces + per_block - 1) / per_block, 1), 8192);
    floor_stream_read_kernel<<<dim3(blocks), dim3(kFloorThreads), 0, s>>>(
        reinterpret_cast<const v4u*>(p), pieces, sink);
    return hipGetLastError();
}

}  // namespace bl

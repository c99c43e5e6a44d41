// Measurement aids for the roofline report: the two floors a kernel of the
// library is compared with.  An empty kernel gives the launch floor; a
// read-only pass over a buffer, with the 16-byte-per-lane coalesced loads the
// decode kernels use, gives the time the same bytes take to stream from HBM.
#include "device_common.h"
#include "internal.h"

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

}  // namespace

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

// 2-bit packing of ternary weights (unite.ai BitNet.cpp article, Ternäres
// Gewichtssystem / Das Konzept: three states per weight).  code = w + 1;
// the 16 weights of a group form one uint32 with weight e = 4j + b at bit
// 8b + 2j, so that a shift by 2j and a mask 0x03030303 yield four byte-lane
// codes in natural order -- the operand form of the int8 dot products and
// MFMAs of the forward kernels.
//
// One thread per output word: a 16-byte load of the 16 weights, a 4-byte
// store.  Entries outside {-1, 0, +1} are stored as code 3 and counted with
// one atomic per wave.
#include "device_common.h"
#include "internal.h"

namespace bl {
namespace {

__global__ __launch_bounds__(256) void pack_kernel(const int8_t* __restrict__ w, int64_t words,
                                                   uint32_t* __restrict__ out,
                                                   int32_t* __restrict__ bad) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int nbad = 0;
    if (i < words) {
        uint4 v = reinterpret_cast<const uint4*>(w)[i];
        uint32_t d[4] = {v.x, v.y, v.z, v.w};
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                int val = (int)(int8_t)(d[j] >> (8 * b));
                uint32_t code;
                if (val >= -1 && val <= 1) {
                    code = (uint32_t)(val + 1);
                } else {
                    code = 3u;
                    ++nbad;
                }
                word |= code << (8 * b + 2 * j);
            }
        }
        out[i] = word;
    }
    if (bad) {
        int tot = wave_sum_i(nbad);
        if ((threadIdx.x % kWave) == 0 && tot) atomicAdd(bad, tot);
    }
}

__global__ void zero_int_kernel(int32_t* p) { *p = 0; }

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ y,
                                                        int32_t* __restrict__ acc, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * 256) {
        if (y) y[i] = 0.0f;
        if (acc) acc[i] = 0;
    }
}

}  // namespace

hipError_t launch_pack(const int8_t* w, int64_t N, int64_t K, uint32_t* packed, int32_t* bad,
                       hipStream_t s) {
    if (bad) {
        zero_int_kernel<<<1, 1, 0, s>>>(bad);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t words = N * (K / 16);
    if (words == 0) return hipSuccess;
    const int64_t blocks = (words + 255) / 256;
    pack_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(w, words, packed, bad);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* y, int32_t* acc, int64_t count, hipStream_t s) {
    if (count == 0) return hipSuccess;
    int64_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    fill_zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(y, acc, count);
    return hipGetLastError();
}

}  // namespace bl

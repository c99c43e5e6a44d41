// Host-only stand-ins for the device launchers of libbitlinear, for the CPU
// sanitizer build of the C ABI's argument validation (api.cpp with the shape
// rules of shapes.cpp).  Each launcher accepts its arguments, launches
// nothing and returns hipSuccess; a validation path that reaches a launcher
// therefore behaves as on a device whose launch succeeded.  Test
// infrastructure only: never linked into the library.
#include "internal.h"

namespace bl {

hipError_t launch_quant_act(const void*, int, int64_t, int64_t, const float*, float, int8_t*, float*,
                            hipStream_t) { return hipSuccess; }
hipError_t launch_quant_gemv(const void*, bool, int, const float*, float, const uint32_t*, int, float,
                             float*, int32_t*, int8_t*, float*, hipStream_t) { return hipSuccess; }
hipError_t launch_silu_mul_quant(const float*, const float*, int64_t, int64_t, float*, int8_t*, float*,
                                 hipStream_t) { return hipSuccess; }
hipError_t launch_silu_mul_quant_acc(const int32_t*, const float*, int64_t, int64_t, float, float,
                                     float*, int8_t*, float*, hipStream_t) { return hipSuccess; }
hipError_t launch_pack(const int8_t*, int64_t, int64_t, uint32_t*, int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_fill_zero(float*, int32_t*, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_gemv_valu(const int8_t*, const float*, int, int, const uint32_t*, int, float, float*,
                            int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_skinny_mfma(const int8_t*, const float*, int, int, const uint32_t*, int, float, float*,
                              int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_decode_lds(const int8_t*, const float*, int, int, const uint32_t*, int, float, float*,
                             int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_decode_lds_grouped(const int8_t*, const float*, int, int, int, const uint32_t*, int,
                                     const float*, float*, int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_decode_lds1(const int8_t*, const float*, int, int, const uint32_t*, int, float, float*,
                              int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_quant_decode1(const void*, bool, int, const float*, float, const uint32_t*, int, float,
                                float*, int32_t*, int8_t*, float*, hipStream_t) { return hipSuccess; }
hipError_t launch_pairwise_mean(const float*, int64_t, int64_t, int64_t, bool, int, double*, double*,
                                float*, hipStream_t) { return hipSuccess; }
hipError_t launch_binarize(const float*, int64_t, int64_t, uint32_t*, int8_t*, double*, float*, double*,
                           float*, hipStream_t) { return hipSuccess; }
hipError_t launch_pack1(const int8_t*, int64_t, int64_t, uint32_t*, int*, hipStream_t) { return hipSuccess; }
hipError_t launch_forward1(const int8_t*, const float*, int, int, const uint32_t*, int, float, float*,
                           int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_ternarize(const float*, int64_t, int64_t, uint32_t*, int8_t*, float*, double*,
                            hipStream_t) { return hipSuccess; }
hipError_t launch_quant_act_grouped(const void*, int, int64_t, int64_t, int64_t, const float*, float,
                                    int8_t*, float*, hipStream_t) { return hipSuccess; }
hipError_t launch_group_sum(const int32_t*, const float*, const float*, int64_t, int64_t, int64_t, float*,
                            hipStream_t) { return hipSuccess; }
hipError_t launch_pack3(const int8_t*, int64_t, int64_t, uint32_t*, int*, hipStream_t) { return hipSuccess; }
hipError_t launch_forward3(const int8_t*, const float*, int, int, const uint32_t*, int, float, float*,
                           int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_gemm_dma(const int8_t*, const float*, int, int, const uint32_t*, int, float, float*,
                           int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_gemm_mfma(const int8_t*, const float*, int, int, const uint32_t*, int, float, float*,
                            int32_t*, hipStream_t) { return hipSuccess; }
bool gemm_dma_supports(int, int, int) { return true; }
hipError_t launch_floor_empty(hipStream_t) { return hipSuccess; }
hipError_t launch_floor_stream_read(const void*, int64_t, uint32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_floor_mfma(const int8_t*, int, int, const uint32_t*, int, uint32_t*, hipStream_t) { return hipSuccess; }

}  // namespace bl

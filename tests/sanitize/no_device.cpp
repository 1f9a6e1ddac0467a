// Stand-ins for the HIP runtime and the kernel launchers, for the host-only
// sanitizer build of the C ABI (api.cpp, plan.cpp): every device query reports
// that there is no device, as on a machine without a GPU, so each entry point
// runs its argument checks and planning and then returns Q8_ERR_DEVICE.  No
// launcher is ever reached; they exist only to link.
#include <hip/hip_runtime_api.h>

#include "launch.hpp"

extern "C" hipError_t hipGetDevice(int *device) {
    if (device) *device = -1;
    return hipErrorNoDevice;
}

extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *, int) { return hipErrorNoDevice; }

namespace q8k {

hipError_t launch_quantize(const float *, int64_t, int64_t, int64_t, int, void *, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_repack(const void *, int64_t, int64_t, void *, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gemv(const void *, int64_t, const void *, int, int64_t, int64_t, float *, int64_t, void *,
                       hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_gemv_f32(const float *, int64_t, int64_t, const void *, int, int64_t, int64_t, float *, int64_t,
                           void *, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_gemv_sequence(const SeqHostStep *, int, int64_t, void *, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gemv_sequence_scratch(const SeqHostStep *, int, int64_t, int32_t *, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_rmsnorm_quantize(const float *, const float *, float *, const float *, int64_t, int64_t, float,
                                   void *, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_moe_route(const float *, int64_t, int64_t, int, int, int32_t *, float *, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_swiglu_quantize(const float *, int64_t, const float *, int64_t, int64_t, int64_t, void *,
                                  hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_moe_combine(const float *, int64_t, const float *, int64_t, int, int64_t, float *, int64_t,
                              hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_kv_write(const float *, int64_t, int, int, int, const int32_t *, int64_t, const float *,
                           const float *, const float *, const float *, float, const int32_t *, int64_t, float *,
                           int8_t *, float *, int8_t *, float *, int32_t *, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_attention_decode(const float *, int64_t, int, int, int, const int8_t *, const float *,
                                   const int8_t *, const float *, int64_t, const int32_t *, const int32_t *, int64_t,
                                   float, float *, void *, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_gemm(const void *, int64_t, const void *, int64_t, int64_t, float *, int64_t, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_grouped(const void *, int64_t, int, const int32_t *, int64_t, int, const void *, int64_t, int64_t,
                          int64_t, int64_t, float *, void *, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_stream_read(const void *, size_t, uint32_t *, hipStream_t) { return hipErrorNoDevice; }

}  // namespace q8k

// abi_stubs.hip - stand-ins for the kernel launchers behind the C ABI, for
// the sanitizer build of the host validation layer (mxq_api.hip) on a
// machine without a GPU.  Test infrastructure: the validation tests never
// pass a call that reaches a launcher; if one did, it reports no device.
#include <hip/hip_runtime.h>

#include "../../mxfp4_precision_numerics_amd/csrc/launch.h"

namespace mxq {

hipError_t launch_quantize_per_tensor(const void*, int, int64_t, int64_t, int64_t, int, float*, int, float*, float*,
                                      float*, uint8_t*, uint8_t*, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_quantize_mx(const void*, int, int64_t, int64_t, int64_t, int, uint8_t*, uint8_t*, uint8_t*,
                              uint8_t*, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_swiglu_quantize_mx(const void*, int, int64_t, int64_t, int64_t, int, uint8_t*, uint8_t*,
                                     hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_repack_fp4_to_fp8(const uint8_t*, const uint8_t*, const int32_t*, int64_t, int64_t, int64_t,
                                    uint8_t*, uint8_t*, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_fp4_row_to_fp8_col(const uint8_t*, const uint8_t*, int64_t, int64_t, uint8_t*, uint8_t*,
                                     hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_scaled_gemm(const GemmArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_grouped_swiglu(const GemmArgs&, hipStream_t) { return hipErrorNoDevice; }

}  // namespace mxq

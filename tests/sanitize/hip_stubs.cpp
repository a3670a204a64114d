// Stand-ins, for the CPU sanitizer build, of the HIP runtime calls and the
// kernel launchers that the library's host code uses.  Every one reports
// that there is no device, so each entry point runs all of its argument and
// descriptor checks and then fails with LBF_E_HIP at the first step that
// would reach a GPU.  Test infrastructure: nothing here is part of the
// library.
#include <hip/hip_runtime_api.h>

#include "lbf_internal.h"

extern "C" {
hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }
hipError_t hipFuncSetAttribute(const void*, hipFuncAttribute, int) { return hipErrorNoDevice; }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { return hipErrorNoDevice; }
hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int*, const void*, int, size_t) { return hipErrorNoDevice; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipErrorNoDevice; }
}

namespace lbf {
hipError_t launch_decode(const lbf_desc&, const uint8_t*, uint16_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_verify(const lbf_desc&, const uint8_t*, uint32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_crc32(const uint8_t*, uint64_t, uint32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_hist(const uint16_t*, uint64_t, uint32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_pack(const uint16_t*, const lbf_desc&, uint8_t*, uint32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gemv(const GroupArg*, int, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gemm(const GroupArg*, int, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gemv_gated(const GroupArg&, const GroupArg&, int, void*, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_hcount(const lbf_desc&, const uint8_t*, uint32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_hwoff(const lbf_desc&, const uint8_t*, const uint8_t[16], uint32_t*, uint32_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_hpack(const lbf_desc&, const uint8_t*, const HCode&, const uint32_t*, uint32_t*, uint64_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_hfill(const lbf_hdesc&, uint8_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_hdecode(const lbf_hdesc&, const HCode&, const uint8_t*, uint16_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t encode_scratch(void**) { return hipErrorNoDevice; }
}  // namespace lbf

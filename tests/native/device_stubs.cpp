// Stand-ins for the device-side launchers (kv_kernels.hip, scratch.hip) so
// the library's host code, api.cpp and block_manager.cpp, can be built with
// g++ and the sanitizers, with no device code.  Every launcher reports that
// there is no device, so the host runtime's argument checks, planning and
// block manager run under AddressSanitizer and UndefinedBehaviorSanitizer
// while nothing is launched (tests/test_host_sanitizers.py).
#include "launch.h"

namespace pa {

hipError_t scratch_buffer(void**) { return hipErrorNoDevice; }
hipError_t launch_zero(void*, int64_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_write_kv(const PoolDesc&, const void*, const void*, const int32_t*, int32_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_copy_blocks(const PoolDesc&, const int32_t*, int32_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_swap_blocks(const PoolDesc&, const int32_t*, int32_t, void*, bool, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_decode(const PoolDesc&, const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t decode_capacity(const PoolDesc&, int32_t, int32_t, int32_t, DecodeCapacity*) { return hipErrorNoDevice; }

}  // namespace pa

// Decode kernels instantiated for f32 pools (see decode_impl.h).
#include "decode_impl.h"

namespace pa {

hipError_t launch_decode_f32(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream) {
  return dec::launch_dtype<kF32>(p, a, stream);
}

}  // namespace pa

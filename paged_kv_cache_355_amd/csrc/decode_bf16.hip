// Decode kernels instantiated for bf16 pools (see decode_impl.h).
#include "decode_impl.h"

namespace pa {

hipError_t launch_decode_bf16(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream) {
  return dec::launch_dtype<kBF16>(p, a, stream);
}

}  // namespace pa

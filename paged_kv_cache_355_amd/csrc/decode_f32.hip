// Decode kernels instantiated for f32 pools (see decode_impl.h).
#include "decode_impl.h"

namespace pa {

hipError_t launch_decode_f32(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream) {
  return dec::launch_dtype<kF32>(p, a, stream);
}

hipError_t decode_grid_f32(const PoolDesc& p, int32_t group, int32_t num_seqs, int32_t max_ctx, int32_t* grid,
                           int32_t* partition_capacity) {
  return dec::grid_dtype<kF32>(p, group, num_seqs, max_ctx, grid, partition_capacity);
}

}  // namespace pa

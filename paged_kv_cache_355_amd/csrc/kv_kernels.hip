// Slot-mapped KV write, copy-on-write block copy and block swap for gfx950.
//
// [P2] "PagedAttention：操作系统级 KV 缓存虚拟内存管理" §3.2.2 step 3 (the new
// token's K/V goes into its slot), §3.4 (a shared block is copied before a
// divergent write) and §5 / §8 (inactive blocks move out to CPU memory and
// back, as pages are swapped).  All are pure byte moves: every lane moves one
// 16-byte vector, consecutive lanes move consecutive bytes of a token row or
// block, so each wavefront issues fully coalesced 1 KiB loads and stores.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

// One thread per 16-byte chunk of one (row, kv-head) of K or V
// (blockIdx.y selects the tensor).  Rows with slot < 0, or a slot outside the
// pool, are skipped.
__global__ __launch_bounds__(kThreads) void write_kv_kernel(
    char* __restrict__ k_pool, char* __restrict__ v_pool, const char* __restrict__ k_new,
    const char* __restrict__ v_new, const int32_t* __restrict__ slots, int32_t n, int32_t kv_heads,
    int32_t block_size, int32_t chunks_per_row, int32_t row_bytes, int32_t total_slots) {
  const int64_t per_tensor = static_cast<int64_t>(n) * kv_heads * chunks_per_row;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= per_tensor) return;
  const int32_t c = static_cast<int32_t>(idx % chunks_per_row);
  const int64_t rh = idx / chunks_per_row;
  const int32_t h = static_cast<int32_t>(rh % kv_heads);
  const int32_t i = static_cast<int32_t>(rh / kv_heads);
  const int32_t slot = slots[i];
  if (slot < 0 || slot >= total_slots) return;
  const int32_t block = slot / block_size;
  const int32_t off = slot - block * block_size;
  const bool is_v = blockIdx.y != 0;
  const char* src = (is_v ? v_new : k_new) + (rh * row_bytes + c * 16);
  char* dst = (is_v ? v_pool : k_pool) +
              ((static_cast<int64_t>(block) * kv_heads + h) * block_size + off) * row_bytes + c * 16;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

// Grid: x = pair × chunk-groups, y = tensor (K, V).  Each thread copies one
// 16-byte chunk per iteration of a grid-stride loop over the block.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(char* __restrict__ k_pool,
                                                               char* __restrict__ v_pool,
                                                               const int32_t* __restrict__ pairs,
                                                               int32_t groups_per_pair, int64_t block_bytes,
                                                               int32_t num_blocks) {
  const int32_t pair = blockIdx.x / groups_per_pair;
  const int32_t grp = blockIdx.x - pair * groups_per_pair;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  char* base = blockIdx.y ? v_pool : k_pool;
  const char* from = base + static_cast<int64_t>(src) * block_bytes;
  char* to = base + static_cast<int64_t>(dst) * block_bytes;
  const int64_t stride = static_cast<int64_t>(groups_per_pair) * kThreads * 16;
  for (int64_t off = (static_cast<int64_t>(grp) * kThreads + threadIdx.x) * 16; off < block_bytes; off += stride) {
    *reinterpret_cast<uint4*>(to + off) = *reinterpret_cast<const uint4*>(from + off);
  }
}

// Grid: x = block × chunk-groups, y = tensor (K, V).  Host layout: block i's
// K tile (all kv-heads) then its V tile, [n][2][block_bytes].  OUT moves pool
// → host, else host → pool; the host side is pinned memory the device maps,
// so the bytes cross the host link once, with no staging copy in HBM.  Block
// ids outside the pool are skipped.
template <bool OUT>
__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(char* __restrict__ k_pool, char* __restrict__ v_pool,
                                                               char* __restrict__ host,
                                                               const int32_t* __restrict__ blocks,
                                                               int32_t groups_per_block, int64_t block_bytes,
                                                               int32_t num_blocks) {
  const int32_t i = blockIdx.x / groups_per_block;
  const int32_t grp = blockIdx.x - i * groups_per_block;
  const int32_t b = blocks[i];
  if (b < 0 || b >= num_blocks) return;
  char* pool_blk = (blockIdx.y ? v_pool : k_pool) + static_cast<int64_t>(b) * block_bytes;
  char* host_blk = host + (2 * static_cast<int64_t>(i) + blockIdx.y) * block_bytes;
  const int64_t stride = static_cast<int64_t>(groups_per_block) * kThreads * 16;
  for (int64_t off = (static_cast<int64_t>(grp) * kThreads + threadIdx.x) * 16; off < block_bytes; off += stride) {
    if constexpr (OUT) {
      *reinterpret_cast<uint4*>(host_blk + off) = *reinterpret_cast<const uint4*>(pool_blk + off);
    } else {
      *reinterpret_cast<uint4*>(pool_blk + off) = *reinterpret_cast<const uint4*>(host_blk + off);
    }
  }
}

}  // namespace

hipError_t launch_swap_blocks(const PoolDesc& p, const int32_t* blocks, int32_t n, void* host_dev, bool out,
                              hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t chunks = p.block_bytes / 16;
  int32_t groups = static_cast<int32_t>((chunks + kThreads - 1) / kThreads);
  if (groups > 16) groups = 16;
  const int64_t grid = static_cast<int64_t>(n) * groups;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (out) {
    hipLaunchKernelGGL(swap_blocks_kernel<true>, dim3(static_cast<uint32_t>(grid), 2), dim3(kThreads), 0, stream,
                       static_cast<char*>(p.k), static_cast<char*>(p.v), static_cast<char*>(host_dev), blocks,
                       groups, p.block_bytes, p.num_blocks);
  } else {
    hipLaunchKernelGGL(swap_blocks_kernel<false>, dim3(static_cast<uint32_t>(grid), 2), dim3(kThreads), 0, stream,
                       static_cast<char*>(p.k), static_cast<char*>(p.v), static_cast<char*>(host_dev), blocks,
                       groups, p.block_bytes, p.num_blocks);
  }
  return hipGetLastError();
}

hipError_t launch_write_kv(const PoolDesc& p, const void* k_new, const void* v_new, const int32_t* slots,
                           int32_t n, hipStream_t stream) {
  const int32_t row_bytes = p.head_dim * elem_bytes(p.dtype);
  const int32_t chunks = row_bytes / 16;
  const int64_t per_tensor = static_cast<int64_t>(n) * p.kv_heads * chunks;
  const int64_t blocks = (per_tensor + kThreads - 1) / kThreads;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(write_kv_kernel, dim3(static_cast<uint32_t>(blocks), 2), dim3(kThreads), 0, stream,
                     static_cast<char*>(p.k), static_cast<char*>(p.v), static_cast<const char*>(k_new),
                     static_cast<const char*>(v_new), slots, n, p.kv_heads, p.block_size, chunks, row_bytes,
                     p.num_blocks * p.block_size);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const PoolDesc& p, const int32_t* pairs, int32_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t chunks = p.block_bytes / 16;
  int32_t groups = static_cast<int32_t>((chunks + kThreads - 1) / kThreads);
  if (groups > 16) groups = 16;  // ≤ 64 KiB per workgroup per pass; loop covers the rest
  const int64_t grid = static_cast<int64_t>(n) * groups;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<uint32_t>(grid), 2), dim3(kThreads), 0, stream,
                     static_cast<char*>(p.k), static_cast<char*>(p.v), pairs, groups, p.block_bytes,
                     p.num_blocks);
  return hipGetLastError();
}

hipError_t launch_decode(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream) {
  switch (p.dtype) {
    case kF32: return launch_decode_f32(p, a, stream);
    case kF16: return launch_decode_f16(p, a, stream);
    case kBF16: return launch_decode_bf16(p, a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t decode_capacity(const PoolDesc& p, int32_t group, int32_t num_seqs, int32_t max_context_len,
                           DecodeCapacity* cap) {
  switch (p.dtype) {
    case kF32: return decode_capacity_f32(p, group, num_seqs, max_context_len, cap);
    case kF16: return decode_capacity_f16(p, group, num_seqs, max_context_len, cap);
    case kBF16: return decode_capacity_bf16(p, group, num_seqs, max_context_len, cap);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa

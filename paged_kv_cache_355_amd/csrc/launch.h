// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace pa {

enum DType : int32_t { kF32 = 0, kF16 = 1, kBF16 = 2 };

constexpr int32_t elem_bytes(int32_t dt) { return dt == kF32 ? 4 : 2; }

// Largest grid of the balanced decode kernel (its merge tree holds at most
// 16^3 records per unit, and a unit meets at most grid + 1 workgroups).
constexpr int32_t kMaxBalancedGrid = 4095;
// Levels of the balanced kernel's merge tree.
constexpr int32_t kMergeLevels = 3;
// Its merge counters: one int32 per slice boundary (0 … kMaxBalancedGrid) per
// level.  A unit cut by the slices owns the boundaries strictly inside it, so
// the counters of different units never meet, and their number does not
// depend on the batch.  Every plan that uses a workspace reserves this region
// at its front (zero-filled once; every balanced call leaves it zero) and puts
// its partial records after it, so calls of any split mode can share one
// workspace without writing over the counters.
constexpr int32_t kCounterSlots = kMaxBalancedGrid + 1;
constexpr int64_t kCounterBytes = int64_t{kMergeLevels} * kCounterSlots * 4;   // 48 KiB, a multiple of 256

// Waves per decode workgroup, and block ids a workgroup stages at a time.
constexpr int32_t kDecodeWaves = 4;
constexpr int32_t kTableBatch = 512;
// Fixed partitions of at most this many tokens are taken one per wave, four to
// a workgroup (DecodeArgs::wave_tokens).
constexpr int32_t kGroupedPartitionTokens = 512;

// Tokens per chunk of the decode inner loops: the 16-token matrix-core tile
// (16-bit K/V, blocks of ≥ 16 tokens, ≥ 4 query rows per kv-head), else four
// (one for blocks shorter than a load) wave-wide 16-byte loads of
// 64 / (head_dim · element bytes / 16) tokens each.  decode_impl.h checks that
// its loops use the same.
constexpr int32_t decode_chunk_tokens(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t group) {
  return (dtype != kF32 && block_size >= 16 && group >= 4)
             ? 16
             : (block_size < 64 / (head_dim * elem_bytes(dtype) / 16) ? 1 : 4) *
                   (64 / (head_dim * elem_bytes(dtype) / 16));
}

struct PoolDesc {
  int32_t num_blocks, block_size, kv_heads, head_dim, dtype;
  void* k;
  void* v;
  int64_t block_bytes;  // kv_heads * block_size * head_dim * elem (one tensor)
};

struct DecodeArgs {
  void* out;
  int32_t out_dtype;
  const void* q;
  int32_t num_seqs, q_heads;
  const int32_t* block_tables;
  int32_t table_stride;
  const int32_t* context_lens;
  int32_t max_context_len;
  float scale_log2;        // logit scale × log2(e)
  // Balanced split (balanced = true): one resident grid of `grid` workgroups
  // sharing the work evenly; partial records live in num_slots slots.
  bool balanced;
  int32_t grid;
  int32_t num_slots;       // num_seqs * kv_heads + grid
  int32_t* counters;       // [kMergeLevels][kCounterSlots], zero on entry and exit
  // Uniform split (uniform = true): `grid` workgroups, all resident at once;
  // the device picks one partition length that fits the batch's partitions
  // into them.  Partial records: [grid][group] rows; unit_desc[num_seqs ×
  // kv_heads][2] = (first task, partitions) of every unit.
  bool uniform = false;
  int32_t* unit_desc = nullptr;
  // Fixed partitions (balanced = false, uniform = false).
  int32_t partition_tokens;
  int32_t max_parts;       // partitions covering max_context_len
  // > 0: each partition of partition_tokens is kDecodeWaves consecutive runs
  // of wave_tokens tokens, one per wave of its workgroup (the caller's
  // partitions, merged in LDS before the record is written); 0: each wave
  // takes one contiguous quarter of the partition's chunks.
  int32_t wave_tokens = 0;
  // Partial records.  Fixed partitions: [num_seqs][q_heads][max_parts] rows;
  // balanced: [num_slots][group] rows; uniform: [grid][group] rows.
  float* part_ml;          // rows × (max, sum)
  float* part_o;           // rows × head_dim
  // Shared prefixes (fixed partitions only; all null/0 for plain decode):
  // group k is batch positions [group_start[k], group_start[k+1]) whose first
  // seq_prefix tokens sit in the same physical blocks.  max_parts then counts
  // the prefix's partitions plus the context's.
  const int32_t* group_start = nullptr;   // device [num_groups + 1]
  const int32_t* seq_prefix = nullptr;    // device [num_seqs]
  int32_t num_groups = 0;
  int32_t max_group_size = 0;
  int32_t max_prefix = 0;
  // pa_decode_append (whole sequences, fixed partitions or the uniform split):
  // the workgroup holding sequence s's last token first writes k_new/v_new
  // [num_seqs][kv_heads][head_dim] row s into slot kv_slots[s].  Null for a
  // plain decode.
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  const int32_t* kv_slots = nullptr;
};

// The library-held workspace of pa_decode_noalloc: one array of this many
// bytes per GPU (a file-scope device array in scratch.hip).
constexpr int64_t kScratchBytes = int64_t{16} << 20;

// Device address of that array on the current device, looked up once per
// device (hipGetSymbolAddress) and cached.
hipError_t scratch_buffer(void** ptr);
// Zero `bytes` (a multiple of 16) at p with a fill kernel on stream (no
// memset node, so the call can be captured into a graph).
hipError_t launch_zero(void* p, int64_t bytes, hipStream_t stream);

// True when the shared-prefix kernels exist for this pool (16-bit K/V, blocks
// of at least 16 tokens: the matrix-core tile).
inline bool shared_prefix_supported(int32_t dtype, int32_t block_size) {
  return dtype != kF32 && block_size >= 16;
}

// True when the decode kernels are instantiated for these sizes.
bool decode_supported(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t group);

hipError_t launch_write_kv(const PoolDesc& p, const void* k_new, const void* v_new, const int32_t* slots,
                           int32_t n, hipStream_t stream);
hipError_t launch_copy_blocks(const PoolDesc& p, const int32_t* pairs, int32_t n, hipStream_t stream);
// host_dev: the device address of pinned host memory of n × 2 × block_bytes.
hipError_t launch_swap_blocks(const PoolDesc& p, const int32_t* blocks, int32_t n, void* host_dev, bool out,
                              hipStream_t stream);
hipError_t launch_decode(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream);

// Workgroups the current device holds at once, per decode kernel.
struct DecodeCapacity {
  int32_t balanced_grid;   // the balanced kernel's grid for these sizes (PA_DECODE_GRID overrides)
  int32_t partition;       // fixed-partition workgroups resident at once
  int32_t uniform;         // uniform-split workgroups resident at once
};
hipError_t decode_capacity(const PoolDesc& p, int32_t group, int32_t num_seqs, int32_t max_context_len,
                           DecodeCapacity* cap);

// Per-dtype decode launchers and grid queries (decode_<dtype>.hip).
hipError_t launch_decode_f32(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_f16(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_bf16(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream);
hipError_t decode_capacity_f32(const PoolDesc& p, int32_t group, int32_t num_seqs, int32_t max_ctx,
                               DecodeCapacity* cap);
hipError_t decode_capacity_f16(const PoolDesc& p, int32_t group, int32_t num_seqs, int32_t max_ctx,
                               DecodeCapacity* cap);
hipError_t decode_capacity_bf16(const PoolDesc& p, int32_t group, int32_t num_seqs, int32_t max_ctx,
                               DecodeCapacity* cap);

}  // namespace pa

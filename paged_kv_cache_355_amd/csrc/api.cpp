// C ABI of libpa.so (declared in include/pa.h): argument validation, pool
// ownership, decode planning and kernel launches, and the block-manager
// wrappers.  Host code only; the kernels live in the .hip files.
#include "pa.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "block_manager.h"
#include "launch.h"

struct pa_pool {
  pa::PoolDesc d;
  bool owns;
};

struct pa_bm {
  explicit pa_bm(int32_t nb, int32_t bs, const std::vector<int32_t>& order) : impl(nb, bs, order) {}
  pa::BlockManager impl;
};

namespace {

thread_local std::string g_last_error;

pa_status fail(pa_status code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

pa_status hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Read on every device call so a process can switch it per call.
bool debug_validate() {
  const char* v = std::getenv("PA_DEBUG_VALIDATE");
  return v && *v && std::strcmp(v, "0") != 0;
}

int32_t env_int(const char* name, int32_t dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return static_cast<int32_t>(std::strtol(v, nullptr, 10));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool supported_block_size(int32_t bs) { return bs == 4 || bs == 8 || bs == 16 || bs == 32 || bs == 64; }

pa_status map_bm(pa::BmResult r, const std::string& why) {
  switch (r) {
    case pa::BmResult::ok: return PA_OK;
    case pa::BmResult::invalid: return fail(PA_ERR_INVALID, why);
    case pa::BmResult::no_blocks: return fail(PA_ERR_NO_BLOCKS, why);
    case pa::BmResult::not_found: return fail(PA_ERR_NOT_FOUND, why);
    case pa::BmResult::exists: return fail(PA_ERR_EXISTS, why);
  }
  return fail(PA_ERR_INVALID, why);
}

// Copy n int32 from device to host on `stream` and wait (debug validation only).
pa_status fetch_ints(const int32_t* dev, int64_t n, std::vector<int32_t>* host, hipStream_t stream) {
  host->resize(static_cast<size_t>(n));
  if (n == 0) return PA_OK;
  hipError_t e = hipMemcpyAsync(host->data(), dev, static_cast<size_t>(n) * sizeof(int32_t), hipMemcpyDeviceToHost,
                                stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "PA_DEBUG_VALIDATE copy");
  return PA_OK;
}

// How pa_decode splits the work for these sizes, and where its workspace
// pieces sit.  Every plan that keeps partial results reserves the balanced
// split's merge counters at the front of the workspace (kCounterBytes, used
// only by that split) and lays its records out after them, so no split mode
// writes where another one counts.
struct DecodePlan {
  bool balanced = false;
  bool uniform = false;          // uniform split: `grid` workgroups, unit descriptors at desc_off
  int64_t desc_off = 0;
  int32_t partition_tokens = 0;  // fixed partitions: tokens per workgroup
  int32_t wave_tokens = 0;       // > 0: the caller's partition length, one partition per wave
  int32_t max_parts = 1;
  int32_t grid = 0;              // balanced split
  int32_t num_slots = 0;
  int64_t ml_off = 0, o_off = 0, bytes = 0;
};

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

// Record layout after the counter region: (max, sum) rows, then output rows.
void layout_records(DecodePlan* plan, int64_t rows, int32_t head_dim) {
  plan->ml_off = pa::kCounterBytes;
  plan->o_off = plan->ml_off + round256(rows * 2 * 4);
  plan->bytes = plan->o_off + rows * head_dim * 4;
}

// The kernels add a partition length to a partition's first token, and round
// lengths up to whole blocks, in int32: the planners keep every token count
// they accept at most 2^30.
constexpr int32_t kMaxDecodeTokens = int32_t{1} << 30;

pa_status check_token_counts(int32_t max_context_len, int32_t partition_tokens, int32_t max_prefix) {
  if (max_context_len > kMaxDecodeTokens || max_prefix > kMaxDecodeTokens)
    return fail(PA_ERR_INVALID, "max_context_len and max_prefix_tokens must be <= 2^30");
  if (partition_tokens > kMaxDecodeTokens) return fail(PA_ERR_INVALID, "partition_tokens must be <= 2^30");
  return PA_OK;
}

// How to split: an explicit positive partition length (a multiple of
// block_size), PA_PARTITION_BALANCED or PA_PARTITION_UNIFORM; for 0, the
// PA_PARTITION_TOKENS override, else whole sequences (one workgroup per
// (sequence, kv-head), in batch order) when the batch's units fill the
// device, else the uniform split.
pa_status plan_decode(const pa_pool* pool, int32_t num_seqs, int32_t q_heads, int32_t max_context_len,
                      int32_t requested, DecodePlan* plan) {
  const pa::PoolDesc& d = pool->d;
  if (requested < 0 && requested != PA_PARTITION_BALANCED && requested != PA_PARTITION_UNIFORM)
    return fail(PA_ERR_INVALID, "partition_tokens must be >= 0, PA_PARTITION_BALANCED or PA_PARTITION_UNIFORM");
  if (pa_status s = check_token_counts(max_context_len, requested, 0)) return s;
  *plan = DecodePlan{};
  if (q_heads % d.kv_heads != 0 || !pa::decode_supported(d.dtype, d.head_dim, d.block_size, q_heads / d.kv_heads))
    return fail(PA_ERR_UNSUPPORTED, "group size " + std::to_string(q_heads / d.kv_heads) +
                                        " (q_heads must be kv_heads x 1, 2, 4 or 8)");
  const int32_t group = q_heads / d.kv_heads;
  const int64_t units = static_cast<int64_t>(num_seqs) * d.kv_heads;
  int32_t p = requested > 0 ? requested : (requested == 0 ? env_int("PA_PARTITION_TOKENS", 0) : 0);
  if (pa_status s = check_token_counts(max_context_len, p, 0)) return s;
  pa::DecodeCapacity cap{};
  bool uniform = requested == PA_PARTITION_UNIFORM;
  if (p <= 0) {
    hipError_t e = pa::decode_capacity(d, group, num_seqs, max_context_len, &cap);
    if (e != hipSuccess) return hip_fail(e, "decode grid query");
    if (requested == 0) {
      if (units >= cap.partition)   // whole sequences keep every CU busy
        p = static_cast<int32_t>(ceil_div(std::max(max_context_len, 1), d.block_size) * d.block_size);
      else
        uniform = true;
    }
  }
  if (p > 0) {
    if (p % d.block_size != 0)
      return fail(PA_ERR_INVALID, "partition_tokens must be a positive multiple of block_size (" +
                                      std::to_string(d.block_size) + ")");
    plan->partition_tokens = p;
    plan->max_parts = static_cast<int32_t>(std::max<int64_t>(1, ceil_div(max_context_len, p)));
    // Short partitions are taken one per wave, kDecodeWaves consecutive ones
    // to a workgroup: each wave streams its partition as one run and the
    // workgroup merges their (max, sum, output) in LDS before it writes one
    // record, so the reduce kernel reads a quarter of the records.
    const int32_t ct = pa::decode_chunk_tokens(d.dtype, d.head_dim, d.block_size, group);
    if (plan->max_parts > 1 && p <= pa::kGroupedPartitionTokens && p % ct == 0 &&
        int64_t{pa::kDecodeWaves} * p <= int64_t{pa::kTableBatch} * d.block_size) {
      plan->wave_tokens = p;
      plan->partition_tokens = pa::kDecodeWaves * p;
      plan->max_parts =
          static_cast<int32_t>(std::max<int64_t>(1, ceil_div(max_context_len, plan->partition_tokens)));
    }
    if (plan->max_parts > 1) layout_records(plan, static_cast<int64_t>(num_seqs) * q_heads * plan->max_parts, d.head_dim);
    return PA_OK;
  }
  if (uniform) {
    // One resident grid (PA_DECODE_GRID overrides), at least one workgroup
    // per unit, at most one per block of every unit.
    int64_t W = cap.uniform;
    const int32_t forced = env_int("PA_DECODE_GRID", 0);
    if (forced > 0) W = forced;
    W = std::min<int64_t>(W, units * std::max<int64_t>(1, ceil_div(max_context_len, d.block_size)));
    W = std::max<int64_t>(W, units);
    if (W >= (int64_t{1} << 31)) return fail(PA_ERR_INVALID, "too many sequences x kv-heads");
    plan->uniform = true;
    plan->grid = static_cast<int32_t>(W);
    layout_records(plan, W * group, d.head_dim);
    plan->desc_off = round256(plan->bytes);
    plan->bytes = plan->desc_off + units * 2 * 4;
    return PA_OK;
  }
  const int32_t grid = cap.balanced_grid;
  plan->balanced = true;
  if (units * std::max<int64_t>(max_context_len, 1) >= (int64_t{1} << 40))
    return fail(PA_ERR_INVALID, "num_seqs * kv_heads * max_context_len must be < 2^40");
  if (units + grid >= (int64_t{1} << 31)) return fail(PA_ERR_INVALID, "too many sequences x kv-heads");
  plan->grid = grid;
  plan->num_slots = static_cast<int32_t>(units + grid);
  layout_records(plan, static_cast<int64_t>(plan->num_slots) * group, d.head_dim);
  return PA_OK;
}

// The shared-prefix call's split: fixed partitions always (its prefix pass
// and the suffix pass write partial records that decode_reduce_kernel
// merges).  partition_tokens > 0 is used as given; 0 picks whole contexts
// when the batch's (sequence, kv-head) units fill the device, else 512
// tokens.  max_parts = prefix partitions + context partitions.
pa_status plan_shared_prefix(const pa_pool* pool, int32_t num_seqs, int32_t q_heads, int32_t max_context_len,
                             int32_t max_prefix, int32_t requested, DecodePlan* plan) {
  const pa::PoolDesc& d = pool->d;
  if (requested < 0) return fail(PA_ERR_INVALID, "partition_tokens must be >= 0 for a shared-prefix decode");
  if (pa_status s = check_token_counts(max_context_len, requested, max_prefix)) return s;
  if (q_heads % d.kv_heads != 0 || !pa::decode_supported(d.dtype, d.head_dim, d.block_size, q_heads / d.kv_heads))
    return fail(PA_ERR_UNSUPPORTED, "group size " + std::to_string(q_heads / d.kv_heads) +
                                        " (q_heads must be kv_heads x 1, 2, 4 or 8)");
  *plan = DecodePlan{};
  int32_t p = requested;
  if (p == 0) {
    pa::DecodeCapacity cap{};
    hipError_t e = pa::decode_capacity(d, q_heads / d.kv_heads, num_seqs, max_context_len, &cap);
    if (e != hipSuccess) return hip_fail(e, "decode grid query");
    const int64_t units = static_cast<int64_t>(num_seqs) * d.kv_heads;
    p = units >= cap.partition
            ? static_cast<int32_t>(ceil_div(std::max(max_context_len, 1), d.block_size) * d.block_size)
            : 512;
  }
  if (p % d.block_size != 0)
    return fail(PA_ERR_INVALID, "partition_tokens must be a positive multiple of block_size (" +
                                    std::to_string(d.block_size) + ")");
  plan->partition_tokens = p;
  plan->max_parts = static_cast<int32_t>(std::max<int64_t>(1, ceil_div(max_prefix, p) + ceil_div(max_context_len, p)));
  layout_records(plan, static_cast<int64_t>(num_seqs) * q_heads * plan->max_parts, d.head_dim);
  return PA_OK;
}

// The arguments every decode launch shares; scale ≤ 0 selects 1/sqrt(head_dim).
pa::DecodeArgs decode_args(const pa::PoolDesc& d, void* out, pa_dtype out_dtype, const void* q, int32_t num_seqs,
                           int32_t q_heads, const int32_t* block_tables, int32_t stride, const int32_t* context_lens,
                           int32_t max_context_len, float scale) {
  pa::DecodeArgs a{};
  a.out = out;
  a.out_dtype = out_dtype;
  a.q = q;
  a.num_seqs = num_seqs;
  a.q_heads = q_heads;
  a.block_tables = block_tables;
  a.table_stride = stride;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  const double sc = scale > 0.f ? static_cast<double>(scale) : 1.0 / std::sqrt(static_cast<double>(d.head_dim));
  a.scale_log2 = static_cast<float>(sc * 1.4426950408889634);  // log2(e)
  return a;
}

// Host checks of pa_decode's device-resident indices (PA_DEBUG_VALIDATE).
pa_status validate_decode_indices(const pa::PoolDesc& d, int32_t num_seqs, const int32_t* block_tables,
                                  int32_t stride, const int32_t* context_lens, int32_t max_context_len,
                                  hipStream_t st, std::vector<int32_t>* lens, std::vector<int32_t>* tables) {
  if (pa_status s = fetch_ints(context_lens, num_seqs, lens, st)) return s;
  if (pa_status s = fetch_ints(block_tables, static_cast<int64_t>(num_seqs) * stride, tables, st)) return s;
  for (int32_t i = 0; i < num_seqs; ++i) {
    if ((*lens)[i] < 0 || (*lens)[i] > max_context_len)
      return fail(PA_ERR_INVALID, "context_lens[" + std::to_string(i) + "] outside [0, max_context_len]");
    const int64_t nblk = ceil_div((*lens)[i], d.block_size);
    for (int64_t j = 0; j < nblk; ++j) {
      const int32_t b = (*tables)[static_cast<size_t>(i) * stride + j];
      if (b < 0 || b >= d.num_blocks)
        return fail(PA_ERR_INVALID, "block_tables[" + std::to_string(i) + "][" + std::to_string(j) + "] = " +
                                        std::to_string(b) + " outside the pool");
    }
  }
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------------------
// pool
// ---------------------------------------------------------------------------
pa_status pa_alloc_pool(int32_t num_blocks, int32_t block_size, int32_t kv_heads, int32_t head_dim,
                        pa_dtype dtype, void* k_mem, void* v_mem, pa_pool** out) {
  if (!out) return fail(PA_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || kv_heads <= 0) return fail(PA_ERR_INVALID, "num_blocks and kv_heads must be positive");
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "dtype");
  if (!supported_block_size(block_size)) return fail(PA_ERR_UNSUPPORTED, "block_size must be 4, 8, 16, 32 or 64");
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t{1} << 31))
    return fail(PA_ERR_INVALID, "num_blocks * block_size must be < 2^31");
  if ((k_mem == nullptr) != (v_mem == nullptr)) return fail(PA_ERR_INVALID, "pass both k_mem and v_mem or neither");
  if (k_mem && (!aligned(k_mem, 256) || !aligned(v_mem, 256)))
    return fail(PA_ERR_INVALID, "pool memory must be 256-byte aligned");
  pa::PoolDesc d{};
  d.num_blocks = num_blocks;
  d.block_size = block_size;
  d.kv_heads = kv_heads;
  d.head_dim = head_dim;
  d.dtype = dtype;
  d.block_bytes = static_cast<int64_t>(kv_heads) * block_size * head_dim * pa::elem_bytes(dtype);
  bool owns = false;
  if (!k_mem) {
    const size_t bytes = static_cast<size_t>(d.block_bytes) * num_blocks;
    hipError_t e = hipMalloc(&d.k, bytes);
    if (e != hipSuccess) return fail(PA_ERR_NO_MEMORY, std::string("hipMalloc K: ") + hipGetErrorString(e));
    e = hipMalloc(&d.v, bytes);
    if (e != hipSuccess) {
      (void)hipFree(d.k);
      return fail(PA_ERR_NO_MEMORY, std::string("hipMalloc V: ") + hipGetErrorString(e));
    }
    owns = true;
  } else {
    d.k = k_mem;
    d.v = v_mem;
  }
  *out = new pa_pool{d, owns};
  return PA_OK;
}

void pa_free_pool(pa_pool* pool) {
  if (!pool) return;
  if (pool->owns) {
    (void)hipFree(pool->d.k);
    (void)hipFree(pool->d.v);
  }
  delete pool;
}

pa_status pa_pool_info(const pa_pool* pool, void** k, void** v, int64_t* block_bytes) {
  if (!pool) return fail(PA_ERR_INVALID, "pool is NULL");
  if (k) *k = pool->d.k;
  if (v) *v = pool->d.v;
  if (block_bytes) *block_bytes = pool->d.block_bytes;
  return PA_OK;
}

// ---------------------------------------------------------------------------
// KV write / block copy
// ---------------------------------------------------------------------------
pa_status pa_write_kv(pa_pool* pool, const void* k_new, const void* v_new, const int32_t* slot_mapping, int32_t n,
                      void* stream) {
  if (!pool) return fail(PA_ERR_INVALID, "pool is NULL");
  if (n < 0) return fail(PA_ERR_INVALID, "n must be >= 0");
  if (n == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping) return fail(PA_ERR_INVALID, "NULL pointer");
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(PA_ERR_INVALID, "k_new/v_new must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_validate()) {
    std::vector<int32_t> slots;
    if (pa_status s = fetch_ints(slot_mapping, n, &slots, st)) return s;
    const int64_t total = static_cast<int64_t>(pool->d.num_blocks) * pool->d.block_size;
    std::vector<char> seen(static_cast<size_t>(total), 0);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t sl = slots[i];
      if (sl < -1 || sl >= total) return fail(PA_ERR_INVALID, "slot " + std::to_string(sl) + " outside the pool");
      if (sl >= 0 && seen[sl]++) return fail(PA_ERR_INVALID, "slot " + std::to_string(sl) + " written twice");
    }
  }
  hipError_t e = pa::launch_write_kv(pool->d, k_new, v_new, slot_mapping, n, st);
  return e == hipSuccess ? PA_OK : hip_fail(e, "write_kv launch");
}

pa_status pa_copy_blocks(pa_pool* pool, const int32_t* pairs, int32_t n, void* stream) {
  if (!pool) return fail(PA_ERR_INVALID, "pool is NULL");
  if (n < 0) return fail(PA_ERR_INVALID, "n must be >= 0");
  if (n == 0) return PA_OK;
  if (!pairs) return fail(PA_ERR_INVALID, "pairs is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_validate()) {
    std::vector<int32_t> h;
    if (pa_status s = fetch_ints(pairs, 2 * static_cast<int64_t>(n), &h, st)) return s;
    std::vector<char> role(static_cast<size_t>(pool->d.num_blocks), 0);  // 1 = src, 2 = dst
    for (int32_t i = 0; i < n; ++i) {
      const int32_t a = h[2 * i], b = h[2 * i + 1];
      if (a < 0 || a >= pool->d.num_blocks || b < 0 || b >= pool->d.num_blocks)
        return fail(PA_ERR_INVALID, "copy pair outside the pool");
      role[a] = 1;
    }
    // every destination once, and never a block that any pair reads
    for (int32_t i = 0; i < n; ++i) {
      const int32_t b = h[2 * i + 1];
      if (role[b] != 0) return fail(PA_ERR_INVALID, "destination block repeats or is a source");
      role[b] = 2;
    }
  }
  hipError_t e = pa::launch_copy_blocks(pool->d, pairs, n, st);
  return e == hipSuccess ? PA_OK : hip_fail(e, "copy_blocks launch");
}

// Shared checks of pa_swap_out / pa_swap_in; *host_dev receives the device
// address of the pinned host buffer.
static pa_status swap_args(const pa_pool* pool, const int32_t* blocks, int32_t n, const void* host,
                           int64_t host_bytes, bool in, hipStream_t st, void** host_dev) {
  if (!pool) return fail(PA_ERR_INVALID, "pool is NULL");
  if (n < 0) return fail(PA_ERR_INVALID, "n must be >= 0");
  if (n == 0) return PA_OK;
  if (!blocks || !host) return fail(PA_ERR_INVALID, "NULL pointer");
  if (host_bytes < static_cast<int64_t>(n) * 2 * pool->d.block_bytes)
    return fail(PA_ERR_INVALID, "host buffer smaller than n x 2 x block_bytes");
  if (!aligned(host, 16)) return fail(PA_ERR_INVALID, "host buffer must be 16-byte aligned");
  // Two independent checks that the device may touch this memory: the
  // runtime knows it as page-locked host memory, and maps it for the device.
  hipPointerAttribute_t attr{};
  hipError_t e = hipPointerGetAttributes(&attr, host);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(PA_ERR_INVALID, "host buffer is not pinned host memory (hipHostMalloc or pin_memory=True)");
  }
  e = hipHostGetDevicePointer(host_dev, const_cast<void*>(host), 0);
  if (e != hipSuccess || !*host_dev) {
    (void)hipGetLastError();
    return fail(PA_ERR_INVALID, "host buffer is not mapped for the device");
  }
  if (debug_validate()) {
    std::vector<int32_t> h;
    if (pa_status s = fetch_ints(blocks, n, &h, st)) return s;
    std::vector<char> seen(static_cast<size_t>(pool->d.num_blocks), 0);
    for (int32_t i = 0; i < n; ++i) {
      if (h[i] < 0 || h[i] >= pool->d.num_blocks) return fail(PA_ERR_INVALID, "block outside the pool");
      if (in && seen[h[i]]++) return fail(PA_ERR_INVALID, "a block is swapped in twice");
    }
  }
  return PA_OK;
}

pa_status pa_swap_out(const pa_pool* pool, const int32_t* blocks, int32_t n, void* host, int64_t host_bytes,
                      void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* host_dev = nullptr;
  if (pa_status s = swap_args(pool, blocks, n, host, host_bytes, false, st, &host_dev)) return s;
  if (n == 0) return PA_OK;
  hipError_t e = pa::launch_swap_blocks(pool->d, blocks, n, host_dev, true, st);
  return e == hipSuccess ? PA_OK : hip_fail(e, "swap_out launch");
}

pa_status pa_swap_in(pa_pool* pool, const int32_t* blocks, int32_t n, const void* host, int64_t host_bytes,
                     void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* host_dev = nullptr;
  if (pa_status s = swap_args(pool, blocks, n, host, host_bytes, true, st, &host_dev)) return s;
  if (n == 0) return PA_OK;
  hipError_t e = pa::launch_swap_blocks(pool->d, blocks, n, host_dev, false, st);
  return e == hipSuccess ? PA_OK : hip_fail(e, "swap_in launch");
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------
pa_status pa_decode_partition_tokens(const pa_pool* pool, int32_t num_seqs, int32_t q_heads, int32_t max_context_len,
                                     int32_t partition_tokens, int32_t* resolved) {
  if (!pool || !resolved) return fail(PA_ERR_INVALID, "NULL pointer");
  if (num_seqs < 0 || q_heads <= 0 || q_heads % pool->d.kv_heads != 0 || max_context_len < 0)
    return fail(PA_ERR_INVALID, "bad sizes");
  DecodePlan plan;
  if (pa_status s = plan_decode(pool, num_seqs, q_heads, max_context_len, partition_tokens, &plan)) return s;
  *resolved = plan.balanced  ? PA_PARTITION_BALANCED
              : plan.uniform ? PA_PARTITION_UNIFORM
              : plan.wave_tokens > 0 ? plan.wave_tokens
                                     : plan.partition_tokens;
  return PA_OK;
}

pa_status pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs, int32_t q_heads, int32_t max_context_len,
                                    int32_t partition_tokens, int64_t* bytes) {
  if (!pool || !bytes) return fail(PA_ERR_INVALID, "NULL pointer");
  if (num_seqs < 0 || q_heads <= 0 || q_heads % pool->d.kv_heads != 0 || max_context_len < 0)
    return fail(PA_ERR_INVALID, "bad sizes");
  DecodePlan plan;
  if (num_seqs == 0) {
    *bytes = 0;
    return PA_OK;
  }
  if (pa_status s = plan_decode(pool, num_seqs, q_heads, max_context_len, partition_tokens, &plan)) return s;
  *bytes = plan.bytes;
  return PA_OK;
}

namespace {
// pa_decode, and pa_decode_append when k_new is not null (then v_new and
// slot_mapping are its KV write's arguments, checked by the caller).
pa_status decode_call(const pa_pool* pool, void* out, pa_dtype out_dtype, const void* q, int32_t num_seqs,
                      int32_t q_heads, const int32_t* block_tables, int32_t block_table_stride,
                      const int32_t* context_lens, int32_t max_context_len, float scale, int32_t partition_tokens,
                      void* workspace, int64_t workspace_bytes, const void* k_new, const void* v_new,
                      const int32_t* slot_mapping, void* stream) {
  if (!pool) return fail(PA_ERR_INVALID, "pool is NULL");
  if (num_seqs < 0 || num_seqs > 65535) return fail(PA_ERR_INVALID, "num_seqs must be in [0, 65535]");
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !block_tables || !context_lens) return fail(PA_ERR_INVALID, "NULL pointer");
  const pa::PoolDesc& d = pool->d;
  if (q_heads <= 0 || q_heads % d.kv_heads != 0)
    return fail(PA_ERR_INVALID, "q_heads must be a positive multiple of kv_heads");
  const int32_t group = q_heads / d.kv_heads;
  if (!pa::decode_supported(d.dtype, d.head_dim, d.block_size, group))
    return fail(PA_ERR_UNSUPPORTED, "group size " + std::to_string(group) + " (supported: 1, 2, 4, 8)");
  if (out_dtype != d.dtype && out_dtype != PA_F32)
    return fail(PA_ERR_UNSUPPORTED, "out_dtype must be the pool dtype or PA_F32");
  if (d.kv_heads > 65535 || q_heads > 65535) return fail(PA_ERR_INVALID, "kv_heads and q_heads must be <= 65535");
  if (max_context_len < 0) return fail(PA_ERR_INVALID, "max_context_len must be >= 0");
  if (block_table_stride < ceil_div(max_context_len, d.block_size))
    return fail(PA_ERR_INVALID, "block_table_stride shorter than ceil(max_context_len / block_size)");
  if (!aligned(q, 16)) return fail(PA_ERR_INVALID, "q must be 16-byte aligned");
  DecodePlan plan;
  if (pa_status s = plan_decode(pool, num_seqs, q_heads, max_context_len, partition_tokens, &plan)) return s;
  if (plan.bytes > 0 && (!workspace || workspace_bytes < plan.bytes || !aligned(workspace, 256)))
    return fail(PA_ERR_INVALID,
                "workspace must be 256-byte aligned and hold " + std::to_string(plan.bytes) + " bytes");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_validate()) {
    std::vector<int32_t> lens, tables;
    if (pa_status s = validate_decode_indices(d, num_seqs, block_tables, block_table_stride, context_lens,
                                              max_context_len, st, &lens, &tables))
      return s;
    if (k_new) {   // each live slot is the one that holds token len−1 of its sequence
      std::vector<int32_t> slots;
      if (pa_status s = fetch_ints(slot_mapping, num_seqs, &slots, st)) return s;
      for (int32_t i = 0; i < num_seqs; ++i) {
        const int32_t sl = slots[i], len = lens[i];
        if (sl < 0) continue;
        const int32_t want = len > 0 ? tables[static_cast<size_t>(i) * block_table_stride + (len - 1) / d.block_size] *
                                               d.block_size + (len - 1) % d.block_size
                                     : -2;
        if (sl != want)
          return fail(PA_ERR_INVALID, "slot_mapping[" + std::to_string(i) + "] = " + std::to_string(sl) +
                                          " is not the slot of token context_lens - 1");
      }
    }
    if (plan.balanced) {
      std::vector<int32_t> ctr;
      const int64_t n = pa::kCounterBytes / 4;
      if (pa_status s = fetch_ints(static_cast<const int32_t*>(workspace), n, &ctr, st)) return s;
      for (int64_t i = 0; i < n; ++i)
        if (ctr[static_cast<size_t>(i)] != 0)
          return fail(PA_ERR_INVALID, "workspace merge counters are not zero (zero-fill a new workspace once)");
    }
  }
  pa::DecodeArgs a = decode_args(d, out, out_dtype, q, num_seqs, q_heads, block_tables, block_table_stride,
                                 context_lens, max_context_len, scale);
  a.balanced = plan.balanced;
  a.uniform = plan.uniform;
  a.grid = plan.grid;
  a.num_slots = plan.num_slots;
  a.partition_tokens = plan.partition_tokens;
  a.wave_tokens = plan.wave_tokens;
  a.max_parts = plan.max_parts;
  if (plan.bytes > 0) {
    char* ws = static_cast<char*>(workspace);
    a.counters = plan.balanced ? reinterpret_cast<int32_t*>(ws) : nullptr;
    a.part_ml = reinterpret_cast<float*>(ws + plan.ml_off);
    a.part_o = reinterpret_cast<float*>(ws + plan.o_off);
    a.unit_desc = plan.uniform ? reinterpret_cast<int32_t*>(ws + plan.desc_off) : nullptr;
  }
  if (k_new) {
    if (plan.balanced) {   // its pieces have no single owner of the last token: write first
      hipError_t e = pa::launch_write_kv(d, k_new, v_new, slot_mapping, num_seqs, st);
      if (e != hipSuccess) return hip_fail(e, "write_kv launch");
    } else {
      a.k_new = k_new;
      a.v_new = v_new;
      a.kv_slots = slot_mapping;
    }
  }
  hipError_t e = pa::launch_decode(d, a, st);
  return e == hipSuccess ? PA_OK : hip_fail(e, "decode launch");
}
}  // namespace

pa_status pa_decode(const pa_pool* pool, void* out, pa_dtype out_dtype, const void* q, int32_t num_seqs,
                    int32_t q_heads, const int32_t* block_tables, int32_t block_table_stride,
                    const int32_t* context_lens, int32_t max_context_len, float scale, int32_t partition_tokens,
                    void* workspace, int64_t workspace_bytes, void* stream) {
  return decode_call(pool, out, out_dtype, q, num_seqs, q_heads, block_tables, block_table_stride, context_lens,
                     max_context_len, scale, partition_tokens, workspace, workspace_bytes, nullptr, nullptr, nullptr,
                     stream);
}

pa_status pa_decode_noalloc(const pa_pool* pool, void* out, pa_dtype out_dtype, const void* q, int32_t num_seqs,
                            int32_t q_heads, const int32_t* block_tables, int32_t block_table_stride,
                            const int32_t* context_lens, int32_t max_context_len, float scale,
                            int32_t partition_tokens, void* stream) {
  if (!pool) return fail(PA_ERR_INVALID, "pool is NULL");
  if (num_seqs < 0 || num_seqs > 65535) return fail(PA_ERR_INVALID, "num_seqs must be in [0, 65535]");
  if (num_seqs == 0) return PA_OK;
  if (q_heads <= 0 || q_heads % pool->d.kv_heads != 0)
    return fail(PA_ERR_INVALID, "q_heads must be a positive multiple of kv_heads");
  if (max_context_len < 0) return fail(PA_ERR_INVALID, "max_context_len must be >= 0");
  DecodePlan plan;
  if (pa_status s = plan_decode(pool, num_seqs, q_heads, max_context_len, partition_tokens, &plan)) return s;
  if (plan.bytes > pa::kScratchBytes)
    return fail(PA_ERR_INVALID, "this split keeps " + std::to_string(plan.bytes) +
                                    " bytes of partial results; pa_decode_noalloc holds " +
                                    std::to_string(pa::kScratchBytes) +
                                    " (pass pa_decode a workspace, or choose fewer partitions)");
  void* ws = nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (plan.bytes > 0) {
    hipError_t e = pa::scratch_buffer(&ws);
    if (e != hipSuccess) return hip_fail(e, "static workspace address");
    // the array keeps the previous call's contents: the balanced split's
    // merge counters must start at zero
    if (plan.balanced) {
      e = pa::launch_zero(ws, pa::kCounterBytes, st);
      if (e != hipSuccess) return hip_fail(e, "zero the merge counters");
    }
  }
  return decode_call(pool, out, out_dtype, q, num_seqs, q_heads, block_tables, block_table_stride, context_lens,
                     max_context_len, scale, partition_tokens, ws, ws ? pa::kScratchBytes : 0, nullptr, nullptr,
                     nullptr, stream);
}

pa_status pa_decode_append(pa_pool* pool, const void* k_new, const void* v_new, const int32_t* slot_mapping,
                           void* out, pa_dtype out_dtype, const void* q, int32_t num_seqs, int32_t q_heads,
                           const int32_t* block_tables, int32_t block_table_stride, const int32_t* context_lens,
                           int32_t max_context_len, float scale, int32_t partition_tokens, void* workspace,
                           int64_t workspace_bytes, void* stream) {
  if (!pool) return fail(PA_ERR_INVALID, "pool is NULL");
  if (num_seqs < 0 || num_seqs > 65535) return fail(PA_ERR_INVALID, "num_seqs must be in [0, 65535]");
  if (num_seqs == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping) return fail(PA_ERR_INVALID, "NULL pointer");
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(PA_ERR_INVALID, "k_new/v_new must be 16-byte aligned");
  if (debug_validate()) {   // pa_write_kv's own checks of the slots
    std::vector<int32_t> slots;
    if (pa_status s = fetch_ints(slot_mapping, num_seqs, &slots, static_cast<hipStream_t>(stream))) return s;
    const int64_t total = static_cast<int64_t>(pool->d.num_blocks) * pool->d.block_size;
    std::vector<char> seen(static_cast<size_t>(total), 0);
    for (int32_t i = 0; i < num_seqs; ++i) {
      const int32_t sl = slots[i];
      if (sl < -1 || sl >= total) return fail(PA_ERR_INVALID, "slot " + std::to_string(sl) + " outside the pool");
      if (sl >= 0 && seen[sl]++) return fail(PA_ERR_INVALID, "slot " + std::to_string(sl) + " written twice");
    }
  }
  return decode_call(pool, out, out_dtype, q, num_seqs, q_heads, block_tables, block_table_stride, context_lens,
                     max_context_len, scale, partition_tokens, workspace, workspace_bytes, k_new, v_new, slot_mapping,
                     stream);
}

pa_status pa_decode_shared_prefix_workspace_bytes(const pa_pool* pool, int32_t num_seqs, int32_t q_heads,
                                                  int32_t max_context_len, int32_t max_prefix_tokens,
                                                  int32_t partition_tokens, int64_t* bytes) {
  if (!pool || !bytes) return fail(PA_ERR_INVALID, "NULL pointer");
  if (num_seqs < 0 || q_heads <= 0 || q_heads % pool->d.kv_heads != 0 || max_context_len < 0 ||
      max_prefix_tokens < 0 || max_prefix_tokens > max_context_len)
    return fail(PA_ERR_INVALID, "bad sizes");
  *bytes = 0;
  if (num_seqs == 0) return PA_OK;
  if (!pa::shared_prefix_supported(pool->d.dtype, pool->d.block_size) || max_prefix_tokens == 0)
    return pa_decode_workspace_bytes(pool, num_seqs, q_heads, max_context_len, partition_tokens, bytes);
  DecodePlan plan;
  if (pa_status s = plan_shared_prefix(pool, num_seqs, q_heads, max_context_len, max_prefix_tokens, partition_tokens,
                                       &plan))
    return s;
  *bytes = plan.bytes;
  return PA_OK;
}

pa_status pa_decode_shared_prefix(const pa_pool* pool, void* out, pa_dtype out_dtype, const void* q,
                                  int32_t num_seqs, int32_t q_heads, const int32_t* block_tables,
                                  int32_t block_table_stride, const int32_t* context_lens, int32_t max_context_len,
                                  float scale, int32_t num_groups, const int32_t* group_start,
                                  const int32_t* prefix_tokens, int32_t max_group_size, int32_t max_prefix_tokens,
                                  int32_t partition_tokens, void* workspace, int64_t workspace_bytes,
                                  void* stream) {
  if (!pool) return fail(PA_ERR_INVALID, "pool is NULL");
  const pa::PoolDesc& d = pool->d;
  if (num_groups < 0 || num_groups > num_seqs || max_prefix_tokens < 0 || max_prefix_tokens > max_context_len ||
      max_group_size < 0 || max_group_size > std::max(num_seqs, 0))
    return fail(PA_ERR_INVALID, "bad group sizes");
  if (!pa::shared_prefix_supported(d.dtype, d.block_size) || max_prefix_tokens == 0)
    return pa_decode(pool, out, out_dtype, q, num_seqs, q_heads, block_tables, block_table_stride, context_lens,
                     max_context_len, scale, partition_tokens, workspace, workspace_bytes, stream);
  if (num_seqs < 0 || num_seqs > 65535) return fail(PA_ERR_INVALID, "num_seqs must be in [0, 65535]");
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !block_tables || !context_lens) return fail(PA_ERR_INVALID, "NULL pointer");
  if (num_groups > 0 && (!group_start || !prefix_tokens || max_group_size < 1))
    return fail(PA_ERR_INVALID, "group_start, prefix_tokens and max_group_size are needed with groups");
  if (q_heads <= 0 || q_heads % d.kv_heads != 0)
    return fail(PA_ERR_INVALID, "q_heads must be a positive multiple of kv_heads");
  const int32_t group = q_heads / d.kv_heads;
  if (out_dtype != d.dtype && out_dtype != PA_F32)
    return fail(PA_ERR_UNSUPPORTED, "out_dtype must be the pool dtype or PA_F32");
  if (d.kv_heads > 65535 || q_heads > 65535) return fail(PA_ERR_INVALID, "kv_heads and q_heads must be <= 65535");
  const int64_t tiles = ceil_div(std::max(max_group_size, 1), 16 / group);
  if (static_cast<int64_t>(d.kv_heads) * tiles > 65535)
    return fail(PA_ERR_INVALID, "kv_heads x member tiles must be <= 65535");
  if (block_table_stride < ceil_div(max_context_len, d.block_size))
    return fail(PA_ERR_INVALID, "block_table_stride shorter than ceil(max_context_len / block_size)");
  if (!aligned(q, 16)) return fail(PA_ERR_INVALID, "q must be 16-byte aligned");
  DecodePlan plan;
  if (pa_status s = plan_shared_prefix(pool, num_seqs, q_heads, max_context_len, max_prefix_tokens, partition_tokens,
                                       &plan))
    return s;
  if (!workspace || workspace_bytes < plan.bytes || !aligned(workspace, 256))
    return fail(PA_ERR_INVALID,
                "workspace must be 256-byte aligned and hold " + std::to_string(plan.bytes) + " bytes");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_validate()) {
    std::vector<int32_t> lens, tables, gs, pre;
    if (pa_status s = validate_decode_indices(d, num_seqs, block_tables, block_table_stride, context_lens,
                                              max_context_len, st, &lens, &tables))
      return s;
    if (num_groups > 0) {
      if (pa_status s = fetch_ints(group_start, num_groups + 1, &gs, st)) return s;
      if (pa_status s = fetch_ints(prefix_tokens, num_seqs, &pre, st)) return s;
      if (gs[0] != 0 || gs[num_groups] != num_seqs)
        return fail(PA_ERR_INVALID, "group_start must run from 0 to num_seqs");
      for (int32_t k = 0; k < num_groups; ++k) {
        const int32_t a = gs[k], b = gs[k + 1];
        if (b < a) return fail(PA_ERR_INVALID, "group_start must not decrease");
        if (b - a > max_group_size) return fail(PA_ERR_INVALID, "a group is larger than max_group_size");
        for (int32_t i = a; i < b; ++i) {
          const int32_t pi = pre[i];
          if (pi != pre[a]) return fail(PA_ERR_INVALID, "prefix_tokens differ inside group " + std::to_string(k));
          if (pi < 0 || pi % d.block_size != 0 || pi > lens[i] || pi > max_prefix_tokens)
            return fail(PA_ERR_INVALID, "prefix_tokens[" + std::to_string(i) +
                                            "] must be a multiple of block_size in [0, min(length, max_prefix)]");
          for (int32_t j = 0; j < pi / d.block_size; ++j)
            if (tables[static_cast<size_t>(i) * block_table_stride + j] !=
                tables[static_cast<size_t>(a) * block_table_stride + j])
              return fail(PA_ERR_INVALID, "sequence " + std::to_string(i) +
                                              " does not hold its group's prefix in the same blocks");
        }
      }
    }
  }
  pa::DecodeArgs a = decode_args(d, out, out_dtype, q, num_seqs, q_heads, block_tables, block_table_stride,
                                 context_lens, max_context_len, scale);
  a.partition_tokens = plan.partition_tokens;
  a.max_parts = plan.max_parts;
  char* ws = static_cast<char*>(workspace);
  a.part_ml = reinterpret_cast<float*>(ws + plan.ml_off);
  a.part_o = reinterpret_cast<float*>(ws + plan.o_off);
  if (num_groups > 0) {
    a.group_start = group_start;
    a.seq_prefix = prefix_tokens;
    a.num_groups = num_groups;
    a.max_group_size = max_group_size;
    a.max_prefix = max_prefix_tokens;
  }
  hipError_t e = pa::launch_decode(d, a, st);
  return e == hipSuccess ? PA_OK : hip_fail(e, "shared-prefix decode launch");
}

// ---------------------------------------------------------------------------
// block manager
// ---------------------------------------------------------------------------
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order, pa_bm** out) {
  if (!out) return fail(PA_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0) return fail(PA_ERR_INVALID, "num_blocks and block_size must be positive");
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t{1} << 31))
    return fail(PA_ERR_INVALID, "num_blocks * block_size must be < 2^31");
  std::vector<int32_t> order;
  if (initial_free_order) {
    if (!pa::BlockManager::is_permutation(initial_free_order, num_blocks))
      return fail(PA_ERR_INVALID, "initial_free_order is not a permutation of 0..num_blocks-1");
    order.assign(initial_free_order, initial_free_order + num_blocks);
  }
  try {
    *out = new pa_bm(num_blocks, block_size, order);
  } catch (...) {
    return fail(PA_ERR_NO_MEMORY, "block manager allocation");
  }
  return PA_OK;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq_id, int32_t num_tokens) {
  if (!bm) return fail(PA_ERR_INVALID, "bm is NULL");
  std::string why;
  return map_bm(bm->impl.add_seq(seq_id, num_tokens, &why), why);
}

pa_status pa_bm_fork(pa_bm* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return fail(PA_ERR_INVALID, "bm is NULL");
  std::string why;
  return map_bm(bm->impl.fork(parent_id, child_id, &why), why);
}

pa_status pa_bm_append_slot(pa_bm* bm, int64_t seq_id, int32_t* slot, int32_t* cow_src, int32_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return fail(PA_ERR_INVALID, "NULL pointer");
  std::string why;
  return map_bm(bm->impl.append_slot(seq_id, slot, cow_src, cow_dst, &why), why);
}

static void write_rows(const pa::BlockManager& m, const int64_t* ids, int32_t n, int32_t* tables, int32_t stride,
                       int32_t* lens) {
  for (int32_t i = 0; i < n; ++i) {
    int32_t len = 0;
    const std::vector<int32_t>* t = m.table(ids[i], &len);
    if (tables) {
      int32_t* row = tables + static_cast<int64_t>(i) * stride;
      const int32_t nb = static_cast<int32_t>(t->size());
      if (nb > 0) std::memcpy(row, t->data(), sizeof(int32_t) * nb);   // an empty table has no data()
      for (int32_t j = nb; j < stride; ++j) row[j] = -1;
    }
    if (lens) lens[i] = len;
  }
}

pa_status pa_bm_step(pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* slot_mapping, int32_t* cow_pairs,
                     int32_t* n_cow, int32_t* block_tables, int32_t stride, int32_t* context_lens) {
  if (!bm) return fail(PA_ERR_INVALID, "bm is NULL");
  if (n < 0 || (n > 0 && !seq_ids)) return fail(PA_ERR_INVALID, "bad batch");
  if (n_cow) *n_cow = 0;
  const int32_t bs = bm->impl.block_size();
  if (block_tables) {
    if (stride <= 0) return fail(PA_ERR_INVALID, "stride must be positive");
    for (int32_t i = 0; i < n; ++i) {
      int32_t len = 0;
      if (bm->impl.table(seq_ids[i], &len) && ceil_div(static_cast<int64_t>(len) + 1, bs) > stride)
        return fail(PA_ERR_INVALID, "stride shorter than sequence " + std::to_string(seq_ids[i]) + "'s table");
    }
  }
  std::vector<int32_t> pairs;
  std::string why;
  pa::BmResult r = bm->impl.step(seq_ids, n, slot_mapping, &pairs, &why);
  if (r != pa::BmResult::ok) return map_bm(r, why);
  if (cow_pairs && !pairs.empty()) std::memcpy(cow_pairs, pairs.data(), sizeof(int32_t) * pairs.size());
  if (n_cow) *n_cow = static_cast<int32_t>(pairs.size() / 2);
  write_rows(bm->impl, seq_ids, n, block_tables, stride, context_lens);
  return PA_OK;
}

pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq_id) {
  if (!bm) return fail(PA_ERR_INVALID, "bm is NULL");
  std::string why;
  return map_bm(bm->impl.free_seq(seq_id, &why), why);
}

pa_status pa_bm_block_table(const pa_bm* bm, int64_t seq_id, int32_t* out, int32_t cap, int32_t* n_blocks,
                            int32_t* n_tokens) {
  if (!bm) return fail(PA_ERR_INVALID, "bm is NULL");
  int32_t len = 0;
  const std::vector<int32_t>* t = bm->impl.table(seq_id, &len);
  if (!t) return fail(PA_ERR_NOT_FOUND, "unknown sequence " + std::to_string(seq_id));
  const int32_t nb = static_cast<int32_t>(t->size());
  if (n_blocks) *n_blocks = nb;
  if (n_tokens) *n_tokens = len;
  if (out) {
    if (cap < nb) return fail(PA_ERR_INVALID, "cap smaller than the table");
    if (nb > 0) std::memcpy(out, t->data(), sizeof(int32_t) * nb);
  }
  return PA_OK;
}

pa_status pa_bm_token_slots(const pa_bm* bm, int64_t seq_id, int32_t first, int32_t count, int32_t* out) {
  if (!bm || (count > 0 && !out)) return fail(PA_ERR_INVALID, "NULL pointer");
  int32_t len = 0;
  const std::vector<int32_t>* t = bm->impl.table(seq_id, &len);
  if (!t) return fail(PA_ERR_NOT_FOUND, "unknown sequence " + std::to_string(seq_id));
  if (first < 0 || count < 0 || static_cast<int64_t>(first) + count > len)
    return fail(PA_ERR_INVALID, "token range outside the sequence");
  const int32_t bs = bm->impl.block_size();
  for (int32_t i = 0; i < count; ++i) {
    const int32_t tok = first + i;
    out[i] = (*t)[tok / bs] * bs + tok % bs;
  }
  return PA_OK;
}

pa_status pa_bm_tables(const pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* block_tables, int32_t stride,
                       int32_t* context_lens) {
  if (!bm || n < 0 || (n > 0 && !seq_ids)) return fail(PA_ERR_INVALID, "bad arguments");
  for (int32_t i = 0; i < n; ++i) {
    const std::vector<int32_t>* t = bm->impl.table(seq_ids[i], nullptr);
    if (!t) return fail(PA_ERR_NOT_FOUND, "unknown sequence " + std::to_string(seq_ids[i]));
    if (block_tables && static_cast<int32_t>(t->size()) > stride)
      return fail(PA_ERR_INVALID, "stride shorter than sequence " + std::to_string(seq_ids[i]) + "'s table");
  }
  write_rows(bm->impl, seq_ids, n, block_tables, stride, context_lens);
  return PA_OK;
}

pa_status pa_bm_dispatch_order(const pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* order) {
  if (!bm || n < 0 || (n > 0 && (!seq_ids || !order))) return fail(PA_ERR_INVALID, "bad arguments");
  std::string why;
  return map_bm(bm->impl.dispatch_order(seq_ids, n, order, &why), why);
}

pa_status pa_bm_prefix_groups(const pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* group_start,
                              int32_t* prefix_tokens, int32_t* num_groups, int32_t* max_group_size) {
  if (!bm || n < 0 || !group_start || !num_groups || !max_group_size || (n > 0 && (!seq_ids || !prefix_tokens)))
    return fail(PA_ERR_INVALID, "bad arguments");
  std::string why;
  return map_bm(bm->impl.prefix_groups(seq_ids, n, group_start, prefix_tokens, num_groups, max_group_size, &why),
                why);
}

static pa_status bm_swap(pa_bm* bm, int64_t seq_id, int32_t* blocks, int32_t cap, int32_t* n_blocks, bool out) {
  if (!bm || !n_blocks || cap < 0 || (cap > 0 && !blocks)) return fail(PA_ERR_INVALID, "bad arguments");
  // the table length is known before anything changes, so a short buffer changes nothing
  int64_t need = 0;
  if (out) {
    const std::vector<int32_t>* t = bm->impl.table(seq_id, nullptr);
    if (!t) return fail(PA_ERR_NOT_FOUND, "unknown sequence " + std::to_string(seq_id));
    need = static_cast<int64_t>(t->size());
  } else {
    const int32_t len = bm->impl.swapped_length(seq_id);
    if (len < 0) return fail(PA_ERR_NOT_FOUND, "sequence " + std::to_string(seq_id) + " is not swapped out");
    need = ceil_div(len, bm->impl.block_size());
  }
  *n_blocks = static_cast<int32_t>(need);
  if (cap < need) return fail(PA_ERR_INVALID, "cap smaller than the block table");
  std::vector<int32_t> got;
  std::string why;
  const pa::BmResult r = out ? bm->impl.swap_out(seq_id, &got, &why) : bm->impl.swap_in(seq_id, &got, &why);
  if (r != pa::BmResult::ok) return map_bm(r, why);
  if (!got.empty()) std::memcpy(blocks, got.data(), sizeof(int32_t) * got.size());
  return PA_OK;
}

pa_status pa_bm_swap_out(pa_bm* bm, int64_t seq_id, int32_t* blocks, int32_t cap, int32_t* n_blocks) {
  return bm_swap(bm, seq_id, blocks, cap, n_blocks, true);
}

pa_status pa_bm_swap_in(pa_bm* bm, int64_t seq_id, int32_t* blocks, int32_t cap, int32_t* n_blocks) {
  return bm_swap(bm, seq_id, blocks, cap, n_blocks, false);
}

pa_status pa_bm_refcount(const pa_bm* bm, int32_t block, int32_t* rc) {
  if (!bm || !rc) return fail(PA_ERR_INVALID, "NULL pointer");
  if (block < 0 || block >= bm->impl.num_blocks()) return fail(PA_ERR_INVALID, "block outside the pool");
  *rc = bm->impl.refcount(block);
  return PA_OK;
}

pa_status pa_bm_free_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n) {
  if (!bm) return fail(PA_ERR_INVALID, "bm is NULL");
  const auto& fl = bm->impl.free_list();
  const int32_t cnt = static_cast<int32_t>(fl.size());
  if (n) *n = cnt;
  if (out) {
    if (cap < cnt) return fail(PA_ERR_INVALID, "cap smaller than the free list");
    int32_t i = 0;
    for (int32_t b : fl) out[i++] = b;
  }
  return PA_OK;
}

pa_status pa_bm_stats(const pa_bm* bm, pa_bm_stats_t* out) {
  if (!bm || !out) return fail(PA_ERR_INVALID, "NULL pointer");
  const pa::BmStats s = bm->impl.stats();
  out->num_blocks = s.num_blocks;
  out->block_size = s.block_size;
  out->free_blocks = s.free_blocks;
  out->used_blocks = s.used_blocks;
  out->shared_blocks = s.shared_blocks;
  out->num_seqs = s.num_seqs;
  out->logical_tokens = s.logical_tokens;
  out->logical_blocks = s.logical_blocks;
  out->filled_slots = s.filled_slots;
  out->cow_copies = s.cow_copies;
  out->swapped_seqs = s.swapped_seqs;
  out->reserved = 0;
  out->swapped_tokens = s.swapped_tokens;
  return PA_OK;
}

}  // extern "C"

namespace pa {
bool decode_supported(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t group) {
  return (dtype == kF32 || dtype == kF16 || dtype == kBF16) && (head_dim == 64 || head_dim == 128) &&
         supported_block_size(block_size) && (group == 1 || group == 2 || group == 4 || group == 8);
}
}  // namespace pa

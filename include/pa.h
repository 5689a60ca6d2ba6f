/*
 * pa.h — paged KV cache and paged decode attention for AMD Instinct MI355X
 * (gfx950).  The library is libpa.so; this header is its whole public
 * interface.
 *
 * What it computes (pages cited by title and section):
 *   [P1] "Paged Attention：大模型推理显存优化的核心方案" (learnblockchain.cn)
 *   [P2] "PagedAttention：操作系统级 KV 缓存虚拟内存管理" (freeguideonline.com)
 *   [P3] "PagedAttention 和 vLLM" (aiunderstanding.org)
 *
 *   - The KV cache is a pool of fixed-size blocks, each holding the K and V of
 *     block_size tokens; a sequence's blocks are scattered through the pool and
 *     found through its block table ([P1] "Paged Attention 的工作原理",
 *     "块表（Block Table）"; [P2] §2.1, §2.3).
 *   - A decode step appends the new token's K/V into its slot, opening a block
 *     when the last one is full, then attends over every cached token
 *     ([P2] §3.2.2).
 *   - Attention is softmax(q Kᵀ/√d) V ([P2] §1.1), one query row per head.
 *   - Free blocks live in a pool any request may draw from; finished requests
 *     return theirs ([P2] §3.3).  Shared blocks are refcounted and read-only;
 *     a write into one copies it first ([P2] §3.4; [P3] "技术洞察").
 *
 * Conventions
 *   - Every function returns pa_status: PA_OK (0) or a negative error code;
 *     pa_last_error() gives a message for the calling thread's last failure.
 *   - Device calls (pa_write_kv, pa_copy_blocks, pa_decode) validate their
 *     host-side arguments synchronously, enqueue kernels on `stream` (a
 *     hipStream_t; NULL = the default stream) and return without synchronising.
 *     Device pointers belong to the caller, who keeps them alive until the
 *     stream has passed the call.  The library keeps no caller pointer after
 *     a call returns (except a pool's caller-provided memory, see
 *     pa_alloc_pool).
 *   - Device-resident indices (block tables, context lengths, slot mappings,
 *     copy pairs) are not read on the host unless the environment variable
 *     PA_DEBUG_VALIDATE=1 is set; then each device call copies them to the
 *     host, synchronises the stream and rejects out-of-range or aliasing
 *     entries with PA_ERR_INVALID before launching anything.
 *   - Kernel faults are asynchronous and surface as PA_ERR_HIP from a later
 *     call that checks the stream.
 *   - Sizes and indices are int32_t; byte counts int64_t.
 *
 * Pool layout (device memory, one array each for K and V):
 *     [num_blocks][kv_heads][block_size][head_dim] elements of the pool dtype,
 *   so the tile of one (block, kv-head) is block_size*head_dim contiguous
 *   elements (the pages ask only that each block be contiguous inside, [P2]
 *   §4.2).  Slot s means (block s / block_size, offset s % block_size).
 */
#ifndef PA_H
#define PA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pa_status;
#define PA_OK               0
#define PA_ERR_INVALID     -1  /* bad size, pointer or index                   */
#define PA_ERR_UNSUPPORTED -2  /* dtype / head_dim / block_size / group size   */
#define PA_ERR_NO_BLOCKS   -3  /* free list cannot supply the blocks; no change */
#define PA_ERR_READ_ONLY   -4  /* write into a shared (refcount > 1) block      */
#define PA_ERR_NOT_FOUND   -5  /* unknown sequence id                           */
#define PA_ERR_EXISTS      -6  /* sequence id already present                   */
#define PA_ERR_HIP         -7  /* HIP runtime or kernel launch failure          */
#define PA_ERR_NO_MEMORY   -8  /* device or host allocation failed              */

typedef int32_t pa_dtype;
#define PA_F32  0
#define PA_F16  1
#define PA_BF16 2

typedef struct pa_pool pa_pool;
typedef struct pa_bm pa_bm;

/* Message for the calling thread's most recent error ("" if none). */
const char* pa_last_error(void);

/* ------------------------------------------------------------------------ */
/* KV block pool ([P1] "Paged Attention 的工作原理"; [P2] §2.1, §3.1, §4.2)   */
/* ------------------------------------------------------------------------ */

/* Describe (and optionally allocate) a pool of num_blocks blocks.
 *   block_size ∈ {4, 8, 16, 32, 64}; head_dim ∈ {64, 128};
 *   dtype ∈ {PA_F32, PA_F16, PA_BF16}; kv_heads ≥ 1;
 *   num_blocks * block_size < 2^31 (slots are int32).
 *   k_mem, v_mem: both NULL → the library allocates both arrays on the current
 *   HIP device and frees them in pa_free_pool; both non-NULL → caller-owned
 *   device memory of at least num_blocks * pa block bytes each, 256-byte
 *   aligned, which must outlive the pool.  Contents start undefined.
 * Errors: PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_NO_MEMORY. */
pa_status pa_alloc_pool(int32_t num_blocks, int32_t block_size, int32_t kv_heads,
                        int32_t head_dim, pa_dtype dtype, void* k_mem, void* v_mem,
                        pa_pool** out);

/* Release the descriptor (and the arrays if the library allocated them).
 * NULL is ignored.  Work already enqueued on the pool must have completed. */
void pa_free_pool(pa_pool* pool);

/* Device addresses of the K and V arrays and the bytes of one block of one of
 * them (kv_heads * block_size * head_dim * element size).  Any out pointer may
 * be NULL. */
pa_status pa_pool_info(const pa_pool* pool, void** k, void** v, int64_t* block_bytes);

/* ------------------------------------------------------------------------ */
/* Slot-mapped KV write — decode step 3 of [P2] §3.2.2, prefill of §3.2.1   */
/* ------------------------------------------------------------------------ */

/* For each row i < n with slot_mapping[i] ≥ 0, copy k_new[i] and v_new[i]
 * (each kv_heads*head_dim elements of the pool dtype) into that slot of every
 * kv-head's tile; rows with slot -1 are skipped.  Bit-exact byte copy.
 *   k_new, v_new: device [n][kv_heads][head_dim], contiguous, 16-byte aligned.
 *   slot_mapping: device int32[n]; live slots must be distinct and
 *   < num_blocks*block_size (checked only under PA_DEBUG_VALIDATE).
 * n = 0 is a no-op.  Errors: PA_ERR_INVALID, PA_ERR_HIP. */
pa_status pa_write_kv(pa_pool* pool, const void* k_new, const void* v_new,
                      const int32_t* slot_mapping, int32_t n, void* stream);

/* ------------------------------------------------------------------------ */
/* Copy-on-write block copy ([P2] §3.4)                                     */
/* ------------------------------------------------------------------------ */

/* For each of the n (src, dst) pairs, copy block src to block dst (K and V,
 * every kv-head, every slot).  Pairs act as if simultaneous.
 *   pairs: device int32[n][2]; destinations must be distinct and disjoint
 *   from sources, all in [0, num_blocks) (checked only under
 *   PA_DEBUG_VALIDATE).  Enqueue before the pa_write_kv that writes into the
 *   copies; stream order then makes the write land on the copied block.
 * n = 0 is a no-op.  Errors: PA_ERR_INVALID, PA_ERR_HIP. */
pa_status pa_copy_blocks(pa_pool* pool, const int32_t* pairs, int32_t n, void* stream);

/* ------------------------------------------------------------------------ */
/* Paged decode attention ([P2] §1.1, §3.2.2 step 4, §4.1, §4.2)            */
/* ------------------------------------------------------------------------ */

/* Bytes of device workspace pa_decode needs for these sizes (0 when no
 * partial results are kept): the partial (max, sum, output) records of the
 * tiled softmax's pieces before they are merged ([P2] §4.1), after the
 * balanced split's merge counters.  partition_tokens as for pa_decode.  The
 * automatic choice and the balanced split depend on the current device's CU
 * count and occupancy, so ask on the device that will decode.
 * Errors: PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_HIP. */
pa_status pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs, int32_t q_heads,
                                    int32_t max_context_len, int32_t partition_tokens,
                                    int64_t* bytes);

/* partition_tokens values that select the balanced and the uniform split
 * (see pa_decode). */
#define PA_PARTITION_BALANCED -1
#define PA_PARTITION_UNIFORM -2

/* How pa_decode will split these sizes into the pieces of [P2] §4.1's tiled
 * softmax, whose lengths differ per sequence ([P2] §4.3: a batch's sequences
 * need different numbers of blocks): the partition length in tokens (a
 * length ≥ max_context_len means one workgroup per (sequence, kv-head)),
 * PA_PARTITION_BALANCED or PA_PARTITION_UNIFORM.
 * Errors: PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_HIP. */
pa_status pa_decode_partition_tokens(const pa_pool* pool, int32_t num_seqs, int32_t q_heads,
                                     int32_t max_context_len, int32_t partition_tokens,
                                     int32_t* resolved);

/* Block swap between the pool and pinned host memory ([P2] §5, §8: blocks
 * of an inactive sequence move to CPU memory and back, as pages are swapped).
 *   blocks: device int32[n], pool block ids; ids outside the pool are skipped.
 *   host: pinned host memory the device can map (hipHostMalloc, or a torch
 *     tensor made with pin_memory=True), 16-byte aligned, host_bytes ≥
 *     n × 2 × block_bytes.  Layout [n][2][block_bytes]: block i's K tile (all
 *     kv-heads) then its V tile, each in the pool's [kv_heads][block_size]
 *     [head_dim] order.
 *   pa_swap_out copies pool → host, pa_swap_in host → pool (blocks distinct).
 *   One kernel moves the bytes straight between HBM and host memory over the
 *   host link: no staging buffer, no allocation.  Asynchronous on stream: the
 *   host reads swapped-out bytes after synchronising the stream, and keeps the
 *   buffer unchanged until a swap-in has completed.
 * Errors: PA_ERR_INVALID (bad pointer or size; host memory that is not
 * pinned and mapped), PA_ERR_HIP. */
pa_status pa_swap_out(const pa_pool* pool, const int32_t* blocks, int32_t n, void* host, int64_t host_bytes,
                      void* stream);
pa_status pa_swap_in(pa_pool* pool, const int32_t* blocks, int32_t n, const void* host, int64_t host_bytes,
                     void* stream);

/* out[s][h] = softmax(q[s][h] · K_sᵀ · scale) · V_s over the context_lens[s]
 * tokens of sequence s, whose token t lives at slot
 * block_tables[s*block_table_stride + t/block_size]*block_size + t%block_size.
 *   q: device [num_seqs][q_heads][head_dim] in the pool dtype.
 *   out: device [num_seqs][q_heads][head_dim] in out_dtype (the pool dtype or
 *     PA_F32); rounding to fp16/bf16 is round-to-nearest-even.
 *   q_heads must be a multiple of kv_heads with group q_heads/kv_heads ∈
 *     {1, 2, 4, 8}; query head h reads kv-head h / group.
 *   block_tables: device int32; row s holds ≥ ceil(context_lens[s]/block_size)
 *     valid block ids; block_table_stride ≥ ceil(max_context_len/block_size).
 *   context_lens: device int32[num_seqs], each in [0, max_context_len];
 *     a length of 0 gives a zero row.  Slots past the length are never used.
 *   max_context_len: host-known bound that sizes the launch, at most 2^30.
 *   scale: the logit scale; ≤ 0 selects 1/sqrt(head_dim).
 *   partition_tokens: how the context is split into work ([P2] §4.1's tiled
 *     softmax, merged with running max and sum):
 *       > 0 — fixed partitions of that many tokens (a multiple of
 *           block_size, at most 2^30), merged by a second reduce kernel
 *           when a sequence has more than one.  Partitions of at most 512
 *           tokens that hold whole chunks of the inner loop (16 tokens for
 *           16-bit K/V with a group of ≥ 4 and blocks of ≥ 16 tokens; 8 to
 *           32 on the vector loop) are taken one per wave, four consecutive
 *           ones to a workgroup, which merges them before it writes one
 *           partial result;
 *           longer ones take one workgroup each;
 *       PA_PARTITION_UNIFORM — one grid of workgroups, all resident at
 *           once; the device picks the shortest partition length (a
 *           multiple of block_size) whose partitions of every (sequence,
 *           kv-head) unit fit in that grid, numbers them densely and runs
 *           one per workgroup, so every XCD gets an equal count; units of
 *           more than one partition are merged by the reduce kernel;
 *       PA_PARTITION_BALANCED — one grid of workgroups, all resident at
 *           once, each taking an equal share of the batch's total KV; pieces
 *           of a sequence that straddle workgroups are merged inside the
 *           same kernel (no second launch);
 *       0 — automatic: PA_PARTITION_TOKENS if set and positive; else, when
 *           the batch has at least as many (sequence, kv-head) units as the
 *           device holds workgroups at once, one workgroup per unit with no
 *           split; else the uniform split.
 *     With fixed partitions (and in the automatic whole-sequence case)
 *     workgroups start in batch order, sequence 0 first; arrange the batch
 *     with pa_bm_dispatch_order to run long sequences first.  Results do not
 *     depend on the order.
 *   workspace: device memory of ≥ pa_decode_workspace_bytes(...) bytes,
 *     256-byte aligned; may be NULL when that is 0.  Its first 48 KiB
 *     (whenever the size is not 0) hold the balanced split's merge counters;
 *     partial results of every split mode follow them.  A new workspace must
 *     be zero-filled once before its first use (at least those 48 KiB); every
 *     call leaves the counters at zero again and no split mode writes them
 *     otherwise, so one workspace serves later calls on the same pool of any
 *     split mode and any sizes whose pa_decode_workspace_bytes (or
 *     pa_decode_shared_prefix_workspace_bytes) fits in it.  Calls that may
 *     run concurrently need separate workspaces.
 * A length above max_context_len, or a block id outside the pool, yields NaN
 * in that sequence's output rows instead of a memory access out of bounds.
 * Errors: PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_HIP. */
pa_status pa_decode(const pa_pool* pool, void* out, pa_dtype out_dtype, const void* q,
                    int32_t num_seqs, int32_t q_heads, const int32_t* block_tables,
                    int32_t block_table_stride, const int32_t* context_lens,
                    int32_t max_context_len, float scale, int32_t partition_tokens,
                    void* workspace, int64_t workspace_bytes, void* stream);

/* pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * arguments and the result are pa_decode's without the workspace: partial
 * results go to a device array that the library holds for each GPU it runs on
 * (16 MiB, kept until the process ends; its address is looked up on the first
 * call on a device).  Nothing is allocated, by this call or any other.
 *   - Splits whose partial results need more than 16 MiB (pa_decode_workspace
 *     _bytes above 16777216) are rejected with PA_ERR_INVALID before
 *     anything is enqueued.
 *   - Every call on a GPU shares that GPU's array and leaves its contents
 *     there.  Before a balanced split the call clears the merge counters with
 *     a fill kernel on `stream` (no memset).  Calls that may overlap on one
 *     GPU (other streams, other threads) race on the array: serialise them.
 * Errors: PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_HIP. */
pa_status pa_decode_noalloc(const pa_pool* pool, void* out, pa_dtype out_dtype, const void* q,
                            int32_t num_seqs, int32_t q_heads, const int32_t* block_tables,
                            int32_t block_table_stride, const int32_t* context_lens,
                            int32_t max_context_len, float scale, int32_t partition_tokens,
                            void* stream);

/* One decode step's KV write and attention in one launch ([P2] §3.2.2: step 3
 * writes the new token's K/V into its slot, step 4 attends over every cached
 * token, the new one included).  The result — pool contents and out — is that
 * of pa_write_kv(pool, k_new, v_new, slot_mapping, num_seqs) followed by
 * pa_decode(...) with the remaining arguments; the attention is bit-identical
 * to that pair of calls.
 *   k_new, v_new: device [num_seqs][kv_heads][head_dim] in the pool dtype,
 *     16-byte aligned: the new token of each sequence, one row per sequence.
 *   slot_mapping: device int32[num_seqs]; slot_mapping[s] is −1 (nothing to
 *     write: the token is already in the pool) or the slot of token
 *     context_lens[s] − 1, the sequence's last, which is what pa_bm_step
 *     returns.  Live slots are distinct.  A slot outside the pool is skipped.
 *   The remaining arguments are pa_decode's, with its workspace rules.
 * The workgroup that attends over the last token of (sequence, kv-head)
 * takes that token's K and V rows from k_new/v_new (staged in LDS with its
 * first block ids) in place of its slot, and stores them into the slot after
 * its token loop, so neither a second launch nor a wait for the store is
 * needed; the values are the same bytes, so the result is unchanged.  The
 * balanced split (PA_PARTITION_BALANCED) has no single owner of the last
 * token: there the library enqueues pa_write_kv's kernel before the decode.  A slot that is not the last token's gives undefined
 * rows (never an access outside the pool); PA_DEBUG_VALIDATE=1 checks the
 * slots against the tables and lengths on the host.
 * Errors: PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_HIP. */
pa_status pa_decode_append(pa_pool* pool, const void* k_new, const void* v_new, const int32_t* slot_mapping,
                           void* out, pa_dtype out_dtype, const void* q, int32_t num_seqs, int32_t q_heads,
                           const int32_t* block_tables, int32_t block_table_stride, const int32_t* context_lens,
                           int32_t max_context_len, float scale, int32_t partition_tokens, void* workspace,
                           int64_t workspace_bytes, void* stream);

/* Sharing-aware decode ([P2] §3.4 and [P1] "跨请求的内存共享": forked samples
 * and beams point their tables at the same physical blocks).  The result is
 * pa_decode's (within fp32 rounding order), for a batch arranged in groups
 * whose members hold their first tokens in the same blocks: each group's
 * prefix is read once per kv-head for all members (the members' query rows
 * share one matrix-core tile), each member's remaining tokens are read as
 * usual, and the two partial softmaxes are merged by running max and sum
 * ([P2] §4.1).
 *   Arguments up to scale are pa_decode's.
 *   num_groups ≥ 0; group_start: device int32[num_groups + 1], group k is
 *     batch positions [group_start[k], group_start[k+1]), from 0 to num_seqs.
 *   prefix_tokens: device int32[num_seqs]; for a member of group k the same
 *     value P_k, a multiple of block_size, ≤ every member's length and
 *     ≤ max_prefix_tokens, such that every member's first P_k / block_size
 *     table entries equal those of the group's first member (0: no prefix).
 *     pa_bm_prefix_groups computes groups and prefixes for a batch.
 *   max_group_size: host bound on group sizes; max_prefix_tokens: host bound
 *     on prefix_tokens (≤ max_context_len).
 *   partition_tokens: > 0 fixed partitions (a multiple of block_size) for
 *     prefixes and the rest; 0 = whole contexts when the batch fills the
 *     device, else 512.  PA_PARTITION_BALANCED is rejected.
 *   workspace: ≥ pa_decode_shared_prefix_workspace_bytes(...) bytes, 256-byte
 *     aligned, zero-filled once before first use, laid out and shareable as
 *     for pa_decode (the shared-prefix kernels write partial results after
 *     the counter region; the fallback below may take pa_decode's balanced
 *     split, which counts there).
 * Pools with fp32 K/V or blocks under 16 tokens, and max_prefix_tokens = 0,
 * take pa_decode itself (the grouping arguments are then ignored).  A
 * violated grouping contract gives wrong rows, never an out-of-bounds
 * access; PA_DEBUG_VALIDATE=1 checks it on the host.
 * Errors: PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_HIP. */
pa_status pa_decode_shared_prefix_workspace_bytes(const pa_pool* pool, int32_t num_seqs, int32_t q_heads,
                                                  int32_t max_context_len, int32_t max_prefix_tokens,
                                                  int32_t partition_tokens, int64_t* bytes);
pa_status pa_decode_shared_prefix(const pa_pool* pool, void* out, pa_dtype out_dtype, const void* q,
                                  int32_t num_seqs, int32_t q_heads, const int32_t* block_tables,
                                  int32_t block_table_stride, const int32_t* context_lens, int32_t max_context_len,
                                  float scale, int32_t num_groups, const int32_t* group_start,
                                  const int32_t* prefix_tokens, int32_t max_group_size, int32_t max_prefix_tokens,
                                  int32_t partition_tokens, void* workspace, int64_t workspace_bytes,
                                  void* stream);

/* ------------------------------------------------------------------------ */
/* Host block manager ([P2] §3.2, §3.3, §3.4; [P1] "跨请求的内存共享")        */
/* Pure host code: needs no GPU.  Not thread-safe per instance.              */
/* ------------------------------------------------------------------------ */
/* Policy (fixed so results are reproducible):
 *   - FIFO free list, initially initial_free_order (NULL = 0..num_blocks-1);
 *     allocation takes the head, release appends to the tail in table order.
 *   - Prefill of n tokens takes ceil(n/block_size) blocks ([P2] §3.2.1).
 *   - Append: if the length is a multiple of block_size a new block is
 *     appended; otherwise, if the last block's refcount is > 1, it is copied
 *     to a new block (a copy-on-write pair), the table entry is repointed and
 *     the old count drops by one.  Sequences in a batch are visited in order,
 *     so the last of k sharers writes in place ([P2] §3.2.2, §3.4).
 *   - A block is read-only while its refcount is > 1.
 *   - Calls that fail leave the manager unchanged. */

typedef struct pa_bm_stats_t {
  int32_t num_blocks, block_size;
  int32_t free_blocks;     /* blocks on the free list                        */
  int32_t used_blocks;     /* blocks with refcount > 0                       */
  int32_t shared_blocks;   /* blocks with refcount > 1                       */
  int32_t num_seqs;
  int64_t logical_tokens;  /* sum of sequence lengths                        */
  int64_t logical_blocks;  /* sum of block-table lengths                     */
  int64_t filled_slots;    /* slots of used blocks holding a token (unique)  */
  int64_t cow_copies;      /* copy-on-write pairs emitted so far             */
  int32_t swapped_seqs;    /* sequences swapped out (not in num_seqs)        */
  int32_t reserved;        /* 0                                              */
  int64_t swapped_tokens;  /* sum of their lengths                           */
} pa_bm_stats_t;

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size,
                       const int32_t* initial_free_order, pa_bm** out);
void pa_bm_destroy(pa_bm* bm);

/* Prefill allocation of num_tokens ≥ 0 tokens for a new sequence.
 * Errors: PA_ERR_EXISTS, PA_ERR_INVALID, PA_ERR_NO_BLOCKS. */
pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq_id, int32_t num_tokens);

/* child shares every block of parent (each refcount +1) and its length
 * ([P1] "跨请求的内存共享": parallel samples, beam branches).
 * Errors: PA_ERR_NOT_FOUND, PA_ERR_EXISTS. */
pa_status pa_bm_fork(pa_bm* bm, int64_t parent_id, int64_t child_id);

/* Append one token to one sequence.  *slot receives its slot; *cow_src and
 * *cow_dst receive the copy pair or -1.  Errors: PA_ERR_NOT_FOUND,
 * PA_ERR_NO_BLOCKS. */
pa_status pa_bm_append_slot(pa_bm* bm, int64_t seq_id, int32_t* slot, int32_t* cow_src,
                            int32_t* cow_dst);

/* Batched decode-step append for n distinct sequences, all or nothing.
 * Outputs (host memory, caller-owned, any may be NULL):
 *   slot_mapping int32[n]; cow_pairs int32[n][2] with *n_cow pairs filled in
 *   decision order; block_tables int32[n][stride] (rows padded with -1;
 *   PA_ERR_INVALID if a table is longer than stride); context_lens int32[n]
 *   (lengths after the append).
 * Errors: PA_ERR_INVALID (duplicate ids, bad stride), PA_ERR_NOT_FOUND,
 * PA_ERR_NO_BLOCKS. */
pa_status pa_bm_step(pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* slot_mapping,
                     int32_t* cow_pairs, int32_t* n_cow, int32_t* block_tables, int32_t stride,
                     int32_t* context_lens);

/* Release a sequence: refcounts drop; blocks reaching 0 rejoin the free list.
 * Errors: PA_ERR_NOT_FOUND. */
pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq_id);

/* Copy a sequence's block table (up to cap entries) into out; *n_blocks and
 * *n_tokens receive its table length and token count.  PA_ERR_INVALID if
 * cap is too small (n_blocks is still set).  Errors: PA_ERR_NOT_FOUND. */
pa_status pa_bm_block_table(const pa_bm* bm, int64_t seq_id, int32_t* out, int32_t cap,
                            int32_t* n_blocks, int32_t* n_tokens);

/* Slots of tokens [first, first+count) of a sequence (for a prefill
 * pa_write_kv).  Errors: PA_ERR_NOT_FOUND, PA_ERR_INVALID (range). */
pa_status pa_bm_token_slots(const pa_bm* bm, int64_t seq_id, int32_t first, int32_t count,
                            int32_t* out);

/* Rows of block tables and lengths for n sequences, as pa_bm_step writes
 * them, without appending. */
pa_status pa_bm_tables(const pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* block_tables,
                       int32_t stride, int32_t* context_lens);

/* Dispatch order for a decode batch of n sequences: order[k] (host int32[n],
 * caller-owned) receives the batch position to place k-th.  pa_decode starts
 * its workgroups in batch order, so a batch arranged this way runs the long
 * sequences first and lets the short ones fill the tail (longest processing
 * time first), and keeps sequences that share a prefix side by side so their
 * common blocks are read at about the same time ([P2] §3.4; [P1]
 * "跨请求的内存共享").  Sequences whose first block is the same physical
 * block form a group; groups are ordered by their longest member
 * (descending), then by their lowest position; members by length
 * (descending), then by position.  An empty sequence is a group of its own
 * with length 0.  With no sharing this is a stable sort by length, longest
 * first.  Duplicate ids are allowed (each position is placed once).
 * Errors: PA_ERR_INVALID, PA_ERR_NOT_FOUND. */
pa_status pa_bm_dispatch_order(const pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* order);

/* Prefix groups of a decode batch for pa_decode_shared_prefix.  Runs of
 * consecutive batch positions whose first block is the same physical block
 * form the groups (arrange the batch with pa_bm_dispatch_order first);
 * group_start (host int32[n + 1]) receives their starts and n, *num_groups
 * their count, *max_group_size the largest.  prefix_tokens (host int32[n])
 * receives, for each member, block_size × the number of leading table
 * entries all members of its group share, counting only blocks that are
 * full in every member; a group of one gets 0.
 * Errors: PA_ERR_INVALID, PA_ERR_NOT_FOUND. */
pa_status pa_bm_prefix_groups(const pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* group_start,
                              int32_t* prefix_tokens, int32_t* num_groups, int32_t* max_group_size);

/* Swap a sequence out ([P2] §5, §8: inactive blocks move to CPU memory, as
 * pages are swapped).  blocks (host int32, cap entries) receives its block
 * table in order — the source blocks for pa_swap_out — and *n_blocks its
 * length; each block's refcount then drops (blocks reaching 0 join the free
 * list in table order) and the sequence keeps only its length.  Until
 * pa_bm_swap_in every other call treats it as unknown, except pa_bm_free_seq.
 * The blocks may be handed out again at once: enqueue pa_swap_out on the
 * stream before any write that could reuse them.
 * Errors: PA_ERR_NOT_FOUND, PA_ERR_INVALID (cap too small; *n_blocks is set,
 * nothing changes). */
pa_status pa_bm_swap_out(pa_bm* bm, int64_t seq_id, int32_t* blocks, int32_t cap, int32_t* n_blocks);

/* Swap a sequence back in: it takes ⌈length / block_size⌉ blocks from the
 * free list (its new table, every block private with refcount 1; blocks it
 * shared before swap-out are not shared again), returned in table order in
 * blocks — the destinations for pa_swap_in.
 * Errors: PA_ERR_NOT_FOUND (not swapped out), PA_ERR_NO_BLOCKS (no change),
 * PA_ERR_INVALID (cap too small; *n_blocks is set, nothing changes). */
pa_status pa_bm_swap_in(pa_bm* bm, int64_t seq_id, int32_t* blocks, int32_t cap, int32_t* n_blocks);

/* The reference count of a physical block: the number of block tables that
 * map one of their entries to it ([P2] §3.4: shared blocks are counted, and
 * a block with a count above 1 is read-only; [P1] "跨请求的内存共享").
 * 0 for a free block.  Errors: PA_ERR_INVALID (NULL pointer, block outside
 * the pool). */
pa_status pa_bm_refcount(const pa_bm* bm, int32_t block, int32_t* rc);

/* Free-list contents from head to tail (up to cap entries); *n receives the
 * number of free blocks ([P2] §3.3: the manager keeps a list of free
 * physical blocks, finished requests return theirs to it, and any free block
 * may serve any request; the head is handed out next).  out may be NULL to
 * ask for the count.  Errors: PA_ERR_INVALID (cap smaller than the list;
 * *n is set). */
pa_status pa_bm_free_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n);

/* The manager's occupancy counters (pa_bm_stats_t above), from which the
 * pages' utilisation measures follow: slots holding a token over slots of the
 * blocks in use — waste only in each sequence's last, part-filled block
 * ([P1] "内存浪费的两种形式" and "Paged Attention 的工作原理": 2/4 of the
 * last block against 6/16 of a contiguous reservation; [P2] §3.3: above 99 %
 * utilisation) — and logical over physical blocks, the saving of blocks
 * shared by refcount ([P2] §3.4).  Errors: PA_ERR_INVALID (NULL pointer). */
pa_status pa_bm_stats(const pa_bm* bm, pa_bm_stats_t* out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */

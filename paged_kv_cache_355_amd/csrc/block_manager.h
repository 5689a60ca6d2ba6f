// Host block manager: free list, refcounts, fork, copy-on-write and slot
// assignment for the paged KV cache.  Pure C++ (no HIP), so it runs and is
// tested without a GPU.
//
// Pages: [P2] "PagedAttention：操作系统级 KV 缓存虚拟内存管理" §3.2.1 (prefill
// takes ⌈n/bs⌉ blocks, last part-filled), §3.2.2 (decode append: a full last
// block means a new block), §3.3 (one free pool, blocks recycled on release),
// §3.4 (refcounted sharing, read-only shared blocks, copy before write);
// [P1] "Paged Attention：大模型推理显存优化的核心方案", "跨请求的内存共享"
// (forked samples / beams share blocks).
#pragma once

#include <cstdint>
#include <deque>
#include <string>
#include <unordered_map>
#include <vector>

namespace pa {

enum class BmResult { ok, invalid, no_blocks, not_found, exists };

struct BmStats {
  int32_t num_blocks, block_size, free_blocks, used_blocks, shared_blocks, num_seqs;
  int64_t logical_tokens, logical_blocks, filled_slots, cow_copies;
  int32_t swapped_seqs, reserved;
  int64_t swapped_tokens;
};

class BlockManager {
 public:
  // initial_free_order: permutation of 0..num_blocks-1 (validated by caller
  // via is_permutation) or empty for the identity order.
  BlockManager(int32_t num_blocks, int32_t block_size, const std::vector<int32_t>& initial_free_order);

  static bool is_permutation(const int32_t* order, int32_t n);

  BmResult add_seq(int64_t id, int32_t num_tokens, std::string* why);
  BmResult fork(int64_t parent, int64_t child, std::string* why);
  BmResult append_slot(int64_t id, int32_t* slot, int32_t* cow_src, int32_t* cow_dst, std::string* why);
  // Batched append in batch order, all or nothing.  slots[n]; cow pairs are
  // appended to `pairs` as src, dst.
  BmResult step(const int64_t* ids, int32_t n, int32_t* slots, std::vector<int32_t>* pairs, std::string* why);
  // Dispatch order for a decode batch: order[k] is the batch position to run
  // k-th.  Sequences whose first block is the same physical block form a
  // group; groups go by their longest member (descending), then by their
  // lowest position; members by length (descending), then position.  Empty
  // sequences are singleton groups of length 0.  With no sharing this is a
  // stable sort by length, longest first.
  BmResult dispatch_order(const int64_t* ids, int32_t n, int32_t* order, std::string* why) const;
  // Prefix groups of a decode batch: runs of consecutive positions whose
  // first block is the same physical block.  group_start[num_groups + 1];
  // prefix_tokens[n] = block_size × the leading table entries every member of
  // the run holds in common, counting only blocks full in every member (0 for
  // a run of one).
  BmResult prefix_groups(const int64_t* ids, int32_t n, int32_t* group_start, int32_t* prefix_tokens,
                         int32_t* num_groups, int32_t* max_group_size, std::string* why) const;
  BmResult free_seq(int64_t id, std::string* why);
  // Swap a resident sequence out: *blocks receives its table (the blocks to
  // copy to host memory, in order), each block's refcount drops (blocks
  // reaching 0 join the free list in table order), and the sequence keeps
  // only its length until swap_in.  A swapped sequence is unknown to every
  // other call except free_seq.  cap < table length: invalid, no change.
  BmResult swap_out(int64_t id, std::vector<int32_t>* blocks, std::string* why);
  // Swap a sequence back in: it takes ⌈length / block_size⌉ blocks from the
  // free list (all private, refcount 1), returned in table order as the
  // destinations of the copy back.  Not enough free blocks: no change.
  BmResult swap_in(int64_t id, std::vector<int32_t>* blocks, std::string* why);
  // Length of a swapped-out sequence, or -1 if id is not swapped out.
  int32_t swapped_length(int64_t id) const {
    auto it = swapped_.find(id);
    return it == swapped_.end() ? -1 : it->second;
  }

  const std::vector<int32_t>* table(int64_t id, int32_t* length) const;
  int32_t refcount(int32_t block) const { return rc_[block]; }
  const std::deque<int32_t>& free_list() const { return free_; }
  BmStats stats() const;

  int32_t num_blocks() const { return num_blocks_; }
  int32_t block_size() const { return block_size_; }

 private:
  struct Seq {
    std::vector<int32_t> table;
    int32_t length = 0;
  };
  int32_t pop_free();
  void append_unchecked(Seq& s, int32_t* slot, int32_t* cow_src, int32_t* cow_dst);

  int32_t num_blocks_, block_size_;
  std::deque<int32_t> free_;
  std::vector<int32_t> rc_;
  std::unordered_map<int64_t, Seq> seqs_;
  std::unordered_map<int64_t, int32_t> swapped_;   // id -> length of swapped-out sequences
  int64_t cow_copies_ = 0;
  std::vector<int32_t> drop_scratch_;  // per-block refcount drops during a step's dry run
};

}  // namespace pa

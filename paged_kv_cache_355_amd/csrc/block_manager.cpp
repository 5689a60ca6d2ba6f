// Host block manager (see block_manager.h for the pages this follows).
#include "block_manager.h"

#include <algorithm>
#include <unordered_set>

namespace pa {

namespace {
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

BlockManager::BlockManager(int32_t num_blocks, int32_t block_size,
                           const std::vector<int32_t>& initial_free_order)
    : num_blocks_(num_blocks), block_size_(block_size), rc_(num_blocks, 0), drop_scratch_(num_blocks, 0) {
  if (initial_free_order.empty()) {
    for (int32_t b = 0; b < num_blocks; ++b) free_.push_back(b);
  } else {
    free_.assign(initial_free_order.begin(), initial_free_order.end());
  }
}

bool BlockManager::is_permutation(const int32_t* order, int32_t n) {
  std::vector<char> seen(n, 0);
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = order[i];
    if (b < 0 || b >= n || seen[b]) return false;
    seen[b] = 1;
  }
  return true;
}

int32_t BlockManager::pop_free() {
  int32_t b = free_.front();
  free_.pop_front();
  rc_[b] = 1;
  return b;
}

BmResult BlockManager::add_seq(int64_t id, int32_t num_tokens, std::string* why) {
  if (num_tokens < 0) {
    *why = "num_tokens must be >= 0";
    return BmResult::invalid;
  }
  if (seqs_.count(id) || swapped_.count(id)) {
    *why = "sequence " + std::to_string(id) + " already exists";
    return BmResult::exists;
  }
  int64_t need = ceil_div(num_tokens, block_size_);
  if (need > static_cast<int64_t>(free_.size())) {
    *why = "prefill needs " + std::to_string(need) + " blocks, " + std::to_string(free_.size()) + " free";
    return BmResult::no_blocks;
  }
  Seq s;
  s.table.reserve(need);
  for (int64_t j = 0; j < need; ++j) s.table.push_back(pop_free());
  s.length = num_tokens;
  seqs_.emplace(id, std::move(s));
  return BmResult::ok;
}

BmResult BlockManager::fork(int64_t parent, int64_t child, std::string* why) {
  auto it = seqs_.find(parent);
  if (it == seqs_.end()) {
    *why = "unknown parent " + std::to_string(parent);
    return BmResult::not_found;
  }
  if (seqs_.count(child) || swapped_.count(child)) {
    *why = "sequence " + std::to_string(child) + " already exists";
    return BmResult::exists;
  }
  Seq c = it->second;  // copy of table and length
  for (int32_t b : c.table) ++rc_[b];
  seqs_.emplace(child, std::move(c));
  return BmResult::ok;
}

// One append whose block needs were already checked against the free list.
void BlockManager::append_unchecked(Seq& s, int32_t* slot, int32_t* cow_src, int32_t* cow_dst) {
  const int32_t t = s.length;
  *cow_src = *cow_dst = -1;
  if (t % block_size_ == 0) {
    s.table.push_back(pop_free());
  } else {
    int32_t last = s.table.back();
    if (rc_[last] > 1) {  // shared, part-filled: copy before writing
      int32_t fresh = pop_free();
      --rc_[last];
      s.table.back() = fresh;
      *cow_src = last;
      *cow_dst = fresh;
      ++cow_copies_;
    }
  }
  *slot = s.table[t / block_size_] * block_size_ + t % block_size_;
  s.length = t + 1;
}

BmResult BlockManager::append_slot(int64_t id, int32_t* slot, int32_t* cow_src, int32_t* cow_dst,
                                   std::string* why) {
  auto it = seqs_.find(id);
  if (it == seqs_.end()) {
    *why = "unknown sequence " + std::to_string(id);
    return BmResult::not_found;
  }
  Seq& s = it->second;
  bool needs = (s.length % block_size_ == 0) || rc_[s.table.back()] > 1;
  if (needs && free_.empty()) {
    *why = "free list empty";
    return BmResult::no_blocks;
  }
  append_unchecked(s, slot, cow_src, cow_dst);
  return BmResult::ok;
}

BmResult BlockManager::step(const int64_t* ids, int32_t n, int32_t* slots, std::vector<int32_t>* pairs,
                            std::string* why) {
  std::vector<Seq*> batch;
  batch.reserve(n);
  {
    std::unordered_set<int64_t> seen;
    seen.reserve(static_cast<size_t>(n) * 2);
    for (int32_t i = 0; i < n; ++i) {
      if (!seen.insert(ids[i]).second) {
        *why = "sequence " + std::to_string(ids[i]) + " appears twice in one step";
        return BmResult::invalid;
      }
      auto it = seqs_.find(ids[i]);
      if (it == seqs_.end()) {
        *why = "unknown sequence " + std::to_string(ids[i]);
        return BmResult::not_found;
      }
      batch.push_back(&it->second);
    }
  }
  // Dry run: blocks this batch takes, counting refcount drops from copies
  // decided earlier in the same batch.
  int64_t need = 0;
  std::vector<int32_t> touched;
  for (Seq* s : batch) {
    if (s->length % block_size_ == 0) {
      ++need;
    } else {
      int32_t last = s->table.back();
      if (rc_[last] - drop_scratch_[last] > 1) {
        ++need;
        if (drop_scratch_[last]++ == 0) touched.push_back(last);
      }
    }
  }
  for (int32_t b : touched) drop_scratch_[b] = 0;
  if (need > static_cast<int64_t>(free_.size())) {
    *why = "step needs " + std::to_string(need) + " blocks, " + std::to_string(free_.size()) + " free";
    return BmResult::no_blocks;
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t slot, src, dst;
    append_unchecked(*batch[i], &slot, &src, &dst);
    if (slots) slots[i] = slot;
    if (src >= 0 && pairs) {
      pairs->push_back(src);
      pairs->push_back(dst);
    }
  }
  return BmResult::ok;
}

BmResult BlockManager::dispatch_order(const int64_t* ids, int32_t n, int32_t* order, std::string* why) const {
  struct Key {
    int32_t group_len, group_pos, len, pos;
  };
  struct Group {
    int32_t len, pos;
  };
  std::vector<Key> keys(n);
  std::vector<int32_t> first(n);
  std::unordered_map<int32_t, Group> groups;   // first block -> longest member, lowest position
  groups.reserve(static_cast<size_t>(n) * 2);
  for (int32_t i = 0; i < n; ++i) {
    auto it = seqs_.find(ids[i]);
    if (it == seqs_.end()) {
      *why = "unknown sequence " + std::to_string(ids[i]);
      return BmResult::not_found;
    }
    const Seq& s = it->second;
    first[i] = s.table.empty() ? -1 : s.table.front();
    keys[i] = {s.length, i, s.length, i};
    if (first[i] >= 0) {
      auto g = groups.emplace(first[i], Group{s.length, i});
      if (!g.second) g.first->second.len = std::max(g.first->second.len, s.length);
    }
  }
  for (int32_t i = 0; i < n; ++i) {
    if (first[i] >= 0) {
      const Group& g = groups[first[i]];
      keys[i].group_len = g.len;
      keys[i].group_pos = g.pos;
    }
  }
  std::sort(keys.begin(), keys.end(), [](const Key& a, const Key& b) {
    if (a.group_len != b.group_len) return a.group_len > b.group_len;
    if (a.group_pos != b.group_pos) return a.group_pos < b.group_pos;
    if (a.len != b.len) return a.len > b.len;
    return a.pos < b.pos;
  });
  for (int32_t k = 0; k < n; ++k) order[k] = keys[k].pos;
  return BmResult::ok;
}

BmResult BlockManager::prefix_groups(const int64_t* ids, int32_t n, int32_t* group_start, int32_t* prefix_tokens,
                                     int32_t* num_groups, int32_t* max_group_size, std::string* why) const {
  std::vector<const Seq*> batch(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = seqs_.find(ids[i]);
    if (it == seqs_.end()) {
      *why = "unknown sequence " + std::to_string(ids[i]);
      return BmResult::not_found;
    }
    batch[i] = &it->second;
  }
  int32_t groups = 0, largest = 0;
  for (int32_t a = 0; a < n;) {
    int32_t b = a + 1;
    if (!batch[a]->table.empty())
      while (b < n && !batch[b]->table.empty() && batch[b]->table.front() == batch[a]->table.front()) ++b;
    int64_t blocks = 0;
    if (b - a > 1) {
      blocks = static_cast<int64_t>(batch[a]->table.size());
      for (int32_t i = a; i < b; ++i) {
        const std::vector<int32_t>& t = batch[i]->table;
        blocks = std::min<int64_t>(blocks, batch[i]->length / block_size_);   // full blocks only
        int64_t j = 0;
        while (j < blocks && t[j] == batch[a]->table[j]) ++j;
        blocks = j;
      }
    }
    group_start[groups++] = a;
    for (int32_t i = a; i < b; ++i) prefix_tokens[i] = static_cast<int32_t>(blocks * block_size_);
    largest = std::max(largest, b - a);
    a = b;
  }
  group_start[groups] = n;
  *num_groups = groups;
  *max_group_size = largest;
  return BmResult::ok;
}

BmResult BlockManager::swap_out(int64_t id, std::vector<int32_t>* blocks, std::string* why) {
  auto it = seqs_.find(id);
  if (it == seqs_.end()) {
    *why = "unknown sequence " + std::to_string(id);
    return BmResult::not_found;
  }
  *blocks = it->second.table;
  for (int32_t b : it->second.table) {
    if (--rc_[b] == 0) free_.push_back(b);
  }
  swapped_[id] = it->second.length;
  seqs_.erase(it);
  return BmResult::ok;
}

BmResult BlockManager::swap_in(int64_t id, std::vector<int32_t>* blocks, std::string* why) {
  auto it = swapped_.find(id);
  if (it == swapped_.end()) {
    *why = "sequence " + std::to_string(id) + " is not swapped out";
    return BmResult::not_found;
  }
  const int64_t need = ceil_div(it->second, block_size_);
  if (need > static_cast<int64_t>(free_.size())) {
    *why = "swap-in needs " + std::to_string(need) + " blocks, " + std::to_string(free_.size()) + " free";
    return BmResult::no_blocks;
  }
  Seq s;
  s.length = it->second;
  s.table.reserve(need);
  for (int64_t j = 0; j < need; ++j) s.table.push_back(pop_free());
  *blocks = s.table;
  seqs_.emplace(id, std::move(s));
  swapped_.erase(it);
  return BmResult::ok;
}

BmResult BlockManager::free_seq(int64_t id, std::string* why) {
  if (swapped_.erase(id)) return BmResult::ok;   // its blocks were released at swap-out
  auto it = seqs_.find(id);
  if (it == seqs_.end()) {
    *why = "unknown sequence " + std::to_string(id);
    return BmResult::not_found;
  }
  for (int32_t b : it->second.table) {
    if (--rc_[b] == 0) free_.push_back(b);
  }
  seqs_.erase(it);
  return BmResult::ok;
}

const std::vector<int32_t>* BlockManager::table(int64_t id, int32_t* length) const {
  auto it = seqs_.find(id);
  if (it == seqs_.end()) return nullptr;
  if (length) *length = it->second.length;
  return &it->second.table;
}

BmStats BlockManager::stats() const {
  BmStats st{};
  st.num_blocks = num_blocks_;
  st.block_size = block_size_;
  st.free_blocks = static_cast<int32_t>(free_.size());
  std::vector<int32_t> fill(num_blocks_, 0);
  for (const auto& kv : seqs_) {
    const Seq& s = kv.second;
    st.logical_tokens += s.length;
    st.logical_blocks += static_cast<int64_t>(s.table.size());
    for (size_t j = 0; j < s.table.size(); ++j) {
      int64_t n = std::min<int64_t>(block_size_, s.length - static_cast<int64_t>(j) * block_size_);
      fill[s.table[j]] = std::max<int32_t>(fill[s.table[j]], static_cast<int32_t>(n));
    }
  }
  for (int32_t b = 0; b < num_blocks_; ++b) {
    if (rc_[b] > 0) {
      ++st.used_blocks;
      if (rc_[b] > 1) ++st.shared_blocks;
      st.filled_slots += fill[b];
    }
  }
  st.num_seqs = static_cast<int32_t>(seqs_.size());
  st.cow_copies = cow_copies_;
  st.swapped_seqs = static_cast<int32_t>(swapped_.size());
  for (const auto& kv : swapped_) st.swapped_tokens += kv.second;
  return st;
}

}  // namespace pa

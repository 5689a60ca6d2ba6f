// Randomised exercise of the host block manager, built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py (g++, no
// GPU).  After every operation it checks the invariants the paged cache
// relies on:
//   * a block's refcount equals the number of block tables holding it;
//   * the free list holds exactly the blocks with refcount 0, each once;
//   * every table has ceil(length / block_size) entries;
//   * the slots of one step are distinct and lie in their sequence's table;
//   * a copy-on-write pair copies the writer's old last block into a block
//     that was free, and calls that fail change nothing;
//   * a dispatch order is a permutation of the batch positions with groups
//     (same first block) contiguous and longest members never rising;
//   * swap-out returns the table and releases it; swap-in takes blocks from
//     the head of the free list, private, as many as the length needs, and a
//     failed swap-in changes nothing.
// Exit status 0 means every check held; a sanitizer report aborts.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <string>
#include <vector>

#include "block_manager.h"

using pa::BlockManager;
using pa::BmResult;

static int g_fail = 0;
#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c);  \
      ++g_fail;                                                           \
      if (g_fail > 20) std::exit(1);                                      \
    }                                                                     \
  } while (0)

struct Snapshot {
  std::vector<int32_t> rc, free_list;
  std::map<int64_t, std::pair<std::vector<int32_t>, int32_t>> tables;
};

static Snapshot snap(const BlockManager& bm, const std::set<int64_t>& ids) {
  Snapshot s;
  for (int32_t b = 0; b < bm.num_blocks(); ++b) s.rc.push_back(bm.refcount(b));
  s.free_list.assign(bm.free_list().begin(), bm.free_list().end());
  for (int64_t id : ids) {
    int32_t len = 0;
    const std::vector<int32_t>* t = bm.table(id, &len);
    if (t) s.tables[id] = {*t, len};
  }
  return s;
}

static bool same(const Snapshot& a, const Snapshot& b) {
  return a.rc == b.rc && a.free_list == b.free_list && a.tables == b.tables;
}

static void check_invariants(const BlockManager& bm, const std::set<int64_t>& ids) {
  const int32_t nb = bm.num_blocks(), bs = bm.block_size();
  std::vector<int32_t> owners(nb, 0);
  for (int64_t id : ids) {
    int32_t len = -1;
    const std::vector<int32_t>* t = bm.table(id, &len);
    CHECK(t != nullptr);
    if (!t) continue;
    CHECK(static_cast<int64_t>(t->size()) == (static_cast<int64_t>(len) + bs - 1) / bs);
    for (int32_t b : *t) {
      CHECK(b >= 0 && b < nb);
      if (b >= 0 && b < nb) ++owners[b];
    }
  }
  std::vector<int32_t> on_free(nb, 0);
  for (int32_t b : bm.free_list()) {
    CHECK(b >= 0 && b < nb);
    if (b >= 0 && b < nb) ++on_free[b];
  }
  for (int32_t b = 0; b < nb; ++b) {
    CHECK(bm.refcount(b) == owners[b]);
    CHECK(on_free[b] == (owners[b] == 0 ? 1 : 0));
  }
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
  std::mt19937_64 rng(12345);
  for (int round = 0; round < 4; ++round) {
    const int32_t bs = std::vector<int32_t>{1, 4, 16, 32}[round];
    const int32_t nb = 64 + round * 37;
    std::vector<int32_t> order(nb);
    for (int32_t i = 0; i < nb; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    BlockManager bm(nb, bs, order);
    std::set<int64_t> ids;
    std::map<int64_t, int32_t> swapped;   // id -> length
    int64_t next_id = 0;
    std::string why;
    for (int it = 0; it < iters; ++it) {
      const int op = static_cast<int>(rng() % 100);
      const Snapshot before = snap(bm, ids);
      if (op < 20) {  // prefill a new sequence
        const int32_t n = static_cast<int32_t>(rng() % (3 * bs + 2));
        const BmResult r = bm.add_seq(next_id, n, &why);
        if (r == BmResult::ok) ids.insert(next_id++);
        else CHECK(r == BmResult::no_blocks && same(before, snap(bm, ids)));
      } else if (op < 30 && !ids.empty()) {  // fork
        auto p = ids.begin();
        std::advance(p, static_cast<long>(rng() % ids.size()));
        CHECK(bm.fork(*p, next_id, &why) == BmResult::ok);
        ids.insert(next_id++);
      } else if (op < 80 && !ids.empty()) {  // batched decode-step append
        std::vector<int64_t> batch(ids.begin(), ids.end());
        std::shuffle(batch.begin(), batch.end(), rng);
        batch.resize(1 + rng() % batch.size());
        std::vector<int32_t> slots(batch.size(), -7), pairs;
        const std::set<int32_t> free_before(bm.free_list().begin(), bm.free_list().end());
        std::map<int64_t, int32_t> last_before;
        for (int64_t id : batch) {
          int32_t len = 0;
          const std::vector<int32_t>* t = bm.table(id, &len);
          last_before[id] = t->empty() ? -1 : t->back();
        }
        const BmResult r = bm.step(batch.data(), static_cast<int32_t>(batch.size()), slots.data(), &pairs, &why);
        if (r == BmResult::ok) {
          std::vector<int32_t> order(batch.size(), -1);
          CHECK(bm.dispatch_order(batch.data(), static_cast<int32_t>(batch.size()), order.data(), &why) ==
                BmResult::ok);
          std::vector<int32_t> sorted_order(order);
          std::sort(sorted_order.begin(), sorted_order.end());
          for (size_t i = 0; i < batch.size(); ++i) CHECK(sorted_order[i] == static_cast<int32_t>(i));
          std::set<int32_t> done_groups;
          int32_t prev_group = -2, prev_max = 1 << 30;
          for (size_t k = 0; k < order.size(); ++k) {
            int32_t len = 0;
            const std::vector<int32_t>* t = bm.table(batch[order[k]], &len);
            const int32_t group = t->empty() ? -1 - order[k] : t->front();
            if (group != prev_group) {
              CHECK(done_groups.insert(group).second);   // a group appears in one run
              int32_t longest = 0;
              for (int64_t id : batch) {
                int32_t l2 = 0;
                const std::vector<int32_t>* t2 = bm.table(id, &l2);
                if (!t2->empty() && !t->empty() && t2->front() == group) longest = std::max(longest, l2);
              }
              if (t->empty()) longest = len;
              CHECK(longest <= prev_max);
              prev_max = longest;
              prev_group = group;
            }
          }
          std::set<int32_t> seen;
          for (size_t i = 0; i < batch.size(); ++i) {
            CHECK(seen.insert(slots[i]).second);
            int32_t len = 0;
            const std::vector<int32_t>* t = bm.table(batch[i], &len);
            const int32_t tok = len - 1;
            CHECK(slots[i] == (*t)[tok / bs] * bs + tok % bs);
          }
          for (size_t k = 0; k < pairs.size(); k += 2) {
            CHECK(free_before.count(pairs[k + 1]) == 1);   // destination was free
            bool from_a_writer = false;
            for (const auto& kv : last_before) from_a_writer = from_a_writer || kv.second == pairs[k];
            CHECK(from_a_writer);
          }
        } else {
          CHECK(r == BmResult::no_blocks && same(before, snap(bm, ids)));
        }
      } else if (op < 85) {  // errors leave the manager unchanged
        std::vector<int64_t> dup = {next_id + 5, next_id + 5};
        CHECK(bm.step(dup.data(), 2, nullptr, nullptr, &why) != BmResult::ok);
        CHECK(bm.fork(next_id + 9, next_id + 10, &why) == BmResult::not_found);
        CHECK(bm.free_seq(next_id + 11, &why) == BmResult::not_found);
        CHECK(same(before, snap(bm, ids)));
      } else if (op < 90 && !ids.empty()) {  // swap out
        auto p = ids.begin();
        std::advance(p, static_cast<long>(rng() % ids.size()));
        int32_t len = 0;
        const std::vector<int32_t> table = *bm.table(*p, &len);
        std::vector<int32_t> blocks;
        CHECK(bm.swap_out(*p, &blocks, &why) == BmResult::ok);
        CHECK(blocks == table && bm.table(*p, nullptr) == nullptr && bm.swapped_length(*p) == len);
        swapped[*p] = len;
        ids.erase(p);
      } else if (op < 95 && !swapped.empty()) {  // swap in
        auto p = swapped.begin();
        std::advance(p, static_cast<long>(rng() % swapped.size()));
        const std::vector<int32_t> free_before(bm.free_list().begin(), bm.free_list().end());
        std::vector<int32_t> blocks;
        const BmResult r = bm.swap_in(p->first, &blocks, &why);
        const size_t need = static_cast<size_t>((static_cast<int64_t>(p->second) + bs - 1) / bs);
        if (r == BmResult::ok) {
          CHECK(blocks.size() == need);
          CHECK(std::equal(blocks.begin(), blocks.end(), free_before.begin()));
          for (int32_t b : blocks) CHECK(bm.refcount(b) == 1);
          ids.insert(p->first);
          swapped.erase(p);
        } else {
          CHECK(r == BmResult::no_blocks && need > free_before.size() && same(before, snap(bm, ids)));
        }
      } else if (!ids.empty() || !swapped.empty()) {  // release (resident or swapped)
        if (!swapped.empty() && (ids.empty() || rng() % 4 == 0)) {
          auto p = swapped.begin();
          CHECK(bm.free_seq(p->first, &why) == BmResult::ok);
          swapped.erase(p);
        } else {
          auto p = ids.begin();
          std::advance(p, static_cast<long>(rng() % ids.size()));
          CHECK(bm.free_seq(*p, &why) == BmResult::ok);
          ids.erase(p);
        }
      }
      check_invariants(bm, ids);
    }
    const pa::BmStats st = bm.stats();
    CHECK(st.free_blocks + st.used_blocks == nb);
    CHECK(st.swapped_seqs == static_cast<int32_t>(swapped.size()));
  }
  std::printf("bm_fuzz: %d failed checks\n", g_fail);
  return g_fail == 0 ? 0 : 1;
}

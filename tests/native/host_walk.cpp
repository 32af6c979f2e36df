// Seeded walks over the library's host C++ (the continuous-batching scheduler
// with its prefix cache, and the per-step block allocator with sharing),
// built with g++ and the address and undefined-behaviour sanitizers against
// stand-ins for the device calls.  The walks check block conservation after
// every step (every block is free, listed by a table entry or held by the
// prefix cache, never free and used at once); the sanitizers check every
// access.  Exit status 0 = all walks passed.
#include <cstdint>
#include <cstdio>
#include <random>
#include <set>
#include <vector>

#include "../../include/pagedkv.h"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                    \
    }                                                              \
  } while (0)

static int sched_walk(unsigned seed, int slots, int layers, int budget, int num_blocks, int n_req) {
  std::mt19937 rng(seed);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  const int max_blocks = 24;
  pkv_sched* s = nullptr;
  CHECK(pkv_sched_create(&s, slots, layers, max_blocks, num_blocks, budget) == PKV_OK);
  std::vector<std::vector<int32_t>> systems(3);
  for (auto& v : systems) {
    v.resize(uni(20, 200));
    for (auto& t : v) t = uni(0, 999);
  }
  for (int i = 0; i < n_req; ++i) {
    std::vector<int32_t> toks(systems[uni(0, 2)]);
    toks.resize(uni(1, (int)toks.size()));
    for (int k = uni(0, 60); k > 0; --k) toks.push_back(uni(0, 999));
    const int new_tokens = uni(1, 8);
    if ((int)toks.size() + new_tokens - 1 > max_blocks * PKV_BLOCK_SIZE) continue;
    const int rc = uni(0, 5) ? pkv_sched_submit_tokens(s, i, toks.data(), (int)toks.size(), new_tokens)
                             : pkv_sched_submit(s, i, (int)toks.size(), new_tokens);
    CHECK(rc == PKV_OK || rc == PKV_ERR_CAPACITY);
  }
  std::vector<pkv_bf16*> dummy(layers, reinterpret_cast<pkv_bf16*>(16));
  for (int it_n = 0;; ++it_n) {
    CHECK(it_n < 100000);
    pkv_sched_iter it;
    CHECK(pkv_sched_next(s, &it) == PKV_OK);
    CHECK(it.n_tokens <= budget);
    int32_t bt_dummy[4], meta_dummy[4];
    CHECK(pkv_sched_run(s, &it, dummy.data(), dummy.data(), (const pkv_bf16* const*)dummy.data(), dummy.data(),
                        dummy[0], dummy[0], bt_dummy, meta_dummy, 32, 8, 64, reinterpret_cast<const float*>(16),
                        4096, 0.125f, dummy[0], 1 << 20, nullptr) == PKV_OK);
    pkv_sched_state st;
    CHECK(pkv_sched_info(s, &st) == PKV_OK);
    std::vector<char> seen(num_blocks, 0);
    for (int i = 0; i < st.n_free; ++i) {
      const int b = st.free_list[i];
      CHECK(b >= 0 && b < num_blocks && !seen[b]);
      seen[b] = 1;
    }
    std::set<int> used;
    for (int64_t e = 0; e < (int64_t)slots * layers * max_blocks; ++e)
      if (st.table[e] >= 0) used.insert(st.table[e]);
    for (int i = 0; i < st.n_cache_blocks; ++i) used.insert(st.cache_blocks[i]);
    for (int b : used) {
      CHECK(b >= 0 && b < num_blocks && !seen[b]);
      seen[b] = 1;
    }
    for (int b = 0; b < num_blocks; ++b) CHECK(seen[b]);
    if (it.n_tokens == 0 && it.n_patch == 0) break;
  }
  pkv_sched_state st;
  CHECK(pkv_sched_info(s, &st) == PKV_OK);
  CHECK(st.n_active == 0 && st.n_queued == 0 && st.n_free + st.n_cache_blocks == num_blocks);
  CHECK(pkv_sched_destroy(s) == PKV_OK);
  return 0;
}

static int blocks_walk(unsigned seed) {
  std::mt19937 rng(seed);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  const int slots = 6, max_blocks = 10, num_blocks = 48;
  std::vector<int32_t> bt(slots * max_blocks, -1), free_list(num_blocks), refcount(num_blocks, 0);
  for (int i = 0; i < num_blocks; ++i) free_list[i] = i;
  int n_free = num_blocks;
  std::vector<int> len(slots, 0);
  std::vector<int32_t> off(4 * max_blocks * slots), val(off.size()), cs(off.size()), cd(off.size());
  for (int step = 0; step < 3000; ++step) {
    const int op = uni(0, 9);
    const int sl = uni(0, slots - 1);
    int n_patch = 0, n_copy = 0;
    if (op == 0) {
      CHECK(pkv_blocks_release_shared(bt.data(), max_blocks, slots, max_blocks, sl, free_list.data(), &n_free,
                                      num_blocks, refcount.data(), num_blocks, off.data(), val.data(),
                                      &n_patch) == PKV_OK);
      len[sl] = 0;
    } else if (op == 1 && len[sl] == 0) {
      const int src = uni(0, slots - 1);
      if (src != sl && len[src] > 0) {
        const int n = uni(1, len[src]);
        if (pkv_blocks_share(bt.data(), max_blocks, slots, max_blocks, src, sl, n, refcount.data(), num_blocks,
                             off.data(), val.data(), &n_patch) == PKV_OK)
          len[sl] = n;
      }
    } else {
      std::vector<int32_t> sid, pos;
      for (int k = uni(1, 5); k > 0 && len[sl] + (int)pos.size() < max_blocks * PKV_BLOCK_SIZE; --k) {
        sid.push_back(sl);
        pos.push_back(len[sl] + (int)pos.size());
      }
      if (sid.empty()) continue;
      const int rc = pkv_blocks_assign_shared(bt.data(), max_blocks, slots, max_blocks, free_list.data(), &n_free,
                                              refcount.data(), num_blocks, sid.data(), pos.data(), (int)sid.size(),
                                              off.data(), val.data(), &n_patch, cs.data(), cd.data(), &n_copy);
      CHECK(rc == PKV_OK || rc == PKV_ERR_CAPACITY);
      if (rc == PKV_OK) len[sl] += (int)sid.size();
    }
    // counts equal the entries listing each block; free blocks are unlisted
    std::vector<int> cnt(num_blocks, 0);
    for (int32_t b : bt)
      if (b >= 0) ++cnt[b];
    for (int b = 0; b < num_blocks; ++b) CHECK(cnt[b] == refcount[b]);
    for (int i = 0; i < n_free; ++i) CHECK(refcount[free_list[i]] == 0);
    int used = 0;
    for (int b = 0; b < num_blocks; ++b) used += refcount[b] > 0;
    CHECK(used + n_free == num_blocks);
  }
  return 0;
}

int main() {
  int rc = 0;
  rc |= sched_walk(1, 4, 2, 48, 120, 60);
  rc |= sched_walk(2, 6, 1, 6, 40, 80);      // tight pool: evictions
  rc |= sched_walk(3, 3, 3, 300, 400, 40);
  for (unsigned seed = 10; seed < 14; ++seed) rc |= blocks_walk(seed);
  if (rc == 0) std::printf("host walks passed\n");
  return rc;
}

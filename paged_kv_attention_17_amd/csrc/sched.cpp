// Continuous batching on the host: a fixed set of sequence slots filled from a
// FIFO queue of requests, one iteration at a time under a token budget
// (pkv_sched_*), and the device half of an iteration (pkv_sched_run).
//
// Source: "An Inference Engine in 1,500 Lines of CUDA: The Map", section "The
// path of one inference": every buffer and the block pool are allocated once;
// prompts wait in a queue; a free slot takes the next prompt, which is
// prefilled; a decode step gives every active slot one token; a slot whose
// request is finished returns to the free set; the loop stops when no slot is
// active and the queue is empty.  The category page's mini-sglang chapter-3
// title adds the per-step token budget and chunked prefill: when several
// requests wait, the step takes only as many tokens as the budget allows and
// prefills a long prompt over several steps.
//
// Policy of one iteration (this library's reading where the pages are
// silent):
//   1. slots whose request produced its last token in the previous iteration
//      are released: their blocks go back to the free list, their table
//      entries to -1;
//   2. admission, first come first served: the head of the queue takes the
//      lowest free slot if the blocks it can ever need (every layer, prompt +
//      max_new_tokens - 1 cached tokens) are still unreserved; otherwise the
//      queue waits (no request overtakes the head, none is preempted);
//   3. decode rows: every request whose prompt is cached and that still owes
//      tokens caches its newest token (one row each; the budget is at least
//      the slot count, so they always fit), oldest admission first;
//   4. prefill chunks: what is left of the budget goes to requests whose
//      prompt is not yet cached, oldest admission first, each taking
//      min(uncached prompt tokens, budget left);
//   5. blocks leave the free list only when a token opens a 16-token chunk
//      (the pages' rule), from the request's reservation, so an admitted
//      request never runs out of blocks.
// A request's prompt yields its first new token in the iteration that caches
// the prompt's last chunk; every decode row yields one more; the request is
// finished after max_new_tokens tokens (the last one is never cached).
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/pagedkv.h"
#include "kv_policy.h"

namespace pkv {
// paging.hip: write (offset, value) pairs with distinct offsets through kernel arguments
int patch_distinct(int32_t* bt_dev, int64_t bt_elems, const int32_t* off, const int32_t* val, int n_patch,
                   void* stream);
}  // namespace pkv

namespace {

struct Request {
  int64_t id = -1;
  int prompt = 0;       // prompt tokens
  int max_new = 0;      // tokens to produce
  int cached = 0;       // tokens in the cache
  int produced = 0;     // tokens produced so far
  int reserved = 0;     // blocks reserved and not yet taken from the free list
  int64_t order = 0;    // admission order
  std::vector<int32_t> tokens;   // prompt token ids (empty: the request takes no part in prefix caching)
  std::vector<int> path;         // prefix-cache nodes its first table entries list, in block order
};

// A node of the prefix cache: one full 16-token block of some prompt, under
// the node of the block before it.  Its blocks (one per layer) hold the K/V of
// those tokens after exactly that prefix, so any request whose prompt starts
// with the same tokens can list them instead of prefilling them again.
struct Node {
  int parent = -1;
  int32_t key[PKV_BLOCK_SIZE];           // the block's token ids
  std::vector<int32_t> blocks;           // pool block per layer
  std::unordered_map<uint64_t, int> kids;  // key hash -> child
  int ref = 0;                           // active requests whose rows list it
  int64_t last_use = 0;
  bool live = false;
};

uint64_t key_hash(const int32_t* t) {
  uint64_t h = 1469598103934665603ull;   // FNV-1a over the 16 ids
  for (int i = 0; i < PKV_BLOCK_SIZE; ++i) {
    h ^= (uint32_t)t[i];
    h *= 1099511628211ull;
  }
  return h;
}

int blocks_needed(int tokens) { return (tokens + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE; }

}  // namespace

struct pkv_sched {
  int num_slots = 0, n_layers = 0, max_blocks = 0, num_blocks = 0, budget = 0;
  std::vector<int32_t> table;          // [slots][layers][max_blocks]
  std::vector<int32_t> free_list;      // popped from the end
  int n_free = 0;
  int reserved = 0;                    // sum of the active requests' reservations
  std::deque<Request> queue;
  std::vector<Request> slot;           // id == -1: free slot
  std::vector<char> finished;          // released at the start of the next iteration
  int64_t admissions = 0;

  // the iteration handed out by the last pkv_sched_next (valid until the next call)
  std::vector<int32_t> decode_slots, decode_lens, chunk_slots, chunk_start, cu_chunk, token_slots, token_pos,
      patch_off, patch_val;
  std::vector<int64_t> decode_ids, chunk_ids, done_ids, admitted_ids;
  std::vector<int32_t> admitted_slots, admitted_cached;

  // prefix cache: node 0 is the root (no blocks); evictable = live nodes with
  // no children that no active request lists, oldest use first
  std::vector<Node> nodes;
  std::vector<int> dead_nodes;
  std::set<std::pair<int64_t, int>> evictable;
  int64_t tick = 0;
  int cache_nodes = 0;                 // live nodes besides the root
  int64_t hit_tokens = 0;              // prompt tokens taken from the cache
  mutable std::vector<int32_t> cache_list;   // pkv_sched_info's list of the cache's blocks

  int64_t entry(int s, int l, int j) const { return ((int64_t)s * n_layers + l) * max_blocks + j; }
};

extern "C" int pkv_sched_create(pkv_sched** out, int num_slots, int n_layers, int max_blocks_per_seq, int num_blocks,
                                int token_budget) {
  if (!out) return PKV_ERR_NULL;
  *out = nullptr;
  if (num_slots <= 0 || n_layers <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || token_budget < num_slots)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)num_slots * n_layers * max_blocks_per_seq > INT32_MAX) return PKV_ERR_INVALID_ARG;
  pkv_sched* s = new pkv_sched;
  s->num_slots = num_slots;
  s->n_layers = n_layers;
  s->max_blocks = max_blocks_per_seq;
  s->num_blocks = num_blocks;
  s->budget = token_budget;
  s->table.assign((size_t)num_slots * n_layers * max_blocks_per_seq, -1);
  // numbered once, 0 .. num_blocks - 1, the lowest id popped first
  s->free_list.resize(num_blocks);
  for (int i = 0; i < num_blocks; ++i) s->free_list[i] = num_blocks - 1 - i;
  s->n_free = num_blocks;
  s->slot.resize(num_slots);
  s->finished.assign(num_slots, 0);
  s->nodes.resize(1);
  s->nodes[0].live = true;
  *out = s;
  return PKV_OK;
}

extern "C" int pkv_sched_destroy(pkv_sched* s) {
  delete s;
  return PKV_OK;
}

extern "C" int pkv_sched_submit_tokens(pkv_sched* s, int64_t request_id, const int32_t* prompt_tokens_host,
                                       int prompt_len, int max_new_tokens) {
  if (!s) return PKV_ERR_NULL;
  if (request_id < 0 || prompt_len <= 0 || max_new_tokens <= 0) return PKV_ERR_INVALID_ARG;
  const int64_t tokens = (int64_t)prompt_len + max_new_tokens - 1;
  if (tokens > (int64_t)s->max_blocks * PKV_BLOCK_SIZE) return PKV_ERR_CAPACITY;
  if ((int64_t)blocks_needed((int)tokens) * s->n_layers > s->num_blocks) return PKV_ERR_CAPACITY;
  Request r;
  r.id = request_id;
  r.prompt = prompt_len;
  r.max_new = max_new_tokens;
  if (prompt_tokens_host) r.tokens.assign(prompt_tokens_host, prompt_tokens_host + prompt_len);
  s->queue.push_back(std::move(r));
  return PKV_OK;
}

extern "C" int pkv_sched_submit(pkv_sched* s, int64_t request_id, int prompt_len, int max_new_tokens) {
  return pkv_sched_submit_tokens(s, request_id, nullptr, prompt_len, max_new_tokens);
}

namespace {

// Give the token at `pos` of slot `si` a block in every layer (from the
// request's reservation) and record the table changes.
void open_chunk(pkv_sched* s, int si, int pos) {
  Request& r = s->slot[si];
  const int j = pos / PKV_BLOCK_SIZE;
  for (int l = 0; l < s->n_layers; ++l) {
    const int64_t e = s->entry(si, l, j);
    if (s->table[e] != -1) continue;
    const int32_t blk = s->free_list[--s->n_free];
    s->table[e] = blk;
    --r.reserved;
    --s->reserved;
    s->patch_off.push_back((int32_t)e);
    s->patch_val.push_back(blk);
  }
}

// ---- prefix cache ----------------------------------------------------------

void touch(pkv_sched* s, int n) {
  Node& x = s->nodes[n];
  if (x.ref == 0 && x.kids.empty()) s->evictable.erase({x.last_use, n});
  x.last_use = ++s->tick;
  if (x.ref == 0 && x.kids.empty()) s->evictable.insert({x.last_use, n});
}

void add_ref(pkv_sched* s, int n, int d) {
  Node& x = s->nodes[n];
  if (x.ref == 0 && x.kids.empty()) s->evictable.erase({x.last_use, n});
  x.ref += d;
  if (x.ref == 0 && x.kids.empty()) s->evictable.insert({x.last_use, n});
}

// The child of `n` whose key is tokens t[0..16), or -1.
int find_child(const pkv_sched* s, int n, const int32_t* t) {
  const Node& x = s->nodes[n];
  auto it = x.kids.find(key_hash(t));
  if (it == x.kids.end()) return -1;
  const Node& c = s->nodes[it->second];
  return std::equal(t, t + PKV_BLOCK_SIZE, c.key) ? it->second : -1;
}

// Longest run of the prompt's full blocks in the cache, leaving at least one
// prompt token to prefill (its row gives the first new token).
std::vector<int> match(const pkv_sched* s, const Request& r) {
  std::vector<int> path;
  if (r.tokens.empty()) return path;
  int n = 0;
  for (int j = 0; (j + 1) * PKV_BLOCK_SIZE < r.prompt; ++j) {
    const int c = find_child(s, n, r.tokens.data() + j * PKV_BLOCK_SIZE);
    if (c < 0) break;
    path.push_back(c);
    n = c;
  }
  return path;
}

// Drop the least recently used evictable node; its blocks go back to the
// free list (no table lists them).
void evict_one(pkv_sched* s) {
  const int n = s->evictable.begin()->second;
  s->evictable.erase(s->evictable.begin());
  Node& x = s->nodes[n];
  for (int32_t b : x.blocks) s->free_list[s->n_free++] = b;
  Node& p = s->nodes[x.parent];
  p.kids.erase(key_hash(x.key));
  if (x.parent != 0 && p.ref == 0 && p.kids.empty()) s->evictable.insert({p.last_use, x.parent});
  x = Node();
  s->dead_nodes.push_back(n);
  --s->cache_nodes;
}

// The request in slot si has just cached its whole prompt: publish its full
// prompt blocks after the ones it already lists from the cache.  Stops at a
// block another request has published meanwhile (this row keeps its own copy).
void publish(pkv_sched* s, int si) {
  Request& r = s->slot[si];
  if (r.tokens.empty()) return;
  int parent = r.path.empty() ? 0 : r.path.back();
  for (int j = (int)r.path.size(); (j + 1) * PKV_BLOCK_SIZE <= r.prompt; ++j) {
    const int32_t* t = r.tokens.data() + j * PKV_BLOCK_SIZE;
    if (s->nodes[parent].kids.count(key_hash(t))) break;
    int n;
    if (!s->dead_nodes.empty()) {
      n = s->dead_nodes.back();
      s->dead_nodes.pop_back();
    } else {
      n = (int)s->nodes.size();
      s->nodes.emplace_back();
    }
    Node& x = s->nodes[n];
    x.live = true;
    x.parent = parent;
    std::copy(t, t + PKV_BLOCK_SIZE, x.key);
    x.blocks.resize(s->n_layers);
    for (int l = 0; l < s->n_layers; ++l) x.blocks[l] = s->table[s->entry(si, l, j)];
    x.ref = 1;
    x.last_use = ++s->tick;
    Node& p = s->nodes[parent];
    if (parent != 0 && p.ref == 0 && p.kids.empty()) s->evictable.erase({p.last_use, parent});
    p.kids[key_hash(t)] = n;
    r.path.push_back(n);
    ++s->cache_nodes;
    parent = n;
  }
}

void release(pkv_sched* s, int si) {
  Request& r = s->slot[si];
  const int shared = (int)r.path.size();       // entries listing cache blocks stay allocated
  for (int l = 0; l < s->n_layers; ++l)
    for (int j = 0; j < s->max_blocks; ++j) {
      const int64_t e = s->entry(si, l, j);
      if (s->table[e] == -1) continue;
      if (j >= shared) s->free_list[s->n_free++] = s->table[e];
      s->table[e] = -1;
      s->patch_off.push_back((int32_t)e);
      s->patch_val.push_back(-1);
    }
  for (int n : r.path) {
    touch(s, n);
    add_ref(s, n, -1);
  }
  s->reserved -= r.reserved;
  r = Request();
}

}  // namespace

extern "C" int pkv_sched_next(pkv_sched* s, pkv_sched_iter* it) {
  if (!s || !it) return PKV_ERR_NULL;
  for (auto* v : {&s->decode_slots, &s->decode_lens, &s->chunk_slots, &s->chunk_start, &s->cu_chunk,
                  &s->token_slots, &s->token_pos, &s->patch_off, &s->patch_val, &s->admitted_slots})
    v->clear();
  s->decode_ids.clear();
  s->chunk_ids.clear();
  s->done_ids.clear();
  s->admitted_ids.clear();
  s->admitted_cached.clear();

  // 1. release the slots finished last time
  for (int si = 0; si < s->num_slots; ++si)
    if (s->finished[si]) {
      release(s, si);
      s->finished[si] = 0;
    }
  // 2. admission (first come first served, no overtaking): the prompt's
  // longest cached prefix is listed, not prefilled; cache blocks nobody lists
  // are evicted (least recently used first) when the free list is short
  while (!s->queue.empty()) {
    const Request& h = s->queue.front();
    int si = 0;
    while (si < s->num_slots && s->slot[si].id >= 0) ++si;
    if (si == s->num_slots) break;
    std::vector<int> path = match(s, h);
    const int need = (blocks_needed(h.prompt + h.max_new - 1) - (int)path.size()) * s->n_layers;
    for (int n : path) add_ref(s, n, 1);          // not evictable while admitting
    while (need > s->n_free - s->reserved && !s->evictable.empty()) evict_one(s);
    if (need > s->n_free - s->reserved) {
      for (int n : path) add_ref(s, n, -1);
      break;
    }
    Request r = std::move(s->queue.front());
    s->queue.pop_front();
    r.reserved = need;
    r.order = s->admissions++;
    r.path = std::move(path);
    r.cached = (int)r.path.size() * PKV_BLOCK_SIZE;
    s->hit_tokens += r.cached;
    for (int j = 0; j < (int)r.path.size(); ++j) {
      touch(s, r.path[j]);
      for (int l = 0; l < s->n_layers; ++l) {
        const int64_t e = s->entry(si, l, j);
        s->table[e] = s->nodes[r.path[j]].blocks[l];
        s->patch_off.push_back((int32_t)e);
        s->patch_val.push_back(s->table[e]);
      }
    }
    s->reserved += need;
    s->admitted_ids.push_back(r.id);
    s->admitted_slots.push_back(si);
    s->admitted_cached.push_back(r.cached);
    s->slot[si] = std::move(r);
  }
  // active slots by admission order
  std::vector<int> order;
  for (int si = 0; si < s->num_slots; ++si)
    if (s->slot[si].id >= 0) order.push_back(si);
  std::sort(order.begin(), order.end(), [&](int a, int b) { return s->slot[a].order < s->slot[b].order; });

  // 3. decode rows: the newest token of every request whose prompt is cached
  int left = s->budget;
  for (int si : order) {
    Request& r = s->slot[si];
    if (r.cached < r.prompt || r.produced >= r.max_new) continue;
    const int pos = r.cached;
    open_chunk(s, si, pos);
    r.cached = pos + 1;
    ++r.produced;
    s->decode_slots.push_back(si);
    s->decode_lens.push_back(pos + 1);
    s->decode_ids.push_back(r.id);
    --left;
  }
  // 4. prefill chunks in what is left of the budget
  s->cu_chunk.push_back(0);
  for (int si : order) {
    if (left <= 0) break;
    Request& r = s->slot[si];
    if (r.cached >= r.prompt) continue;
    const int n = std::min(r.prompt - r.cached, left);
    const int start = r.cached;
    for (int p = start; p < start + n; ++p) {
      if (p % PKV_BLOCK_SIZE == 0 || p == start) open_chunk(s, si, p);
      s->token_slots.push_back(si);
      s->token_pos.push_back(p);
    }
    r.cached = start + n;
    if (r.cached == r.prompt) {
      r.produced = 1;                           // the prompt's last row gives the first token
      publish(s, si);
    }
    s->chunk_slots.push_back(si);
    s->chunk_start.push_back(start);
    s->chunk_ids.push_back(r.id);
    s->cu_chunk.push_back((int32_t)s->token_slots.size());
    left -= n;
  }
  // requests that produced their last token in this iteration
  for (int si : order) {
    Request& r = s->slot[si];
    if (r.produced >= r.max_new && !s->finished[si]) {
      s->finished[si] = 1;
      s->done_ids.push_back(r.id);
    }
  }

  std::memset(it, 0, sizeof(*it));
  it->n_decode = (int)s->decode_slots.size();
  it->decode_slots = s->decode_slots.data();
  it->decode_lens = s->decode_lens.data();
  it->decode_ids = s->decode_ids.data();
  it->n_chunks = (int)s->chunk_slots.size();
  it->chunk_slots = s->chunk_slots.data();
  it->chunk_start = s->chunk_start.data();
  it->cu_chunk = s->cu_chunk.data();
  it->chunk_ids = s->chunk_ids.data();
  it->n_prefill_tokens = (int)s->token_slots.size();
  it->token_slots = s->token_slots.data();
  it->token_pos = s->token_pos.data();
  it->n_tokens = it->n_decode + it->n_prefill_tokens;
  it->n_patch = (int)s->patch_off.size();
  it->patch_off = s->patch_off.data();
  it->patch_val = s->patch_val.data();
  it->n_done = (int)s->done_ids.size();
  it->done_ids = s->done_ids.data();
  it->n_admitted = (int)s->admitted_ids.size();
  it->admitted_ids = s->admitted_ids.data();
  it->admitted_slots = s->admitted_slots.data();
  it->admitted_cached = s->admitted_cached.data();
  return PKV_OK;
}

namespace {
void s_list_cache(const pkv_sched* s) {
  auto& v = s->cache_list;
  v.clear();
  for (size_t n = 1; n < s->nodes.size(); ++n)
    if (s->nodes[n].live) v.insert(v.end(), s->nodes[n].blocks.begin(), s->nodes[n].blocks.end());
}
}  // namespace

extern "C" int pkv_sched_info(const pkv_sched* s, pkv_sched_state* st) {
  if (!s || !st) return PKV_ERR_NULL;
  st->num_slots = s->num_slots;
  st->n_layers = s->n_layers;
  st->max_blocks_per_seq = s->max_blocks;
  st->num_blocks = s->num_blocks;
  st->token_budget = s->budget;
  st->n_queued = (int)s->queue.size();
  int active = 0;
  for (const Request& r : s->slot) active += r.id >= 0;
  st->n_active = active;
  st->n_free = s->n_free;
  st->n_reserved = s->reserved;
  st->table = s->table.data();
  st->free_list = s->free_list.data();
  s_list_cache(s);
  st->n_cache_nodes = s->cache_nodes;
  st->n_cache_blocks = (int)s->cache_list.size();
  st->cache_blocks = s->cache_list.data();
  st->n_evictable = (int)s->evictable.size();
  st->cache_hit_tokens = s->hit_tokens;
  st->meta_elems = pkv_sched_meta_elems(s->num_slots, s->budget);
  return PKV_OK;
}

extern "C" int64_t pkv_sched_meta_elems(int num_slots, int token_budget) {
  if (num_slots <= 0 || token_budget <= 0) return 0;
  return (int64_t)num_slots + 6 * (int64_t)token_budget + 1;
}

extern "C" int pkv_sched_run(const pkv_sched* s, const pkv_sched_iter* it, pkv_bf16* const* q, pkv_bf16* const* k,
                             const pkv_bf16* const* v, pkv_bf16* const* out, pkv_bf16* k_pool, pkv_bf16* v_pool,
                             int32_t* bt_dev, int32_t* meta_dev, int n_q_heads, int n_kv_heads, int head_dim,
                             const float* cos_sin, int max_pos, float scale, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!s || !it) return PKV_ERR_NULL;
  if (it->n_tokens == 0 && it->n_patch == 0) return PKV_OK;
  if (!bt_dev || !meta_dev || !k_pool || !v_pool) return PKV_ERR_NULL;
  if (it->n_tokens > 0 && (!q || !k || !v || !out || !cos_sin)) return PKV_ERR_NULL;
  const int nd = it->n_decode, nt = it->n_prefill_tokens, nc = it->n_chunks, ns = s->num_slots, bud = s->budget;
  if (nd < 0 || nt < 0 || nc < 0 || nd > ns || nd + nt > bud || nc > bud || it->n_tokens != nd + nt)
    return PKV_ERR_INVALID_ARG;
  const int64_t bt_elems = (int64_t)ns * s->n_layers * s->max_blocks;
  int rc = pkv_block_table_patch(bt_dev, bt_elems, it->patch_off, it->patch_val, it->n_patch, stream);
  if (rc != PKV_OK || it->n_tokens == 0) return rc;

  // device metadata [context lengths (per slot) | decode slot ids | prefill
  // token slots | token positions | chunk offsets (budget + 1) | chunk starts
  // | chunk slots], sent in kernel arguments
  const int64_t o_dsl = ns, o_tsl = o_dsl + bud, o_tpo = o_tsl + bud, o_cu = o_tpo + bud, o_cst = o_cu + bud + 1,
                o_csl = o_cst + bud;
  thread_local std::vector<int32_t> off, val;
  off.clear();
  val.clear();
  auto put = [&](int64_t o, int32_t x) {
    off.push_back((int32_t)o);
    val.push_back(x);
  };
  for (int b = 0; b < nd; ++b) {
    put(it->decode_slots[b], it->decode_lens[b]);
    put(o_dsl + b, it->decode_slots[b]);
  }
  for (int t = 0; t < nt; ++t) {
    put(o_tsl + t, it->token_slots[t]);
    put(o_tpo + t, it->token_pos[t]);
  }
  int max_q = 0;
  for (int c = 0; c < nc; ++c) {
    put(o_cst + c, it->chunk_start[c]);
    put(o_csl + c, it->chunk_slots[c]);
    max_q = std::max(max_q, it->cu_chunk[c + 1] - it->cu_chunk[c]);
  }
  for (int c = 0; c <= nc; ++c) put(o_cu + c, it->cu_chunk[c]);
  // every offset above appears once (a slot is a decode row or has one chunk)
  rc = pkv::patch_distinct(meta_dev, pkv_sched_meta_elems(ns, bud), off.data(), val.data(), (int)off.size(), stream);
  if (rc != PKV_OK) return rc;

  int max_ctx = 0;
  for (int b = 0; b < nd; ++b) max_ctx = std::max(max_ctx, it->decode_lens[b]);
  // decode rows that list the same prefix-cache blocks read them with cached
  // loads (a block two requests list is its first node's, at least)
  bool shared = false;
  for (int b = 0; b < nd && !shared; ++b) {
    const int sl = it->decode_slots[b];
    if (sl < 0 || sl >= ns) continue;
    const std::vector<int>& path = s->slot[sl].path;
    shared = !path.empty() && s->nodes[path[0]].ref >= 2;
  }
  const pkv::KvReadScope kv_read(shared ? PKV_KV_READ_REUSE : 0);
  const int64_t row_stride = (int64_t)s->n_layers * s->max_blocks;
  const int64_t q_row = (int64_t)n_q_heads * head_dim, kv_row = (int64_t)n_kv_heads * head_dim;
  for (int l = 0; l < s->n_layers; ++l) {
    const int32_t* bt_l = bt_dev + (int64_t)l * s->max_blocks;
    if (nd > 0) {
      rc = pkv_paged_decode_fused(out[l], q[l], k[l], v[l], k_pool, v_pool, s->num_blocks, bt_l, row_stride, ns,
                                  s->max_blocks, meta_dev + o_dsl, meta_dev, it->decode_lens, nd, max_ctx, n_q_heads,
                                  n_kv_heads, head_dim, cos_sin, max_pos, scale, 0, workspace, workspace_bytes,
                                  stream);
      if (rc != PKV_OK) return rc;
    }
    if (nt > 0) {
      pkv_bf16* qp = q[l] + nd * q_row;
      pkv_bf16* kp = k[l] + nd * kv_row;
      rc = pkv_rope_decode(qp, kp, meta_dev + o_tpo, nt, n_q_heads, n_kv_heads, head_dim, cos_sin, max_pos, stream);
      if (rc != PKV_OK) return rc;
      rc = pkv_paged_kv_append(k_pool, v_pool, s->num_blocks, kp, v[l] + nd * kv_row, bt_l, row_stride, ns,
                               s->max_blocks, meta_dev + o_tsl, meta_dev + o_tpo, nt, n_kv_heads, head_dim, stream);
      if (rc != PKV_OK) return rc;
      rc = pkv_paged_attn_prefill(out[l] + nd * q_row, qp, meta_dev + o_cu, meta_dev + o_cst, meta_dev + o_csl,
                                  k_pool, v_pool, s->num_blocks, bt_l, row_stride, ns, s->max_blocks, nc, nt, max_q,
                                  n_q_heads, n_kv_heads, head_dim, scale, it->cu_chunk, it->chunk_start, stream);
      if (rc != PKV_OK) return rc;
    }
  }
  return PKV_OK;
}

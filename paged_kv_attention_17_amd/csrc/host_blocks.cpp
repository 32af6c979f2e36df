// Host-only part of libpagedkv: status text, the per-step block allocator and
// the block-table validator.  No HIP calls; this file also builds with g++ for
// sanitizer runs.
//
// The allocator follows "An Inference Engine in 1,500 Lines of CUDA: The Map",
// section "The path of one inference", step (4): the pool is numbered once into
// a free list, a table per (slot, layer) maps each 16-token chunk of a sequence
// to a block, and -1 marks an entry that has no block yet.  A decode step pops a
// block for every sequence whose new token opens a chunk.
#include <cstdint>
#include <cstring>
#include <vector>
#include <unordered_map>
#include <unordered_set>

#include "../../include/pagedkv.h"

extern "C" const char* pkv_status_str(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "null pointer argument";
    case PKV_ERR_MISALIGNED: return "device pointer misaligned (16 bytes for bf16/float buffers, 4 for int32)";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape (head_dim must be 64, q/kv head ratio 1, 2, 4 or 8)";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_BAD_BLOCK: return "block table holds -1 or an out-of-range block inside a context";
    case PKV_ERR_CAPACITY: return "capacity exceeded (workspace, free list or table row)";
    case PKV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" int pkv_abi_version(void) { return (1 << 16) | 0; }

extern "C" int pkv_blocks_assign(int32_t* bt, int64_t stride, int num_slots, int max_blocks,
                                 int32_t* free_list, int* n_free, const int32_t* slot_ids,
                                 const int32_t* positions, int num_tokens, int32_t* patch_off,
                                 int32_t* patch_val, int* n_patch) {
  if (num_tokens < 0 || num_slots < 0 || max_blocks < 0 || stride < max_blocks) return PKV_ERR_INVALID_ARG;
  if (num_tokens == 0) {
    if (n_patch) *n_patch = 0;
    return PKV_OK;
  }
  if (!bt || !free_list || !n_free || !slot_ids || !positions || !patch_off || !patch_val || !n_patch)
    return PKV_ERR_NULL;
  if (*n_free < 0) return PKV_ERR_INVALID_ARG;
  // First pass: find the entries that need a block (each at most once, even if
  // several tokens of one chunk arrive together) and check capacity, so that a
  // failure leaves every array untouched.
  std::vector<int64_t> need;
  std::unordered_set<int64_t> seen;
  for (int t = 0; t < num_tokens; ++t) {
    const int s = slot_ids[t], p = positions[t];
    if (s < 0 || s >= num_slots || p < 0) return PKV_ERR_INVALID_ARG;
    const int j = p / PKV_BLOCK_SIZE;
    if (j >= max_blocks) return PKV_ERR_CAPACITY;
    const int64_t off = (int64_t)s * stride + j;
    if (bt[off] == -1 && seen.insert(off).second) need.push_back(off);
  }
  if ((int64_t)need.size() > *n_free) return PKV_ERR_CAPACITY;
  int np = 0;
  for (int64_t off : need) {
    const int32_t blk = free_list[--(*n_free)];
    bt[off] = blk;
    patch_off[np] = (int32_t)off;
    patch_val[np] = blk;
    ++np;
  }
  *n_patch = np;
  return PKV_OK;
}

extern "C" int pkv_blocks_release(int32_t* bt, int64_t stride, int num_slots, int max_blocks, int slot,
                                  int32_t* free_list, int* n_free, int free_capacity,
                                  int32_t* patch_off, int32_t* patch_val, int* n_patch) {
  if (!bt || !free_list || !n_free || !patch_off || !patch_val || !n_patch) return PKV_ERR_NULL;
  if (slot < 0 || slot >= num_slots || max_blocks < 0 || stride < max_blocks || *n_free < 0)
    return PKV_ERR_INVALID_ARG;
  int32_t* row = bt + (int64_t)slot * stride;
  int cnt = 0;
  for (int j = 0; j < max_blocks; ++j) cnt += row[j] != -1;
  if (*n_free + cnt > free_capacity) return PKV_ERR_CAPACITY;
  int np = 0;
  for (int j = 0; j < max_blocks; ++j) {
    if (row[j] == -1) continue;
    free_list[(*n_free)++] = row[j];
    row[j] = -1;
    patch_off[np] = (int32_t)((int64_t)slot * stride + j);
    patch_val[np] = -1;
    ++np;
  }
  *n_patch = np;
  return PKV_OK;
}

extern "C" int pkv_check_block_table(const int32_t* bt, int64_t stride, int num_slots, int max_blocks,
                                     const int32_t* slot_ids, const int32_t* context_lens, int batch,
                                     int num_blocks, int* bad_row, int* bad_idx) {
  if (bad_row) *bad_row = -1;
  if (bad_idx) *bad_idx = -1;
  if (batch < 0 || num_slots < 0 || max_blocks < 0 || num_blocks < 0 || stride < max_blocks)
    return PKV_ERR_INVALID_ARG;
  if (batch == 0) return PKV_OK;
  if (!bt || !context_lens) return PKV_ERR_NULL;
  std::vector<uint8_t> used((size_t)num_blocks, 0);
  for (int b = 0; b < batch; ++b) {
    const int s = slot_ids ? slot_ids[b] : b;
    auto fail = [&](int idx) {
      if (bad_row) *bad_row = b;
      if (bad_idx) *bad_idx = idx;
      return PKV_ERR_BAD_BLOCK;
    };
    if (s < 0 || s >= num_slots) return fail(-2);
    const int n = context_lens[s];
    if (n < 0) return fail(-1);
    const int nb = (n + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;
    if (nb > max_blocks) return fail(-1);
    // A slot listed twice in slot_ids is checked once.
    bool repeat_row = false;
    for (int b2 = 0; b2 < b && !repeat_row; ++b2) repeat_row = (slot_ids ? slot_ids[b2] : b2) == s;
    if (repeat_row) continue;
    const int32_t* row = bt + (int64_t)s * stride;
    for (int j = 0; j < nb; ++j) {
      const int32_t blk = row[j];
      if (blk < 0 || blk >= num_blocks || used[blk]) return fail(j);
      used[blk] = 1;
    }
  }
  return PKV_OK;
}

// Prefix sharing.  The category page "code-series" lists, in its mini-sglang
// series, a chapter on a radix cache: requests that open with the same prompt
// reuse that prefix's cached K/V instead of computing it again.  The pages give
// no mechanism; here a block may be listed by several table entries,
// refcount[b] counts the entries listing b, and a block is written only through
// an entry that lists it alone: an entry about to receive a token while its
// block is shared first moves to a private copy (copy on write; the caller
// copies the block contents with pkv_blocks_copy before appending).

extern "C" int pkv_blocks_share(int32_t* bt, int64_t stride, int num_slots, int max_blocks, int src_slot,
                                int dst_slot, int n_tokens, int32_t* refcount, int num_blocks, int32_t* patch_off,
                                int32_t* patch_val, int* n_patch) {
  if (num_slots < 0 || max_blocks < 0 || stride < max_blocks || num_blocks < 0 || n_tokens < 0)
    return PKV_ERR_INVALID_ARG;
  if (src_slot < 0 || src_slot >= num_slots || dst_slot < 0 || dst_slot >= num_slots || src_slot == dst_slot)
    return PKV_ERR_INVALID_ARG;
  if (n_tokens == 0) {
    if (n_patch) *n_patch = 0;
    return PKV_OK;
  }
  if (!bt || !refcount || !patch_off || !patch_val || !n_patch) return PKV_ERR_NULL;
  const int nb = (n_tokens + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;
  if (nb > max_blocks) return PKV_ERR_CAPACITY;
  const int32_t* src = bt + (int64_t)src_slot * stride;
  int32_t* dst = bt + (int64_t)dst_slot * stride;
  // Check everything first: a failure changes nothing.
  for (int j = 0; j < nb; ++j) {
    const int32_t blk = src[j];
    if (blk < 0 || blk >= num_blocks) return PKV_ERR_BAD_BLOCK;
    if (refcount[blk] < 1 || refcount[blk] == INT32_MAX) return PKV_ERR_INVALID_ARG;
    if (dst[j] != -1) return PKV_ERR_INVALID_ARG;
  }
  for (int j = 0; j < nb; ++j) {
    dst[j] = src[j];
    ++refcount[src[j]];
    patch_off[j] = (int32_t)((int64_t)dst_slot * stride + j);
    patch_val[j] = src[j];
  }
  *n_patch = nb;
  return PKV_OK;
}

extern "C" int pkv_blocks_assign_shared(int32_t* bt, int64_t stride, int num_slots, int max_blocks,
                                        int32_t* free_list, int* n_free, int32_t* refcount, int num_blocks,
                                        const int32_t* slot_ids, const int32_t* positions, int num_tokens,
                                        int32_t* patch_off, int32_t* patch_val, int* n_patch, int32_t* copy_src,
                                        int32_t* copy_dst, int* n_copy) {
  if (num_tokens < 0 || num_slots < 0 || max_blocks < 0 || stride < max_blocks || num_blocks < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_tokens == 0) {
    if (n_patch) *n_patch = 0;
    if (n_copy) *n_copy = 0;
    return PKV_OK;
  }
  if (!bt || !free_list || !n_free || !refcount || !slot_ids || !positions || !patch_off || !patch_val ||
      !n_patch || !copy_src || !copy_dst || !n_copy)
    return PKV_ERR_NULL;
  if (*n_free < 0) return PKV_ERR_INVALID_ARG;
  // First pass: the entries that change, in token order (each once), and for
  // a shared block the count it will have when its entry is reached (earlier
  // rows of this call may already have moved off it), so that a failure leaves
  // every array untouched.
  struct Change {
    int64_t off;
    int32_t old;   // -1: fresh block; else the shared block being copied
  };
  std::vector<Change> changes;
  std::unordered_set<int64_t> seen;
  std::unordered_map<int32_t, int> moved;   // block -> entries already moved off it
  for (int t = 0; t < num_tokens; ++t) {
    const int s = slot_ids[t], p = positions[t];
    if (s < 0 || s >= num_slots || p < 0) return PKV_ERR_INVALID_ARG;
    const int j = p / PKV_BLOCK_SIZE;
    if (j >= max_blocks) return PKV_ERR_CAPACITY;
    const int64_t off = (int64_t)s * stride + j;
    if (!seen.insert(off).second) continue;
    const int32_t blk = bt[off];
    if (blk == -1) {
      changes.push_back({off, -1});
      continue;
    }
    if (blk < 0 || blk >= num_blocks) return PKV_ERR_BAD_BLOCK;
    if (refcount[blk] < 1) return PKV_ERR_INVALID_ARG;
    if (refcount[blk] - moved[blk] > 1) {
      changes.push_back({off, blk});
      ++moved[blk];
    }
  }
  if ((int64_t)changes.size() > *n_free) return PKV_ERR_CAPACITY;
  for (size_t i = 0; i < changes.size(); ++i) {
    const int32_t blk = free_list[*n_free - 1 - (int64_t)i];
    if (blk < 0 || blk >= num_blocks || refcount[blk] != 0) return PKV_ERR_INVALID_ARG;
  }
  int np = 0, nc = 0;
  for (const Change& c : changes) {
    const int32_t blk = free_list[--(*n_free)];
    refcount[blk] = 1;
    if (c.old != -1) {
      --refcount[c.old];
      copy_src[nc] = c.old;
      copy_dst[nc] = blk;
      ++nc;
    }
    bt[c.off] = blk;
    patch_off[np] = (int32_t)c.off;
    patch_val[np] = blk;
    ++np;
  }
  *n_patch = np;
  *n_copy = nc;
  return PKV_OK;
}

extern "C" int pkv_blocks_release_shared(int32_t* bt, int64_t stride, int num_slots, int max_blocks, int slot,
                                         int32_t* free_list, int* n_free, int free_capacity, int32_t* refcount,
                                         int num_blocks, int32_t* patch_off, int32_t* patch_val, int* n_patch) {
  if (!bt || !free_list || !n_free || !refcount || !patch_off || !patch_val || !n_patch) return PKV_ERR_NULL;
  if (slot < 0 || slot >= num_slots || max_blocks < 0 || stride < max_blocks || *n_free < 0 || num_blocks < 0)
    return PKV_ERR_INVALID_ARG;
  int32_t* row = bt + (int64_t)slot * stride;
  std::unordered_map<int32_t, int> drop;   // block -> entries of this row listing it
  for (int j = 0; j < max_blocks; ++j) {
    if (row[j] == -1) continue;
    if (row[j] < 0 || row[j] >= num_blocks) return PKV_ERR_BAD_BLOCK;
    ++drop[row[j]];
  }
  int freed = 0;
  for (const auto& d : drop) {
    if (refcount[d.first] < d.second) return PKV_ERR_INVALID_ARG;
    freed += refcount[d.first] == d.second;
  }
  if ((int64_t)*n_free + freed > free_capacity) return PKV_ERR_CAPACITY;
  int np = 0;
  for (int j = 0; j < max_blocks; ++j) {
    if (row[j] == -1) continue;
    if (--refcount[row[j]] == 0) free_list[(*n_free)++] = row[j];
    row[j] = -1;
    patch_off[np] = (int32_t)((int64_t)slot * stride + j);
    patch_val[np] = -1;
    ++np;
  }
  *n_patch = np;
  return PKV_OK;
}

// Native driver for one decode step of an n-layer engine (pkv_decode_step).
//
// Follows "An Inference Engine in 1,500 Lines of CUDA: The Map", section "The
// path of one inference": each decode step advances every active slot by one
// token; a block leaves the free list when a sequence's new token opens a
// 16-token chunk; the block table maps chunks to blocks per (slot, layer).
// The per-layer work is RoPE on the new q/k, the append of k/v into the cache
// and paged attention, fused into one kernel (pkv_paged_decode_fused), so the
// whole step is one call from the host language and one launch per layer
// (plus the metadata patches).
#include <cstdint>
#include <vector>

#include "../../include/pagedkv.h"

extern "C" int pkv_decode_step(int n_layers, pkv_bf16* const* q, pkv_bf16* const* k, const pkv_bf16* const* v,
                               pkv_bf16* const* out, pkv_bf16* k_pool, pkv_bf16* v_pool, int num_blocks,
                               int32_t* bt_host, int32_t* bt_dev, int num_slots, int max_blocks_per_seq,
                               int32_t* free_list_host, int* n_free, int32_t* cached_lens_host, int32_t* meta_dev,
                               const int32_t* slot_ids_host, int batch, int n_q_heads, int n_kv_heads, int head_dim,
                               const float* cos_sin, int max_pos, float scale, int max_context_len,
                               int partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  if (n_layers < 0 || batch < 0 || num_slots < 0 || max_blocks_per_seq < 0) return PKV_ERR_INVALID_ARG;
  if (n_layers == 0 || batch == 0) return PKV_OK;
  if (!q || !k || !v || !out || !bt_host || !bt_dev || !free_list_host || !n_free || !cached_lens_host ||
      !meta_dev || !slot_ids_host)
    return PKV_ERR_NULL;
  if (*n_free < 0) return PKV_ERR_INVALID_ARG;
  const int64_t layer_stride = max_blocks_per_seq;
  const int64_t row_stride = (int64_t)n_layers * max_blocks_per_seq;
  const int64_t bt_elems = (int64_t)num_slots * row_stride;
  if (bt_elems > INT32_MAX) return PKV_ERR_INVALID_ARG;

  // 1. Host allocation, checked for capacity before anything changes.
  int64_t need = 0;
  for (int b = 0; b < batch; ++b) {
    const int s = slot_ids_host[b];
    if (s < 0 || s >= num_slots) return PKV_ERR_INVALID_ARG;
    for (int b2 = 0; b2 < b; ++b2)
      if (slot_ids_host[b2] == s) return PKV_ERR_INVALID_ARG;   // one new token per slot per step
    const int p = cached_lens_host[s];
    if (p < 0) return PKV_ERR_INVALID_ARG;
    if (p / PKV_BLOCK_SIZE >= max_blocks_per_seq) return PKV_ERR_CAPACITY;
    for (int l = 0; l < n_layers; ++l)
      need += bt_host[s * row_stride + l * layer_stride + p / PKV_BLOCK_SIZE] == -1;
  }
  if (need > *n_free) return PKV_ERR_CAPACITY;

  thread_local std::vector<int32_t> t_off, t_val, m_off, m_val;
  t_off.clear();
  t_val.clear();
  m_off.clear();
  m_val.clear();
  for (int b = 0; b < batch; ++b) {
    const int s = slot_ids_host[b];
    const int p = cached_lens_host[s];
    for (int l = 0; l < n_layers; ++l) {
      const int64_t off = s * row_stride + l * layer_stride + p / PKV_BLOCK_SIZE;
      if (bt_host[off] != -1) continue;
      const int32_t blk = free_list_host[--(*n_free)];
      bt_host[off] = blk;
      t_off.push_back((int32_t)off);
      t_val.push_back(blk);
    }
  }
  // 2. Context lengths, positions and slot ids for the kernels.
  for (int b = 0; b < batch; ++b) {
    const int s = slot_ids_host[b];
    const int p = cached_lens_host[s];
    cached_lens_host[s] = p + 1;
    m_off.push_back(s);
    m_val.push_back(p + 1);
    m_off.push_back(num_slots + b);
    m_val.push_back(p);
    m_off.push_back(num_slots + batch + b);
    m_val.push_back(s);
  }
  const int64_t meta_elems = (int64_t)num_slots + 2 * (int64_t)batch;
  int rc = pkv_block_table_patch(bt_dev, bt_elems, t_off.data(), t_val.data(), (int)t_off.size(), stream);
  if (rc != PKV_OK) return rc;
  rc = pkv_block_table_patch(meta_dev, meta_elems, m_off.data(), m_val.data(), (int)m_off.size(), stream);
  if (rc != PKV_OK) return rc;

  // 3. Per layer: RoPE, append and attention in one launch.  An identity
  // batch (row b = slot b) passes no slot ids, which saves the kernels one
  // dependent memory read before their first K/V load.
  bool identity = batch <= num_slots;
  for (int b = 0; b < batch && identity; ++b) identity = slot_ids_host[b] == b;
  thread_local std::vector<int32_t> row_lens;
  row_lens.resize(batch);
  for (int b = 0; b < batch; ++b) row_lens[b] = cached_lens_host[slot_ids_host[b]];
  const int32_t* ctx_dev = meta_dev;
  const int32_t* sid_dev = identity ? nullptr : meta_dev + num_slots + batch;
  for (int l = 0; l < n_layers; ++l) {
    const int32_t* bt_l = bt_dev + l * layer_stride;
    rc = pkv_paged_decode_fused(out[l], q[l], k[l], v[l], k_pool, v_pool, num_blocks, bt_l, row_stride, num_slots,
                                max_blocks_per_seq, sid_dev, ctx_dev, row_lens.data(), batch, max_context_len, n_q_heads,
                                n_kv_heads, head_dim, cos_sin, max_pos, scale, partition_size, workspace,
                                workspace_bytes, stream);
    if (rc != PKV_OK) return rc;
  }
  return PKV_OK;
}

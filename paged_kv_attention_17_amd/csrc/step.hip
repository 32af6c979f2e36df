// Native driver for one decode step of an n-layer engine (pkv_decode_step).
//
// Follows "An Inference Engine in 1,500 Lines of CUDA: The Map", section "The
// path of one inference": each decode step advances every active slot by one
// token; a block leaves the free list when a sequence's new token opens a
// 16-token chunk; the block table maps chunks to blocks per (slot, layer).
// The per-layer work is RoPE on the new q/k, the append of k/v into the cache
// and paged attention, fused into one kernel (pkv_paged_decode_fused), so the
// whole step is one call from the host language and one launch per layer
// (plus the metadata patches and one merge of rows cut by workgroup shares).
//
// The step also comes in two halves for a device half captured once as a HIP
// graph and replayed every step (the category page's mini-sglang chapter on
// kernel-argument metadata and CUDA graphs): the host half allocates blocks
// and writes the table changes, the step's metadata and the streaming
// kernel's plan into a staging area; the device half copies nothing itself
// and launches a fixed sequence (apply the staging area, one streaming launch
// per layer reading its plan from the staged copy, one merge) whose shapes do
// not depend on the lengths.
#include <cstdint>
#include <cstring>
#include <vector>

#include "common.h"
#include "decode_api.h"

namespace pkv {
int patch_two(int32_t* a, int64_t a_elems, const int32_t* a_off, const int32_t* a_val, int n_a, int32_t* b,
              int64_t b_elems, const int32_t* b_off, const int32_t* b_val, int n_b, void* stream);
}

using namespace pkv;

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
  const hipStream_t st = static_cast<hipStream_t>(stream);

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

  // 2. Every layer's attention launch, planned and checked before anything
  // changes or is enqueued.  The layers share the rows and their lengths, so
  // their streaming launches chain: each merges the previous layer's rows cut
  // by share ends in its prologue, and one merge launch follows the last.  An
  // identity batch (row b = slot b) passes no device slot ids.
  bool identity = batch <= num_slots;
  for (int b = 0; b < batch && identity; ++b) identity = slot_ids_host[b] == b;
  thread_local std::vector<int32_t> row_lens;
  row_lens.resize(batch);
  for (int b = 0; b < batch; ++b) row_lens[b] = cached_lens_host[slot_ids_host[b]] + 1;
  const int32_t* ctx_dev = meta_dev;
  const int32_t* sid_dev = identity ? nullptr : meta_dev + num_slots + batch;
  thread_local std::vector<DecodeLaunch> launches;
  launches.resize(n_layers);
  bool chain = false;
  const size_t plan_off = decode_plan_offset(n_q_heads);
  StreamPlan* plan_ws = n_layers > 1 && workspace && n_q_heads > 0 && workspace_bytes >= plan_off + kStreamPlanBytes
                            ? reinterpret_cast<StreamPlan*>(static_cast<char*>(workspace) + plan_off)
                            : nullptr;
  for (int l = 0; l < n_layers; ++l) {
    DecodeCall c{};
    c.fused = true;
    c.out = out[l];
    c.q = q[l];
    c.k_new = k[l];
    c.v_new = v[l];
    c.k_pool = k_pool;
    c.v_pool = v_pool;
    c.num_blocks = num_blocks;
    c.block_table = bt_dev + l * layer_stride;
    c.bt_row_stride = row_stride;
    c.num_slots = num_slots;
    c.max_blocks_per_seq = max_blocks_per_seq;
    c.slot_ids = sid_dev;
    c.slot_ids_host = slot_ids_host;
    c.context_lens = ctx_dev;
    c.row_lens_host = row_lens.data();
    c.batch = batch;
    c.max_context_len = max_context_len;
    c.n_q_heads = n_q_heads;
    c.n_kv_heads = n_kv_heads;
    c.head_dim = head_dim;
    c.cos_sin = cos_sin;
    c.max_pos = max_pos;
    c.scale = scale;
    c.partition_size = partition_size;
    c.workspace = workspace;
    c.workspace_bytes = workspace_bytes;
    c.chain_plan = n_layers > 1;
    // chained launches: the first stores its plan in the workspace, the others
    // read it from there (small kernel arguments)
    if (l == 0 && plan_ws) c.plan_out = plan_ws;
    if (chain) {
      c.records_half = l & 1;
      c.out_prev = out[l - 1];
      c.plan_dev = plan_ws;
    }
    const int rc = decode_prepare(c, &launches[l]);
    if (rc != PKV_OK) return rc;
    if (l == 0) chain = n_layers > 1 && decode_chainable(launches[0]);
  }

  // 3. Allocation and the step's metadata (context lengths, positions, slot
  // ids), carried to the device in kernel arguments.
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
  // the table changes name distinct entries (one block per (slot, layer) per
  // step) and so do the metadata pairs: one launch carries both when they fit
  int rc = patch_two(bt_dev, bt_elems, t_off.data(), t_val.data(), (int)t_off.size(), meta_dev, meta_elems,
                     m_off.data(), m_val.data(), (int)m_off.size(), stream);
  if (rc != PKV_OK) return rc;

  // 4. Per layer: RoPE, append and attention in one launch.
  for (int l = 0; l < n_layers; ++l)
    if ((rc = decode_enqueue(launches[l], st, !chain)) != PKV_OK) return rc;
  return chain ? decode_finish(launches[n_layers - 1], st) : PKV_OK;
}

// ------------------------------------------------------------ two halves --

namespace {

// Staging area of the two-half step (int32 words): a header, the full step
// metadata (context lengths per slot | positions | slot ids), room for one
// table change per (row, layer), then the streaming kernel's plan.
constexpr int kHdr = 4;                  // n_tpatch, batch, n_layers, num_slots

struct StagingLayout {
  size_t meta, patches, plan, bytes;     // word offsets (plan: 16-byte aligned), total bytes
};

StagingLayout staging_layout(int n_layers, int batch, int num_slots) {
  StagingLayout L;
  L.meta = kHdr;
  L.patches = L.meta + (size_t)num_slots + 2 * (size_t)batch;
  L.plan = (L.patches + 2 * (size_t)batch * n_layers + 3) / 4 * 4;
  L.bytes = L.plan * 4 + sizeof(StreamPlan);
  return L;
}

// Apply a staged step: table changes into bt_dev, the metadata into meta_dev.
__global__ __launch_bounds__(256) void apply_staging_kernel(const int32_t* __restrict__ st, int32_t* __restrict__ bt,
                                                            int64_t bt_elems, int32_t* __restrict__ meta,
                                                            int meta_elems, int patch_off, int max_patches) {
  const int np = min(st[0], max_patches);
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    const int off = st[patch_off + 2 * i];
    if (off >= 0 && off < bt_elems) bt[off] = st[patch_off + 2 * i + 1];
  }
  for (int i = threadIdx.x; i < meta_elems; i += blockDim.x) meta[i] = st[kHdr + i];
}

}  // namespace

extern "C" size_t pkv_decode_step_staging_bytes(int n_layers, int batch, int num_slots) {
  if (n_layers <= 0 || batch <= 0 || batch > kStreamMaxSeqs || num_slots <= 0) return 0;
  return staging_layout(n_layers, batch, num_slots).bytes;
}

extern "C" int pkv_decode_step_host(int n_layers, int32_t* bt_host, int num_slots, int max_blocks_per_seq,
                                    int32_t* free_list_host, int* n_free, int32_t* cached_lens_host,
                                    const int32_t* slot_ids_host, int batch, void* staging_host) {
  if (n_layers <= 0 || batch <= 0 || num_slots <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
  if (batch > kStreamMaxSeqs) return PKV_ERR_UNSUPPORTED;
  if (!bt_host || !free_list_host || !n_free || !cached_lens_host || !slot_ids_host || !staging_host)
    return PKV_ERR_NULL;
  if (*n_free < 0) return PKV_ERR_INVALID_ARG;
  const int64_t layer_stride = max_blocks_per_seq;
  const int64_t row_stride = (int64_t)n_layers * max_blocks_per_seq;
  if ((int64_t)num_slots * row_stride > INT32_MAX) return PKV_ERR_INVALID_ARG;
  // checks and the new lengths, before anything changes
  int64_t need = 0;
  thread_local std::vector<int32_t> row_lens;
  row_lens.resize(batch);
  for (int b = 0; b < batch; ++b) {
    const int s = slot_ids_host[b];
    if (s < 0 || s >= num_slots) return PKV_ERR_INVALID_ARG;
    for (int b2 = 0; b2 < b; ++b2)
      if (slot_ids_host[b2] == s) return PKV_ERR_INVALID_ARG;
    const int p = cached_lens_host[s];
    if (p < 0) return PKV_ERR_INVALID_ARG;
    if (p / PKV_BLOCK_SIZE >= max_blocks_per_seq) return PKV_ERR_CAPACITY;
    for (int l = 0; l < n_layers; ++l)
      need += bt_host[s * row_stride + l * layer_stride + p / PKV_BLOCK_SIZE] == -1;
    row_lens[b] = p + 1;
  }
  if (need > *n_free) return PKV_ERR_CAPACITY;
  // the rows must suit the streaming kernel and, over several layers, the
  // chained prologue merge
  thread_local StreamPlan plan;
  int merge = 0;
  const bool chain = n_layers > 1;
  const int pr = stream_plan_build(batch, row_lens.data(), max_blocks_per_seq, slot_ids_host, true, num_slots, chain,
                                   &plan, &merge);
  if (pr < 0 || (chain && pr != 0)) return PKV_ERR_UNSUPPORTED;
  const StagingLayout SL = staging_layout(n_layers, batch, num_slots);
  int32_t* st = static_cast<int32_t*>(staging_host);
  std::memcpy(st + SL.plan, &plan, sizeof(StreamPlan));
  // allocation, as pkv_decode_step
  int np = 0;
  int32_t* pairs = st + SL.patches;
  for (int b = 0; b < batch; ++b) {
    const int s = slot_ids_host[b];
    const int p = cached_lens_host[s];
    for (int l = 0; l < n_layers; ++l) {
      const int64_t off = s * row_stride + l * layer_stride + p / PKV_BLOCK_SIZE;
      if (bt_host[off] != -1) continue;
      const int32_t blk = free_list_host[--(*n_free)];
      bt_host[off] = blk;
      pairs[2 * np] = (int32_t)off;
      pairs[2 * np + 1] = blk;
      ++np;
    }
  }
  for (int b = 0; b < batch; ++b) cached_lens_host[slot_ids_host[b]] += 1;
  int32_t* meta = st + SL.meta;
  for (int s = 0; s < num_slots; ++s) meta[s] = cached_lens_host[s];
  for (int b = 0; b < batch; ++b) {
    meta[num_slots + b] = cached_lens_host[slot_ids_host[b]] - 1;
    meta[num_slots + batch + b] = slot_ids_host[b];
  }
  st[0] = np;
  st[1] = batch;
  st[2] = n_layers;
  st[3] = num_slots;
  return PKV_OK;
}

extern "C" int pkv_decode_step_device(int n_layers, pkv_bf16* const* q, pkv_bf16* const* k,
                                      const pkv_bf16* const* v, pkv_bf16* const* out, pkv_bf16* k_pool,
                                      pkv_bf16* v_pool, int num_blocks, int32_t* bt_dev, int num_slots,
                                      int max_blocks_per_seq, int32_t* meta_dev, int batch, int n_q_heads,
                                      int n_kv_heads, int head_dim, const float* cos_sin, int max_pos, float scale,
                                      const void* staging_host, const void* staging_dev, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (n_layers <= 0 || batch <= 0 || num_slots <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
  if (batch > kStreamMaxSeqs) return PKV_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out || !bt_dev || !meta_dev || !staging_host || !staging_dev) return PKV_ERR_NULL;
  if (!aligned16(staging_dev)) return PKV_ERR_MISALIGNED;
  const int64_t layer_stride = max_blocks_per_seq;
  const int64_t row_stride = (int64_t)n_layers * max_blocks_per_seq;
  const int64_t bt_elems = (int64_t)num_slots * row_stride;
  if (bt_elems > INT32_MAX) return PKV_ERR_INVALID_ARG;
  const StagingLayout SL = staging_layout(n_layers, batch, num_slots);
  const int32_t* sth = static_cast<const int32_t*>(staging_host);
  if (sth[1] != batch || sth[2] != n_layers || sth[3] != num_slots) return PKV_ERR_INVALID_ARG;
  const StreamPlan* plan_h = reinterpret_cast<const StreamPlan*>(sth + SL.plan);
  const StreamPlan* plan_d = reinterpret_cast<const StreamPlan*>(static_cast<const int32_t*>(staging_dev) + SL.plan);
  // the lengths of the staged step, used to check the launches (the kernels
  // read the plan from the device copy at every launch)
  thread_local std::vector<int32_t> row_lens, sids;
  row_lens.assign(plan_h->row_n, plan_h->row_n + batch);
  sids.assign(sth + SL.meta + num_slots + batch, sth + SL.meta + num_slots + 2 * batch);
  const int32_t* ctx_dev = meta_dev;
  const int32_t* sid_dev = meta_dev + num_slots + batch;
  thread_local std::vector<DecodeLaunch> launches;
  launches.resize(n_layers);
  for (int l = 0; l < n_layers; ++l) {
    DecodeCall c{};
    c.fused = true;
    c.out = out[l];
    c.q = q[l];
    c.k_new = k[l];
    c.v_new = v[l];
    c.k_pool = k_pool;
    c.v_pool = v_pool;
    c.num_blocks = num_blocks;
    c.block_table = bt_dev + l * layer_stride;
    c.bt_row_stride = row_stride;
    c.num_slots = num_slots;
    c.max_blocks_per_seq = max_blocks_per_seq;
    c.slot_ids = sid_dev;
    c.slot_ids_host = sids.data();
    c.context_lens = ctx_dev;
    c.row_lens_host = row_lens.data();
    c.batch = batch;
    c.max_context_len = max_blocks_per_seq * PKV_BLOCK_SIZE;
    c.n_q_heads = n_q_heads;
    c.n_kv_heads = n_kv_heads;
    c.head_dim = head_dim;
    c.cos_sin = cos_sin;
    c.max_pos = max_pos;
    c.scale = scale;
    c.workspace = workspace;
    c.workspace_bytes = workspace_bytes;
    c.plan_dev = plan_d;
    c.fixed_shape = true;
    c.chain_plan = n_layers > 1;
    if (n_layers > 1) {
      c.records_half = l & 1;
      c.out_prev = l > 0 ? out[l - 1] : nullptr;
    }
    const int rc = decode_prepare(c, &launches[l]);
    if (rc != PKV_OK) return rc;
    if (launches[l].path != 1) return PKV_ERR_UNSUPPORTED;
    if (n_layers > 1 && !decode_chainable(launches[l])) return PKV_ERR_CAPACITY;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int32_t* std_ = static_cast<const int32_t*>(staging_dev);
  const int meta_elems = num_slots + 2 * batch;
  const int patch_off = (int)SL.patches;
  const int max_patches = batch * n_layers;
  void* args[] = {&std_, &bt_dev, const_cast<int64_t*>(&bt_elems), &meta_dev, const_cast<int*>(&meta_elems),
                  const_cast<int*>(&patch_off), const_cast<int*>(&max_patches)};
  int rc = launch_status(hipLaunchKernel((const void*)apply_staging_kernel, dim3(1), dim3(256), args, 0, st));
  if (rc != PKV_OK) return rc;
  for (int l = 0; l < n_layers; ++l)
    if ((rc = decode_enqueue(launches[l], st, n_layers == 1)) != PKV_OK) return rc;
  return n_layers > 1 ? decode_finish(launches[n_layers - 1], st) : PKV_OK;
}

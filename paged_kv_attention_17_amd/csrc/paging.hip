// KV-cache writes and reads through the block table, for gfx950.
//
// Source: "An Inference Engine in 1,500 Lines of CUDA: The Map", section "The
// path of one inference", step (4): one pool cut into 16-token blocks and a
// block table per (slot, layer) mapping each 16-token chunk of a sequence to
// its block (-1 = none yet); the series' sixth chapter title (reading
// non-contiguous blocks through the table).
//
// Token p of table row s lives at pool[table[s][p / 16]][p % 16][head][:].
// Each thread moves one 16-byte chunk (8 bf16) of one head's row, so a K or V
// row of 128 bytes is eight adjacent lanes and every load/store is a full
// dwordx4.  Every index that comes from device data is range-checked before
// it is used as an address.
#include "common.h"

#include <algorithm>
#include <unordered_set>
#include <vector>

namespace pkv {

constexpr int kChunks = kHeadDim * 2 / 16;   // 16-byte chunks per head row

__global__ __launch_bounds__(256) void append_kernel(uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
                                                     int num_blocks, const uint4* __restrict__ k_new,
                                                     const uint4* __restrict__ v_new,
                                                     const int32_t* __restrict__ bt, int64_t stride,
                                                     int num_slots, int max_blocks,
                                                     const int32_t* __restrict__ slot_ids,
                                                     const int32_t* __restrict__ positions, int num_tokens,
                                                     int n_kv) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = (int64_t)n_kv * kChunks * 2;
  if (gid >= (int64_t)num_tokens * per_token) return;
  const int t = (int)(gid / per_token);
  const int rem = (int)(gid % per_token);
  const int which = rem / (n_kv * kChunks);            // 0 = K, 1 = V
  const int hc = rem % (n_kv * kChunks);                // head * kChunks + chunk
  const int s = slot_ids[t];
  const int p = positions[t];
  if (s < 0 || s >= num_slots || p < 0 || p / kBlock >= max_blocks) return;
  const int blk = bt[(int64_t)s * stride + p / kBlock];
  if (blk < 0 || blk >= num_blocks) return;
  const int64_t dst = ((int64_t)blk * kBlock + p % kBlock) * n_kv * kChunks + hc;
  const int64_t src = (int64_t)t * n_kv * kChunks + hc;
  if (which == 0)
    k_pool[dst] = k_new[src];
  else
    v_pool[dst] = v_new[src];
}

__global__ __launch_bounds__(256) void gather_kernel(uint4* __restrict__ k_dense, uint4* __restrict__ v_dense,
                                                     const uint4* __restrict__ k_pool,
                                                     const uint4* __restrict__ v_pool, int num_blocks,
                                                     const int32_t* __restrict__ row, int context_len,
                                                     int n_kv) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = (int64_t)n_kv * kChunks;
  if (gid >= (int64_t)context_len * per_token) return;
  const int p = (int)(gid / per_token);
  const int hc = (int)(gid % per_token);
  const int blk = row[p / kBlock];
  uint4 kv = make_uint4(0, 0, 0, 0), vv = kv;
  if (blk >= 0 && blk < num_blocks) {
    const int64_t src = ((int64_t)blk * kBlock + p % kBlock) * per_token + hc;
    kv = k_pool[src];
    vv = v_pool[src];
  }
  k_dense[gid] = kv;
  v_dense[gid] = vv;
}

constexpr int kPatchPerLaunch = 500;   // (offset, value) pairs carried in one kernel's arguments (< 4 KB)

struct PatchArgs {
  int32_t off[kPatchPerLaunch];
  int32_t val[kPatchPerLaunch];
};

__global__ __launch_bounds__(512) void patch_kernel(int32_t* __restrict__ bt, int64_t elems, PatchArgs pa, int n) {
  const int i = threadIdx.x;
  if (i < n && pa.off[i] >= 0 && pa.off[i] < elems) bt[pa.off[i]] = pa.val[i];
}

// Two arrays in one launch: pairs [0, n_a) go to a, pairs [n_a, n) to b.
__global__ __launch_bounds__(512) void patch2_kernel(int32_t* __restrict__ a, int64_t a_elems, int n_a,
                                                     int32_t* __restrict__ b, int64_t b_elems, PatchArgs pa, int n) {
  const int i = threadIdx.x;
  if (i >= n) return;
  int32_t* t = i < n_a ? a : b;
  const int64_t el = i < n_a ? a_elems : b_elems;
  if (pa.off[i] >= 0 && pa.off[i] < el) t[pa.off[i]] = pa.val[i];
}

// Write n (offset, value) pairs whose offsets are distinct: each launch takes
// up to kPatchPerLaunch of them in its arguments, one thread per pair.
int patch_distinct(int32_t* bt_dev, int64_t bt_elems, const int32_t* off, const int32_t* val, int n_patch,
                   void* stream) {
  for (int base = 0; base < n_patch; base += kPatchPerLaunch) {
    PatchArgs pa;
    const int n = n_patch - base < kPatchPerLaunch ? n_patch - base : kPatchPerLaunch;
    std::copy(off + base, off + base + n, pa.off);
    std::copy(val + base, val + base + n, pa.val);
    int32_t* bt = bt_dev;
    int64_t el = bt_elems;
    int nn = n;
    void* args[] = {&bt, &el, &pa, &nn};
    const int st = launch_status(hipLaunchKernel((const void*)patch_kernel, dim3(1), dim3(512), args, 0,
                                                 (hipStream_t)stream));
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

// Distinct (offset, value) pairs into two arrays: when both lists fit one
// launch's arguments they go in one launch, else one launch per list.
int patch_two(int32_t* a, int64_t a_elems, const int32_t* a_off, const int32_t* a_val, int n_a, int32_t* b,
              int64_t b_elems, const int32_t* b_off, const int32_t* b_val, int n_b, void* stream) {
  if (n_a == 0) return patch_distinct(b, b_elems, b_off, b_val, n_b, stream);
  if (n_b == 0 || n_a + n_b > kPatchPerLaunch) {
    const int rc = patch_distinct(a, a_elems, a_off, a_val, n_a, stream);
    return rc != PKV_OK ? rc : patch_distinct(b, b_elems, b_off, b_val, n_b, stream);
  }
  PatchArgs pa;
  std::copy(a_off, a_off + n_a, pa.off);
  std::copy(a_val, a_val + n_a, pa.val);
  std::copy(b_off, b_off + n_b, pa.off + n_a);
  std::copy(b_val, b_val + n_b, pa.val + n_a);
  int n = n_a + n_b;
  void* args[] = {&a, &a_elems, &n_a, &b, &b_elems, &pa, &n};
  return launch_status(hipLaunchKernel((const void*)patch2_kernel, dim3(1), dim3(512), args, 0,
                                       (hipStream_t)stream));
}

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_paged_kv_append(pkv_bf16* k_pool, pkv_bf16* v_pool, int num_blocks, const pkv_bf16* k_new,
                                   const pkv_bf16* v_new, const int32_t* block_table, int64_t bt_row_stride,
                                   int num_slots, int max_blocks_per_seq, const int32_t* slot_ids,
                                   const int32_t* positions, int num_tokens, int n_kv_heads, int head_dim,
                                   void* stream) {
  if (num_tokens < 0 || num_blocks < 0 || n_kv_heads <= 0 || num_slots < 0 || max_blocks_per_seq < 0 ||
      bt_row_stride < max_blocks_per_seq)
    return PKV_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !block_table || !slot_ids || !positions) return PKV_ERR_NULL;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new) ||
      !aligned4(block_table) || !aligned4(slot_ids) || !aligned4(positions))
    return PKV_ERR_MISALIGNED;
  const int64_t total = (int64_t)num_tokens * n_kv_heads * kChunks * 2;
  const int64_t grid = (total + 255) / 256;
  if (grid > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  uint4* kp = reinterpret_cast<uint4*>(k_pool);
  uint4* vp = reinterpret_cast<uint4*>(v_pool);
  const uint4* kn = reinterpret_cast<const uint4*>(k_new);
  const uint4* vn = reinterpret_cast<const uint4*>(v_new);
  int nb = num_blocks, ns = num_slots, mb = max_blocks_per_seq, nt = num_tokens, nk = n_kv_heads;
  int64_t st = bt_row_stride;
  const int32_t *bt = block_table, *si = slot_ids, *po = positions;
  void* args[] = {&kp, &vp, &nb, &kn, &vn, &bt, &st, &ns, &mb, &si, &po, &nt, &nk};
  return launch_status(hipLaunchKernel((const void*)append_kernel, dim3((unsigned)grid), dim3(256), args, 0,
                                       (hipStream_t)stream));
}

extern "C" int pkv_paged_gather(pkv_bf16* k_dense, pkv_bf16* v_dense, const pkv_bf16* k_pool,
                                const pkv_bf16* v_pool, int num_blocks, const int32_t* block_table,
                                int64_t bt_row_stride, int max_blocks_per_seq, int slot, int context_len,
                                int n_kv_heads, int head_dim, void* stream) {
  if (context_len < 0 || num_blocks < 0 || n_kv_heads <= 0 || slot < 0 || max_blocks_per_seq < 0 ||
      bt_row_stride < max_blocks_per_seq)
    return PKV_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return PKV_ERR_UNSUPPORTED;
  if (context_len == 0) return PKV_OK;
  if ((context_len + kBlock - 1) / kBlock > max_blocks_per_seq) return PKV_ERR_CAPACITY;
  if (!k_dense || !v_dense || !k_pool || !v_pool || !block_table) return PKV_ERR_NULL;
  if (!aligned16(k_dense) || !aligned16(v_dense) || !aligned16(k_pool) || !aligned16(v_pool))
    return PKV_ERR_MISALIGNED;
  const int64_t total = (int64_t)context_len * n_kv_heads * kChunks;
  const int64_t grid = (total + 255) / 256;
  uint4* kd = reinterpret_cast<uint4*>(k_dense);
  uint4* vd = reinterpret_cast<uint4*>(v_dense);
  const uint4* kp = reinterpret_cast<const uint4*>(k_pool);
  const uint4* vp = reinterpret_cast<const uint4*>(v_pool);
  const int32_t* row = block_table + (int64_t)slot * bt_row_stride;
  int nb = num_blocks, cl = context_len, nk = n_kv_heads;
  void* args[] = {&kd, &vd, &kp, &vp, &nb, &row, &cl, &nk};
  return launch_status(hipLaunchKernel((const void*)gather_kernel, dim3((unsigned)grid), dim3(256), args, 0,
                                       (hipStream_t)stream));
}

namespace pkv {

// Whole-block copies for copy on write of a shared block: workgroup 2 i + w
// copies pool w (0 = K, 1 = V) of pair i, the block's 16 rows of every head
// (16 KB at 8 KV heads) as 16-byte words, consecutive lanes on consecutive
// words.  The pairs travel in the kernel arguments.
constexpr int kCopyPerLaunch = 480;

struct CopyArgs {
  int32_t src[kCopyPerLaunch];
  int32_t dst[kCopyPerLaunch];
};
static_assert(sizeof(CopyArgs) + 64 <= 4096, "kernel argument block");

__global__ __launch_bounds__(256) void block_copy_kernel(uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
                                                         int num_blocks, int64_t words_per_block, CopyArgs c,
                                                         int n) {
  const int i = blockIdx.x >> 1;
  if (i >= n) return;
  const int32_t a = c.src[i], b = c.dst[i];
  if (a < 0 || a >= num_blocks || b < 0 || b >= num_blocks) return;
  uint4* pool = (blockIdx.x & 1) ? v_pool : k_pool;
  const uint4* from = pool + (int64_t)a * words_per_block;
  uint4* to = pool + (int64_t)b * words_per_block;
  for (int64_t w = threadIdx.x; w < words_per_block; w += blockDim.x) to[w] = from[w];
}

}  // namespace pkv

extern "C" int pkv_blocks_copy(pkv_bf16* k_pool, pkv_bf16* v_pool, int num_blocks, int n_kv_heads, int head_dim,
                               const int32_t* src_host, const int32_t* dst_host, int n_copy, void* stream) {
  if (n_copy < 0 || num_blocks < 0 || n_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return PKV_ERR_UNSUPPORTED;
  if (n_copy == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src_host || !dst_host) return PKV_ERR_NULL;
  if (!aligned16(k_pool) || !aligned16(v_pool)) return PKV_ERR_MISALIGNED;
  // Every copy reads the pool as it was before the call: ids in range, no
  // block written twice, and no block both written and read.
  std::vector<uint8_t> role((size_t)num_blocks, 0);   // bit 0: read, bit 1: written
  for (int i = 0; i < n_copy; ++i) {
    const int32_t a = src_host[i], b = dst_host[i];
    if (a < 0 || a >= num_blocks || b < 0 || b >= num_blocks) return PKV_ERR_BAD_BLOCK;
    if (role[b] & 2) return PKV_ERR_INVALID_ARG;
    role[a] |= 1;
    role[b] |= 2;
  }
  for (int i = 0; i < n_copy; ++i)
    if (role[src_host[i]] & 2) return PKV_ERR_INVALID_ARG;
  const int64_t words = (int64_t)kBlock * n_kv_heads * kChunks;
  for (int base = 0; base < n_copy; base += kCopyPerLaunch) {
    CopyArgs c;
    const int n = n_copy - base < kCopyPerLaunch ? n_copy - base : kCopyPerLaunch;
    for (int i = 0; i < n; ++i) {
      c.src[i] = src_host[base + i];
      c.dst[i] = dst_host[base + i];
    }
    uint4* kp = reinterpret_cast<uint4*>(k_pool);
    uint4* vp = reinterpret_cast<uint4*>(v_pool);
    int nbk = num_blocks;
    int64_t w = words;
    int nn = n;
    void* args[] = {&kp, &vp, &nbk, &w, &c, &nn};
    const int st = launch_status(hipLaunchKernel((const void*)block_copy_kernel, dim3(2 * n), dim3(256), args, 0,
                                                 (hipStream_t)stream));
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

extern "C" int pkv_block_table_patch(int32_t* bt_dev, int64_t bt_elems, const int32_t* patch_offsets_host,
                                     const int32_t* patch_values_host, int n_patch, void* stream) {
  if (n_patch < 0 || bt_elems < 0) return PKV_ERR_INVALID_ARG;
  if (n_patch == 0) return PKV_OK;
  if (!bt_dev || !patch_offsets_host || !patch_values_host) return PKV_ERR_NULL;
  if (!aligned4(bt_dev)) return PKV_ERR_MISALIGNED;
  // The list is applied in order: when an entry appears more than once (a row
  // released and reused in one step) only its last pair is kept, so the pairs
  // that reach the device name distinct entries and their order within a
  // launch does not matter.
  thread_local std::vector<int32_t> off, val;
  off.clear();
  val.clear();
  {
    std::unordered_set<int32_t> seen;
    seen.reserve((size_t)n_patch * 2);
    for (int i = n_patch - 1; i >= 0; --i)
      if (seen.insert(patch_offsets_host[i]).second) {
        off.push_back(patch_offsets_host[i]);
        val.push_back(patch_values_host[i]);
      }
  }
  return patch_distinct(bt_dev, bt_elems, off.data(), val.data(), (int)off.size(), stream);
}

namespace pkv {

// Grid-stride read of n 16-byte words (consecutive threads read consecutive
// words; the hardware keeps several iterations' loads in flight per wave).
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, size_t n, uint32_t* sink) {
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) *sink = acc;
}

}  // namespace pkv

extern "C" int pkv_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return PKV_OK;
  if (!buf || !sink) return PKV_ERR_NULL;
  if (!pkv::aligned16(buf) || !pkv::aligned4(sink) || bytes % 16) return PKV_ERR_MISALIGNED;
  const uint4* p = static_cast<const uint4*>(buf);
  size_t n = bytes / 16;
  void* args[] = {&p, &n, &sink};
  return pkv::launch_status(hipLaunchKernel((const void*)pkv::read_probe_kernel, dim3(2048), dim3(256), args, 0,
                                            (hipStream_t)stream));
}

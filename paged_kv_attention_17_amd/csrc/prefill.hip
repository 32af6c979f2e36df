// Chunked causal prefill attention over the paged KV cache, on gfx950 MFMA.
//
// Source: "An Inference Engine in 1,500 Lines of CUDA: The Map", section "The
// path of one inference", closing paragraph (prefill pushes every prompt token
// through at once, so attention is matrix x matrix; decode has its own kernels)
// and the category page's chapter title on chunked prefill (a prompt may arrive
// in chunks; a chunk's queries also see the keys of earlier chunks).
//
// Tiling.  A workgroup of 4 wave64s owns (sequence, KV head, 32 query tokens).
// Wave w computes query head g*G + w (looping when G > 4) for those 32 tokens,
// so the 4 GQA heads share every K/V tile staged in LDS.  Per 32-key tile:
//   S^T[key][query] = K . Q^T   four v_mfma_f32_32x32x16_bf16 over the 64 dims
//   online softmax per query    (a lane owns one query column: its 16 keys are
//                                in-lane, the other 16 in lane ^ 32)
//   O^T[dim][query] += V^T . P^T  four MFMAs (2 dim halves x 2 key halves)
// Computing the transposed products keeps the per-query max/sum/rescale in one
// lane.  MFMA contracts A's k slots against B's k slots of the same lane group,
// so any consistent assignment of dims (or keys) to k slots is correct; the key
// assignment used for P^T is the one the S^T accumulator layout already has
// (keys 8*(i/4) + 4*(lane/32) + i%4 for accumulator i), and V^T is read from a
// transposed LDS copy with the same assignment.  Keys past the sequence's cached
// length get V = 0 in LDS and scores of -inf by select, so NaN in unused pool
// slots never reaches the output; causal masking is a select as well.
#include "common.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQTile = 32;            // query tokens per workgroup
constexpr int kKTile = 32;            // keys per step
constexpr int kPfWaves = 4;
constexpr int kKsStride = kHeadDim + 8;   // padded LDS row (bf16) for K tiles
constexpr int kVtStride = kKTile + 8;     // padded LDS row (bf16) for transposed V tiles

struct PrefillArgs {
  uint16_t* out;
  const uint16_t* q;
  const int32_t* cu_q;
  const int32_t* q_start;
  const int32_t* slot_ids;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* bt;
  int64_t bt_stride;
  int num_blocks;
  int num_slots;
  int max_blocks;
  int n_q;
  int n_kv;
  int q_tiles;        // tiles in the grid's x dimension
  int total_q;
  float scale_log2e;
};

__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

template <int G>
__global__ __launch_bounds__(kPfWaves * kWave) void prefill_kernel(PrefillArgs a) {
  const int tile = a.q_tiles - 1 - (int)blockIdx.x;   // heavy (late) tiles first
  const int g = blockIdx.y;
  const int seq = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = wave_uniform(tid >> 6);
  const int col = lane & 31;        // query column of this lane
  const int half = lane >> 5;       // which k half of an MFMA operand

  const int q0 = a.cu_q[seq];
  const int q_len = a.cu_q[seq + 1] - q0;
  if (q0 < 0 || q_len <= 0 || q0 + q_len > a.total_q || tile * kQTile >= q_len) return;
  const int slot = a.slot_ids ? a.slot_ids[seq] : seq;
  if (slot < 0 || slot >= a.num_slots) return;
  const int start = a.q_start[seq];
  const int tok0 = tile * kQTile;                        // first query token of the tile (chunk-relative)
  const int n_q_tile = min(kQTile, q_len - tok0);
  int n_keys = start + q_len;                            // keys cached for this sequence
  n_keys = min(n_keys, a.max_blocks * kBlock);
  const int last_pos = start + tok0 + n_q_tile - 1;      // largest query position in the tile
  const int key_end = min(last_pos + 1, n_keys);
  const int n_ktiles = (key_end + kKTile - 1) / kKTile;
  const int32_t* btrow = a.bt + (int64_t)slot * a.bt_stride;
  const int64_t row_elems = (int64_t)a.n_kv * kHeadDim;

  __shared__ __attribute__((aligned(16))) uint16_t ks[kKTile * kKsStride];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kHeadDim * kVtStride];

  // This lane's query: column col of the tile.
  const int my_q = tok0 + col;                     // chunk-relative token
  const bool q_ok = col < n_q_tile;
  const int my_pos = start + my_q;

  // Loader role: thread -> (key row, 16-byte chunk).
  const int ld_key = tid >> 3;
  const int ld_chunk = tid & 7;

  for (int hh = w; hh < (G > kPfWaves ? G : kPfWaves); hh += kPfWaves) {
    const bool head_active = hh < G;
    const int h = g * G + (head_active ? hh : 0);
    // Q^T operand: 4 k-steps of 8 dims each.
    uint4 qb[4];
#pragma unroll
    for (int ks_ = 0; ks_ < 4; ++ks_) {
      qb[ks_] = make_uint4(0, 0, 0, 0);
      if (q_ok && head_active)
        qb[ks_] = *reinterpret_cast<const uint4*>(a.q + ((int64_t)(q0 + my_q) * a.n_q + h) * kHeadDim + ks_ * 16 +
                                                  half * 8);
    }
    f32x16 o0 = {}, o1 = {};
    float m = -1.0e30f, l = 0.f;

    for (int kt = 0; kt < n_ktiles; ++kt) {
      const int kbase = kt * kKTile;
      // Stage the K tile (row-major) and the V tile (transposed) in LDS.
      {
        const int kk = kbase + ld_key;
        uint4 kv = make_uint4(0, 0, 0, 0), vv = kv;
        if (kk < n_keys) {
          const int blk = btrow[kk / kBlock];
          if (blk >= 0 && blk < a.num_blocks) {
            const int64_t off = ((int64_t)blk * kBlock + kk % kBlock) * row_elems + g * kHeadDim + ld_chunk * 8;
            kv = *reinterpret_cast<const uint4*>(a.k_pool + off);
            vv = *reinterpret_cast<const uint4*>(a.v_pool + off);
          }
        }
        __syncthreads();   // previous tile fully consumed
        *reinterpret_cast<uint4*>(&ks[ld_key * kKsStride + ld_chunk * 8]) = kv;
        const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vt[(ld_chunk * 8 + 2 * j) * kVtStride + ld_key] = (uint16_t)(vw[j] & 0xffffu);
          vt[(ld_chunk * 8 + 2 * j + 1) * kVtStride + ld_key] = (uint16_t)(vw[j] >> 16);
        }
        __syncthreads();
      }
      if (!head_active) continue;

      // S^T = K . Q^T  (rows: keys of the tile, cols: queries)
      f32x16 s = {};
#pragma unroll
      for (int ks_ = 0; ks_ < 4; ++ks_) {
        const uint4 ka = *reinterpret_cast<const uint4*>(&ks[col * kKsStride + ks_ * 16 + half * 8]);
        s = mfma32(ka, qb[ks_], s);
      }
      // Mask and running max for this lane's query.
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kbase + 8 * (i / 4) + 4 * half + (i % 4);
        const bool ok = q_ok && key <= my_pos && key < n_keys;
        s[i] = ok ? s[i] * a.scale_log2e : -INFINITY;
        tmax = fmaxf(tmax, s[i]);
      }
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
      const float mn = fmaxf(m, tmax);
      const float alpha = fast_exp2(m - mn);
      float psum = 0.f;
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(s[i] - mn);
        psum += p[i];
      }
      psum += shfl_xor(psum, 32);
      l = l * alpha + psum;
      m = mn;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        o0[i] *= alpha;
        o1[i] *= alpha;
      }
      // P^T operands: k-step 0 = accumulators 0..7, k-step 1 = 8..15.
      uint4 pb[2];
      pb[0] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                         pack_bf16x2(p[6], p[7]));
      pb[1] = make_uint4(pack_bf16x2(p[8], p[9]), pack_bf16x2(p[10], p[11]), pack_bf16x2(p[12], p[13]),
                         pack_bf16x2(p[14], p[15]));
      // O^T += V^T . P^T ; V^T rows are dims, k slots the same keys as P^T.
#pragma unroll
      for (int kstep = 0; kstep < 2; ++kstep) {
        const int key_a = kstep * 16 + 4 * half;   // keys key_a..+3 and key_a+8..+11
        const uint2 a0lo = *reinterpret_cast<const uint2*>(&vt[col * kVtStride + key_a]);
        const uint2 a0hi = *reinterpret_cast<const uint2*>(&vt[col * kVtStride + key_a + 8]);
        const uint2 a1lo = *reinterpret_cast<const uint2*>(&vt[(col + 32) * kVtStride + key_a]);
        const uint2 a1hi = *reinterpret_cast<const uint2*>(&vt[(col + 32) * kVtStride + key_a + 8]);
        o0 = mfma32(make_uint4(a0lo.x, a0lo.y, a0hi.x, a0hi.y), pb[kstep], o0);
        o1 = mfma32(make_uint4(a1lo.x, a1lo.y, a1hi.x, a1hi.y), pb[kstep], o1);
      }
    }
    if (!head_active || !q_ok) continue;
    // O^T accumulator i holds dim 8*(i/4) + 4*half + i%4 (+32 for o1) of this lane's query.
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* orow = a.out + ((int64_t)(q0 + my_q) * a.n_q + h) * kHeadDim;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int d = 8 * grp + 4 * half;
      uint2 v0, v1;
      v0.x = pack_bf16x2(o0[4 * grp + 0] * inv, o0[4 * grp + 1] * inv);
      v0.y = pack_bf16x2(o0[4 * grp + 2] * inv, o0[4 * grp + 3] * inv);
      v1.x = pack_bf16x2(o1[4 * grp + 0] * inv, o1[4 * grp + 1] * inv);
      v1.y = pack_bf16x2(o1[4 * grp + 2] * inv, o1[4 * grp + 3] * inv);
      *reinterpret_cast<uint2*>(orow + d) = v0;
      *reinterpret_cast<uint2*>(orow + 32 + d) = v1;
    }
  }
}

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_paged_attn_prefill(pkv_bf16* out, const pkv_bf16* q, const int32_t* cu_q_lens,
                                      const int32_t* q_start_pos, const int32_t* slot_ids, const pkv_bf16* k_pool,
                                      const pkv_bf16* v_pool, int num_blocks, const int32_t* block_table,
                                      int64_t bt_row_stride, int num_slots, int max_blocks_per_seq, int num_seqs,
                                      int total_q, int max_q_len, int n_q_heads, int n_kv_heads, int head_dim,
                                      float scale, void* stream) {
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || num_blocks < 0 || num_slots < 0 ||
      max_blocks_per_seq < 0 || bt_row_stride < max_blocks_per_seq || !(scale == scale))
    return PKV_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads) return PKV_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || !ratio_supported(n_q_heads, n_kv_heads)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PKV_OK;
  if (!out || !q || !cu_q_lens || !q_start_pos || !k_pool || !v_pool || !block_table) return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned4(block_table) ||
      !aligned4(cu_q_lens) || !aligned4(q_start_pos) || (slot_ids && !aligned4(slot_ids)))
    return PKV_ERR_MISALIGNED;
  if (num_seqs > 65535 || n_kv_heads > 65535) return PKV_ERR_INVALID_ARG;
  PrefillArgs a;
  a.out = out;
  a.q = q;
  a.cu_q = cu_q_lens;
  a.q_start = q_start_pos;
  a.slot_ids = slot_ids;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.bt = block_table;
  a.bt_stride = bt_row_stride;
  a.num_blocks = num_blocks;
  a.num_slots = num_slots;
  a.max_blocks = max_blocks_per_seq;
  a.n_q = n_q_heads;
  a.n_kv = n_kv_heads;
  a.q_tiles = (max_q_len + kQTile - 1) / kQTile;
  a.total_q = total_q;
  a.scale_log2e = scale * 1.4426950408889634f;
  const int G = n_q_heads / n_kv_heads;
  const void* fn = G == 1 ? (const void*)prefill_kernel<1>
                 : G == 2 ? (const void*)prefill_kernel<2>
                 : G == 4 ? (const void*)prefill_kernel<4>
                          : (const void*)prefill_kernel<8>;
  void* args[] = {&a};
  return launch_status(hipLaunchKernel(fn, dim3(a.q_tiles, n_kv_heads, num_seqs), dim3(kPfWaves * kWave), args, 0,
                                       (hipStream_t)stream));
}

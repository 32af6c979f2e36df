// Paged single-query (decode) attention for gfx950: split-context partitions
// plus a merge kernel.
//
// Source: the Korean page of "An Inference Engine in 1,500 Lines of CUDA: The
// Map" ("What is in the box" table: online softmax and PagedAttention inside
// pagedAttentionKernel, four query heads per KV head), the English page's
// section "The build: two files, two backends" (lane exchanges inside that
// kernel are where the 32- vs 64-lane width matters) and the sixth chapter's
// title (each decode step re-reads every cached K/V of the sequence through the
// block table).
//
// What one workgroup does.  A workgroup of kWaves wave64s owns one
// (sequence, KV head, context partition) and serves all G query heads that
// share the KV head, so each K/V byte is fetched from HBM once for G queries.
// The waves take the partition's 16-token blocks round-robin.  Inside a wave,
// lane = 8 * r + c: c picks 8 of the 64 dims (one 16-byte chunk), r picks rows
// r and r + 8 of the block, so one dwordx4 load per lane covers 8 token rows of
// 128 contiguous bytes (the pool layout [block][16][kv head][64] keeps a head's
// row contiguous).  Scores use the bf16 dot2 instruction (no widening of K);
// the 8 partial dots of a row are summed with three DPP steps.  Every lane
// keeps its own running (max, sum, 8 output dims) per query head over the rows
// it saw; rows are merged at the end: across r with lane exchanges, across
// waves through LDS.  Scores are kept in log2 units (scale * log2 e folded in)
// so the exponentials are single v_exp_f32.  Masked rows (past the context) are
// removed by selects, never by multiplying, so NaN in unused slots cannot leak.
//
// A sequence whose context fits one partition is finished in place (output
// written as bf16); otherwise each partition leaves (max, sum, unnormalised
// output) in the workspace and decode_merge_kernel combines them.
#include "common.h"

namespace pkv {

constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;   // running-max start value (finite: no inf - inf)

struct DecodeArgs {
  uint16_t* out;
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* bt;
  const int32_t* slot_ids;
  const int32_t* ctx_lens;
  float* ws_ml;   // [B][n_q][P][2]  running max (log2 units) and sum per partition
  float* ws_o;    // [B][n_q][P][64] unnormalised output per partition
  int64_t bt_stride;
  int num_blocks;
  int num_slots;
  int max_blocks;
  int n_q;
  int n_kv;
  int P;          // partitions in the grid
  int ps;         // tokens per partition (multiple of 16)
  float scale_log2e;
};

// Context length of batch row b after clipping to the table, and the number of
// partitions that hold tokens of it (the last one runs to the end).
__device__ __forceinline__ void seq_extent(const DecodeArgs& a, int b, int& slot, int& n, int& nparts) {
  slot = a.slot_ids ? a.slot_ids[b] : b;
  n = 0;
  if (slot >= 0 && slot < a.num_slots) {
    n = a.ctx_lens[slot];
    n = n < 0 ? 0 : n;
    n = n > a.max_blocks * kBlock ? a.max_blocks * kBlock : n;
  }
  nparts = (n + a.ps - 1) / a.ps;
  nparts = nparts > a.P ? a.P : nparts;
}

template <int G>
__global__ __launch_bounds__(kWaves * kWave) void decode_partition_kernel(DecodeArgs a) {
  const int kvh = blockIdx.x;
  const int part = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = wave_uniform(threadIdx.x >> 6);
  const int c = lane & 7;
  const int r = lane >> 3;

  int slot, n, nparts;
  seq_extent(a, b, slot, n, nparts);
  if (part >= (nparts > 0 ? nparts : 1)) return;   // partition 0 always runs (zero row for n == 0)
  const int t_begin = part * a.ps;
  const int t_end = (part == nparts - 1) ? n : (nparts == 0 ? 0 : t_begin + a.ps);

  // q chunk for each of the G heads: 8 bf16 = 4 packed dwords.
  uint4 qv[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qv[h] = *reinterpret_cast<const uint4*>(a.q + ((int64_t)b * a.n_q + kvh * G + h) * kHeadDim + c * 8);

  float m[G], l[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[h][i] = 0.f;
  }

  const int jb_begin = t_begin / kBlock;
  const int jb_end = (t_end + kBlock - 1) / kBlock;
  const int64_t row_elems = (int64_t)a.n_kv * kHeadDim;          // elements between token rows
  const int32_t* btrow = a.bt + (int64_t)slot * a.bt_stride;
  const int64_t lane_off = (int64_t)r * row_elems + kvh * kHeadDim + c * 8;
  const int64_t block_elems = (int64_t)kBlock * row_elems;

  auto block_base = [&](int jb) -> int64_t {
    int blk = wave_uniform(btrow[jb]);
    blk = (blk >= 0 && blk < a.num_blocks) ? blk : -1;
    return blk < 0 ? -1 : (int64_t)blk * block_elems;
  };

  int jb = jb_begin + w;
  uint4 k0 = make_uint4(0, 0, 0, 0), k1 = k0, v0 = k0, v1 = k0;
  int64_t base = -1;
  if (jb < jb_end) {
    base = block_base(jb);
    if (base >= 0) {
      const uint16_t* kp = a.k_pool + base + lane_off;
      const uint16_t* vp = a.v_pool + base + lane_off;
      k0 = *reinterpret_cast<const uint4*>(kp);
      k1 = *reinterpret_cast<const uint4*>(kp + 8 * row_elems);
      v0 = *reinterpret_cast<const uint4*>(vp);
      v1 = *reinterpret_cast<const uint4*>(vp + 8 * row_elems);
    }
  }

  for (; jb < jb_end; jb += kWaves) {
    // Issue the next block's loads before working on this one.
    const int jn = jb + kWaves;
    uint4 nk0 = make_uint4(0, 0, 0, 0), nk1 = nk0, nv0 = nk0, nv1 = nk0;
    int64_t nbase = -1;
    if (jn < jb_end) {
      nbase = block_base(jn);
      if (nbase >= 0) {
        const uint16_t* kp = a.k_pool + nbase + lane_off;
        const uint16_t* vp = a.v_pool + nbase + lane_off;
        nk0 = *reinterpret_cast<const uint4*>(kp);
        nk1 = *reinterpret_cast<const uint4*>(kp + 8 * row_elems);
        nv0 = *reinterpret_cast<const uint4*>(vp);
        nv1 = *reinterpret_cast<const uint4*>(vp + 8 * row_elems);
      }
    }

    if (base >= 0) {
      const int tok0 = jb * kBlock + r;
      const bool ok0 = tok0 < t_end;
      const bool ok1 = tok0 + 8 < t_end;
      float s0[G], s1[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d0 = dot2_bf16(qv[h].x, k0.x, 0.f);
        float d1 = dot2_bf16(qv[h].x, k1.x, 0.f);
        d0 = dot2_bf16(qv[h].y, k0.y, d0);
        d1 = dot2_bf16(qv[h].y, k1.y, d1);
        d0 = dot2_bf16(qv[h].z, k0.z, d0);
        d1 = dot2_bf16(qv[h].z, k1.z, d1);
        d0 = dot2_bf16(qv[h].w, k0.w, d0);
        d1 = dot2_bf16(qv[h].w, k1.w, d1);
        s0[h] = ok0 ? sum8(d0) * a.scale_log2e : -INFINITY;
        s1[h] = ok1 ? sum8(d1) * a.scale_log2e : -INFINITY;
      }
      const uint4 z = make_uint4(0, 0, 0, 0);
      const uint4 va = ok0 ? v0 : z;
      const uint4 vb = ok1 ? v1 : z;
      float fa[8] = {bf16_lo(va.x), bf16_hi(va.x), bf16_lo(va.y), bf16_hi(va.y),
                     bf16_lo(va.z), bf16_hi(va.z), bf16_lo(va.w), bf16_hi(va.w)};
      float fb[8] = {bf16_lo(vb.x), bf16_hi(vb.x), bf16_lo(vb.y), bf16_hi(vb.y),
                     bf16_lo(vb.z), bf16_hi(vb.z), bf16_lo(vb.w), bf16_hi(vb.w)};
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mx = fmaxf(s0[h], s1[h]);
        const float mn = fmaxf(m[h], mx);
        const float alpha = fast_exp2(m[h] - mn);
        const float p0 = fast_exp2(s0[h] - mn);
        const float p1 = fast_exp2(s1[h] - mn);
        l[h] = l[h] * alpha + p0 + p1;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[h][i] = o[h][i] * alpha + p0 * fa[i] + p1 * fb[i];
        m[h] = mn;
      }
    }
    k0 = nk0;
    k1 = nk1;
    v0 = nv0;
    v1 = nv1;
    base = nbase;
  }

  // Merge the 8 row groups of the wave (lane bits 3..5).
#pragma unroll
  for (int step = 0; step < 3; ++step) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float m2, l2;
      if (step == 0) {
        m2 = dpp<kDppRowRor8>(m[h]);
        l2 = dpp<kDppRowRor8>(l[h]);
      } else {
        m2 = shfl_xor(m[h], 8 << step);
        l2 = shfl_xor(l[h], 8 << step);
      }
      const float mm = fmaxf(m[h], m2);
      const float a1 = fast_exp2(m[h] - mm);
      const float a2 = fast_exp2(m2 - mm);
      l[h] = l[h] * a1 + l2 * a2;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float o2 = step == 0 ? dpp<kDppRowRor8>(o[h][i]) : shfl_xor(o[h][i], 8 << step);
        o[h][i] = o[h][i] * a1 + o2 * a2;
      }
      m[h] = mm;
    }
  }

  // Merge the waves through LDS.
  __shared__ float sm_ml[kWaves][G][2];
  __shared__ float sm_o[kWaves][G][kHeadDim];
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sm_o[w][h][c * 8 + i] = o[h][i];
      if (c == 0) {
        sm_ml[w][h][0] = m[h];
        sm_ml[w][h][1] = l[h];
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * kHeadDim; e += kWaves * kWave) {
    const int h = e / kHeadDim;
    const int d = e % kHeadDim;
    float mm = sm_ml[0][h][0];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) mm = fmaxf(mm, sm_ml[ww][h][0]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = fast_exp2(sm_ml[ww][h][0] - mm);
      L += sm_ml[ww][h][1] * f;
      O += sm_o[ww][h][d] * f;
    }
    const int64_t row = (int64_t)b * a.n_q + kvh * G + h;
    if (nparts <= 1) {
      a.out[row * kHeadDim + d] = to_bf16(L > 0.f ? O / L : 0.f);
    } else {
      const int64_t pr = row * a.P + part;
      a.ws_o[pr * kHeadDim + d] = O;
      if (d == 0) {
        a.ws_ml[pr * 2 + 0] = mm;
        a.ws_ml[pr * 2 + 1] = L;
      }
    }
  }
}

// One wave per (batch row, query head); lane = output dim.
__global__ __launch_bounds__(kWaves * kWave) void decode_merge_kernel(DecodeArgs a) {
  const int w = threadIdx.x >> 6;
  const int d = threadIdx.x & (kWave - 1);
  const int h = blockIdx.x * kWaves + w;
  const int b = blockIdx.y;
  if (h >= a.n_q) return;
  int slot, n, nparts;
  seq_extent(a, b, slot, n, nparts);
  if (nparts <= 1) return;   // finished by the partition kernel
  const int64_t row = (int64_t)b * a.n_q + h;
  const float* ml = a.ws_ml + row * a.P * 2;
  const float* op = a.ws_o + row * a.P * kHeadDim + d;
  float mm = ml[0];
  for (int p = 1; p < nparts; ++p) mm = fmaxf(mm, ml[2 * p]);
  float L = 0.f, O = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float f = fast_exp2(ml[2 * p] - mm);
    L += ml[2 * p + 1] * f;
    O += op[(int64_t)p * kHeadDim] * f;
  }
  a.out[row * kHeadDim + d] = to_bf16(L > 0.f ? O / L : 0.f);
}

static int auto_partition(int batch, int n_kv, int max_ctx) {
  // Largest partition that still gives the grid about 16 workgroups per CU
  // (256 CUs); never below one block per wave.
  const int target = 4096;
  const int cands[] = {1024, 512, 256, 128};
  for (int ps : cands) {
    const int64_t parts = ((int64_t)max_ctx + ps - 1) / ps;
    if ((int64_t)batch * n_kv * (parts > 0 ? parts : 1) >= target) return ps;
  }
  return kBlock * kWaves;
}

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_decode_partition_size(int batch, int n_kv_heads, int max_context_len) {
  if (batch < 0 || n_kv_heads <= 0 || max_context_len < 0) return 0;
  return auto_partition(batch, n_kv_heads, max_context_len);
}

static int64_t decode_parts(int max_context_len, int ps) {
  const int64_t p = ((int64_t)max_context_len + ps - 1) / ps;
  return p > 0 ? p : 1;
}

extern "C" size_t pkv_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                             int max_context_len, int partition_size) {
  if (batch <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim != kHeadDim || max_context_len < 0)
    return 0;
  const int ps = partition_size > 0 ? partition_size : auto_partition(batch, n_kv_heads, max_context_len);
  const int64_t P = decode_parts(max_context_len, ps);
  if (P <= 1) return 0;
  return (size_t)batch * n_q_heads * P * (2 + kHeadDim) * sizeof(float);
}

extern "C" int pkv_paged_attn_decode(pkv_bf16* out, const pkv_bf16* q, const pkv_bf16* k_pool,
                                     const pkv_bf16* v_pool, int num_blocks, const int32_t* block_table,
                                     int64_t bt_row_stride, int num_slots, int max_blocks_per_seq,
                                     const int32_t* slot_ids, const int32_t* context_lens, int batch,
                                     int max_context_len, int n_q_heads, int n_kv_heads, int head_dim,
                                     float scale, int partition_size, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  if (batch < 0 || num_blocks < 0 || num_slots < 0 || max_blocks_per_seq < 0 ||
      bt_row_stride < max_blocks_per_seq || max_context_len < 0 || partition_size < 0 ||
      partition_size % kBlock || !(scale == scale))
    return PKV_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads) return PKV_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || !ratio_supported(n_q_heads, n_kv_heads)) return PKV_ERR_UNSUPPORTED;
  if (batch == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_table || !context_lens) return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned4(block_table) ||
      !aligned4(context_lens) || (slot_ids && !aligned4(slot_ids)) || (workspace && !aligned16(workspace)))
    return PKV_ERR_MISALIGNED;
  if (batch > 65535) return PKV_ERR_INVALID_ARG;

  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.bt = block_table;
  a.slot_ids = slot_ids;
  a.ctx_lens = context_lens;
  a.bt_stride = bt_row_stride;
  a.num_blocks = num_blocks;
  a.num_slots = num_slots;
  a.max_blocks = max_blocks_per_seq;
  a.n_q = n_q_heads;
  a.n_kv = n_kv_heads;
  a.ps = partition_size > 0 ? partition_size : auto_partition(batch, n_kv_heads, max_context_len);
  const int64_t P = decode_parts(max_context_len, a.ps);
  if (P > 65535) return PKV_ERR_INVALID_ARG;
  a.P = (int)P;
  a.scale_log2e = scale * kLog2e;
  const size_t need = pkv_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_context_len,
                                                 a.ps);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_CAPACITY;
  a.ws_ml = static_cast<float*>(workspace);
  a.ws_o = need > 0 ? a.ws_ml + (size_t)batch * n_q_heads * P * 2 : nullptr;

  const int G = n_q_heads / n_kv_heads;
  const void* fn = G == 1 ? (const void*)decode_partition_kernel<1>
                 : G == 2 ? (const void*)decode_partition_kernel<2>
                 : G == 4 ? (const void*)decode_partition_kernel<4>
                          : (const void*)decode_partition_kernel<8>;
  void* args[] = {&a};
  hipStream_t st = (hipStream_t)stream;
  int rc = launch_status(hipLaunchKernel(fn, dim3(n_kv_heads, a.P, batch), dim3(kWaves * kWave), args, 0, st));
  if (rc != PKV_OK || P <= 1) return rc;
  return launch_status(hipLaunchKernel((const void*)decode_merge_kernel,
                                       dim3((n_q_heads + kWaves - 1) / kWaves, batch), dim3(kWaves * kWave), args,
                                       0, st));
}

// Paged single-query (decode) attention for gfx950, optionally fused with the
// step's RoPE and KV append.
//
// Source: the Korean page of "An Inference Engine in 1,500 Lines of CUDA: The
// Map" ("What is in the box" table: online softmax and PagedAttention inside
// pagedAttentionKernel, four query heads per KV head), the English page's
// section "The build: two files, two backends" (lane exchanges inside that
// kernel are where the 32- vs 64-lane width matters) and the sixth chapter's
// title (each decode step re-reads every cached K/V of the sequence through the
// block table).
//
// With host-known row lengths the call goes to the streaming kernel
// (decode_stream.hip: one workgroup per CU over an equal share of all blocks);
// this file's kernels serve the other cases (lengths only on the device,
// shapes the streaming kernel does not cover).
//
// Work split.  A workgroup of 4 wave64s owns one (sequence, KV head, context
// partition) and serves all G query heads that share the KV head, so each K/V
// byte leaves HBM once for G queries.  The workgroups of one (sequence,
// partition) are placed on one XCD (see decode_item).  The waves take the
// partition's 16-token blocks round-robin, two blocks in flight per wave
// (unconditional, clamped loads into two register sets, so the compiler can
// wait for exactly the older set).  A partition's block ids are read once into
// a VGPR (lane i = block i) and picked with v_readlane, so no scalar load sits
// in the loop.  The per-block arithmetic (scores, lazy-rescaled online
// softmax, p . V, masking by selects) is attn_block.h's.
//
// Merge.  The 8 row groups of a wave are summed pairwise with DPP and the rest
// through LDS together with the other waves (each wave carries its own max).
// A context that fits one partition is finished in place.  Otherwise every
// partition stores (max, sum, unnormalised output) in the workspace and a
// second, small kernel merges them (the kernel boundary orders the memory
// traffic; merging inside the first kernel would need an agent-scope release
// per workgroup, an L2 write-back on this chip, which costs far more).
//
// Fused variant (the decode step).  The query and the new token's key are
// rotated in registers from the RoPE table (same arithmetic as the RoPE
// kernel), the new token (position context_len - 1) takes part in the
// attention from registers, and the workgroup of the last partition writes the
// rotated key and the value into their pool row at the end of the kernel.
#include "attn_block.h"
#include "decode_api.h"
#include "kv_policy.h"

#include <algorithm>
#include <atomic>
#include <mutex>

namespace pkv {

constexpr int kWaves = 4;
constexpr int kMaxPlanSeqs = 256;     // batch rows a host schedule can describe

struct DecodeArgs {
  uint16_t* out;
  const uint16_t* q;
  const uint16_t* k_new;       // fused: new keys (before RoPE) [B][n_kv][64]
  const uint16_t* v_new;       // fused: new values [B][n_kv][64]
  uint16_t* k_pool;
  uint16_t* v_pool;
  const int32_t* bt;
  const int32_t* slot_ids;
  const int32_t* ctx_lens;
  const float2* rope;          // fused: cos/sin table [max_pos][32]
  float* ws_o;                 // [B][n_kv][P][G][64] unnormalised partial outputs
  float* ws_ml;                // [B][n_kv][P][G][2]  partial (max, sum)
  uint32_t* errors;            // device error flags (errors.hip), or null
  int64_t bt_stride;
  int num_blocks;
  int num_slots;
  int max_blocks;
  int n_q;
  int n_kv;
  int P;                       // partitions in the grid
  int ps;                      // tokens per partition (multiple of 16)
  int max_pos;
  int batch;
  float scale_log2e;
  int kv_nt;                   // K/V loads marked non-temporal
  // Host schedule (plan_seqs > 0), built from host-known row lengths.  Row b
  // has length plan_n[b] and is cut into partitions of plan_ps[b] * 16
  // tokens (only its last one shorter).  Items [0, full_items) are the
  // partitions that are not a row's last one, row b owning items plan_pre[b]
  // .. plan_pre[b+1]-1; item full_items + j is the last partition of row
  // plan_last[j], longest first.
  int plan_seqs;
  int full_items;
  int n_items;
  int32_t plan_pre[kMaxPlanSeqs + 1];
  int32_t plan_n[kMaxPlanSeqs];
  uint16_t plan_ps[kMaxPlanSeqs];
  uint16_t plan_last[kMaxPlanSeqs];
};

// One workgroup's share: row b (table row `slot`), KV head kvh, partition
// `part` of `nparts` covering tokens [t_begin, t_end) of the n in context.
struct Item {
  int b, kvh, part, slot, n, nparts, t_begin, t_end;
};

// Workgroup id -> (KV head, partition, sequence).  Workgroups are handed to the
// 8 XCDs round-robin by linear id, so ids are arranged in groups of 8 items
// (item = sequence * P + partition) x n_kv heads with the item's low 3 bits in
// the id's low 3 bits: all KV heads of an item run on the same XCD at about the
// same time and fetch the 128-byte head rows of each 1 KB token row together.
// (One XCD per head instead costs about 15% of HBM bandwidth on this layout.)
// Without a host schedule, item = sequence * P + partition over the grid that
// max_context_len implies (items past a sequence's length exit at once); with
// one, only real partitions are launched, longest first.
__device__ __forceinline__ int clip_len(const DecodeArgs& a, int n) {
  if (n > a.max_blocks * kBlock && threadIdx.x == 0) report_error(a.errors, PKV_DEVERR_LONG_CONTEXT);
  return n < 0 ? 0 : (n > a.max_blocks * kBlock ? a.max_blocks * kBlock : n);
}

// Row b's extent from the host schedule (no memory access) or, without one,
// from context_lens on the device with the uniform partition size.
__device__ __forceinline__ void row_extent(const DecodeArgs& a, int b, int& slot, int& n, int& nparts, int& ps) {
  slot = a.slot_ids ? a.slot_ids[b] : b;
  const bool slot_ok = slot >= 0 && slot < a.num_slots && a.num_blocks > 0;
  if (!(slot >= 0 && slot < a.num_slots) && threadIdx.x == 0) report_error(a.errors, PKV_DEVERR_BAD_SLOT);
  slot = slot_ok ? slot : 0;
  if (a.plan_seqs > 0) {
    n = slot_ok ? a.plan_n[b] : 0;
    nparts = n > 0 ? a.plan_pre[b + 1] - a.plan_pre[b] + 1 : 0;
    ps = a.plan_ps[b] * kBlock;
  } else {
    n = slot_ok ? clip_len(a, a.ctx_lens[slot]) : 0;
    nparts = (n + a.ps - 1) / a.ps;
    nparts = nparts > a.P ? a.P : nparts;
    ps = a.ps;
  }
}

__device__ __forceinline__ bool decode_item(const DecodeArgs& a, Item& it) {
  const int id = blockIdx.x;
  const int grp = id / (8 * a.n_kv);
  const int in = id - grp * 8 * a.n_kv;
  it.kvh = in >> 3;
  const int item = grp * 8 + (in & 7);
  int ps;
  if (a.plan_seqs > 0) {
    if (item >= a.n_items) return false;
    bool last;
    if (item < a.full_items) {
      int lo = 0, hi = a.plan_seqs;            // plan_pre[lo] <= item < plan_pre[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.plan_pre[mid] <= item) lo = mid; else hi = mid;
      }
      it.b = lo;
      it.part = item - a.plan_pre[lo];
      last = false;
    } else {
      it.b = a.plan_last[item - a.full_items];
      last = true;
    }
    if (it.b >= a.batch) return false;
    row_extent(a, it.b, it.slot, it.n, it.nparts, ps);
    if (last) it.part = it.nparts > 0 ? it.nparts - 1 : 0;
  } else {
    it.b = item / a.P;
    it.part = item - it.b * a.P;
    if (it.b >= a.batch) return false;
    row_extent(a, it.b, it.slot, it.n, it.nparts, ps);
    // partition 0 always runs (it writes the zero row of an empty context)
    if (it.part >= (it.nparts > 0 ? it.nparts : 1)) return false;
  }
  it.t_begin = it.part * ps;
  it.t_end = (it.part == it.nparts - 1) ? it.n : (it.nparts == 0 ? 0 : it.t_begin + ps);
  return true;
}

template <int G, bool FUSED, bool NT>
__global__ __launch_bounds__(kWaves * kWave) void decode_kernel(DecodeArgs a) {
  Item it;
  if (!decode_item(a, it)) return;
  const int kvh = it.kvh, part = it.part, b = it.b, slot = it.slot, n = it.n, nparts = it.nparts;
  const int t_begin = it.t_begin, t_end = it.t_end;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = wave_uniform(tid >> 6);
  const int c = lane & 7;
  const int r = lane >> 3;
  const int32_t* btrow = a.bt + (int64_t)slot * a.bt_stride;
  const int jb_begin = t_begin / kBlock;
  const int64_t row_elems = (int64_t)a.n_kv * kHeadDim;

  // This lane's chunk of the G query heads (rotated here when fused).
  uint4 qv[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qv[h] = *reinterpret_cast<const uint4*>(a.q + ((int64_t)b * a.n_q + kvh * G + h) * kHeadDim + c * 8);
  const int pos_new = n - 1;              // the token appended this step (fused)
  uint4 knew = make_uint4(0, 0, 0, 0), vnew = knew;
  if constexpr (FUSED) {
    if (n > 0) {
      knew = *reinterpret_cast<const uint4*>(a.k_new + ((int64_t)b * a.n_kv + kvh) * kHeadDim + c * 8);
      vnew = *reinterpret_cast<const uint4*>(a.v_new + ((int64_t)b * a.n_kv + kvh) * kHeadDim + c * 8);
      if (pos_new < a.max_pos) {
        float2 cs[8];
        const float2* trow = a.rope + (int64_t)pos_new * (kHeadDim / 2) + (c & 3) * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) cs[j] = trow[j];
#pragma unroll
        for (int h = 0; h < G; ++h) qv[h] = rope_chunk(qv[h], cs, c);
        knew = rope_chunk(knew, cs, c);
      }
    }
  }

  OnlineSoftmax<G> acc;
  acc.reset();
  const float C = a.scale_log2e;
  const float invC = 1.0f / C;

  // In the fused step the new token's pool row is not read: it joins from
  // registers after the loop.
  const int t_loop_end = (FUSED && part == nparts - 1 && n > 0) ? n - 1 : t_end;
  const int nb = (t_loop_end + kBlock - 1) / kBlock - jb_begin;
  const uint32_t block_bytes = (uint32_t)(kBlock * row_elems * 2);
  const uint32_t lane_off = (uint32_t)(((int64_t)r * row_elems + kvh * kHeadDim + c * 8) * 2);
  const uint32_t lane_off8 = lane_off + (uint32_t)(8 * row_elems * 2);   // row r + 8
  const char* kbase = reinterpret_cast<const char*>(a.k_pool);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool);

  for (int cb = 0; cb < nb; cb += kWave) {
    const int ncb = min(kWave, nb - cb);
    int tab = btrow[jb_begin + cb + min(lane, ncb - 1)];
    if (lane < ncb && !(tab >= 0 && tab < a.num_blocks)) report_error(a.errors, PKV_DEVERR_BAD_BLOCK);
    tab = (tab >= 0 && tab < a.num_blocks && lane < ncb) ? tab : -1;
    if (w >= ncb) continue;

    auto issue = [&](KVRegs& R, int i) {
      int blk = __builtin_amdgcn_readlane(tab, min(i, ncb - 1));
      blk = blk < 0 ? 0 : blk;
      const auto rk = buf_rsrc(kbase + (size_t)blk * block_bytes, block_bytes);
      const auto rv = buf_rsrc(vbase + (size_t)blk * block_bytes, block_bytes);
      buf_load_kv4<NT>(rk, lane_off, lane_off8, rv, lane_off, lane_off8, R.k0, R.k1, R.v0, R.v1);
    };

    // One block: branch-free apart from the rare rescale.  Rows past the
    // context and rows of an unusable block are removed by selects.
    auto process = [&](const KVRegs& R, int i) {
      const bool blk_ok = __builtin_amdgcn_readlane(tab, i) >= 0;
      const int tok0 = (jb_begin + cb + i) * kBlock + r;
      acc.block(qv, R, blk_ok && tok0 < t_loop_end, blk_ok && tok0 + 8 < t_loop_end, C, invC);
    };

    KVRegs X, Y;
    issue(X, w);
    issue(Y, w + kWaves);
    for (int i = w;; i += 2 * kWaves) {
      process(X, i);
      issue(X, i + 2 * kWaves);
      if (i + kWaves >= ncb) break;
      process(Y, i + kWaves);
      issue(Y, i + 3 * kWaves);
      if (i + 2 * kWaves >= ncb) break;
    }
  }

  if constexpr (FUSED) {
    // The new token, from registers, counted once (row group 0 of wave 0).
    if (part == nparts - 1 && n > 0 && w == 0) acc.token(qv, knew, vnew, r == 0, C, invC);
  }

  // ---- merge: row-group pairs by DPP, the rest through LDS ----------------
#pragma unroll
  for (int h = 0; h < G; ++h) {
    acc.l[h] += dpp<kDppRowRor8>(acc.l[h]);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc.o[h][j] += dpp<kDppRowRor8>(acc.o[h][j]);
  }
  __shared__ float sm_o[kWaves][4][G][kHeadDim];
  __shared__ float sm_l[kWaves][4][G];
  __shared__ float sm_m[kWaves][G];
  if ((r & 1) == 0) {
    const int grp = r >> 1;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      *reinterpret_cast<float4*>(&sm_o[w][grp][h][c * 8]) =
          make_float4(acc.o[h][0], acc.o[h][1], acc.o[h][2], acc.o[h][3]);
      *reinterpret_cast<float4*>(&sm_o[w][grp][h][c * 8 + 4]) =
          make_float4(acc.o[h][4], acc.o[h][5], acc.o[h][6], acc.o[h][7]);
      if (c == 0) sm_l[w][grp][h] = acc.l[h];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) sm_m[w][h] = acc.m[h];
  }
  __syncthreads();

  const int64_t grp_row = (int64_t)b * a.n_kv + kvh;          // (sequence, kv head)
  for (int e = tid; e < G * kHeadDim; e += kWaves * kWave) {
    const int h = e / kHeadDim;
    const int d = e % kHeadDim;
    float mm = sm_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) mm = fmaxf(mm, sm_m[ww][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = fast_exp2(sm_m[ww][h] - mm);
      L += f * (sm_l[ww][0][h] + sm_l[ww][1][h] + sm_l[ww][2][h] + sm_l[ww][3][h]);
      O += f * (sm_o[ww][0][h][d] + sm_o[ww][1][h][d] + sm_o[ww][2][h][d] + sm_o[ww][3][h][d]);
    }
    if (nparts <= 1) {
      a.out[((int64_t)b * a.n_q + kvh * G + h) * kHeadDim + d] = to_bf16(L > 0.f ? O / L : 0.f);
    } else {
      const int64_t pr = (grp_row * a.P + part) * G + h;
      a.ws_o[pr * kHeadDim + d] = O;
      if (d == 0) {
        a.ws_ml[pr * 2 + 0] = mm;
        a.ws_ml[pr * 2 + 1] = L;
      }
    }
  }

  if constexpr (FUSED) {
    // Append the rotated key and the value of the new token (one 128-byte row
    // each); no workgroup reads this row during the call.
    if (part == nparts - 1 && n > 0 && tid < 8) {
      const int blk = btrow[pos_new / kBlock];
      if (!(blk >= 0 && blk < a.num_blocks)) report_error(a.errors, PKV_DEVERR_BAD_BLOCK);
      if (blk >= 0 && blk < a.num_blocks) {
        const int64_t off = ((int64_t)blk * kBlock + pos_new % kBlock) * row_elems + kvh * kHeadDim + tid * 8;
        *reinterpret_cast<uint4*>(a.k_pool + off) = knew;
        *reinterpret_cast<uint4*>(a.v_pool + off) = vnew;
      }
    }
  }
}

// Split-context merge: one workgroup per (sequence, KV head), thread = (head,
// dim).  M = max_p m_p, L = sum_p 2^(m_p - M) l_p, out = sum_p 2^(m_p - M) o_p / L,
// taken eight partitions at a time (independent loads) with a running merge.
template <int G>
__global__ __launch_bounds__(kWaves * kWave) void decode_merge_kernel(DecodeArgs a) {
  const int kvh = blockIdx.x;
  const int b = blockIdx.y;
  int slot, n, nparts, ps;
  row_extent(a, b, slot, n, nparts, ps);
  if (nparts <= 1) return;            // finished by the partition kernel
  const int64_t grp_row = (int64_t)b * a.n_kv + kvh;
  for (int e = threadIdx.x; e < G * kHeadDim; e += kWaves * kWave) {
    const int h = e / kHeadDim;
    const int d = e % kHeadDim;
    const int64_t base = grp_row * a.P * G + h;
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int p0 = 0; p0 < nparts; p0 += 8) {
      float mv[8], lv[8], ov[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool in = p0 + j < nparts;
        const int64_t pr = base + (int64_t)(in ? p0 + j : p0) * G;
        mv[j] = in ? a.ws_ml[pr * 2] : -INFINITY;
        lv[j] = a.ws_ml[pr * 2 + 1];
        ov[j] = a.ws_o[pr * kHeadDim + d];
      }
      float mm = M;
#pragma unroll
      for (int j = 0; j < 8; ++j) mm = fmaxf(mm, mv[j]);
      const float f0 = M == -INFINITY ? 0.f : fast_exp2(M - mm);
      L *= f0;
      O *= f0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float f = mv[j] == -INFINITY ? 0.f : fast_exp2(mv[j] - mm);
        L += f * lv[j];
        O += f * ov[j];
      }
      M = mm;
    }
    a.out[((int64_t)b * a.n_q + kvh * G + h) * kHeadDim + d] = to_bf16(L > 0.f ? O / L : 0.f);
  }
}

static int auto_partition(int batch, int n_kv, int max_ctx) {
  // Largest partition that still gives the grid about 16 workgroups per CU
  // (256 CUs); never below two blocks per wave.
  const int target = 4096;
  const int cands[] = {1024, 512, 256};
  for (int ps : cands) {
    const int64_t parts = ((int64_t)max_ctx + ps - 1) / ps;
    if ((int64_t)batch * n_kv * (parts > 0 ? parts : 1) >= target) return ps;
  }
  return 2 * kBlock * kWaves;
}

static int64_t decode_parts(int max_context_len, int ps) {
  const int64_t p = ((int64_t)max_context_len + ps - 1) / ps;
  return p > 0 ? p : 1;
}

struct WsLayout {
  size_t o_bytes, ml_bytes, total;
};

static WsLayout ws_layout(int batch, int n_q, int n_kv, int64_t P) {
  WsLayout L;
  if (P <= 1) {
    L.o_bytes = L.ml_bytes = L.total = 0;
    return L;
  }
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  L.o_bytes = up((size_t)batch * n_q * P * kHeadDim * sizeof(float));
  L.ml_bytes = up((size_t)batch * n_q * P * 2 * sizeof(float));
  L.total = L.o_bytes + L.ml_bytes;
  return L;
}

template <bool FUSED, bool NT>
static const void* pick_kernel_nt(int G) {
  return G == 1 ? (const void*)decode_kernel<1, FUSED, NT>
       : G == 2 ? (const void*)decode_kernel<2, FUSED, NT>
       : G == 4 ? (const void*)decode_kernel<4, FUSED, NT>
                : (const void*)decode_kernel<8, FUSED, NT>;
}
template <bool FUSED>
static const void* pick_kernel(int G, bool nt) {
  return nt ? pick_kernel_nt<FUSED, true>(G) : pick_kernel_nt<FUSED, false>(G);
}

// Longest-first schedule from host-known row lengths.  Row b (n tokens) is
// cut into round(n / ps) partitions of equal, block-aligned size (so no
// partition is a sliver), at most P of them.  Every non-last partition comes
// first, then each row's last partition by decreasing length, so the in-order
// hardware dispatcher acts as a longest-first list scheduler.  Rows of length
// 0 keep their partition 0 (the zero row).
static void build_plan(DecodeArgs& a, const int32_t* row_lens_host, int batch) {
  a.plan_pre[0] = 0;
  int last_len[kMaxPlanSeqs];
  uint16_t order[kMaxPlanSeqs];
  for (int b = 0; b < batch; ++b) {
    int n = row_lens_host[b];
    n = n < 0 ? 0 : (n > a.max_blocks * kBlock ? a.max_blocks * kBlock : n);
    int np = n > 0 ? (n + a.ps / 2) / a.ps : 0;
    np = n > 0 && np < 1 ? 1 : np;
    np = np > a.P ? a.P : np;
    int ps_b = np > 0 ? ((n + np - 1) / np + kBlock - 1) / kBlock * kBlock : a.ps;
    np = n > 0 ? (n + ps_b - 1) / ps_b : 0;
    a.plan_n[b] = n;
    a.plan_ps[b] = (uint16_t)(ps_b / kBlock);
    a.plan_pre[b + 1] = a.plan_pre[b] + (np > 1 ? np - 1 : 0);
    last_len[b] = np > 0 ? n - (np - 1) * ps_b : 0;
    order[b] = (uint16_t)b;
  }
  for (int i = 1; i < batch; ++i) {     // stable, by decreasing last-partition length
    const uint16_t o = order[i];
    int j = i;
    while (j > 0 && last_len[order[j - 1]] < last_len[o]) { order[j] = order[j - 1]; --j; }
    order[j] = o;
  }
  for (int i = 0; i < batch; ++i) a.plan_last[i] = order[i];
  a.plan_seqs = batch;
  a.full_items = a.plan_pre[batch];
  a.n_items = a.full_items + batch;
}

// The per-partition kernels (and their merge) for a checked call.
static int partition_launch(bool fused, DecodeArgs& a, int batch, int max_context_len, int partition_size,
                            const int32_t* row_lens_host, void* workspace, hipStream_t st) {
  a.ps = partition_size > 0 ? partition_size : auto_partition(batch, a.n_kv, max_context_len);
  const int64_t P = decode_parts(max_context_len, a.ps);
  a.P = (int)P;
  const WsLayout L = ws_layout(batch, a.n_q, a.n_kv, P);
  char* ws = static_cast<char*>(workspace);
  a.ws_o = L.total ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_ml = L.total ? reinterpret_cast<float*>(ws + L.o_bytes) : nullptr;
  const int G = a.n_q / a.n_kv;
  a.batch = batch;
  a.plan_seqs = 0;
  if (row_lens_host && batch <= kMaxPlanSeqs && a.max_blocks <= 0xffff) build_plan(a, row_lens_host, batch);
  const int64_t items = a.plan_seqs > 0 ? (int64_t)a.n_items : (int64_t)batch * a.P;
  const int64_t grid = (items + 7) / 8 * 8 * a.n_kv;
  const void* fn = fused ? pick_kernel<true>(G, a.kv_nt != 0) : pick_kernel<false>(G, a.kv_nt != 0);
  void* args[] = {&a};
  const int rc = launch_status(hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kWaves * kWave), args, 0, st));
  if (rc != PKV_OK || P <= 1) return rc;
  const void* mg = G == 1 ? (const void*)decode_merge_kernel<1>
                 : G == 2 ? (const void*)decode_merge_kernel<2>
                 : G == 4 ? (const void*)decode_merge_kernel<4>
                          : (const void*)decode_merge_kernel<8>;
  return launch_status(hipLaunchKernel(mg, dim3(a.n_kv, batch), dim3(kWaves * kWave), args, 0, st));
}

__global__ void zero_kernel(uint32_t* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_decode_partition_size(int batch, int n_kv_heads, int max_context_len) {
  if (batch < 0 || n_kv_heads <= 0 || max_context_len < 0) return 0;
  return auto_partition(batch, n_kv_heads, max_context_len);
}

extern "C" size_t pkv_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                             int max_context_len, int partition_size) {
  if (batch <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim != kHeadDim || max_context_len < 0 ||
      partition_size < 0)
    return 0;
  const int ps = partition_size > 0 ? partition_size : auto_partition(batch, n_kv_heads, max_context_len);
  return std::max(ws_layout(batch, n_q_heads, n_kv_heads, decode_parts(max_context_len, ps)).total,
                  decode_plan_offset(n_q_heads) + kStreamPlanBytes);
}

extern "C" int pkv_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes == 0) return PKV_OK;
  if (!workspace) return PKV_ERR_NULL;
  if (!aligned16(workspace)) return PKV_ERR_MISALIGNED;
  uint32_t* p = static_cast<uint32_t*>(workspace);
  size_t n = workspace_bytes / 4;
  const size_t grid = (n + 255) / 256;
  if (grid > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  void* args[] = {&p, &n};
  return launch_status(hipLaunchKernel((const void*)zero_kernel, dim3((unsigned)grid), dim3(256), args, 0,
                                       (hipStream_t)stream));
}

static int decode_common_checks(const pkv_bf16* out, const pkv_bf16* q, const pkv_bf16* k_pool,
                                const pkv_bf16* v_pool, int num_blocks, const int32_t* block_table,
                                int64_t bt_row_stride, int num_slots, int max_blocks_per_seq,
                                const int32_t* slot_ids, const int32_t* context_lens, int batch,
                                int max_context_len, int n_q_heads, int n_kv_heads, int head_dim, float scale,
                                int partition_size, void* workspace) {
  if (batch < 0 || num_blocks < 0 || num_slots < 0 || max_blocks_per_seq < 0 ||
      bt_row_stride < max_blocks_per_seq || max_context_len < 0 || partition_size < 0 ||
      partition_size % kBlock || !(scale > 0.f && scale < 3.0e38f))
    return PKV_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads) return PKV_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || !ratio_supported(n_q_heads, n_kv_heads)) return PKV_ERR_UNSUPPORTED;
  if (batch == 0) return -1;   // nothing to do
  if (!out || !q || !k_pool || !v_pool || !block_table || !context_lens) return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned4(block_table) ||
      !aligned4(context_lens) || (slot_ids && !aligned4(slot_ids)) || (workspace && !aligned16(workspace)))
    return PKV_ERR_MISALIGNED;
  if (batch > 65535 || n_kv_heads > 65535) return PKV_ERR_INVALID_ARG;
  if ((int64_t)kBlock * n_kv_heads * kHeadDim * 2 * (int64_t)num_blocks <= 0 && num_blocks > 0)
    return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

static DecodeArgs base_args(const DecodeCall& c) {
  DecodeArgs a{};
  a.out = c.out;
  a.q = c.q;
  a.k_new = c.k_new;
  a.v_new = c.v_new;
  a.k_pool = c.k_pool;
  a.v_pool = c.v_pool;
  a.bt = c.block_table;
  a.slot_ids = c.slot_ids;
  a.ctx_lens = c.context_lens;
  a.rope = reinterpret_cast<const float2*>(c.cos_sin);
  a.max_pos = c.max_pos;
  a.bt_stride = c.bt_row_stride;
  a.num_blocks = c.num_blocks;
  a.num_slots = c.num_slots;
  a.max_blocks = c.max_blocks_per_seq;
  a.n_q = c.n_q_heads;
  a.n_kv = c.n_kv_heads;
  a.scale_log2e = c.scale * kLog2e;
  a.errors = device_errors_ptr();
  return a;
}

namespace pkv {

namespace {
std::atomic<int> g_kv_read{PKV_KV_READ_STREAM};   // process-wide K/V read policy
thread_local int t_kv_read = 0;                   // this thread's override, 0 = none
}  // namespace

int kv_read_policy_now() { return t_kv_read ? t_kv_read : g_kv_read.load(std::memory_order_relaxed); }

int kv_read_override(int policy) {
  const int prev = t_kv_read;
  t_kv_read = policy;
  return prev;
}

void kv_read_set(int policy) { g_kv_read.store(policy, std::memory_order_relaxed); }
int kv_read_setting() { return g_kv_read.load(std::memory_order_relaxed); }

int decode_prepare(const DecodeCall& c, DecodeLaunch* L) {
  L->c = c;
  L->path = 0;
  L->kv_nt = kv_read_policy_now() == PKV_KV_READ_STREAM;
  int rc = decode_common_checks(c.out, c.q, c.k_pool, c.v_pool, c.num_blocks, c.block_table, c.bt_row_stride,
                                c.num_slots, c.max_blocks_per_seq, c.slot_ids, c.context_lens, c.batch,
                                c.max_context_len, c.n_q_heads, c.n_kv_heads, c.head_dim, c.scale,
                                c.partition_size, c.workspace);
  if (rc < 0) return c.out_prev ? PKV_ERR_INVALID_ARG : PKV_OK;   // empty batch: nothing to do
  if (rc != PKV_OK) return rc;
  if (c.fused) {
    if (c.max_pos < 1) return PKV_ERR_INVALID_ARG;
    if (!c.k_new || !c.v_new || !c.cos_sin) return PKV_ERR_NULL;
    if (!aligned16(c.k_new) || !aligned16(c.v_new) || !aligned16(c.cos_sin)) return PKV_ERR_MISALIGNED;
  }
  if (c.records_half < 0 || c.records_half > 1) return PKV_ERR_INVALID_ARG;
  // the streaming kernel: host row lengths and room for its records
  const size_t R = stream_records_bytes(c.n_q_heads);
  const size_t need = (size_t)(c.records_half + 1) * R;
  if (c.row_lens_host && c.workspace && c.workspace_bytes >= need && (!c.out_prev || c.workspace_bytes >= 2 * R)) {
    char* ws = static_cast<char*>(c.workspace);
    StreamCall sc{};
    sc.out = c.out;
    sc.q = c.q;
    sc.k_new = c.k_new;
    sc.v_new = c.v_new;
    sc.k_pool = c.k_pool;
    sc.v_pool = c.v_pool;
    sc.num_blocks = c.num_blocks;
    sc.block_table = c.block_table;
    sc.bt_row_stride = c.bt_row_stride;
    sc.num_slots = c.num_slots;
    sc.max_blocks = c.max_blocks_per_seq;
    sc.slot_ids = c.slot_ids;
    sc.slot_ids_host = c.slot_ids_host;
    sc.row_lens_host = c.row_lens_host;
    sc.batch = c.batch;
    sc.n_q = c.n_q_heads;
    sc.n_kv = c.n_kv_heads;
    sc.cos_sin = c.cos_sin;
    sc.max_pos = c.max_pos;
    sc.scale = c.scale;
    sc.records = reinterpret_cast<float*>(ws + c.records_half * R);
    sc.records_bytes = R;
    sc.out_prev = c.out_prev;
    sc.records_prev = c.out_prev ? reinterpret_cast<const float*>(ws + (1 - c.records_half) * R) : nullptr;
    sc.plan_dev = c.plan_dev;
    sc.fixed_shape = c.fixed_shape;
    sc.plan_out = c.plan_out;
    sc.chain_plan = c.chain_plan;
    sc.kv_nt = L->kv_nt;
    if (stream_prepare(c.fused, sc, &L->s) == PKV_OK) {
      L->path = 1;
      return PKV_OK;
    }
  }
  // chaining and device plans exist on the streaming path only
  if (c.out_prev || c.plan_dev) return c.plan_dev ? PKV_ERR_UNSUPPORTED : PKV_ERR_INVALID_ARG;
  // the per-partition kernels
  const int ps = c.partition_size > 0 ? c.partition_size : auto_partition(c.batch, c.n_kv_heads, c.max_context_len);
  const int64_t P = decode_parts(c.max_context_len, ps);
  if (P > 65535) return PKV_ERR_INVALID_ARG;
  const WsLayout W = ws_layout(c.batch, c.n_q_heads, c.n_kv_heads, P);
  if (W.total > 0 && (!c.workspace || c.workspace_bytes < W.total)) return PKV_ERR_CAPACITY;
  const int64_t items = (int64_t)c.batch * P;   // the host schedule launches at most this many
  if ((items + 7) / 8 * 8 * c.n_kv_heads > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  L->path = 2;
  return PKV_OK;
}

size_t decode_plan_offset(int n_q_heads) { return 2 * stream_records_bytes(n_q_heads); }

int decode_retarget(const DecodeLaunch& base, const int32_t* block_table, const StreamPlan* plan_dev,
                    DecodeLaunch* out) {
  if (base.c.out_prev || base.c.plan_dev || base.c.fixed_shape) return PKV_ERR_INVALID_ARG;
  if (base.path != 0 && !block_table) return PKV_ERR_NULL;
  if (base.path != 0 && !aligned4(block_table)) return PKV_ERR_MISALIGNED;
  if (plan_dev && (base.path != 1 || base.c.plan_out != plan_dev)) return PKV_ERR_INVALID_ARG;
  *out = base;
  out->c.block_table = block_table;
  out->c.plan_out = nullptr;
  out->c.plan_dev = plan_dev;
  if (base.path == 1) {
    StreamArgs& a = out->s.a;
    a.bt = block_table;
    a.plan_out = nullptr;
    if (plan_dev) {
      out->s.devplan = true;
      a.plan_dev = plan_dev;
    }
  }
  return PKV_OK;
}

bool decode_chainable(const DecodeLaunch& L) {
  return L.path == 1 && !L.s.long_rows && L.c.workspace_bytes >= decode_plan_offset(L.c.n_q_heads) + kStreamPlanBytes;
}

int decode_enqueue(const DecodeLaunch& L, hipStream_t st, bool merge) {
  if (L.path == 0) return PKV_OK;
  if (L.path == 1) return stream_enqueue(L.s, st, merge);
  DecodeArgs a = base_args(L.c);
  a.kv_nt = L.kv_nt ? 1 : 0;
  return partition_launch(L.c.fused, a, L.c.batch, L.c.max_context_len, L.c.partition_size, L.c.row_lens_host,
                          L.c.workspace, st);
}

int decode_finish(const DecodeLaunch& L, hipStream_t st) {
  return L.path == 1 ? stream_merge_enqueue(L.s, st) : PKV_OK;
}

}  // namespace pkv

extern "C" int pkv_set_kv_read_policy(int policy) {
  if (policy != PKV_KV_READ_STREAM && policy != PKV_KV_READ_REUSE) return PKV_ERR_INVALID_ARG;
  pkv::kv_read_set(policy);
  return PKV_OK;
}

extern "C" int pkv_kv_read_policy(void) { return pkv::kv_read_setting(); }

extern "C" int pkv_paged_read_probe(const pkv_bf16* k_pool, const pkv_bf16* v_pool, int num_blocks,
                                    const int32_t* block_table, int64_t bt_row_stride, int num_slots,
                                    int max_blocks_per_seq, const int32_t* slot_ids, const int32_t* row_lens_host,
                                    int batch, int n_kv_heads, int head_dim, uint32_t* sink, void* stream) {
  if (batch < 0 || num_blocks < 0 || num_slots < 0 || max_blocks_per_seq < 0 || bt_row_stride < max_blocks_per_seq)
    return PKV_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return PKV_ERR_UNSUPPORTED;
  if (batch == 0) return PKV_OK;
  if (!k_pool || !v_pool || !block_table || !row_lens_host || !sink) return PKV_ERR_NULL;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned4(block_table) || !aligned4(sink) ||
      (slot_ids && !aligned4(slot_ids)))
    return PKV_ERR_MISALIGNED;
  if (!slot_ids && batch > num_slots) return PKV_ERR_INVALID_ARG;
  StreamCall c{};
  c.k_pool = const_cast<uint16_t*>(k_pool);
  c.v_pool = const_cast<uint16_t*>(v_pool);
  c.num_blocks = num_blocks;
  c.block_table = block_table;
  c.bt_row_stride = bt_row_stride;
  c.num_slots = num_slots;
  c.max_blocks = max_blocks_per_seq;
  c.slot_ids = slot_ids;
  c.row_lens_host = row_lens_host;
  c.batch = batch;
  c.n_kv = n_kv_heads;
  c.kv_nt = kv_read_policy_now() == PKV_KV_READ_STREAM;
  return stream_read_probe(c, sink, static_cast<hipStream_t>(stream));
}

extern "C" int pkv_paged_attn_decode(pkv_bf16* out, const pkv_bf16* q, const pkv_bf16* k_pool,
                                     const pkv_bf16* v_pool, int num_blocks, const int32_t* block_table,
                                     int64_t bt_row_stride, int num_slots, int max_blocks_per_seq,
                                     const int32_t* slot_ids, const int32_t* context_lens,
                                     const int32_t* row_lens_host, int batch, int max_context_len, int n_q_heads,
                                     int n_kv_heads, int head_dim, float scale, int partition_size,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  DecodeCall c{};
  c.fused = false;
  c.out = out;
  c.q = q;
  c.k_pool = const_cast<pkv_bf16*>(k_pool);
  c.v_pool = const_cast<pkv_bf16*>(v_pool);
  c.num_blocks = num_blocks;
  c.block_table = block_table;
  c.bt_row_stride = bt_row_stride;
  c.num_slots = num_slots;
  c.max_blocks_per_seq = max_blocks_per_seq;
  c.slot_ids = slot_ids;
  c.context_lens = context_lens;
  c.row_lens_host = row_lens_host;
  c.batch = batch;
  c.max_context_len = max_context_len;
  c.n_q_heads = n_q_heads;
  c.n_kv_heads = n_kv_heads;
  c.head_dim = head_dim;
  c.scale = scale;
  c.partition_size = partition_size;
  c.workspace = workspace;
  c.workspace_bytes = workspace_bytes;
  DecodeLaunch L;
  const int rc = decode_prepare(c, &L);
  if (rc != PKV_OK) return rc;
  return decode_enqueue(L, (hipStream_t)stream);
}

extern "C" int pkv_paged_decode_fused(pkv_bf16* out, const pkv_bf16* q, const pkv_bf16* k_new,
                                      const pkv_bf16* v_new, pkv_bf16* k_pool, pkv_bf16* v_pool, int num_blocks,
                                      const int32_t* block_table, int64_t bt_row_stride, int num_slots,
                                      int max_blocks_per_seq, const int32_t* slot_ids, const int32_t* context_lens,
                                      const int32_t* row_lens_host, int batch, int max_context_len, int n_q_heads,
                                      int n_kv_heads, int head_dim,
                                      const float* cos_sin, int max_pos, float scale, int partition_size,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  DecodeCall c{};
  c.fused = true;
  c.out = out;
  c.q = q;
  c.k_new = k_new;
  c.v_new = v_new;
  c.k_pool = k_pool;
  c.v_pool = v_pool;
  c.num_blocks = num_blocks;
  c.block_table = block_table;
  c.bt_row_stride = bt_row_stride;
  c.num_slots = num_slots;
  c.max_blocks_per_seq = max_blocks_per_seq;
  c.slot_ids = slot_ids;
  c.context_lens = context_lens;
  c.row_lens_host = row_lens_host;
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
  DecodeLaunch L;
  const int rc = decode_prepare(c, &L);
  if (rc != PKV_OK) return rc;
  return decode_enqueue(L, (hipStream_t)stream);
}

// ------------------------------------------------------------------------
// The decode step of one layer without a caller workspace, for callers that
// cannot allocate (code under graph capture, serving loops that forbid
// allocation): the partial records live in this file's device array.  Its
// host-side name is only a stand-in for the symbol; the device address is
// looked up once per device (with that device current) and kept.
// ------------------------------------------------------------------------

static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device, or null.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" int pkv_paged_decode_fused_noalloc(pkv_bf16* out, const pkv_bf16* q, const pkv_bf16* k_new,
                                              const pkv_bf16* v_new, pkv_bf16* k_pool, pkv_bf16* v_pool,
                                              int num_blocks, const int32_t* block_table, int64_t bt_row_stride,
                                              int num_slots, int max_blocks_per_seq, const int32_t* slot_ids,
                                              const int32_t* context_lens, const int32_t* row_lens_host, int batch,
                                              int max_context_len, int n_q_heads, int n_kv_heads, int head_dim,
                                              const float* cos_sin, int max_pos, float scale, int partition_size,
                                              void* stream) {
  DecodeCall c{};
  c.fused = true;
  c.out = out;
  c.q = q;
  c.k_new = k_new;
  c.v_new = v_new;
  c.k_pool = k_pool;
  c.v_pool = v_pool;
  c.num_blocks = num_blocks;
  c.block_table = block_table;
  c.bt_row_stride = bt_row_stride;
  c.num_slots = num_slots;
  c.max_blocks_per_seq = max_blocks_per_seq;
  c.slot_ids = slot_ids;
  c.context_lens = context_lens;
  c.row_lens_host = row_lens_host;
  c.batch = batch;
  c.max_context_len = max_context_len;
  c.n_q_heads = n_q_heads;
  c.n_kv_heads = n_kv_heads;
  c.head_dim = head_dim;
  c.cos_sin = cos_sin;
  c.max_pos = max_pos;
  c.scale = scale;
  c.partition_size = partition_size;
  c.workspace_bytes = PKV_NOALLOC_SCRATCH_BYTES;
  // Plan with a stand-in address first (nothing is dereferenced on the host),
  // so that argument errors and a workspace need beyond the array's size are
  // reported before the device is touched.
  c.workspace = reinterpret_cast<void*>((uintptr_t)256);
  DecodeLaunch L;
  int rc = decode_prepare(c, &L);
  if (rc != PKV_OK || L.path == 0) return rc;
  void* p = scratch_ptr();
  if (!p) return PKV_ERR_HIP;
  c.workspace = p;
  if ((rc = decode_prepare(c, &L)) != PKV_OK) return rc;
  return decode_enqueue(L, (hipStream_t)stream);
}

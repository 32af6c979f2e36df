// Streaming decode attention for gfx950: one 1024-thread workgroup per CU,
// each taking an equal, contiguous share of all 16-token blocks of the batch.
//
// Source: the Korean page of "An Inference Engine in 1,500 Lines of CUDA: The
// Map" ("What is in the box" table: online softmax and PagedAttention, four
// query heads per KV head) and the sixth chapter's title (each decode step
// re-reads every cached K/V of the sequence through the block table).  The
// split of the work across the chip is this library's own.
//
// Why.  Decode attention reads every cached block once, so the step is an HBM
// stream of about 2 KB per token and layer.  With one workgroup per
// (sequence, KV head, partition) the launch has a long ramp and tail: each
// workgroup first waits for its table slice and its first blocks, workgroups
// on one CU progress at very different speeds, and the last ones run alone.
// Here the batch's blocks are laid end to end (row by row, the block stream)
// and cut into equal shares, one per CU; every block is read whole (all KV
// heads, 16 KB of K and V each) in whole 128-byte lines.
//
// Work inside a workgroup.  16 waves = n_kv heads x (16 / n_kv) lanes of
// blocks: wave w serves KV head w % n_kv and takes every (16 / n_kv)-th block
// of the share, starting at block w / n_kv, with two blocks in flight.  The
// assignment is fixed, so a row's float32 sums are taken in an order that
// depends only on the row lengths (never on timing or on where the blocks sit
// in the pool): the same inputs give the same bits, under any placement of the
// blocks.  Each wave's first two blocks are looked up and requested before the
// share's table slice and queries are staged in LDS, so the first K/V bytes
// are on their way while the staging waits.
//
// A block's arithmetic runs on the matrix cores: scores S^T = K . Q^T (two
// 16x16x32 products, the G query heads as columns), then O^T += V^T . P^T
// (four 16x16x16 products, V transposed through a per-wave LDS tile), so the
// vector ALU is left with the masks, the exponentials and the rare rescale.
// K is loaded in whole lines (each load brings 8 token rows x 128 bytes) and
// put into the product's operand layout with one DPP row rotation.  When a
// wave's next block belongs to another row it folds its state for the finished
// row into that row's LDS slot, without waiting for the other waves.  After
// the last block one barrier, then the waves of each KV head are merged per
// row: a row that lies inside the share is finished in place, a row cut by the
// share's ends leaves (max, sum, unnormalised output) in one of the share's two
// records.  Those records are merged either by a small kernel after the launch
// or, when launches are chained over the layers of one step (same rows, same
// lengths), in the prologue of the next launch, where their loads overlap that
// launch's own start-up.
//
// Fused variant.  The workgroup holding a row's last block rotates the row's
// new key and keeps key and value in LDS.  Pool reads of that block stop
// before the new token; the wave that processes the block puts the token into
// its K and V registers at the token's slot, so it joins the same products and
// no read waits for a write.  The workgroup writes the token into the pool
// (position context_len - 1) after its stream, which keeps the table lookup
// for that write off the start-up path.
#include "attn_block.h"
#include "decode_stream.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace pkv {

namespace {

constexpr int kWaves = 16;
constexpr int kDepth = 2;             // blocks in flight per wave
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxRows = 4;           // rows one share may touch
constexpr int kMaxQ = 32;             // query heads staged per row
constexpr int kMaxKv = 16;            // KV heads
constexpr int kRec = kStreamRec;
constexpr int kWin = kThreads;        // blocks whose table entries are staged in LDS at a time
constexpr int kPrevSpan = 8;          // shares a row may span for the prologue merge of chained launches
static_assert(kRec == kHeadDim + 4, "record layout: outputs, max, sum, padding to 16 bytes");
static_assert(kMaxRows * kMaxQ * 8 <= kThreads, "one query chunk per thread");

// A 16-bit plan entry at a wave-uniform index, read as its aligned dword (a
// scalar load; there is no 16-bit scalar load).
__device__ __forceinline__ int plan_u16(const uint16_t* arr, int idx) {
  const int i = wave_uniform(idx);
  const uint32_t wd = reinterpret_cast<const uint32_t*>(arr)[i >> 1];
  return (int)((i & 1) ? (wd >> 16) : (wd & 0xffffu));
}

// The rows a share touches (at most kMaxRows = 4), held in registers: their
// starts in the block stream (and the end of the last), lengths and table
// rows.  Accessors take a row index that may differ between lanes.
struct ShareRows {
  int s0, s1, s2, s3, s4;      // starts of rows 0..3, and the start after row 3
  int n0, n1, n2, n3;          // tokens
  int t0, t1, t2, t3;          // table rows (-1: none)
  __device__ __forceinline__ static int sel(int i, int a0, int a1, int a2, int a3) {
    return i == 0 ? a0 : i == 1 ? a1 : i == 2 ? a2 : a3;
  }
  __device__ __forceinline__ int start(int i) const { return i == 4 ? s4 : sel(i, s0, s1, s2, s3); }
  __device__ __forceinline__ int end(int i) const { return start(i + 1); }
  __device__ __forceinline__ int len(int i) const { return sel(i, n0, n1, n2, n3); }
  __device__ __forceinline__ int slot(int i) const { return sel(i, t0, t1, t2, t3); }
};
static_assert(kMaxRows == 4, "ShareRows holds four rows");

// Table row of batch row b (wave-uniform b), or -1.
__device__ __forceinline__ int row_slot_u(const StreamCore& a, const StreamPlan& P, int b) {
  if (P.slots_in_args) {
    const int s = plan_u16(P.row_slot, b);
    return s == 0xffff ? -1 : s;
  }
  const int s = a.slot_ids ? a.slot_ids[wave_uniform(b)] : b;
  return (s >= 0 && s < a.num_slots) ? s : -1;
}

__device__ __forceinline__ int row_slot(const StreamCore& a, const StreamPlan& P, int b) {
  if (P.slots_in_args) {
    const int s = P.row_slot[b];
    return s == 0xffff ? -1 : s;
  }
  const int s = a.slot_ids ? a.slot_ids[b] : b;
  return (s >= 0 && s < a.num_slots) ? s : -1;
}

// Rotate chunk `own` (8 dims starting at 8 * ch) against its pair partner
// chunk (ch ^ 4); t: the (cos, sin) of the chunk's 8 pairs, two per float4
// (pairs 8 (ch % 4) .. + 7 of the position's table row).
__device__ __forceinline__ uint4 rope_own_chunk(uint4 own, uint4 oth, const float4 (&t)[4], int ch) {
  const uint32_t o[4] = {own.x, own.y, own.z, own.w};
  const uint32_t p[4] = {oth.x, oth.y, oth.z, oth.w};
  uint32_t res[4];
  const bool first_half = ch < 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float r[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float mine = e ? bf16_hi(o[j]) : bf16_lo(o[j]);
      const float other = e ? bf16_hi(p[j]) : bf16_lo(p[j]);
      const float c = e ? t[j].z : t[j].x;
      const float sn = e ? t[j].w : t[j].y;
      r[e] = first_half ? rope_first(mine, other, c, sn) : rope_second(other, mine, c, sn);
    }
    res[j] = pack_bf16x2(r[0], r[1]);
  }
  return make_uint4(res[0], res[1], res[2], res[3]);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Element (token, dim) of a wave's 16 x 64 V tile in LDS: rows of 64 dims,
// rotated by 16 dims for every token mod 4, so that the row-wise 16-byte
// writes and the transposed 8-byte reads both spread over the banks.
__device__ __forceinline__ int vt_index(int token, int dim) {
  return token * kHeadDim + ((dim + 16 * (token & 3)) & (kHeadDim - 1));
}

// ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives as its
// element j the (i % 4)-th bf16 of the 8-byte word that lane 4 j + i / 4 of the
// group addresses.
__device__ __forceinline__ uint2 lds_tr16(const uint16_t* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, r);
}

// Lane i of each row of 16 lanes takes the value of lane (i + 8) mod 16.
__device__ __forceinline__ uint4 row_rotate8(uint4 x) {
  auto r = [](uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowRor8, 0xF, 0xF, false);
  };
  return make_uint4(r(x.x), r(x.y), r(x.z), r(x.w));
}

// Scores S^T[token][col] += K[token][k] . Q^T[k][col] over 32 dims: lane l
// brings K row l % 16 and Q column l % 16, 8 dims each from group l / 16, and
// receives S^T rows 4 (l / 16) .. + 3 of column l % 16.
__device__ __forceinline__ f32x4 mfma_qk(uint4 k, uint4 q, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k), __builtin_bit_cast(bf16x8, q), c,
                                                  0, 0, 0);
}
// O^T[dim][col] += V^T[dim][token] . P^T[token][col] over the 16 tokens of a
// block: lane l brings V^T row l % 16 and P^T column l % 16 for tokens
// 4 (l / 16) .. + 3 and keeps O^T rows 4 (l / 16) .. + 3 of column l % 16.
__device__ __forceinline__ f32x4 mfma_pv(uint2 vt, uint2 p, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, vt), __builtin_bit_cast(i16x4, p), c,
                                                    0, 0, 0);
}

// Online-softmax state of one wave on the matrix cores.  Column l % 16 of
// every MFMA tile is one query head of the wave's KV head (columns >= G carry
// zero queries and are never written out).  Lane l keeps, for its column, the
// running max m (log2 units, equal in the four lane groups), the raw-score
// level thr above which m must be raised, its share l of the sum (tokens
// 4 (l / 16) .. + 3 of every block) and O^T dims 16 t + 4 (l / 16) .. + 3.
struct MfmaAcc {
  float m, thr, l;
  f32x4 o[4];

  __device__ __forceinline__ void reset() {
    m = kNegBig;
    thr = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One 16-token block.  k0 / k1: the K operands for dims 0..31 and 32..63
  // (token lane % 16).  V rows go through the wave's LDS tile (rows past the
  // context, or of a block whose id is out of range, are zeroed there so NaN
  // in unused pool slots cannot reach the output); scores of such tokens are
  // replaced by -inf (a select, never a product).  `extra` is a token slot
  // that takes part whatever the block (the fused step's new token), or -1.
  __device__ __forceinline__ void block(uint4 qb0, uint4 qb1, uint4 k0, uint4 k1, uint4 v0, uint4 v1,
                                        uint16_t* vtile, int wr0, int wr1, const int (&rd)[4], int r, int q4,
                                        bool blk_ok, int valid, int extra, float C, float invC) {
    const bool full = blk_ok && valid == kBlock;
    if (!full) {
      const uint4 z = make_uint4(0, 0, 0, 0);
      v0 = sel4((blk_ok && r < valid) || r == extra, v0, z);
      v1 = sel4((blk_ok && r + 8 < valid) || r + 8 == extra, v1, z);
    }
    *reinterpret_cast<uint4*>(vtile + wr0) = v0;
    *reinterpret_cast<uint4*>(vtile + wr1) = v1;

    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
    sc = mfma_qk(k0, qb0, sc);
    sc = mfma_qk(k1, qb1, sc);
    float sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * q4 + j;
      sv[j] = (full || (blk_ok && t < valid) || t == extra) ? sc[j] : -INFINITY;
    }
    const bool need = (sv[0] > thr) | (sv[1] > thr) | (sv[2] > thr) | (sv[3] > thr);
    if (__any(need)) {
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])) * C;
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx);
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] *= alpha;
      m = mn;
      thr = (mn + kTau) * invC;
    }
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = fast_exp2(__builtin_fmaf(sv[j], C, -m));
    const uint2 pp = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
    l = dot2_bf16(pp.x, kOnesBf16x2, l);
    l = dot2_bf16(pp.y, kOnesBf16x2, l);
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = mfma_pv(lds_tr16(vtile + rd[t]), pp, o[t]);
  }
};

// Output element (row b, query head qh, dim d) of a row cut by share ends:
// the records of every share the row spans, combined in share order.  Share
// w holds the row in record 2w when the row contains the share's first block,
// else in record 2w + 1.  Empty rows get zeros; rows inside one share were
// finished by their workgroup and are left alone.
__device__ __forceinline__ void merge_element(const StreamCore& a, const StreamPlan& P, uint16_t* out, const float* ws,
                                              int b, int qh,
                                              int d) {
  const int64_t o = ((int64_t)b * a.n_q + qh) * kHeadDim + d;
  if (P.row_n[b] <= 0) {
    out[o] = 0;
    return;
  }
  const int start = P.row_start[b];
  const int w0 = start / P.share;
  const int w1 = (P.row_start[b + 1] - 1) / P.share;
  if (w0 == w1) return;
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int w = w0; w <= w1; w += 8) {
    float mv[8], lv[8], ov[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ww = w + j <= w1 ? w + j : w1;
      const int rec = 2 * ww + ((ww > w0 || start == w0 * P.share) ? 0 : 1);
      const float* src = ws + ((int64_t)rec * a.n_q + qh) * kRec;
      mv[j] = w + j <= w1 ? src[kHeadDim] : -INFINITY;
      lv[j] = src[kHeadDim + 1];
      ov[j] = src[d];
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
  out[o] = to_bf16(L > 0.f ? O / L : 0.f);
}

// The prologue merge of a chained launch, split so that its loads go out with
// the launch's other staging loads: (row b, query head qh, dim d) of the
// previous launch, whose rows span at most kPrevSpan shares.
struct PrevMerge {
  float m[kPrevSpan], l[kPrevSpan], o[kPrevSpan];
  int64_t at;                  // output element, or -1: nothing to do
  bool empty;                  // the row is empty: write zero
};

__device__ __forceinline__ void prev_load(const StreamCore& a, const StreamPlan& P, int b, int qh, int d, PrevMerge& M) {
  M.at = -1;
  M.empty = false;
  if (b >= a.batch) return;
  const int64_t o = ((int64_t)b * a.n_q + qh) * kHeadDim + d;
  if (P.row_n[b] <= 0) {
    M.at = o;
    M.empty = true;
    return;
  }
  const int start = P.row_start[b];
  const int w0 = start / P.share;
  const int w1 = (P.row_start[b + 1] - 1) / P.share;
  if (w0 == w1) return;
  M.at = o;
  // (max, sum) of a record are the same for every lane: read as constant
  // memory (the previous launch wrote them) they become scalar loads
  const __attribute__((address_space(4))) float* ws_c = (const __attribute__((address_space(4))) float*)a.ws_prev;
#pragma unroll
  for (int j = 0; j < kPrevSpan; ++j) {
    const int ww = w0 + j <= w1 ? w0 + j : w1;
    const int rec = 2 * ww + ((ww > w0 || start == w0 * P.share) ? 0 : 1);
    const int64_t base = ((int64_t)rec * a.n_q + qh) * kRec;
    M.m[j] = w0 + j <= w1 ? ws_c[base + kHeadDim] : -INFINITY;
    M.l[j] = ws_c[base + kHeadDim + 1];
    M.o[j] = a.ws_prev[base + d];
  }
}

__device__ __forceinline__ void prev_finish(const StreamCore& a, const PrevMerge& pm) {
  if (pm.at < 0) return;
  if (pm.empty) {
    a.out_prev[pm.at] = 0;
    return;
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < kPrevSpan; ++j) M = fmaxf(M, pm.m[j]);
  float L = 0.f, O = 0.f;
#pragma unroll
  for (int j = 0; j < kPrevSpan; ++j) {
    const float f = pm.m[j] == -INFINITY ? 0.f : fast_exp2(pm.m[j] - M);
    L += f * pm.l[j];
    O += f * pm.o[j];
  }
  a.out_prev[pm.at] = to_bf16(L > 0.f ? O / L : 0.f);
}

// The kernels' argument block: the core alone when the plan is in device memory.
template <bool DEVPLAN>
using ArgsOf = std::conditional_t<DEVPLAN, StreamCore, StreamArgs>;

template <bool DEVPLAN>
__device__ __forceinline__ const StreamPlan& plan_of(const ArgsOf<DEVPLAN>& a) {
  if constexpr (DEVPLAN)
    return *a.plan_dev;
  else
    return a.plan;
}

template <int G, bool FUSED, bool PREV, bool DEVPLAN, bool NT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void stream_kernel(ArgsOf<DEVPLAN> a) {
  const StreamPlan& P = plan_of<DEVPLAN>(a);
  const int B0 = blockIdx.x * P.share;
  const int B1 = min(B0 + P.share, P.total);
  const int len = B1 - B0;
  if (len <= 0) return;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = wave_uniform(tid >> 6);
  const int c = lane & 7;
  const int r = lane >> 3;
  const int n_kv = a.n_kv;
  const int S = kWaves / n_kv;           // waves per KV head
  const int h = w % n_kv;                // this wave's KV head
  const int s = w / n_kv;                // and its lane of blocks
  const int wr = plan_u16(P.wg_rows, blockIdx.x);
  const int bf = wr >> 3;                // first row of the share
  const int nrows = wr & 7;              // rows it touches
  const int64_t row_elems = (int64_t)n_kv * kHeadDim;
  const float C = a.scale_log2e;
  const float invC = 1.0f / C;
  // the share's rows, read once with scalar loads
  constexpr int kFar = 0x7fffffff;
  const ShareRows RW{P.row_start[bf],
                     nrows >= 1 ? P.row_start[bf + 1] : kFar,
                     nrows >= 2 ? P.row_start[bf + 2] : kFar,
                     nrows >= 3 ? P.row_start[bf + 3] : kFar,
                     nrows >= 4 ? P.row_start[bf + 4] : kFar,
                     nrows > 0 ? P.row_n[bf] : 0,
                     nrows > 1 ? P.row_n[bf + 1] : 0,
                     nrows > 2 ? P.row_n[bf + 2] : 0,
                     nrows > 3 ? P.row_n[bf + 3] : 0,
                     nrows > 0 ? row_slot_u(a, P, bf) : -1,
                     nrows > 1 ? row_slot_u(a, P, bf + 1) : -1,
                     nrows > 2 ? row_slot_u(a, P, bf + 2) : -1,
                     nrows > 3 ? row_slot_u(a, P, bf + 3) : -1};

  __shared__ uint4 sq[kMaxRows][kMaxQ * 8];                 // queries: [row][head][chunk]
  __shared__ uint4 snew[kMaxRows][2][kMaxKv * 8];           // fused: new key / value [row][k|v][head][chunk]
  __shared__ __attribute__((aligned(16))) float spo[kMaxRows][kWaves][G][kHeadDim];  // per-wave partial outputs of each row
  __shared__ float2 spm[kMaxRows][kWaves][G];               // and their (max, sum)
  __shared__ int srow_ok[kMaxRows];                         // the row's table slot is valid
  __shared__ int s_app[kMaxRows];                           // fused: pool block of the row's new token, or -1
  __shared__ uint16_t svt[kWaves][kBlock * kHeadDim];       // per-wave V tile (transposed reads)
  __shared__ int s_tab[kWin];                               // window's blocks: pool block id or -1
  __shared__ int s_meta[kWin];                              // and row << 8 | tokens read from the pool

  const uint32_t block_bytes = (uint32_t)(kBlock * row_elems * 2);
  const uint32_t head_off = (uint32_t)(h * kHeadDim * 2);
  // V: lane = 8 r + c reads dims 8c .. 8c + 7 of token rows r and r + 8
  const uint32_t v_off0 = (uint32_t)(r * row_elems * 2) + head_off + 16u * c;
  const uint32_t v_off1 = v_off0 + (uint32_t)(8 * row_elems * 2);
  // K in whole lines: load A covers token rows 0..7, load B rows 8..15, all 8
  // chunks of each.  Lane l takes chunk l / 16 of row l % 16 when that row is
  // the load's, else chunk 4 + l / 16 of row l % 8 (A) or 8 + l % 8 (B), the
  // piece that lane l ^ 8 needs for the second operand (see fix_k).
  const uint32_t k_offA = (uint32_t)((lane & 7) * row_elems * 2) + head_off +
                          16u * (uint32_t)((lane >> 4) | ((lane & 8) >> 1));
  const uint32_t k_offB = (uint32_t)((8 + (lane & 7)) * row_elems * 2) + head_off +
                          16u * (uint32_t)((lane >> 4) | ((~lane & 8) >> 1));
  const char* kbase = reinterpret_cast<const char*>(a.k_pool);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool);
  // the table seen as constant memory: wave-uniform reads become scalar loads
  const __attribute__((address_space(4))) int32_t* bt_const =
      (const __attribute__((address_space(4))) int32_t*)a.bt;

  // stream block p -> its table entry as read (-1 for none; range-checked by
  // block_ok where it is used, so that nothing waits for the load here) and
  // (row << 8 | tokens to read from the pool; the fused step's new token is
  // not among them)
  auto block_ok = [&](int blk) { return (blk >= 0 && blk < a.num_blocks) ? blk : -1; };
  auto block_info = [&](int p, int& tab, int& meta, uint32_t& err) {
    const int ri = (p >= RW.s1) + (p >= RW.s2) + (p >= RW.s3);
    const int start = RW.start(ri);
    const int n = RW.len(ri);
    const int j = p - start;
    const int slot = RW.slot(ri);
    int valid = (FUSED ? n - 1 : n) - j * kBlock;
    valid = valid > kBlock ? kBlock : (valid < 0 ? 0 : valid);
    tab = -1;
    if (slot >= 0 && j < a.max_blocks && valid > 0) tab = a.bt[(int64_t)slot * a.bt_stride + j];
    meta = (ri << 8) | valid;
    // what to report if the block has tokens to read and no valid entry
    err = slot < 0 ? PKV_DEVERR_BAD_SLOT : (j >= a.max_blocks ? PKV_DEVERR_LONG_CONTEXT : PKV_DEVERR_BAD_BLOCK);
  };
  // Loads of one block for this wave's KV head.  blk < 0 reads nothing (a
  // zero-size buffer returns zeros without a memory access).
  auto issue = [&](KVRegs& R, int blk) {
    const bool ok = blk >= 0;
    const size_t base = ok ? (size_t)blk * block_bytes : 0;
    const auto rk = buf_rsrc(kbase + base, ok ? block_bytes : 0u);
    const auto rv = buf_rsrc(vbase + base, ok ? block_bytes : 0u);
    buf_load_kv4<NT>(rk, k_offA, k_offB, rv, v_off0, v_off1, R.k0, R.k1, R.v0, R.v1);
  };

  // ---- start-up.  A wave's vector loads complete in order, so waiting for
  // a load issued after the first blocks' K/V loads would also wait for those
  // bytes: every load the staging needs is issued first and the K/V loads
  // last.  The first blocks' table entries come through the scalar cache
  // (wave-uniform addresses; nothing in this launch writes the table), which
  // the K/V issue waits for on a counter of its own.
  int tb[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    tb[d] = -1;
    const int p = s + d * S;
    if (p < len) {
      const int pb = B0 + p;
      const int ri = (pb >= RW.s1) + (pb >= RW.s2) + (pb >= RW.s3);
      const int j = wave_uniform(pb - RW.start(ri));
      const int slot = wave_uniform(RW.slot(ri));
      if (slot >= 0 && j < a.max_blocks && j * kBlock < RW.len(ri) - (FUSED ? 1 : 0)) {
        const int blk = bt_const[(int64_t)slot * a.bt_stride + j];
        tb[d] = (blk >= 0 && blk < a.num_blocks) ? blk : -1;
      }
    }
  }
  // the first window's table slice: thread t, block t (written to LDS below)
  int tab = -1, meta = 0;
  uint32_t tab_err = 0;
  if (tid < min(kWin, len)) block_info(B0 + tid, tab, meta, tab_err);

  // queries of the share's rows, one 8-dim chunk per thread (with the chunk
  // holding their RoPE partners and the position's table row when fused)
  const bool q_thread = tid < nrows * a.n_q * 8;
  const int qi = tid / (a.n_q * 8);
  const int qrem = tid - qi * a.n_q * 8;
  const int qch = qrem & 7;
  uint4 qv = make_uint4(0, 0, 0, 0), qp = qv;
  float4 qt[4];
  bool q_rot = false;
  if (q_thread) {
    const uint16_t* qrow = a.q + ((int64_t)(bf + qi) * a.n_q + (qrem >> 3)) * kHeadDim;
    qv = *reinterpret_cast<const uint4*>(qrow + qch * 8);
    if constexpr (FUSED) {
      const int pos = RW.len(qi) - 1;
      if (pos >= 0 && pos < a.max_pos) {
        q_rot = true;
        qp = *reinterpret_cast<const uint4*>(qrow + (qch ^ 4) * 8);
        const float4* tr = reinterpret_cast<const float4*>(a.rope + ((int64_t)pos * (kHeadDim / 2) + (qch & 3) * 8) * 2);
#pragma unroll
        for (int t = 0; t < 4; ++t) qt[t] = tr[t];
      }
    }
  }
  // fused: the new token of every row whose last block is here (rotated key
  // and value go to LDS and join the attention from there; the pool write
  // waits for the end of the workgroup's stream, no workgroup reads that pool
  // row in this launch).  nrows * n_kv * 8 <= kThreads: one chunk per thread.
  const int ni = tid / (n_kv * 8);
  const int nrem = tid - ni * n_kv * 8;
  const int nch = nrem & 7;
  bool n_thread = false, n_rot = false;
  uint4 nk = make_uint4(0, 0, 0, 0), nv = nk, np = nk;
  float4 nt[4];
  int napp = -1;
  if constexpr (FUSED) {
    if (tid < nrows * n_kv * 8) {
      const int b = bf + ni;
      const int n = RW.len(ni);
      const int last = RW.end(ni) - 1;
      if (n > 0 && last >= B0 && last < B1) {
        n_thread = true;
        const int pos = n - 1;
        const uint16_t* krow = a.k_new + ((int64_t)b * n_kv + (nrem >> 3)) * kHeadDim;
        nk = *reinterpret_cast<const uint4*>(krow + nch * 8);
        nv = *reinterpret_cast<const uint4*>(a.v_new + ((int64_t)b * n_kv + (nrem >> 3)) * kHeadDim + nch * 8);
        const int slot = RW.slot(ni);
        if (nrem == 0 && slot >= 0 && pos / kBlock < a.max_blocks)
          napp = a.bt[(int64_t)slot * a.bt_stride + pos / kBlock];
        if (pos < a.max_pos) {
          n_rot = true;
          np = *reinterpret_cast<const uint4*>(krow + (nch ^ 4) * 8);
          const float4* tr = reinterpret_cast<const float4*>(a.rope + ((int64_t)pos * (kHeadDim / 2) + (nch & 3) * 8) * 2);
#pragma unroll
          for (int t = 0; t < 4; ++t) nt[t] = tr[t];
        }
      }
    }
  }
  // ---- the first blocks' K/V ----------------------------------------------
  KVRegs R[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) issue(R[d], wave_uniform(tb[d]));

  // ---- staging (its waits cover the loads above, not the K/V loads) ---------
  if (q_thread) sq[qi][qrem] = q_rot ? rope_own_chunk(qv, qp, qt, qch & 4) : qv;
  if constexpr (FUSED) {
    if (tid < nrows) srow_ok[tid] = RW.slot(tid) >= 0;
    if (n_thread) {
      if (nrem == 0) s_app[ni] = napp;
      snew[ni][0][nrem] = n_rot ? rope_own_chunk(nk, np, nt, nch & 4) : nk;
      snew[ni][1][nrem] = nv;
    }
  }
  if (tid < min(kWin, len)) {
    s_tab[tid] = block_ok(tab);
    s_meta[tid] = meta;
    if ((meta & 0xff) && block_ok(tab) < 0) report_error(a.errors, tab_err);
  }
  __syncthreads();

  MfmaAcc acc;
  acc.reset();
  const int col = lane & 15;             // MFMA column: query head of the KV head's group
  const int q4 = lane >> 4;              // MFMA lane group
  const bool lo8 = (lane & 8) == 0;
  uint4 qb0, qb1;                        // Q^T operands: dims 8 q4 .. and 32 + 8 q4 ..
  int cur = 0;                           // row of the share being accumulated
  int row_last = -1;                     // fused: stream block holding the row's new token, or -1
  auto load_q = [&]() {
    const uint4 z = make_uint4(0, 0, 0, 0);
    qb0 = col < G ? sq[cur][(h * G + col) * 8 + q4] : z;
    qb1 = col < G ? sq[cur][(h * G + col) * 8 + q4 + 4] : z;
    if constexpr (FUSED) {
      const int b = bf + cur;
      row_last = wave_uniform(RW.len(cur) > 0 && srow_ok[cur] ? RW.end(cur) - 1 : -1);
    }
  };
  load_q();

  // Fold the wave's state for row `cur` into its LDS slot (the four lane
  // groups hold different tokens' shares of the sum) and move on.
  auto flush = [&]() {
    float l = acc.l;
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (col < G) {
      float* dst = spo[cur][w][col];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        *reinterpret_cast<float4*>(dst + 16 * t + 4 * q4) = make_float4(acc.o[t][0], acc.o[t][1], acc.o[t][2], acc.o[t][3]);
      if (q4 == 0) spm[cur][w][col] = make_float2(acc.m, l);
    }
    ++cur;
    acc.reset();
    if (cur < nrows) load_q();
  };

  // this wave's V tile in LDS: written row-wise, read transposed
  uint16_t* vtile = svt[w];
  const int v_wr0 = vt_index(r, 8 * c);
  const int v_wr1 = vt_index(r + 8, 8 * c);
  int v_rd[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) v_rd[t] = vt_index(lane >> 2, 16 * t + 4 * (lane & 3));

  for (int w0 = 0; w0 < len; w0 += kWin) {
    const int wl = min(kWin, len - w0);
    if (w0 > 0) {
      __syncthreads();                   // every wave is done with the previous window
      if (tid < wl) {
        block_info(B0 + w0 + tid, tab, meta, tab_err);
        s_tab[tid] = block_ok(tab);
        s_meta[tid] = meta;
        if ((meta & 0xff) && block_ok(tab) < 0) report_error(a.errors, tab_err);
      }
      __syncthreads();
#pragma unroll
      for (int d = 0; d < kDepth; ++d) issue(R[d], s + d * S < wl ? wave_uniform(s_tab[s + d * S]) : -1);
    }
    auto step = [&](const KVRegs& R, int i) {
      const int mt = wave_uniform(s_meta[i]);
      while (cur < (mt >> 8)) flush();
      const bool blk_ok = wave_uniform(s_tab[i]) >= 0;
      const int valid = mt & 0xff;       // tokens read from the pool
      // K operands: lanes whose row is in load A take it from there, the
      // others from load B; the second operand comes from lane l ^ 8
      uint4 k0 = sel4(lo8, R.k0, R.k1);
      uint4 k1 = row_rotate8(sel4(lo8, R.k1, R.k0));
      uint4 v0 = R.v0, v1 = R.v1;
      int extra = -1;                    // fused: slot of the new token in this block
      if constexpr (FUSED) {
        // the row's last block: the new token (rotated key, value) from LDS
        if (B0 + w0 + i == row_last) {
          extra = valid;
          if (col == extra) {
            k0 = snew[cur][0][h * 8 + q4];
            k1 = snew[cur][0][h * 8 + q4 + 4];
          }
          if (r == extra) v0 = snew[cur][1][h * 8 + c];
          if (r + 8 == extra) v1 = snew[cur][1][h * 8 + c];
        }
      }
      acc.block(qb0, qb1, k0, k1, v0, v1, vtile, v_wr0, v_wr1, v_rd, r, q4, blk_ok, valid, extra, C, invC);
    };
    // fixed sequence s, s + S, s + 2S, ... with kDepth blocks in flight in
    // as many register sets; a load past the window reads nothing.  Every set
    // is reissued on every path through the loop body, so the compiler's wait
    // before each block covers exactly the oldest set.
    for (int i = s; i < wl; i += kDepth * S) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int idx = i + d * S;
        if (idx < wl) step(R[d], idx);
        issue(R[d], idx + kDepth * S < wl ? wave_uniform(s_tab[idx + kDepth * S]) : -1);
      }
    }
  }
  while (cur < nrows) flush();
  // ---- chained launches: the previous launch's rows cut by share ends, one
  // (row, query head) pair per wave, pairs grid x 16 apart (a small grid
  // takes several).  At the end of the wave's stream: the oldest waves, which
  // get the pairs and finish first, do it while the others still stream.
  if constexpr (PREV) {
    const int pairs = a.batch * a.n_q;
    for (int pp = blockIdx.x + P.grid * w; pp < pairs; pp += P.grid * kWaves) {
      PrevMerge pm;
      prev_load(a, P, pp / a.n_q, pp % a.n_q, lane, pm);
      prev_finish(a, pm);
    }
  }
  if constexpr (FUSED) {
    // the new token into the pool (position context_len - 1 of its row)
    if (tid < nrows * n_kv * 8) {
      const int n = RW.len(ni);
      const int last = RW.end(ni) - 1;
      const bool here = n > 0 && last >= B0 && last < B1;
      const int blk = here ? s_app[ni] : -1;
      if (here && RW.slot(ni) >= 0 && !(blk >= 0 && blk < a.num_blocks)) report_error(a.errors, PKV_DEVERR_BAD_BLOCK);
      if (blk >= 0 && blk < a.num_blocks) {
        const int pos = n - 1;
        const int64_t off =
            ((int64_t)blk * kBlock + pos % kBlock) * row_elems + (nrem >> 3) * kHeadDim + (nrem & 7) * 8;
        *reinterpret_cast<uint4*>(a.k_pool + off) = snew[ni][0][nrem];
        *reinterpret_cast<uint4*>(a.v_pool + off) = snew[ni][1][nrem];
      }
    }
  }
  __syncthreads();

  // ---- merge the KV heads' waves per row: finish rows inside the share,
  // leave records for rows cut by its ends.  One thread per (row, query
  // head, 8 dims): 16-byte LDS reads, one 16-byte output store ------------------
  for (int e = tid; e < nrows * a.n_q * 8; e += kThreads) {
    const int i = e / (a.n_q * 8);
    const int rem = e - i * a.n_q * 8;
    const int b = bf + i;
    if (RW.len(i) <= 0) continue;
    const int qh = rem >> 3;
    const int c8 = rem & 7;
    const int hh = qh / G;
    const int g = qh % G;
    float M = spm[i][hh][g].x;
    for (int t = 1; t < S; ++t) M = fmaxf(M, spm[i][hh + t * n_kv][g].x);
    float L = 0.f;
    float O[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < S; ++t) {
      const float2 ml = spm[i][hh + t * n_kv][g];
      const float f = fast_exp2(ml.x - M);
      L += f * ml.y;
      const float4* src = reinterpret_cast<const float4*>(&spo[i][hh + t * n_kv][g][8 * c8]);
      const float4 o0 = src[0], o1 = src[1];
      O[0] += f * o0.x;
      O[1] += f * o0.y;
      O[2] += f * o0.z;
      O[3] += f * o0.w;
      O[4] += f * o1.x;
      O[5] += f * o1.y;
      O[6] += f * o1.z;
      O[7] += f * o1.w;
    }
    if (RW.start(i) >= B0 && RW.end(i) <= B1) {
      uint4 v;
      v.x = pack_bf16x2(L > 0.f ? O[0] / L : 0.f, L > 0.f ? O[1] / L : 0.f);
      v.y = pack_bf16x2(L > 0.f ? O[2] / L : 0.f, L > 0.f ? O[3] / L : 0.f);
      v.z = pack_bf16x2(L > 0.f ? O[4] / L : 0.f, L > 0.f ? O[5] / L : 0.f);
      v.w = pack_bf16x2(L > 0.f ? O[6] / L : 0.f, L > 0.f ? O[7] / L : 0.f);
      *reinterpret_cast<uint4*>(a.out + ((int64_t)b * a.n_q + qh) * kHeadDim + 8 * c8) = v;
    } else {
      const int rec = 2 * (int)blockIdx.x + (i == 0 ? 0 : 1);
      float* dst = a.ws + ((int64_t)rec * a.n_q + qh) * kRec;
      reinterpret_cast<float4*>(dst + 8 * c8)[0] = make_float4(O[0], O[1], O[2], O[3]);
      reinterpret_cast<float4*>(dst + 8 * c8)[1] = make_float4(O[4], O[5], O[6], O[7]);
      if (c8 == 0) *reinterpret_cast<float2*>(dst + kHeadDim) = make_float2(M, L);
    }
  }
  if constexpr (!DEVPLAN) {
    // the plan for later launches that read it from device memory (last, so
    // that no global store precedes the start-up loads)
    if (a.plan_out != nullptr && blockIdx.x == 0) {
      constexpr int kWords = (int)(sizeof(StreamPlan) / 4);
      static_assert(kWords <= kThreads, "one word per thread");
      if (tid < kWords)
        reinterpret_cast<uint32_t*>(a.plan_out)[tid] = reinterpret_cast<const uint32_t*>(&a.plan)[tid];
    }
  }
}

// Merge of the records of rows cut by share ends: one workgroup per (row, KV
// head), thread = (query head of the group, dim).
template <int G, bool DEVPLAN>
__global__ __launch_bounds__(256) void stream_merge_kernel(ArgsOf<DEVPLAN> a) {
  const StreamPlan& P = plan_of<DEVPLAN>(a);
  const int kvh = blockIdx.x;
  const int b = blockIdx.y;
  for (int e = threadIdx.x; e < G * kHeadDim; e += blockDim.x)
    merge_element(a, P, a.out, a.ws, b, kvh * G + e / kHeadDim, e % kHeadDim);
}

// The same merge for batches whose rows span many shares (few rows, long
// contexts): one workgroup per (row, query head), 16 groups of 64 threads
// (thread = dim); group j takes records j, j + 16, ..., eight of them with
// their loads in flight at once, and the groups' partial (max, sum, output)
// are combined through LDS in group order.  More workgroups and shorter chains
// of dependent loads per thread than the kernel above, which leaves a batch of
// one row on n_kv workgroups walking hundreds of records each.
template <bool DEVPLAN>
__global__ __launch_bounds__(1024) void stream_merge_wide_kernel(ArgsOf<DEVPLAN> a) {
  const StreamPlan& P = plan_of<DEVPLAN>(a);
  constexpr int kGroups = 16;
  __shared__ float part[kGroups][kHeadDim][3];
  const int qh = blockIdx.x;
  const int b = blockIdx.y;
  const int n = P.row_n[b];
  const int d = threadIdx.x % kHeadDim;
  const int grp = threadIdx.x / kHeadDim;
  const int64_t obase = ((int64_t)b * a.n_q + qh) * kHeadDim;
  if (n <= 0) {
    if (grp == 0) a.out[obase + d] = 0;
    return;
  }
  const int start = P.row_start[b];
  const int w0 = start / P.share;
  const int w1 = (P.row_start[b + 1] - 1) / P.share;
  if (w0 == w1) return;
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int w = w0 + grp; w <= w1; w += 8 * kGroups) {
    float mv[8], lv[8], ov[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int wj = w + j * kGroups;
      const int ww = wj <= w1 ? wj : w1;
      const int rec = 2 * ww + ((ww > w0 || start == w0 * P.share) ? 0 : 1);
      const float* src = a.ws + ((int64_t)rec * a.n_q + qh) * kRec;
      mv[j] = wj <= w1 ? src[kHeadDim] : -INFINITY;
      lv[j] = src[kHeadDim + 1];
      ov[j] = src[d];
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
  part[grp][d][0] = M;
  part[grp][d][1] = L;
  part[grp][d][2] = O;
  __syncthreads();
  if (grp > 0) return;
  for (int j = 1; j < kGroups; ++j) {
    const float m2 = part[j][d][0];
    const float mm = fmaxf(M, m2);
    if (mm == -INFINITY) continue;
    const float f1 = M == -INFINITY ? 0.f : fast_exp2(M - mm);
    const float f2 = m2 == -INFINITY ? 0.f : fast_exp2(m2 - mm);
    L = L * f1 + part[j][d][1] * f2;
    O = O * f1 + part[j][d][2] * f2;
    M = mm;
  }
  a.out[obase + d] = to_bf16(L > 0.f ? O / L : 0.f);
}

// Diagnostic, off the attention path: the streaming kernel's K/V reads with
// nothing else (same plan, same table window in LDS, same wave split, the
// same four 16-byte loads per lane and block, kDepth blocks in flight per
// wave); the data are XOR-ed into `sink` under a condition they never meet.
// It gives the time that reading a batch's blocks in this pattern takes on
// its own.
template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_read_probe_kernel(StreamArgs a, uint32_t* sink) {
  const StreamPlan& P = a.plan;
  const int B0 = blockIdx.x * P.share;
  const int B1 = min(B0 + P.share, P.total);
  const int len = B1 - B0;
  if (len <= 0) return;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = wave_uniform(tid >> 6);
  const int c = lane & 7;
  const int r = lane >> 3;
  const int n_kv = a.n_kv;
  const int S = kWaves / n_kv;
  const int h = w % n_kv;
  const int s = w / n_kv;
  const int wr = P.wg_rows[blockIdx.x];
  const int bf = wr >> 3;
  const int nrows = wr & 7;
  const int64_t row_elems = (int64_t)n_kv * kHeadDim;
  __shared__ int s_tab[kWin];
  const uint32_t block_bytes = (uint32_t)(kBlock * row_elems * 2);
  const uint32_t head_off = (uint32_t)(h * kHeadDim * 2);
  const uint32_t v_off0 = (uint32_t)(r * row_elems * 2) + head_off + 16u * c;
  const uint32_t v_off1 = v_off0 + (uint32_t)(8 * row_elems * 2);
  const uint32_t k_offA = (uint32_t)((lane & 7) * row_elems * 2) + head_off +
                          16u * (uint32_t)((lane >> 4) | ((lane & 8) >> 1));
  const uint32_t k_offB = (uint32_t)((8 + (lane & 7)) * row_elems * 2) + head_off +
                          16u * (uint32_t)((lane >> 4) | ((~lane & 8) >> 1));
  const char* kbase = reinterpret_cast<const char*>(a.k_pool);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool);
  // block t of the share (t = thread): its pool block id, or -1
  if (tid < len) {
    const int p = B0 + tid;
    int ri = 0;
    for (int i = 1; i < nrows; ++i) ri = p >= P.row_start[bf + i] ? i : ri;
    const int j = p - P.row_start[bf + ri];
    const int slot = row_slot(a, P, bf + ri);
    int blk = -1;
    if (slot >= 0 && j < a.max_blocks && j * kBlock < P.row_n[bf + ri]) {
      const int b = a.bt[(int64_t)slot * a.bt_stride + j];
      blk = (b >= 0 && b < a.num_blocks) ? b : -1;
    }
    s_tab[tid] = blk;
  }
  __syncthreads();
  auto issue = [&](KVRegs& R, int blk) {
    const bool ok = blk >= 0;
    const size_t base = ok ? (size_t)blk * block_bytes : 0;
    const auto rk = buf_rsrc(kbase + base, ok ? block_bytes : 0u);
    const auto rv = buf_rsrc(vbase + base, ok ? block_bytes : 0u);
    buf_load_kv4<NT>(rk, k_offA, k_offB, rv, v_off0, v_off1, R.k0, R.k1, R.v0, R.v1);
  };
  KVRegs R[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) issue(R[d], s + d * S < len ? wave_uniform(s_tab[s + d * S]) : -1);
  uint32_t x = 0;
  for (int i = s; i < len; i += kDepth * S) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int idx = i + d * S;
      // every loaded dword takes part, so that no load is narrowed
      x ^= R[d].k0.x ^ R[d].k0.y ^ R[d].k0.z ^ R[d].k0.w ^ R[d].k1.x ^ R[d].k1.y ^ R[d].k1.z ^ R[d].k1.w;
      x ^= R[d].v0.x ^ R[d].v0.y ^ R[d].v0.z ^ R[d].v0.w ^ R[d].v1.x ^ R[d].v1.y ^ R[d].v1.z ^ R[d].v1.w;
      issue(R[d], idx + kDepth * S < len ? wave_uniform(s_tab[idx + kDepth * S]) : -1);
    }
  }
  if (x == 0x9e3779b9u) *sink = x;
}

int device_cus() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cus[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <bool FUSED, bool PREV, bool DEVPLAN, bool NT>
const void* pick_stream_nt(int G) {
  return G == 1 ? (const void*)stream_kernel<1, FUSED, PREV, DEVPLAN, NT>
       : G == 2 ? (const void*)stream_kernel<2, FUSED, PREV, DEVPLAN, NT>
                : (const void*)stream_kernel<4, FUSED, PREV, DEVPLAN, NT>;
}
template <bool FUSED, bool PREV, bool DEVPLAN>
const void* pick_stream(int G, bool nt) {
  return nt ? pick_stream_nt<FUSED, PREV, DEVPLAN, true>(G) : pick_stream_nt<FUSED, PREV, DEVPLAN, false>(G);
}

template <bool DEVPLAN>
const void* pick_merge(int G) {
  return G == 1 ? (const void*)stream_merge_kernel<1, DEVPLAN>
       : G == 2 ? (const void*)stream_merge_kernel<2, DEVPLAN>
                : (const void*)stream_merge_kernel<4, DEVPLAN>;
}

}  // namespace

size_t stream_records_bytes(int n_q) {
  return n_q > 0 ? (size_t)2 * kStreamMaxGrid * n_q * kRec * sizeof(float) : 0;
}

int stream_launch_grid() {
  const int cus = device_cus();
  return cus <= 0 ? 0 : std::min(cus, kStreamMaxGrid);
}

namespace {

// Rows touched by each share of `share` blocks, into P->wg_rows (the row of a
// block is the last row whose start is at or before it: empty rows share
// their start with the next row and are passed over).  False when a share
// would touch more than kMaxRows rows, empty rows in between included.
bool plan_shares(StreamPlan* P, int batch, int share, int grid_max) {
  const int grid = (int)((P->total + (int64_t)share - 1) / share);
  if (grid > grid_max) return false;
  P->share = share;
  P->grid = grid;
  for (int g = 0, b = 0; g < grid; ++g) {
    const int p0 = g * share;
    const int p1 = std::min(p0 + share, P->total) - 1;
    while (b + 1 < batch && P->row_start[b + 1] <= p0) ++b;
    int e = b;
    while (e + 1 < batch && P->row_start[e + 1] <= p1) ++e;
    if (e - b + 1 > kMaxRows) return false;
    P->wg_rows[g] = (uint16_t)(b << 3 | (e - b + 1));
  }
  return true;
}

}  // namespace

int stream_plan_build(int batch, const int32_t* row_lens_host, int max_blocks, const int32_t* slot_ids_host,
                      bool slot_ids_dev, int num_slots, bool chain, StreamPlan* P, int* merge_kind) {
  if (!row_lens_host || batch <= 0 || batch > kStreamMaxSeqs) return -1;
  *P = StreamPlan{};
  // each row's slot in the plan when the host knows it (one dependent memory
  // read less before the first K/V load)
  if (slot_ids_host && num_slots <= 0xffff) {
    P->slots_in_args = 1;
    for (int b = 0; b < batch; ++b) {
      const int s = slot_ids_host[b];
      P->row_slot[b] = (uint16_t)((s >= 0 && s < num_slots) ? s : 0xffff);
    }
  } else if (!slot_ids_dev && batch <= num_slots && num_slots <= 0xffff) {
    P->slots_in_args = 1;
    for (int b = 0; b < batch; ++b) P->row_slot[b] = (uint16_t)b;
  }
  // the block stream: rows end to end, each ceil(n / 16) blocks
  int64_t total = 0;
  int longest = 0;
  P->row_start[0] = 0;
  for (int b = 0; b < batch; ++b) {
    int n = row_lens_host[b];
    n = n < 0 ? 0 : (n > max_blocks * kBlock ? max_blocks * kBlock : n);
    P->row_n[b] = n;
    const int nb = (n + kBlock - 1) / kBlock;
    longest = std::max(longest, nb);
    total += nb;
    if (total > 0x3fffffff) return -1;
    P->row_start[b + 1] = (int32_t)total;
  }
  if (total == 0) return -1;
  const int grid_max = stream_launch_grid();
  if (grid_max <= 0) return -1;
  P->total = (int)total;
  const int even = (int)((total + grid_max - 1) / grid_max);
  // a row of n blocks spans at most ceil((n - 1) / share) + 1 shares
  const int chained = std::max(even, (longest - 1 + kPrevSpan - 2) / (kPrevSpan - 1));
  if (!(chain && chained > even && plan_shares(P, batch, chained, grid_max)) && !plan_shares(P, batch, even, grid_max))
    return -1;
  // a merge launch is needed for empty rows and rows cut by share ends; rows
  // that span many shares (few rows) are merged per query head
  int most = 1;
  bool need = false;
  for (int b = 0; b < batch; ++b) {
    if (P->row_n[b] <= 0) {
      need = true;
      continue;
    }
    const int span = (P->row_start[b + 1] - 1) / P->share - P->row_start[b] / P->share + 1;
    need |= span > 1;
    most = std::max(most, span);
  }
  *merge_kind = !need ? 0 : (most > 32 ? 2 : 1);
  return most > kPrevSpan ? 1 : 0;
}

int stream_prepare(bool fused, const StreamCall& c, StreamLaunch* L) {
  const int G = c.n_kv > 0 ? c.n_q / c.n_kv : 0;
  if (!c.row_lens_host || c.batch <= 0 || c.batch > kStreamMaxSeqs || G > 4 || c.n_q > kMaxQ ||
      c.n_kv > kWaves || kWaves % c.n_kv || !c.records)
    return -1;
  StreamArgs& a = L->a;
  a = StreamArgs{};
  a.out = c.out;
  a.q = c.q;
  a.k_new = c.k_new;
  a.v_new = c.v_new;
  a.k_pool = c.k_pool;
  a.v_pool = c.v_pool;
  a.bt = c.block_table;
  a.slot_ids = c.slot_ids;
  a.rope = c.cos_sin;
  a.bt_stride = c.bt_row_stride;
  a.num_blocks = c.num_blocks;
  a.num_slots = c.num_slots;
  a.max_blocks = c.max_blocks;
  a.n_q = c.n_q;
  a.n_kv = c.n_kv;
  a.max_pos = c.max_pos;
  a.batch = c.batch;
  a.scale_log2e = c.scale * kLog2e;
  a.errors = device_errors_ptr();
  a.kv_nt = c.kv_nt ? 1 : 0;
  int merge = 0;
  const int pr = stream_plan_build(c.batch, c.row_lens_host, c.max_blocks, c.slot_ids_host, c.slot_ids != nullptr,
                                   c.num_slots, c.chain_plan, &a.plan, &merge);
  if (pr < 0) return -1;
  L->long_rows = pr > 0;                // a row spans more shares than a chained prologue merges
  const int launched = c.fixed_shape ? stream_launch_grid() : a.plan.grid;
  if (c.records_bytes < (size_t)2 * launched * c.n_q * kRec * sizeof(float)) return -1;
  a.ws = c.records;
  L->prev = c.out_prev != nullptr;
  if (L->prev) {
    if (!c.records_prev || L->long_rows) return -1;
    a.out_prev = c.out_prev;
    a.ws_prev = c.records_prev;
  }
  L->devplan = c.plan_dev != nullptr;
  if (L->devplan) {
    a.plan_dev = c.plan_dev;
    if (c.fixed_shape) {
      // the plan may change between replays: the launch shapes may not depend
      // on it (one workgroup per CU, workgroups past the plan's shares exit;
      // a merge launch always follows: per KV head for chained launches,
      // whose rows span at most kPrevSpan shares, else per query head)
      if (c.chain_plan && L->long_rows) return -1;
      merge = c.chain_plan ? 1 : 2;
    }
  } else if (c.fixed_shape) {
    return -1;
  }
  a.plan_out = c.plan_out;
  L->grid = launched;
  L->fused = fused;
  L->G = G;
  L->merge = merge;
  return PKV_OK;
}

int stream_enqueue(const StreamLaunch& L, hipStream_t st, bool merge) {
  StreamArgs a = L.a;
  StreamCore core = L.a;               // device-plan launches pass the core alone
  void* args[] = {L.devplan ? static_cast<void*>(&core) : static_cast<void*>(&a)};
  const bool nt = L.a.kv_nt != 0;
  const void* fn;
  if (L.devplan)
    fn = L.prev ? pick_stream<true, true, true>(L.G, nt) : pick_stream<true, false, true>(L.G, nt);
  else
    fn = L.fused ? (L.prev ? pick_stream<true, true, false>(L.G, nt) : pick_stream<true, false, false>(L.G, nt))
                 : (L.prev ? pick_stream<false, true, false>(L.G, nt) : pick_stream<false, false, false>(L.G, nt));
  const int rc = launch_status(hipLaunchKernel(fn, dim3(L.grid), dim3(kThreads), args, 0, st));
  if (rc != PKV_OK || !merge) return rc;
  return stream_merge_enqueue(L, st);
}

int stream_read_probe(const StreamCall& c, uint32_t* sink, hipStream_t st) {
  if (!c.row_lens_host || c.batch <= 0 || c.batch > kStreamMaxSeqs || c.n_kv <= 0 || c.n_kv > kWaves ||
      kWaves % c.n_kv)
    return PKV_ERR_UNSUPPORTED;
  StreamArgs a{};
  a.k_pool = c.k_pool;
  a.v_pool = c.v_pool;
  a.bt = c.block_table;
  a.slot_ids = c.slot_ids;
  a.bt_stride = c.bt_row_stride;
  a.num_blocks = c.num_blocks;
  a.num_slots = c.num_slots;
  a.max_blocks = c.max_blocks;
  a.n_kv = c.n_kv;
  a.batch = c.batch;
  a.kv_nt = c.kv_nt ? 1 : 0;
  int merge = 0;
  if (stream_plan_build(c.batch, c.row_lens_host, c.max_blocks, c.slot_ids_host, c.slot_ids != nullptr, c.num_slots,
                        false, &a.plan, &merge) < 0)
    return PKV_ERR_UNSUPPORTED;
  if (a.plan.share > kWin) return PKV_ERR_UNSUPPORTED;     // one table window per share
  void* args[] = {&a, &sink};
  const void* fn = c.kv_nt ? (const void*)stream_read_probe_kernel<true> : (const void*)stream_read_probe_kernel<false>;
  return launch_status(hipLaunchKernel(fn, dim3(a.plan.grid), dim3(kThreads),
                                       args, 0, st));
}

int stream_merge_enqueue(const StreamLaunch& L, hipStream_t st) {
  if (L.merge == 0) return PKV_OK;
  StreamArgs a = L.a;
  StreamCore core = L.a;
  void* args[] = {L.devplan ? static_cast<void*>(&core) : static_cast<void*>(&a)};
  if (L.merge == 2)
    return launch_status(hipLaunchKernel(L.devplan ? (const void*)stream_merge_wide_kernel<true>
                                                   : (const void*)stream_merge_wide_kernel<false>,
                                         dim3(a.n_q, a.batch), dim3(1024), args, 0, st));
  const void* mg = L.devplan ? pick_merge<true>(L.G) : pick_merge<false>(L.G);
  return launch_status(hipLaunchKernel(mg, dim3(a.n_kv, a.batch), dim3(256), args, 0, st));
}

}  // namespace pkv

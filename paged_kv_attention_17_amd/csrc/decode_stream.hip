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
// heads, 16 KB of K and V each), so a CU streams contiguous 1 KB token rows.
//
// Work inside a workgroup.  16 waves = n_kv heads x (16 / n_kv) lanes of
// blocks: wave w serves KV head w % n_kv and takes every (16 / n_kv)-th block
// of the share, with two blocks in flight.  The block's arithmetic runs on the
// matrix cores: scores S^T = K . Q^T (two 16x16x32 products, K straight from
// its loads, the G query heads as columns), then O^T += V^T . P^T (four
// 16x16x16 products, V transposed through a per-wave LDS tile), so the vector
// ALU is left with the masks, the exponentials and the rare rescale.  The rows
// the share touches (at most kMaxRows) have their
// queries staged in LDS, rotated when fused.  When a wave's next block belongs
// to another row it folds its state for the finished row (DPP and lane
// shuffles over the 8 row groups) into that row's LDS slot, without waiting
// for the other waves.  After the last block one barrier, then the waves of
// each KV head are merged per row: a row that lies inside the share is
// finished in place, a row cut by the share's ends leaves (max, sum,
// unnormalised output) in one of the share's two workspace records, and a
// small kernel merges those records.
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

namespace pkv {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxRows = 4;           // rows one share may touch
constexpr int kMaxSeqs = 256;         // batch rows described in the arguments
constexpr int kMaxQ = 32;             // query heads staged per row
constexpr int kMaxGrid = 512;         // workgroups (one per CU)
constexpr int kRec = kHeadDim + 2;    // partial record per query head: o[64], max, sum
constexpr int kWin = kThreads;        // blocks whose table entries are staged in LDS at a time

struct StreamArgs {
  uint16_t* out;
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_pool;
  uint16_t* v_pool;
  const int32_t* bt;
  const int32_t* slot_ids;
  const float2* rope;
  float* ws;                   // records [2 * grid][n_q][kRec]
  int64_t bt_stride;
  int num_blocks;
  int num_slots;
  int max_blocks;
  int n_q;
  int n_kv;
  int max_pos;
  int batch;
  float scale_log2e;
  int share;                   // blocks per workgroup
  int total;                   // blocks in the stream
  int32_t row_start[kMaxSeqs + 1];   // first stream block of each row
  int32_t row_n[kMaxSeqs];           // tokens of each row
  uint16_t wg_rows[kMaxGrid];        // per workgroup: first row << 3 | rows touched
};
static_assert(sizeof(StreamArgs) <= 4096, "kernel argument block");

__device__ __forceinline__ int row_slot(const StreamArgs& a, int b) {
  const int s = a.slot_ids ? a.slot_ids[b] : b;
  return (s >= 0 && s < a.num_slots) ? s : -1;
}

// Rotate chunk `own` (8 dims starting at 8 * ch) against its pair partner
// chunk (ch ^ 4) with the position's cos/sin row.
__device__ __forceinline__ uint4 rope_own_chunk(uint4 own, uint4 oth, const float2* trow, int ch) {
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
      const float2 t = trow[(ch & 3) * 8 + 2 * j + e];
      r[e] = first_half ? rope_first(mine, other, t.x, t.y) : rope_second(other, mine, t.x, t.y);
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

  // One 16-token block: V rows go through the wave's LDS tile (rows past the
  // context, or of a block whose id is out of range, are zeroed there so NaN
  // in unused pool slots cannot reach the output); scores of such tokens are
  // replaced by -inf (a select, never a product).  `extra` is a token slot
  // that takes part whatever the block (the fused step's new token), or -1.
  __device__ __forceinline__ void block(uint4 qb0, uint4 qb1, const KVRegs& R, uint16_t* vtile, int wr0, int wr1,
                                        const int (&rd)[4], int r, int q4, bool blk_ok, int valid, int extra,
                                        float C, float invC) {
    const bool full = blk_ok && valid == kBlock;
    uint4 v0 = R.v0, v1 = R.v1;
    if (!full) {
      const uint4 z = make_uint4(0, 0, 0, 0);
      v0 = sel4((blk_ok && r < valid) || r == extra, v0, z);
      v1 = sel4((blk_ok && r + 8 < valid) || r + 8 == extra, v1, z);
    }
    *reinterpret_cast<uint4*>(vtile + wr0) = v0;
    *reinterpret_cast<uint4*>(vtile + wr1) = v1;

    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
    sc = mfma_qk(R.k0, qb0, sc);
    sc = mfma_qk(R.k1, qb1, sc);
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

template <int G, bool FUSED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void stream_kernel(StreamArgs a) {
  const int B0 = blockIdx.x * a.share;
  const int B1 = min(B0 + a.share, a.total);
  if (B0 >= B1) return;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = wave_uniform(tid >> 6);
  const int c = lane & 7;
  const int r = lane >> 3;
  const int n_kv = a.n_kv;
  const int S = kWaves / n_kv;           // waves per KV head
  const int h = w % n_kv;                // this wave's KV head
  const int s = w / n_kv;                // and its lane of blocks
  const int wr = a.wg_rows[blockIdx.x];
  const int bf = wr >> 3;                // first row of the share
  const int nrows = wr & 7;              // rows it touches
  const int64_t row_elems = (int64_t)n_kv * kHeadDim;
  const float C = a.scale_log2e;
  const float invC = 1.0f / C;

  __shared__ uint4 sq[kMaxRows][kMaxQ * 8];                 // queries: [row][head][chunk]
  __shared__ uint4 snew[kMaxRows][2][kWaves * 8];           // fused: new key / value [row][k|v][head][chunk]
  __shared__ float sp[kMaxRows][kWaves][G][kRec];           // per-wave partials of each row
  __shared__ int srow_ok[kMaxRows];                         // the row's table slot is valid
  __shared__ uint16_t svt[kWaves][kBlock * kHeadDim];       // per-wave V tile (transposed reads)
  __shared__ int s_tab[kWin];                               // window's blocks: pool block id or -1
  __shared__ int s_meta[kWin];                              // and row << 8 | tokens read from the pool
  __shared__ int s_next[kWaves];                            // per KV head: next unclaimed block of the window

  // ---- the share's blocks -------------------------------------------------
  // The share is walked in windows of kWin blocks.  Each window's table slice
  // is computed into LDS (thread t: block t of the window); then the waves of
  // each KV head claim the window's blocks one at a time from the head's LDS
  // counter, so a wave that runs ahead takes more blocks and the waves of the
  // workgroup finish together (with a fixed split the youngest waves of a CU
  // ended long after the oldest).  A wave's claims increase, so it still
  // meets the share's rows in order.
  const int len = B1 - B0;
  const uint32_t block_bytes = (uint32_t)(kBlock * row_elems * 2);
  const uint32_t lane_off = (uint32_t)(((int64_t)r * row_elems + h * kHeadDim + c * 8) * 2);
  const uint32_t lane_off8 = lane_off + (uint32_t)(8 * row_elems * 2);
  // K in the MFMA operand layout: token lane % 16, dims 8 (lane / 16) .. + 7
  // (and the same 32 dims further on for the second operand)
  const uint32_t k_off = (uint32_t)(((int64_t)(lane & 15) * row_elems + h * kHeadDim + 8 * (lane >> 4)) * 2);
  const char* kbase = reinterpret_cast<const char*>(a.k_pool);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool);

  // stream block p -> pool block id and (row << 8 | tokens to read from the
  // pool; the fused step's new token is not among them)
  auto block_info = [&](int p, int& tab, int& meta) {
    int ri = 0;
    for (int i = 1; i < nrows; ++i) ri = p >= a.row_start[bf + i] ? i : ri;
    int start = a.row_start[bf], n = a.row_n[bf];
    for (int i = 1; i < nrows; ++i) {
      start = i == ri ? a.row_start[bf + i] : start;
      n = i == ri ? a.row_n[bf + i] : n;
    }
    const int j = p - start;
    const int slot = row_slot(a, bf + ri);
    int valid = (FUSED ? n - 1 : n) - j * kBlock;
    valid = valid > kBlock ? kBlock : (valid < 0 ? 0 : valid);
    tab = -1;
    if (slot >= 0 && j < a.max_blocks && valid > 0) {
      const int blk = a.bt[(int64_t)slot * a.bt_stride + j];
      tab = (blk >= 0 && blk < a.num_blocks) ? blk : -1;
    }
    meta = (ri << 8) | valid;
  };
  auto issue = [&](KVRegs& R, int blk) {
    blk = blk < 0 ? 0 : blk;
    const auto rk = buf_rsrc(kbase + (size_t)blk * block_bytes, block_bytes);
    const auto rv = buf_rsrc(vbase + (size_t)blk * block_bytes, block_bytes);
    R.k0 = buf_load16(rk, k_off);
    R.k1 = buf_load16(rk, k_off + 64);
    R.v0 = buf_load16(rv, lane_off);
    R.v1 = buf_load16(rv, lane_off8);
  };
  // the first window's table slice is requested before the staging below
  // waits (and written to LDS after it)
  int tab = -1, meta = 0;
  if (tid < min(kWin, len)) block_info(B0 + tid, tab, meta);

  // ---- queries of the share's rows (rotated by position n - 1 when fused) ----
  for (int e = tid; e < nrows * a.n_q * 8; e += kThreads) {
    const int i = e / (a.n_q * 8);
    const int rem = e - i * a.n_q * 8;
    const int ch = rem & 7;
    const int b = bf + i;
    const uint16_t* qrow = a.q + ((int64_t)b * a.n_q + (rem >> 3)) * kHeadDim;
    uint4 v = *reinterpret_cast<const uint4*>(qrow + ch * 8);
    if constexpr (FUSED) {
      const int pos = a.row_n[b] - 1;
      if (pos >= 0 && pos < a.max_pos) {
        const uint4 p = *reinterpret_cast<const uint4*>(qrow + (ch ^ 4) * 8);
        v = rope_own_chunk(v, p, a.rope + (int64_t)pos * (kHeadDim / 2), ch);
      }
    }
    sq[i][rem] = v;
  }
  // ---- fused: the new token of every row whose last block is here: rotated
  // key and value into LDS (it joins the attention from there).  Its pool
  // write waits for the end of the workgroup's stream (no workgroup reads that
  // pool row in this launch), which keeps the table lookup it needs off the
  // start-up path.  nrows * n_kv * 8 <= kMaxRows * kWaves * 8 <= kThreads: one
  // 8-dim chunk per thread.
  int app_blk = -1;                      // pool block of this thread's new-token chunk
  if constexpr (FUSED) {
    if (tid < nrows) srow_ok[tid] = row_slot(a, bf + tid) >= 0;
    if (tid < nrows * n_kv * 8) {
      const int i = tid / (n_kv * 8);
      const int rem = tid - i * n_kv * 8;
      const int ch = rem & 7;
      const int kvh = rem >> 3;
      const int b = bf + i;
      const int n = a.row_n[b];
      const int last = a.row_start[b + 1] - 1;
      if (n > 0 && last >= B0 && last < B1) {
        const int pos = n - 1;
        const uint16_t* krow = a.k_new + ((int64_t)b * n_kv + kvh) * kHeadDim;
        uint4 k = *reinterpret_cast<const uint4*>(krow + ch * 8);
        const uint4 p = *reinterpret_cast<const uint4*>(krow + (ch ^ 4) * 8);
        const uint4 v = *reinterpret_cast<const uint4*>(a.v_new + ((int64_t)b * n_kv + kvh) * kHeadDim + ch * 8);
        const int slot = row_slot(a, b);
        if (slot >= 0) app_blk = a.bt[(int64_t)slot * a.bt_stride + pos / kBlock];
        if (pos < a.max_pos) k = rope_own_chunk(k, p, a.rope + (int64_t)pos * (kHeadDim / 2), ch);
        snew[i][0][rem] = k;
        snew[i][1][rem] = v;
      }
    }
  }
  if (tid < min(kWin, len)) {
    s_tab[tid] = tab;
    s_meta[tid] = meta;
  }
  if (tid < kWaves) s_next[tid] = 0;
  __syncthreads();

  MfmaAcc acc;
  acc.reset();
  const int col = lane & 15;             // MFMA column: query head of the KV head's group
  const int q4 = lane >> 4;              // MFMA lane group
  uint4 qb0, qb1;                        // Q^T operands: dims 8 q4 .. and 32 + 8 q4 ..
  int cur = 0;                           // row of the share being accumulated
  int row_last = -1;                     // fused: stream block holding the row's new token, or -1
  auto load_q = [&]() {
    const uint4 z = make_uint4(0, 0, 0, 0);
    qb0 = col < G ? sq[cur][(h * G + col) * 8 + q4] : z;
    qb1 = col < G ? sq[cur][(h * G + col) * 8 + q4 + 4] : z;
    if constexpr (FUSED) {
      const int b = bf + cur;
      row_last = wave_uniform(a.row_n[b] > 0 && srow_ok[cur] ? a.row_start[b + 1] - 1 : -1);
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
      float* dst = sp[cur][w][col];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        *reinterpret_cast<float4*>(dst + 16 * t + 4 * q4) = make_float4(acc.o[t][0], acc.o[t][1], acc.o[t][2], acc.o[t][3]);
      if (q4 == 0) {
        dst[kHeadDim] = acc.m;
        dst[kHeadDim + 1] = l;
      }
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

  // the next block of this wave's KV head in the current window (wave-uniform)
  auto claim = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(&s_next[h], 1);
    return wave_uniform(v);
  };
  for (int w0 = 0; w0 < len; w0 += kWin) {
    const int wl = min(kWin, len - w0);
    if (w0 > 0) {
      __syncthreads();                   // every wave is done with the previous window
      if (tid < wl) {
        block_info(B0 + w0 + tid, tab, meta);
        s_tab[tid] = tab;
        s_meta[tid] = meta;
      }
      if (tid < kWaves) s_next[tid] = 0;
      __syncthreads();
    }
    auto step = [&](KVRegs R, int i) {
      const int mt = wave_uniform(s_meta[i]);
      while (cur < (mt >> 8)) flush();
      const bool blk_ok = wave_uniform(s_tab[i]) >= 0;
      const int valid = mt & 0xff;       // tokens read from the pool
      int extra = -1;                    // fused: slot of the new token in this block
      if constexpr (FUSED) {
        // the row's last block: the new token (rotated key, value) from LDS
        if (B0 + w0 + i == row_last) {
          extra = valid;
          if (col == extra) {
            R.k0 = snew[cur][0][h * 8 + q4];
            R.k1 = snew[cur][0][h * 8 + q4 + 4];
          }
          if (r == extra) R.v0 = snew[cur][1][h * 8 + c];
          if (r + 8 == extra) R.v1 = snew[cur][1][h * 8 + c];
        }
      }
      acc.block(qb0, qb1, R, vtile, v_wr0, v_wr1, v_rd, r, q4, blk_ok, valid, extra, C, invC);
    };
    // two blocks in flight in two register sets; loads are issued for every
    // claim (a claim past the window reloads the window's last block and is
    // not used), so each step waits for exactly the older set
    KVRegs X, Y;
    int ia = claim();
    issue(X, s_tab[min(ia, wl - 1)]);
    int ib = claim();
    issue(Y, s_tab[min(ib, wl - 1)]);
    while (ia < wl) {
      step(X, ia);
      ia = claim();
      issue(X, s_tab[min(ia, wl - 1)]);
      if (ib >= wl) break;
      step(Y, ib);
      ib = claim();
      issue(Y, s_tab[min(ib, wl - 1)]);
    }
  }
  while (cur < nrows) flush();
  if constexpr (FUSED) {
    // the new token into the pool (position context_len - 1 of its row)
    if (app_blk >= 0 && app_blk < a.num_blocks) {
      const int i = tid / (n_kv * 8);
      const int rem = tid - i * n_kv * 8;
      const int pos = a.row_n[bf + i] - 1;
      const int64_t off = ((int64_t)app_blk * kBlock + pos % kBlock) * row_elems + (rem >> 3) * kHeadDim + (rem & 7) * 8;
      *reinterpret_cast<uint4*>(a.k_pool + off) = snew[i][0][rem];
      *reinterpret_cast<uint4*>(a.v_pool + off) = snew[i][1][rem];
    }
  }
  __syncthreads();

  // ---- merge the KV heads' waves per row: finish rows inside the share,
  // leave records for rows cut by its ends ------------------------------------
  for (int e = tid; e < nrows * a.n_q * kHeadDim; e += kThreads) {
    const int i = e / (a.n_q * kHeadDim);
    const int rem = e - i * a.n_q * kHeadDim;
    const int b = bf + i;
    if (a.row_n[b] <= 0) continue;
    const int qh = rem / kHeadDim;
    const int d = rem % kHeadDim;
    const int hh = qh / G;
    const int g = qh % G;
    float M = sp[i][hh][g][kHeadDim];
    for (int t = 1; t < S; ++t) M = fmaxf(M, sp[i][hh + t * n_kv][g][kHeadDim]);
    float L = 0.f, O = 0.f;
    for (int t = 0; t < S; ++t) {
      const float* src = sp[i][hh + t * n_kv][g];
      const float f = fast_exp2(src[kHeadDim] - M);
      L += f * src[kHeadDim + 1];
      O += f * src[d];
    }
    if (a.row_start[b] >= B0 && a.row_start[b + 1] <= B1) {
      a.out[((int64_t)b * a.n_q + qh) * kHeadDim + d] = to_bf16(L > 0.f ? O / L : 0.f);
    } else {
      const int rec = 2 * (int)blockIdx.x + (i == 0 ? 0 : 1);
      float* dst = a.ws + ((int64_t)rec * a.n_q + qh) * kRec;
      dst[d] = O;
      if (d == 0) {
        dst[kHeadDim] = M;
        dst[kHeadDim + 1] = L;
      }
    }
  }
}

// Merge of the records of rows cut by share ends: one workgroup per (row, KV
// head), thread = (query head, dim).  Share w holds the row in record 2w when
// the row contains the share's first block, else in record 2w + 1.  Empty
// rows get zeros; rows inside one share were finished there.
template <int G>
__global__ __launch_bounds__(256) void stream_merge_kernel(StreamArgs a) {
  const int kvh = blockIdx.x;
  const int b = blockIdx.y;
  const int n = a.row_n[b];
  const int64_t obase = ((int64_t)b * a.n_q + kvh * G) * kHeadDim;
  if (n <= 0) {
    for (int e = threadIdx.x; e < G * kHeadDim; e += blockDim.x) a.out[obase + e] = 0;
    return;
  }
  const int start = a.row_start[b];
  const int w0 = start / a.share;
  const int w1 = (a.row_start[b + 1] - 1) / a.share;
  if (w0 == w1) return;
  for (int e = threadIdx.x; e < G * kHeadDim; e += blockDim.x) {
    const int qh = kvh * G + e / kHeadDim;
    const int d = e % kHeadDim;
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int w = w0; w <= w1; w += 8) {
      float mv[8], lv[8], ov[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ww = w + j <= w1 ? w + j : w1;
        const int rec = 2 * ww + ((ww > w0 || start == w0 * a.share) ? 0 : 1);
        const float* src = a.ws + ((int64_t)rec * a.n_q + qh) * kRec;
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
    a.out[obase + e] = to_bf16(L > 0.f ? O / L : 0.f);
  }
}

// The same merge for batches whose rows span many shares (few rows, long
// contexts): one workgroup per (row, query head), 16 groups of 64 threads
// (thread = dim); group j takes records j, j + 16, ..., eight of them with
// their loads in flight at once, and the groups' partial (max, sum, output)
// are combined through LDS.  More workgroups and shorter chains of dependent
// loads per thread than the kernel above, which leaves a batch of one row
// on n_kv workgroups walking hundreds of records each.
__global__ __launch_bounds__(1024) void stream_merge_wide_kernel(StreamArgs a) {
  constexpr int kGroups = 16;
  __shared__ float part[kGroups][kHeadDim][3];
  const int qh = blockIdx.x;
  const int b = blockIdx.y;
  const int n = a.row_n[b];
  const int d = threadIdx.x % kHeadDim;
  const int grp = threadIdx.x / kHeadDim;
  const int64_t obase = ((int64_t)b * a.n_q + qh) * kHeadDim;
  if (n <= 0) {
    if (grp == 0) a.out[obase + d] = 0;
    return;
  }
  const int start = a.row_start[b];
  const int w0 = start / a.share;
  const int w1 = (a.row_start[b + 1] - 1) / a.share;
  if (w0 == w1) return;
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int w = w0 + grp; w <= w1; w += 8 * kGroups) {
    float mv[8], lv[8], ov[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int wj = w + j * kGroups;
      const int ww = wj <= w1 ? wj : w1;
      const int rec = 2 * ww + ((ww > w0 || start == w0 * a.share) ? 0 : 1);
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

template <bool FUSED>
const void* pick_stream(int G) {
  return G == 1 ? (const void*)stream_kernel<1, FUSED>
       : G == 2 ? (const void*)stream_kernel<2, FUSED>
                : (const void*)stream_kernel<4, FUSED>;
}

}  // namespace

size_t stream_workspace_bytes(int n_q, int n_kv) {
  (void)n_kv;
  return (size_t)2 * kMaxGrid * n_q * kRec * sizeof(float);
}

int stream_decode(bool fused, const StreamCall& c) {
  const int G = c.n_kv > 0 ? c.n_q / c.n_kv : 0;
  if (!c.row_lens_host || c.batch <= 0 || c.batch > kMaxSeqs || G > 4 || c.n_q > kMaxQ ||
      c.n_kv > kWaves || kWaves % c.n_kv || !c.workspace)
    return -1;
  StreamArgs a{};
  a.out = c.out;
  a.q = c.q;
  a.k_new = c.k_new;
  a.v_new = c.v_new;
  a.k_pool = c.k_pool;
  a.v_pool = c.v_pool;
  a.bt = c.block_table;
  a.slot_ids = c.slot_ids;
  a.rope = reinterpret_cast<const float2*>(c.cos_sin);
  a.bt_stride = c.bt_row_stride;
  a.num_blocks = c.num_blocks;
  a.num_slots = c.num_slots;
  a.max_blocks = c.max_blocks;
  a.n_q = c.n_q;
  a.n_kv = c.n_kv;
  a.max_pos = c.max_pos;
  a.batch = c.batch;
  a.scale_log2e = c.scale * kLog2e;
  // the block stream: rows end to end, each ceil(n / 16) blocks
  int64_t total = 0;
  a.row_start[0] = 0;
  for (int b = 0; b < c.batch; ++b) {
    int n = c.row_lens_host[b];
    n = n < 0 ? 0 : (n > c.max_blocks * kBlock ? c.max_blocks * kBlock : n);
    a.row_n[b] = n;
    total += (n + kBlock - 1) / kBlock;
    if (total > 0x3fffffff) return -1;
    a.row_start[b + 1] = (int32_t)total;
  }
  if (total == 0) return -1;
  const int cus = device_cus();
  if (cus <= 0) return -1;
  int grid = std::min(cus, kMaxGrid);
  a.share = (int)((total + grid - 1) / grid);
  grid = (int)((total + a.share - 1) / a.share);
  a.total = (int)total;
  if (c.workspace_bytes < (size_t)2 * grid * c.n_q * kRec * sizeof(float)) return -1;
  a.ws = static_cast<float*>(c.workspace);
  // rows of each share (the row of a block is the last row whose start is at
  // or before it: empty rows share their start with the next row and are
  // passed over); every share must touch at most kMaxRows rows, empty rows in
  // between included
  for (int g = 0, b = 0; g < grid; ++g) {
    const int p0 = g * a.share;
    const int p1 = std::min(p0 + a.share, a.total) - 1;
    while (b + 1 < c.batch && a.row_start[b + 1] <= p0) ++b;
    int e = b;
    while (e + 1 < c.batch && a.row_start[e + 1] <= p1) ++e;
    if (e - b + 1 > kMaxRows) return -1;
    a.wg_rows[g] = (uint16_t)(b << 3 | (e - b + 1));
  }
  void* args[] = {&a};
  hipStream_t st = static_cast<hipStream_t>(c.stream);
  const void* fn = fused ? pick_stream<true>(G) : pick_stream<false>(G);
  int rc = launch_status(hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, st));
  if (rc != PKV_OK) return rc;
  // rows that span many shares (few rows) are merged per query head by 16
  // groups of threads
  int most = 1;
  for (int b = 0; b < c.batch; ++b)
    if (a.row_n[b] > 0) most = std::max(most, (a.row_start[b + 1] - 1) / a.share - a.row_start[b] / a.share + 1);
  if (most > 32)
    return launch_status(hipLaunchKernel((const void*)stream_merge_wide_kernel, dim3(c.n_q, c.batch), dim3(1024),
                                         args, 0, st));
  const void* mg = G == 1 ? (const void*)stream_merge_kernel<1>
                 : G == 2 ? (const void*)stream_merge_kernel<2>
                          : (const void*)stream_merge_kernel<4>;
  return launch_status(hipLaunchKernel(mg, dim3(c.n_kv, c.batch), dim3(256), args, 0, st));
}

}  // namespace pkv

// Chunked causal prefill attention over the paged KV cache, on gfx950 MFMA.
//
// Source: "An Inference Engine in 1,500 Lines of CUDA: The Map", section "The
// path of one inference", closing paragraph (prefill pushes every prompt token
// through at once, so attention is matrix x matrix; decode has its own kernels)
// and the category page's chapter title on chunked prefill (a prompt may arrive
// in chunks; a chunk's queries also see the keys of earlier chunks).
//
// Tiling.  A workgroup of 8 wave64s owns (sequence, KV head, 256 / G query
// tokens): wave w computes query head g*G + w % G for the 32 tokens of query
// subtile w / G, so every K/V tile staged in LDS serves all G heads of the
// group and 256 / G queries.  Per 64-key tile (two 32-key halves) and wave:
//   S^T[key][query] = K . Q^T   four v_mfma_f32_32x32x16_bf16 over the 64 dims
//   online softmax per query    (a lane owns one query column: its 16 keys are
//                                in-lane, the other 16 in lane ^ 32)
//   O^T[dim][query] += V^T . P^T  four MFMAs (2 dim halves x 2 key halves)
// Computing the transposed products keeps the per-query max/sum/rescale in one
// lane.  MFMA contracts A's k slots against B's k slots of the same lane group,
// so any consistent assignment of dims (or keys) to k slots is correct; the key
// assignment used for P^T is the one the S^T accumulator layout already has
// (keys 8*(i/4) + 4*(lane/32) + i%4 for accumulator i).  V stays row-major in
// LDS and the V^T operand is read with the gfx950 transpose load
// (ds_read_b64_tr_b16): within each 16-lane group, lane i's element j comes
// from element i % 4 of the 64-bit word addressed by lane 4j + i / 4, so lanes
// address 4-dim pieces of the keys that the P^T slots hold (the vt_off
// offsets).  V rows are rotated by 16 dims per key (mod 4) and K rows have
// their 16-byte pieces permuted by key (mod 8), so the operand reads hit
// distinct banks without padding.
//
// Pipeline.  K and V tiles travel from the pool straight into a three-stage
// LDS ring by buffer loads that write LDS (no registers, no LDS stores): tile
// kt + 2 is requested while tile kt is computed, each wave waits for its own
// loads of tile kt (s_waitcnt vmcnt) and one barrier per tile publishes them.
// Block ids come from a per-wave table slice (lane j: tile tb + j) read with
// v_readlane.  The running max is shared by a lane and
// lane ^ 32 (both hold the same query) and raised only when a score exceeds it
// by more than 8 (log2 units), so the accumulator rescale and the cross-lane
// exchange are rare; the sum (of the same bf16 weights that multiply V) stays
// per lane until the end.  Masks (causal, and
// keys past the sequence's cached length, which also get V = 0 in LDS) are
// selects applied only on tiles that need them, so NaN in unused pool slots
// never reaches the output.
#include "common.h"

#include <algorithm>
#include <utility>
#include <vector>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kKTile = 64;            // keys per step (two 32-key MFMA blocks)
constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kVsStride = kHeadDim;       // LDS row (bf16) of a V tile, rotated per key
#ifndef PKV_PF_STAGES
#define PKV_PF_STAGES 2
#endif
constexpr int kPfStages = PKV_PF_STAGES;  // steps whose K/V tiles are in LDS at once (ring)
constexpr int kPfDist = kPfStages - 1;    // steps requested ahead of the one computed
constexpr float kPfTau = 8.0f;            // lazy rescale threshold, log2 units
constexpr int kPfMaxItems = 768;          // host-ordered work items carried in the kernel arguments
constexpr uint32_t kOnesBf16 = 0x3F803F80u;  // (1, 1) as a bf16 pair

// Key-tile parities: with G <= 4 the workgroup's waves are split in two
// halves that take the even and the odd key tiles (two tiles per step), and
// the halves' softmax states are merged at the end; with G = 8 every wave is
// one query head and there is one parity.
__host__ __device__ constexpr int pf_parities(int G) { return G <= 4 ? 2 : 1; }
// Query tokens per workgroup for G query heads per KV head (32 per wave).
__host__ __device__ constexpr int pf_qtile(int G) { return 32 * (kPfWaves / (G * pf_parities(G))); }

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
  int q_tiles;        // query tiles per sequence in the grid (fallback order)
  int total_q;
  float scale_log2e;
  uint32_t* errors;   // device error flags (errors.hip), or null
  int n_items;        // > 0: the grid is n_items x n_kv workgroups taking items[id / n_kv]
  uint32_t items[kPfMaxItems];   // (sequence << 12 | query tile), most key tiles first
};

__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

// Element (key, dim) of a V tile in LDS: rows of 64 dims, rotated by 16 dims
// for every key mod 4 (8-dim row pieces and 4-dim read pieces stay contiguous).
__device__ __forceinline__ int vs_index(int key, int dim) { return key * kVsStride + ((dim + 16 * (key & 3)) & 63); }

// Transpose load of 4 bf16 (see the header) from an LDS address.
__device__ __forceinline__ uint2 lds_tr16(const uint16_t* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, r);
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Buffer descriptor words (base, size; gfx9 untyped dword access).
__device__ __forceinline__ v4u rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return v4u{(unsigned)a, (unsigned)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}
// Byte address of a shared-memory location.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
}
// Buffer load of 16 bytes per lane written straight to LDS: lane i's bytes
// land at lds + 16 i; offsets at or past the descriptor's size read zeros.
// Written as assembly so that the compiler neither tracks nor waits for these
// loads: the kernel waits for them itself (s_waitcnt vmcnt, then a barrier).
__device__ __forceinline__ void lds_dma16(v4u rsrc, uint32_t voff, uint32_t lds) {
  // the descriptor and the LDS address are wave-uniform; read them as such so
  // that they sit in scalar registers whatever the compiler inferred
  const v4u r = {(unsigned)__builtin_amdgcn_readfirstlane((int)rsrc[0]),
                 (unsigned)__builtin_amdgcn_readfirstlane((int)rsrc[1]),
                 (unsigned)__builtin_amdgcn_readfirstlane((int)rsrc[2]),
                 (unsigned)__builtin_amdgcn_readfirstlane((int)rsrc[3])};
  const uint32_t l = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  __asm__ volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(r), "s"(l)
                   : "memory", "m0");
}

template <int G>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void prefill_kernel(PrefillArgs a) {
  constexpr int kQTile = pf_qtile(G);
  // Which (sequence, KV head, query tile): from the host's list (most key
  // tiles first, KV heads of one item on consecutive workgroups, hence on
  // different XCDs), else late (heavy) tiles first over all sequences.
  int tile, g, seq;
  if (a.n_items > 0) {
    const int id = blockIdx.x;
    const uint32_t it = a.items[id / a.n_kv];
    g = id % a.n_kv;
    seq = (int)(it >> 12);
    tile = (int)(it & 0xfff);
  } else {
    g = blockIdx.x;
    seq = blockIdx.y;
    tile = a.q_tiles - 1 - (int)blockIdx.z;
  }
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = wave_uniform(tid >> 6);
  const int col = lane & 31;        // query column of this lane
  const int half = lane >> 5;       // which k half of an MFMA operand

  const int q0 = a.cu_q[seq];
  const int q_len = a.cu_q[seq + 1] - q0;
  if (q0 < 0 || q_len <= 0 || q0 + q_len > a.total_q || tile * kQTile >= q_len) return;
  const int slot = a.slot_ids ? a.slot_ids[seq] : seq;
  if (slot < 0 || slot >= a.num_slots) {
    if (threadIdx.x == 0) report_error(a.errors, PKV_DEVERR_BAD_SLOT);
    return;
  }
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

  // kPfStages ring slots, each holding a step's kPar 64-key tiles of K and V
  // (8 KB each), filled by buffer loads that write LDS directly: slot s (16
  // bytes) of K row `key` holds dims 8 (s ^ (key & 7)) .. + 7, slot s of V
  // row `key` holds dims 8 ((s - 2 (key & 3)) & 7) .. + 7 (V element
  // (key, d) sits at vs_index(key, d)); both keep the MFMA-operand reads
  // conflict-free.  After the loop the ring holds the odd parity's softmax
  // states for the merge.
  constexpr int kPar = pf_parities(G);
  constexpr int kSub = kPfWaves / (G * kPar);           // query subtiles per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t kvs[kPfStages][kPar][2][kKTile * kHeadDim];

  // This wave: head hh of the group, query subtile sub, key-tile parity par
  // (tiles kt with kt % kPar == par); this lane: one query.
  const int hh = w % G;
  const int sub = (w / G) % kSub;
  const int par = w / (G * kSub);
  const int h = g * G + hh;
  const int sub0 = tok0 + sub * 32;                // first query of the subtile (chunk-relative)
  const int my_q = sub0 + col;
  const bool q_ok = my_q < tok0 + n_q_tile;
  const int my_pos = start + my_q;
  const int sub_last_pos = start + min(sub0 + 31, tok0 + n_q_tile - 1);   // wave-uniform
  const bool sub_live = sub0 < tok0 + n_q_tile;
  const int sub_key_end = min(sub_last_pos + 1, n_keys);                  // keys this subtile sees
  const int n_steps = (n_ktiles + kPar - 1) / kPar;

  // Loader role: wave w brings keys 8 w .. 8 w + 7 of each of the step's
  // tiles (half of one 16-token block), lane i key 8 w + i / 8 into LDS slot
  // i % 8.  Keys past the cache, and blocks whose id is out of range, read as
  // zeros (offsets beyond the buffer's size), so no NaN from an unused pool
  // slot reaches a product.
  const int ld_row = 8 * (w & 1) + (lane >> 3);              // row inside the block
  const int ld_kx = (lane >> 3) & 7;                         // key & 7
  const uint32_t block_bytes = (uint32_t)(kBlock * row_elems * 2);
  const uint32_t ld_base = (uint32_t)((ld_row * row_elems + g * kHeadDim) * 2);
  const uint32_t ld_koff = ld_base + 16u * (uint32_t)((lane & 7) ^ ld_kx);
  const uint32_t ld_voff = ld_base + 16u * (uint32_t)(((lane & 7) - 2 * (ld_kx & 3)) & 7);
  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  const char* vpool = reinterpret_cast<const char*>(a.v_pool);
  // block ids of this wave's half-blocks for tiles tb .. tb + 63 (lane j: tile tb + j)
  int tb = 0, tabv = -1;
  auto load_table = [&](int t0) {
    tb = t0;
    const int bi = (t0 + lane) * (kKTile / kBlock) + (w >> 1);
    tabv = (t0 + lane) * kKTile < n_keys && bi < a.max_blocks ? btrow[bi] : -1;
    // wait here (vmcnt 0; expcnt and lgkmcnt fields at their maximum), where
    // the compiler sees it, so that no wait for this load is placed on the
    // path every tile takes
    __builtin_amdgcn_s_waitcnt(0x0F70);
  };
  const uint32_t lds_base = lds_addr(&kvs[0][0][0][8 * w * kHeadDim]);   // this wave's rows, slot 0
  constexpr uint32_t kTileBytes = kKTile * kHeadDim * 2;
  // the step's tiles kt = kPar * step + p (a tile past the last reads zeros)
  auto issue = [&](int step, int slot_) {
#pragma unroll
    for (int p = 0; p < kPar; ++p) {
      const int kt = kPar * step + p;
      if (kt - tb >= kWave) load_table(kt);
      const int blk = __builtin_amdgcn_readlane(tabv, kt - tb);
      const bool ok = blk >= 0 && blk < a.num_blocks;
      if (!ok && kt < n_ktiles && kt * kKTile + 8 * w < n_keys && lane == 0)
        report_error(a.errors, PKV_DEVERR_PREFILL_BLOCK);
      const int key = kt * kKTile + 8 * w + (lane >> 3);
      const uint32_t past = key < n_keys ? 0u : 0x80000000u;
      const int64_t boff = (int64_t)(ok ? blk : 0) * block_bytes;
      const uint32_t nrec = ok ? block_bytes : 0u;
      const uint32_t dst = lds_base + (uint32_t)((slot_ * kPar + p) * 2) * kTileBytes;
      lds_dma16(rsrc_words(kpool + boff, nrec), ld_koff | past, dst);
      lds_dma16(rsrc_words(vpool + boff, nrec), ld_voff | past, dst + kTileBytes);
    }
  };

  // Q^T operand: 4 k-steps of 8 dims each.
  uint4 qb[4];
#pragma unroll
  for (int ks_ = 0; ks_ < 4; ++ks_) {
    qb[ks_] = make_uint4(0, 0, 0, 0);
    if (q_ok)
      qb[ks_] = *reinterpret_cast<const uint4*>(a.q + ((int64_t)(q0 + my_q) * a.n_q + h) * kHeadDim + ks_ * 16 +
                                                half * 8);
  }
  // This lane's V^T read offsets inside a 32-key group (key 4 half + kl, dims
  // 16 (g % 2) + 4 (lane % 4) of each dim half; the rotation only depends on kl).
  const int kl = (lane >> 2) & 3;
  const int vdim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int vt_off0 = vs_index(4 * half + kl, vdim);
  const int vt_off1 = vs_index(4 * half + kl, vdim + 32);
  const float C = a.scale_log2e;
  const float invC = 1.0f / C;
  f32x16 o0 = {}, o1 = {};
  float m = -1.0e30f;              // shared by lane and lane ^ 32 (same query)
  float thr = -INFINITY;           // raw-score level above which m must be raised
  float l = 0.f;                   // this lane's half of the sum
  // keys below this bound are visible to this lane's query (none for a
  // padding lane): the causal limit and the cache's end
  const int key_lim = q_ok ? min(my_pos + 1, n_keys) : 0;

  // This lane's K-operand slots: row `col` of each 32-key half, dims
  // 16 ks + 8 half .. + 7, i.e. chunk 2 ks + half at slot (2 ks + half) ^ (col & 7)
  // = 2 (ks ^ kc) + (half ^ (col & 1)) with kc = (col >> 1) & 3.
  const int k_base = col * kHeadDim + 8 * (half ^ (col & 1));
  const int kc = (col >> 1) & 3;

  // Pipeline: step s + kPfDist (kPar tiles) is requested while step s is
  // computed.  Each wave waits for its own loads of step s (2 kPar per step,
  // counted in order), then the barrier makes every wave's part visible and
  // frees the slot that step s + kPfDist overwrites (its previous step,
  // s - 1, is done everywhere).
  load_table(0);
  for (int q = 0; q < kPfDist && q < n_steps; ++q) issue(q, q);
  int st = 0;                                      // ring slot of step s
  for (int step = 0; step < n_steps; ++step) {
    if (kPfDist == 2 && step + 1 < n_steps)
      __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kPar));   // vmcnt(2 kPar): step s + 1's loads may be in flight
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0)
    __syncthreads();
    if (step + kPfDist < n_steps) issue(step + kPfDist, (st + kPfDist) % kPfStages);
    const int kt = kPar * step + par;
    const uint16_t* ks = kvs[st][par][0];
    const uint16_t* vs = kvs[st][par][1];
    st = st == kPfStages - 1 ? 0 : st + 1;
    const int kbase = kt * kKTile;

    if (kt < n_ktiles && sub_live && kbase < sub_key_end) {
      // S^T = K . Q^T for the tile's two 32-key halves (rows: keys, cols: queries)
      f32x16 s[2] = {};
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int ks_ = 0; ks_ < 4; ++ks_) {
          const uint4 ka = *reinterpret_cast<const uint4*>(ks + kh * 32 * kHeadDim + k_base + 16 * (ks_ ^ kc));
          s[kh] = mfma32(ka, qb[ks_], s[kh]);
        }
      }
      // masks only where a key of the tile can lie past a query or the cache
      const bool need_mask = kbase + kKTile - 1 > sub_last_pos - 31 || kbase + kKTile > n_keys;
      if (need_mask) {
        // accumulator i of half kh holds key kbase + 32 kh + 8 (i / 4) + 4 half + i % 4
        const int r = key_lim - kbase - 4 * half;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kh][i] = 32 * kh + 8 * (i / 4) + (i % 4) < r ? s[kh][i] : -INFINITY;
        }
      }
      float tmax = s[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, s[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[1][i]);
      if (__any(tmax > thr)) {
        // raise the shared max of this lane's query (rare)
        const float tm = fmaxf(tmax, shfl_xor(tmax, 32)) * C;
        const float mn = fmaxf(m, tm);
        const float alpha = fast_exp2(m - mn);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          o0[i] *= alpha;
          o1[i] *= alpha;
        }
        m = mn;
        thr = (mn + kPfTau) * invC;
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = fast_exp2(__builtin_fmaf(s[kh][i], C, -m));
        // P^T operands: k-step 0 = accumulators 0..7, k-step 1 = 8..15.
        uint4 pb[2];
        pb[0] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                           pack_bf16x2(p[6], p[7]));
        pb[1] = make_uint4(pack_bf16x2(p[8], p[9]), pack_bf16x2(p[10], p[11]), pack_bf16x2(p[12], p[13]),
                           pack_bf16x2(p[14], p[15]));
        // the sum takes the same bf16 weights as the numerator (dot2 with (1, 1))
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          l = dot2_bf16(pb[u].x, kOnesBf16, l);
          l = dot2_bf16(pb[u].y, kOnesBf16, l);
          l = dot2_bf16(pb[u].z, kOnesBf16, l);
          l = dot2_bf16(pb[u].w, kOnesBf16, l);
        }
        // O^T += V^T . P^T: slot 4u + j of lane (dim, half) must hold key
        // 16 kstep + 8u + 4 half + j (the P^T slot's key), so the addressing
        // lane 16 g + s supplies key ... + 4 (g / 2) + s / 4 and dims
        // 16 (g % 2) + 4 (s % 4) .. + 3 of its dim half.
#pragma unroll
        for (int kstep = 0; kstep < 2; ++kstep) {
          uint2 r[2][2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const uint16_t* row = vs + (kh * 32 + kstep * 16 + 8 * u) * kVsStride;
            r[0][u] = lds_tr16(row + vt_off0);
            r[1][u] = lds_tr16(row + vt_off1);
          }
          o0 = mfma32(make_uint4(r[0][0].x, r[0][0].y, r[0][1].x, r[0][1].y), pb[kstep], o0);
          o1 = mfma32(make_uint4(r[1][0].x, r[1][0].y, r[1][1].x, r[1][1].y), pb[kstep], o1);
        }
      }
    }
  }
  l += shfl_xor(l, 32);
  if constexpr (kPar == 2) {
    // merge the parities, the even one taking the odd one's state from LDS
    // (the ring is free once every wave is past the loop): per lane m, l
    // and the 32 accumulators, in a fixed order
    __syncthreads();
    float* xs = reinterpret_cast<float*>(&kvs[0][0][0][0]) + (w % (G * kSub)) * (34 * kWave);
    if (par == 1) {
      xs[lane] = m;
      xs[kWave + lane] = l;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        xs[(2 + i) * kWave + lane] = o0[i];
        xs[(18 + i) * kWave + lane] = o1[i];
      }
    }
    __syncthreads();
    if (par == 1) return;
    const float m1 = xs[lane];
    const float l1 = xs[kWave + lane];
    const float mm = fmaxf(m, m1);
    const float f0 = fast_exp2(m - mm);
    const float f1 = fast_exp2(m1 - mm);
    l = l * f0 + l1 * f1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      o0[i] = o0[i] * f0 + xs[(2 + i) * kWave + lane] * f1;
      o1[i] = o1[i] * f0 + xs[(18 + i) * kWave + lane] * f1;
    }
  }
  if (!q_ok) return;
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

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_paged_attn_prefill(pkv_bf16* out, const pkv_bf16* q, const int32_t* cu_q_lens,
                                      const int32_t* q_start_pos, const int32_t* slot_ids, const pkv_bf16* k_pool,
                                      const pkv_bf16* v_pool, int num_blocks, const int32_t* block_table,
                                      int64_t bt_row_stride, int num_slots, int max_blocks_per_seq, int num_seqs,
                                      int total_q, int max_q_len, int n_q_heads, int n_kv_heads, int head_dim,
                                      float scale, const int32_t* cu_q_lens_host, const int32_t* q_start_host,
                                      void* stream) {
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || num_blocks < 0 || num_slots < 0 ||
      max_blocks_per_seq < 0 || bt_row_stride < max_blocks_per_seq || !(scale > 0.f && scale < 3.0e38f))
    return PKV_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads) return PKV_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || !ratio_supported(n_q_heads, n_kv_heads)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PKV_OK;
  if (!out || !q || !cu_q_lens || !q_start_pos || !k_pool || !v_pool || !block_table) return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned4(block_table) ||
      !aligned4(cu_q_lens) || !aligned4(q_start_pos) || (slot_ids && !aligned4(slot_ids)))
    return PKV_ERR_MISALIGNED;
  if (num_seqs > 65535 || n_kv_heads > 65535) return PKV_ERR_INVALID_ARG;
  static_assert(sizeof(PrefillArgs) <= 4096, "kernel argument block");
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
  const int G = n_q_heads / n_kv_heads;
  a.q_tiles = (max_q_len + pf_qtile(G) - 1) / pf_qtile(G);
  a.total_q = total_q;
  a.scale_log2e = scale * 1.4426950408889634f;
  a.errors = device_errors_ptr();
  const void* fn = G == 1 ? (const void*)prefill_kernel<1>
                 : G == 2 ? (const void*)prefill_kernel<2>
                 : G == 4 ? (const void*)prefill_kernel<4>
                          : (const void*)prefill_kernel<8>;
  // With the lengths on the host: one workgroup per real (sequence, query
  // tile, KV head), most key tiles first.  The hardware hands workgroups out
  // in id order and places them by id, so a list sorted by work keeps every
  // XCD and shader engine busy to the end (the fallback grid holds empty
  // workgroups for short sequences and groups work by sequence).
  a.n_items = 0;
  if (cu_q_lens_host && q_start_host) {
    const int qt = pf_qtile(G);
    std::vector<std::pair<int, uint32_t>> items;
    bool fits = true;
    for (int s = 0; s < num_seqs && fits; ++s) {
      const int ql = cu_q_lens_host[s + 1] - cu_q_lens_host[s];
      for (int t = 0; t * qt < ql && fits; ++t) {
        const int64_t last = (int64_t)q_start_host[s] + std::min((t + 1) * qt, ql);   // keys seen, at most
        const int nk = (int)std::min<int64_t>((last + kKTile - 1) / kKTile, 1 << 30);
        items.push_back({nk, (uint32_t)s << 12 | (uint32_t)t});
        fits = (int)items.size() <= kPfMaxItems && t < 4096 && s < (1 << 20);
      }
    }
    if (fits && !items.empty()) {
      std::stable_sort(items.begin(), items.end(), [](const auto& x, const auto& y) { return x.first > y.first; });
      for (size_t i = 0; i < items.size(); ++i) a.items[i] = items[i].second;
      a.n_items = (int)items.size();
    }
  }
  void* args[] = {&a};
  const dim3 grid = a.n_items > 0 ? dim3((unsigned)(a.n_items * n_kv_heads)) : dim3(n_kv_heads, num_seqs, a.q_tiles);
  if (a.n_items == 0 && a.q_tiles > 65535) return PKV_ERR_INVALID_ARG;
  return launch_status(hipLaunchKernel(fn, grid, dim3(kPfThreads), args, 0, (hipStream_t)stream));
}

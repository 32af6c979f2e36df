// Per-block arithmetic of paged single-query attention on the vector ALU, used
// by the per-partition decode kernel (the streaming kernel shares the
// constants and register types and does its arithmetic on the matrix cores).
//
// Source: the Korean page of "An Inference Engine in 1,500 Lines of CUDA: The
// Map" ("What is in the box" table: online softmax inside the PagedAttention
// kernel, four query heads per KV head).
//
// Lane layout inside a wave: lane = 8 r + c.  c picks dims 8c..8c+7 (one
// 16-byte chunk), r picks rows r and r + 8 of a 16-token block.  One dwordx4
// load per lane covers rows r of all lanes = 8 contiguous 128-byte head rows
// of the pool layout [block][16][kv head][64].
//   scores   s = q . k with v_dot2_f32_bf16 (bf16 pairs, float32 sum): 4 per
//            (row, head), then a 3-step DPP sum over the 8 lanes of the row;
//   softmax  one running max per head shared by the whole wave, raised only
//            when some score exceeds it by more than 8 (log2 units), so the
//            rescale of the accumulators is rare; p = 2^(s*scale*log2e - m);
//   p . V    p of rows r and r+8 packed as a bf16 pair, V of the same rows
//            packed per dim with v_perm_b32, one v_dot2_f32_bf16 per
//            (head, dim): float32 accumulation of bf16 products;
//   sum      l accumulates the same bf16 p values as the numerator (dot2 with
//            (1, 1)), so numerator and denominator see identical weights.
// Rows past the context (or in a block whose id is out of range) are removed
// by selects on the scores and on V, never by multiplying, so NaN in unused
// pool slots cannot reach the output.
#pragma once

#include "common.h"

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;   // running-max start (finite, so no inf - inf)
constexpr float kTau = 8.0f;          // lazy rescale threshold, log2 units
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;

struct KVRegs {
  uint4 k0, k1, v0, v1;        // rows r and r + 8 of one block, this lane's 8 dims
};

// Element-wise select (keeps the four dwords in registers).
__device__ __forceinline__ uint4 sel4(bool t, uint4 a, uint4 b) {
  return make_uint4(t ? a.x : b.x, t ? a.y : b.y, t ? a.z : b.z, t ? a.w : b.w);
}

// Maximum over the wave; rows repeat across the 8 lanes of a row group.
__device__ __forceinline__ float wave_max_rows(float x) {
  x = fmaxf(x, dpp<kDppRowRor8>(x));
  x = fmaxf(x, shfl_xor(x, 16));
  x = fmaxf(x, shfl_xor(x, 32));
  return x;
}

// Rotate this lane's 8 dims (chunk c) of a 64-dim head vector in place.  The
// pair partner of dim i < 32 is dim i + 32, held by lane c ^ 4 of the row group.
__device__ __forceinline__ uint4 rope_chunk(uint4 v, const float2* cs, int c) {
  uint4 pv;
  pv.x = (uint32_t)__builtin_amdgcn_ds_bpermute(((int)__lane_id() ^ 4) << 2, (int)v.x);
  pv.y = (uint32_t)__builtin_amdgcn_ds_bpermute(((int)__lane_id() ^ 4) << 2, (int)v.y);
  pv.z = (uint32_t)__builtin_amdgcn_ds_bpermute(((int)__lane_id() ^ 4) << 2, (int)v.z);
  pv.w = (uint32_t)__builtin_amdgcn_ds_bpermute(((int)__lane_id() ^ 4) << 2, (int)v.w);
  const uint32_t own[4] = {v.x, v.y, v.z, v.w};
  const uint32_t oth[4] = {pv.x, pv.y, pv.z, pv.w};
  uint32_t res[4];
  const bool first_half = c < 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float r[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float mine = e ? bf16_hi(own[j]) : bf16_lo(own[j]);
      const float other = e ? bf16_hi(oth[j]) : bf16_lo(oth[j]);
      const float2 t = cs[2 * j + e];
      r[e] = first_half ? rope_first(mine, other, t.x, t.y) : rope_second(other, mine, t.x, t.y);
    }
    res[j] = pack_bf16x2(r[0], r[1]);
  }
  return make_uint4(res[0], res[1], res[2], res[3]);
}

// Online-softmax state of one wave for G query heads: the wave-uniform running
// max m (log2 units), the raw-score level thr above which m must be raised,
// and this lane's share of the sum l and of the unnormalised output o (dims
// 8c..8c+7, rows r and r + 8 of every block it saw).
template <int G>
struct OnlineSoftmax {
  float m[G], thr[G], l[G], o[G][8];

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegBig;
      thr[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[h][i] = 0.f;
    }
  }

  // Raise the running max to cover raw scores s0/s1 (rare: only when some
  // score exceeds the current max by more than kTau in log2 units).
  __device__ __forceinline__ void rescale_if_needed(const float (&s0)[G], const float (&s1)[G], float C,
                                                    float invC) {
    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h) need |= (s0[h] > thr[h]) | (s1[h] > thr[h]);
    if (__any(need)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mx = fmaxf(s0[h], s1[h]) * C;
        const float mn = fmaxf(m[h], wave_max_rows(mx));
        const float alpha = fast_exp2(m[h] - mn);
        l[h] *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[h][j] *= alpha;
        m[h] = mn;
        thr[h] = (mn + kTau) * invC;
      }
    }
  }

  // One block: branch-free apart from the rare rescale.  ok0 / ok1 say
  // whether rows r / r + 8 of the block are part of the context.
  __device__ __forceinline__ void block(const uint4 (&qv)[G], const KVRegs& R, bool ok0, bool ok1, float C,
                                        float invC) {
    float s0[G], s1[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d0 = dot2_bf16(qv[h].x, R.k0.x, 0.f);
      float d1 = dot2_bf16(qv[h].x, R.k1.x, 0.f);
      d0 = dot2_bf16(qv[h].y, R.k0.y, d0);
      d1 = dot2_bf16(qv[h].y, R.k1.y, d1);
      d0 = dot2_bf16(qv[h].z, R.k0.z, d0);
      d1 = dot2_bf16(qv[h].z, R.k1.z, d1);
      d0 = dot2_bf16(qv[h].w, R.k0.w, d0);
      d1 = dot2_bf16(qv[h].w, R.k1.w, d1);
      d0 = sum8(d0);
      d1 = sum8(d1);
      // keep the score computation unconditional (no branch around it)
      __asm__ volatile("" : "+v"(d0), "+v"(d1));
      s0[h] = ok0 ? d0 : -INFINITY;
      s1[h] = ok1 ? d1 : -INFINITY;
    }
    rescale_if_needed(s0, s1, C, invC);
    const uint4 z = make_uint4(0, 0, 0, 0);
    const uint4 v0 = sel4(ok0, R.v0, z);
    const uint4 v1 = sel4(ok1, R.v1, z);
    const uint32_t vlo[4] = {pack_lo_halves(v0.x, v1.x), pack_lo_halves(v0.y, v1.y),
                             pack_lo_halves(v0.z, v1.z), pack_lo_halves(v0.w, v1.w)};
    const uint32_t vhi[4] = {pack_hi_halves(v0.x, v1.x), pack_hi_halves(v0.y, v1.y),
                             pack_hi_halves(v0.z, v1.z), pack_hi_halves(v0.w, v1.w)};
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p0 = fast_exp2(__builtin_fmaf(s0[h], C, -m[h]));
      const float p1 = fast_exp2(__builtin_fmaf(s1[h], C, -m[h]));
      const uint32_t pp = pack_bf16x2(p0, p1);
      l[h] = dot2_bf16(pp, kOnesBf16x2, l[h]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[h][2 * j] = dot2_bf16(pp, vlo[j], o[h][2 * j]);
        o[h][2 * j + 1] = dot2_bf16(pp, vhi[j], o[h][2 * j + 1]);
      }
    }
  }

  // One extra token (k, v: this lane's 8 dims), counted by the lanes with
  // `active` (one row group) only.
  __device__ __forceinline__ void token(const uint4 (&qv)[G], uint4 k, uint4 v, bool active, float C,
                                        float invC) {
    float s0[G], s1[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d = dot2_bf16(qv[h].x, k.x, 0.f);
      d = dot2_bf16(qv[h].y, k.y, d);
      d = dot2_bf16(qv[h].z, k.z, d);
      d = dot2_bf16(qv[h].w, k.w, d);
      s0[h] = active ? sum8(d) : -INFINITY;
      s1[h] = -INFINITY;
    }
    rescale_if_needed(s0, s1, C, invC);
    const uint4 v0 = sel4(active, v, make_uint4(0, 0, 0, 0));
    const uint32_t vv[4] = {v0.x, v0.y, v0.z, v0.w};
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint32_t pp = pack_bf16x2(fast_exp2(__builtin_fmaf(s0[h], C, -m[h])), 0.f);
      l[h] = dot2_bf16(pp, kOnesBf16x2, l[h]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[h][2 * j] = dot2_bf16(pp, vv[j] & 0xffffu, o[h][2 * j]);
        o[h][2 * j + 1] = dot2_bf16(pp, vv[j] >> 16, o[h][2 * j + 1]);
      }
    }
  }
};

}  // namespace pkv

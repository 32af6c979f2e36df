// Llama-3-scaled rotary position embedding for gfx950.
//
// Source: "An Inference Engine in 1,500 Lines of CUDA: The Map", section "The
// path of one inference", step (3) (a positional-encoding table built once from
// base 500000 and the scaling numbers 32, 1, 4, 8192) and the paired kernels
// ropeKernel_llama3 / ropeKernelDecode named in the section's closing paragraph.
// The scaling rule itself is the public Llama-3 one (see pagedkv.h).
//
// Design: the table holds float32 (cos, sin) per (position, pair), computed in
// double on the host, so the device never reduces a large angle.  The rotation
// kernel gives each thread eight pairs of one (token, head): the 16-byte chunk
// of dims 8c .. 8c + 7, the chunk 32 dims further on that holds their
// partners, and the pairs' 64 bytes of table, all in 16-byte accesses;
// float32 math, nearest-even bf16 stores.  A decode step's few hundred KB are
// launch-latency bound; a prefill chunk of a few thousand tokens moves tens
// of MB, which the wide accesses stream.
#include <cmath>
#include <vector>

#include "common.h"

namespace pkv {

__global__ __launch_bounds__(256) void rope_kernel(uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                                                   const int32_t* __restrict__ positions, int num_tokens,
                                                   int n_q, int n_kv, const float2* __restrict__ table,
                                                   int max_pos) {
  constexpr int kHalf = kHeadDim / 2;
  constexpr int kChunks = kHalf / 8;     // 8-pair chunks per head row
  const int heads = n_q + (k ? n_kv : 0);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)num_tokens * heads * kChunks;
  if (gid >= total) return;
  const int c = (int)(gid % kChunks);
  const int64_t th = gid / kChunks;
  const int h = (int)(th % heads);
  const int t = (int)(th / heads);
  const int pos = positions[t];
  if (pos < 0 || pos >= max_pos) return;
  uint16_t* row = h < n_q ? q + ((int64_t)t * n_q + h) * kHeadDim
                          : k + ((int64_t)t * n_kv + (h - n_q)) * kHeadDim;
  uint4* r4 = reinterpret_cast<uint4*>(row);
  const uint4 lo = r4[c];                // dims 8c .. 8c + 7
  const uint4 hi = r4[c + kChunks];      // their partners, 32 dims further on
  // (cos, sin) of pairs 8c .. 8c + 7, two pairs per 16-byte load
  const float4* tb = reinterpret_cast<const float4*>(table + (int64_t)pos * kHalf + 8 * c);
  const uint32_t xs[4] = {lo.x, lo.y, lo.z, lo.w};
  const uint32_t ys[4] = {hi.x, hi.y, hi.z, hi.w};
  uint32_t out_lo[4], out_hi[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 cs = tb[j];
    const float x0 = bf16_lo(xs[j]), x1 = bf16_hi(xs[j]);
    const float y0 = bf16_lo(ys[j]), y1 = bf16_hi(ys[j]);
    out_lo[j] = pack_bf16x2(rope_first(x0, y0, cs.x, cs.y), rope_first(x1, y1, cs.z, cs.w));
    out_hi[j] = pack_bf16x2(rope_second(x0, y0, cs.x, cs.y), rope_second(x1, y1, cs.z, cs.w));
  }
  r4[c] = make_uint4(out_lo[0], out_lo[1], out_lo[2], out_lo[3]);
  r4[c + kChunks] = make_uint4(out_hi[0], out_hi[1], out_hi[2], out_hi[3]);
}

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_rope_table_init(float* cos_sin, int max_pos, int head_dim, double theta, double factor,
                                   double low_freq_factor, double high_freq_factor, int original_max_pos,
                                   void* stream) {
  if (!cos_sin) return PKV_ERR_NULL;
  if (!aligned16(cos_sin)) return PKV_ERR_MISALIGNED;
  if (max_pos < 1 || head_dim < 2 || head_dim % 2 || !(theta > 0) || !(factor > 0) ||
      !(high_freq_factor > low_freq_factor) || !(low_freq_factor > 0) || original_max_pos < 1)
    return PKV_ERR_INVALID_ARG;
  const int half = head_dim / 2;
  const double pi = 3.14159265358979323846;
  std::vector<double> f(half);
  const double w_hi = (double)original_max_pos / high_freq_factor;
  const double w_lo = (double)original_max_pos / low_freq_factor;
  for (int i = 0; i < half; ++i) {
    const double base = std::pow(theta, -(2.0 * i) / head_dim);
    const double wl = 2.0 * pi / base;
    if (wl < w_hi) {
      f[i] = base;
    } else if (wl > w_lo) {
      f[i] = base / factor;
    } else {
      const double s = ((double)original_max_pos / wl - low_freq_factor) / (high_freq_factor - low_freq_factor);
      f[i] = (1.0 - s) * base / factor + s * base;
    }
  }
  std::vector<float> host((size_t)max_pos * half * 2);
  for (int p = 0; p < max_pos; ++p)
    for (int i = 0; i < half; ++i) {
      const double a = (double)p * f[i];
      host[((size_t)p * half + i) * 2 + 0] = (float)std::cos(a);
      host[((size_t)p * half + i) * 2 + 1] = (float)std::sin(a);
    }
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(cos_sin, host.data(), host.size() * sizeof(float), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return launch_status(e);
}

extern "C" int pkv_rope_decode(pkv_bf16* q, pkv_bf16* k, const int32_t* positions, int num_tokens,
                               int n_q_heads, int n_kv_heads, int head_dim, const float* cos_sin, int max_pos,
                               void* stream) {
  if (num_tokens < 0 || n_q_heads < 0 || n_kv_heads < 0 || max_pos < 1) return PKV_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!q || !positions || !cos_sin) return PKV_ERR_NULL;
  if (!aligned16(q) || (k && !aligned16(k)) || !aligned4(positions) || !aligned16(cos_sin))
    return PKV_ERR_MISALIGNED;
  const int heads = n_q_heads + (k ? n_kv_heads : 0);
  const int64_t total = (int64_t)num_tokens * heads * (kHeadDim / 16);
  if (total == 0) return PKV_OK;
  const int64_t grid = (total + 255) / 256;
  if (grid > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  uint16_t* qa = q;
  uint16_t* ka = k;
  const int32_t* pa = positions;
  int nt = num_tokens, nq = n_q_heads, nk = n_kv_heads, mp = max_pos;
  const float2* ta = reinterpret_cast<const float2*>(cos_sin);
  void* args[] = {&qa, &ka, &pa, &nt, &nq, &nk, &ta, &mp};
  return launch_status(hipLaunchKernel((const void*)rope_kernel, dim3((unsigned)grid), dim3(256), args, 0,
                                       (hipStream_t)stream));
}

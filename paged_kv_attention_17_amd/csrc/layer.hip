// The rest of a Llama decode layer around the paged attention, for gfx950:
// RMSNorm and the gated-SiLU product as HIP kernels, the projections as plain
// bf16 GEMMs from rocBLAS (float32 accumulation), and pkv_decode_layer, which
// runs one layer's decode step.
//
// Source: "An Inference Engine in 1,500 Lines of CUDA: The Map" -- the engine
// runs Llama 3.2 1B (opening paragraph), has its own RMSNorm kernel (Korean
// page, "What is in the box": rmsNormKernel), keeps a 2048-wide hidden state
// (the buf_2048_* buffers of "A function with 51 parameters") and leaves the
// projections to the vendor GEMM (chapter-4 title).  The formulas are the
// public Llama ones: rmsnorm(x) = x / sqrt(mean(x^2) + eps) * w, the gated
// MLP (silu(x W_gate^T) * (x W_up^T)) W_down^T, residual adds after the
// attention and the MLP.
//
// Design.  At decode batch sizes the projections are matrix x skinny-matrix
// products bound by reading the weights, a plain library GEMM; the row-major
// product C[B][N] = X[B][K] W[N][K]^T is handed to the column-major library
// as C^T = W X^T (op(W) = transpose), and the residual adds ride on the
// GEMM's beta = 1, so h is read, summed in float32 and rounded once.  RMSNorm
// is one workgroup per row: 16-byte loads, a float32 sum of squares reduced
// across the workgroup, one rounding per output.
#include "common.h"

#include <rocblas/rocblas.h>

#include <atomic>
#include <mutex>

namespace pkv {

namespace {

constexpr int kNormThreads = 256;

// out[r] = x[r] / sqrt(mean(x[r]^2) + eps) * w, bf16 in and out, float32 math.
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(uint16_t* __restrict__ out,
                                                               const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ w, int dim, float eps) {
  const int r = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (int64_t)r * dim);
  const uint4* w4 = reinterpret_cast<const uint4*>(w);
  uint4* o4 = reinterpret_cast<uint4*>(out + (int64_t)r * dim);
  const int n4 = dim / 8;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n4; i += kNormThreads) {
    const uint4 v = xr[i];
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_lo(u[j]), b = bf16_hi(u[j]);
      ss = __builtin_fmaf(a, a, ss);
      ss = __builtin_fmaf(b, b, ss);
    }
  }
  __shared__ float part[kNormThreads / kWave];
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) ss += shfl_xor(ss, off);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kNormThreads / kWave; ++i) tot += part[i];
  const float inv = 1.0f / sqrtf(tot / (float)dim + eps);
  for (int i = threadIdx.x; i < n4; i += kNormThreads) {
    const uint4 v = xr[i];
    const uint4 g = w4[i];
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
    uint32_t res[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      res[j] = pack_bf16x2(bf16_lo(u[j]) * inv * bf16_lo(gw[j]), bf16_hi(u[j]) * inv * bf16_hi(gw[j]));
    o4[i] = make_uint4(res[0], res[1], res[2], res[3]);
  }
}

// act[r][i] = silu(gu[r][i]) * gu[r][inter + i], eight outputs per thread.
__global__ __launch_bounds__(256) void silu_mul_kernel(uint16_t* __restrict__ act, const uint16_t* __restrict__ gu,
                                                       int rows, int inter) {
  const int n8 = inter / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)rows * n8) return;
  const int r = (int)(gid / n8);
  const int c = (int)(gid % n8);
  const uint4 g = reinterpret_cast<const uint4*>(gu + (int64_t)r * 2 * inter)[c];
  const uint4 u = reinterpret_cast<const uint4*>(gu + (int64_t)r * 2 * inter + inter)[c];
  const uint32_t gg[4] = {g.x, g.y, g.z, g.w}, uu[4] = {u.x, u.y, u.z, u.w};
  uint32_t res[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float g0 = bf16_lo(gg[j]), g1 = bf16_hi(gg[j]);
    const float s0 = g0 / (1.0f + expf(-g0)), s1 = g1 / (1.0f + expf(-g1));
    res[j] = pack_bf16x2(s0 * bf16_lo(uu[j]), s1 * bf16_hi(uu[j]));
  }
  reinterpret_cast<uint4*>(act + (int64_t)r * inter)[c] = make_uint4(res[0], res[1], res[2], res[3]);
}

// One rocBLAS handle per device, created on first use and kept for the
// process (a handle holds the library's per-device state); calls set the
// stream each time.  Calls on one device from several host threads at once
// must be serialised by the caller (the handle is shared).
rocblas_handle blas_handle() {
  constexpr int kMaxDev = 64;
  static std::atomic<rocblas_handle> handles[kMaxDev];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  rocblas_handle h = handles[dev].load(std::memory_order_acquire);
  if (h) return h;
  std::lock_guard<std::mutex> lock(mu);
  h = handles[dev].load(std::memory_order_relaxed);
  if (!h) {
    if (rocblas_create_handle(&h) != rocblas_status_success) return nullptr;
    handles[dev].store(h, std::memory_order_release);
  }
  return h;
}

}  // namespace

// C[rows][n] = beta * C + X[rows][k] W[n][k]^T, bf16 in and out, float32 sums.
int gemm_xwt(uint16_t* c, const uint16_t* x, const uint16_t* w, int rows, int n, int k, float beta, void* stream) {
  rocblas_handle h = blas_handle();
  if (!h) return PKV_ERR_HIP;
  if (rocblas_set_stream(h, static_cast<hipStream_t>(stream)) != rocblas_status_success) return PKV_ERR_HIP;
  const float alpha = 1.0f;
  // column-major view: C^T [n][rows] = op(W^T [k][n]) X^T [k][rows], op = transpose
  const rocblas_status st = rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, n, rows, k,
                                            &alpha, w, rocblas_datatype_bf16_r, k, x, rocblas_datatype_bf16_r, k,
                                            &beta, c, rocblas_datatype_bf16_r, n, c, rocblas_datatype_bf16_r, n,
                                            rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_rmsnorm(pkv_bf16* out, const pkv_bf16* x, const pkv_bf16* weight, int rows, int dim, float eps,
                           void* stream) {
  if (rows < 0 || dim <= 0 || dim % 8 || !(eps >= 0.f)) return PKV_ERR_INVALID_ARG;
  if (rows == 0) return PKV_OK;
  if (!out || !x || !weight) return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(x) || !aligned16(weight)) return PKV_ERR_MISALIGNED;
  uint16_t* o = out;
  const uint16_t* xx = x;
  const uint16_t* ww = weight;
  int d = dim;
  float e = eps;
  void* args[] = {&o, &xx, &ww, &d, &e};
  return launch_status(hipLaunchKernel((const void*)rmsnorm_kernel, dim3(rows), dim3(kNormThreads), args, 0,
                                       (hipStream_t)stream));
}

extern "C" int pkv_silu_mul(pkv_bf16* act, const pkv_bf16* gate_up, int rows, int intermediate, void* stream) {
  if (rows < 0 || intermediate <= 0 || intermediate % 8) return PKV_ERR_INVALID_ARG;
  if (rows == 0) return PKV_OK;
  if (!act || !gate_up) return PKV_ERR_NULL;
  if (!aligned16(act) || !aligned16(gate_up)) return PKV_ERR_MISALIGNED;
  const int64_t total = (int64_t)rows * (intermediate / 8);
  if ((total + 255) / 256 > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  uint16_t* a = act;
  const uint16_t* g = gate_up;
  int r = rows, in = intermediate;
  void* args[] = {&a, &g, &r, &in};
  return launch_status(hipLaunchKernel((const void*)silu_mul_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                                       args, 0, (hipStream_t)stream));
}

extern "C" int pkv_linear(pkv_bf16* out, const pkv_bf16* x, const pkv_bf16* weight, int rows, int out_features,
                          int in_features, int accumulate, void* stream) {
  if (rows < 0 || out_features <= 0 || in_features <= 0) return PKV_ERR_INVALID_ARG;
  if (rows == 0) return PKV_OK;
  if (!out || !x || !weight) return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(x) || !aligned16(weight)) return PKV_ERR_MISALIGNED;
  return gemm_xwt(out, x, weight, rows, out_features, in_features, accumulate ? 1.0f : 0.0f, stream);
}

extern "C" size_t pkv_decode_layer_scratch_elems(int batch, int hidden, int intermediate, int n_q_heads,
                                                 int n_kv_heads) {
  if (batch <= 0 || hidden <= 0 || intermediate <= 0 || n_q_heads <= 0 || n_kv_heads <= 0) return 0;
  const size_t qd = (size_t)n_q_heads * kHeadDim, kvd = (size_t)n_kv_heads * kHeadDim;
  // a | q | k | v | o | m | gate_up | act, each row-major [batch][width]
  return (size_t)batch * ((size_t)hidden * 2 + qd * 2 + kvd * 2 + (size_t)intermediate * 3);
}

extern "C" int pkv_decode_layer(pkv_bf16* h, const pkv_layer_weights* w, int hidden, int intermediate,
                                pkv_bf16* scratch, size_t scratch_elems, pkv_bf16* k_pool, pkv_bf16* v_pool,
                                int num_blocks, const int32_t* block_table, int64_t bt_row_stride, int num_slots,
                                int max_blocks_per_seq, const int32_t* slot_ids, const int32_t* context_lens,
                                const int32_t* row_lens_host, int batch, int max_context_len, int n_q_heads,
                                int n_kv_heads, const float* cos_sin, int max_pos, float scale, float eps,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0 || hidden <= 0 || intermediate <= 0 || n_q_heads <= 0 || n_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
  if (batch == 0) return PKV_OK;
  if (!h || !w || !scratch || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo || !w->mlp_norm ||
      !w->w_gate_up || !w->w_down)
    return PKV_ERR_NULL;
  if (hidden % 8 || intermediate % 8) return PKV_ERR_INVALID_ARG;
  if (scratch_elems < pkv_decode_layer_scratch_elems(batch, hidden, intermediate, n_q_heads, n_kv_heads))
    return PKV_ERR_CAPACITY;
  if (!aligned16(h) || !aligned16(scratch)) return PKV_ERR_MISALIGNED;
  const int qd = n_q_heads * kHeadDim, kvd = n_kv_heads * kHeadDim;
  pkv_bf16* a = scratch;
  pkv_bf16* q = a + (size_t)batch * hidden;
  pkv_bf16* k = q + (size_t)batch * qd;
  pkv_bf16* v = k + (size_t)batch * kvd;
  pkv_bf16* o = v + (size_t)batch * kvd;
  pkv_bf16* m = o + (size_t)batch * qd;
  pkv_bf16* gu = m + (size_t)batch * hidden;
  pkv_bf16* act = gu + (size_t)batch * 2 * intermediate;
  int rc;
  if ((rc = pkv_rmsnorm(a, h, w->attn_norm, batch, hidden, eps, stream)) != PKV_OK) return rc;
  if ((rc = pkv_linear(q, a, w->wq, batch, qd, hidden, 0, stream)) != PKV_OK) return rc;
  if ((rc = pkv_linear(k, a, w->wk, batch, kvd, hidden, 0, stream)) != PKV_OK) return rc;
  if ((rc = pkv_linear(v, a, w->wv, batch, kvd, hidden, 0, stream)) != PKV_OK) return rc;
  if ((rc = pkv_paged_decode_fused(o, q, k, v, k_pool, v_pool, num_blocks, block_table, bt_row_stride, num_slots,
                                   max_blocks_per_seq, slot_ids, context_lens, row_lens_host, batch, max_context_len,
                                   n_q_heads, n_kv_heads, kHeadDim, cos_sin, max_pos, scale, 0, workspace,
                                   workspace_bytes, stream)) != PKV_OK)
    return rc;
  if ((rc = pkv_linear(h, o, w->wo, batch, hidden, qd, 1, stream)) != PKV_OK) return rc;
  if ((rc = pkv_rmsnorm(m, h, w->mlp_norm, batch, hidden, eps, stream)) != PKV_OK) return rc;
  if ((rc = pkv_linear(gu, m, w->w_gate_up, batch, 2 * intermediate, hidden, 0, stream)) != PKV_OK) return rc;
  if ((rc = pkv_silu_mul(act, gu, batch, intermediate, stream)) != PKV_OK) return rc;
  return pkv_linear(h, act, w->w_down, batch, hidden, intermediate, 1, stream);
}

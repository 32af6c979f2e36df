// The rest of a Llama decode layer around the paged attention, for gfx950:
// RMSNorm and the gated-SiLU product as HIP kernels, the projections as bf16
// products with float32 sums on the library's own MFMA kernel, and
// pkv_decode_layer, which runs one layer's decode step.
//
// Source: "An Inference Engine in 1,500 Lines of CUDA: The Map" -- the engine
// runs Llama 3.2 1B (opening paragraph), has its own RMSNorm kernel (Korean
// page, "What is in the box": rmsNormKernel), keeps a 2048-wide hidden state
// (the buf_2048_* buffers of "A function with 51 parameters") and leaves the
// projections to the vendor GEMM (chapter-4 title); here they are this
// library's own kernel.  The formulas are the public Llama ones: rmsnorm(x) =
// x / sqrt(mean(x^2) + eps) * w, the gated MLP (silu(x W_gate^T) *
// (x W_up^T)) W_down^T, residual adds after the attention and the MLP.
//
// Design.  At decode batch sizes (up to 64 rows) the projections are
// matrix x skinny-matrix products bound by reading the weights once: one
// workgroup per 64 output features and all 64 rows, so each weight byte is
// fetched once and the activations (at most 64 x K, resident in L2) once per
// 64 features; each of the workgroup's four waves takes 16 of its features
// along the workgroup's K range, and where 64-wide feature tiles alone would
// leave the chip's 256 CUs idle K is split over workgroups, whose float32
// partials a second kernel sums in a fixed order (no atomics: the result
// does not depend on scheduling).  The layer's query/key/value product runs
// on a narrow-tile kernel instead (16 features per workgroup, K split over
// its four waves and summed in LDS), which reads the activations once per
// 16 features but needs no partials and no second launch.  Larger batches run
// the same kernel once per 64-row block (a second grid dimension; the weights
// are then read once per row block), and a K or feature count that is not a
// multiple of the tiles is masked, so every shape with K and the feature
// count multiples of 8 runs here.  The residual adds are folded in, so h is
// read, summed in float32 and rounded once.  RMSNorm is one workgroup per
// row: 16-byte loads all requested at once, a float32 sum of squares reduced
// across the workgroup, one rounding per output.
#include "common.h"
#include "decode_api.h"

#include <algorithm>
#include <vector>

namespace pkv {

namespace {

constexpr int kNormThreads = 256;

// out[r] = x[r] / sqrt(mean(x[r]^2) + eps) * w, bf16 in and out, float32 math.
// A thread keeps its first kNormKeep groups of eight features (and their
// weights, requested with them) in registers for the second pass; wider
// rows re-read the rest.
constexpr int kNormKeep = 4;

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(uint16_t* __restrict__ out,
                                                               const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ w, int dim, float eps) {
  const int r = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (int64_t)r * dim);
  const uint4* w4 = reinterpret_cast<const uint4*>(w);
  uint4* o4 = reinterpret_cast<uint4*>(out + (int64_t)r * dim);
  const int n4 = dim / 8;
  float ss = 0.f;
  auto square_sum = [&](uint4 v) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_lo(u[j]), b = bf16_hi(u[j]);
      ss = __builtin_fmaf(a, a, ss);
      ss = __builtin_fmaf(b, b, ss);
    }
  };
  uint4 keep[kNormKeep], wkeep[kNormKeep];
#pragma unroll
  for (int gi = 0; gi < kNormKeep; ++gi) {
    const int i = threadIdx.x + gi * kNormThreads;
    if (i < n4) {
      keep[gi] = xr[i];
      wkeep[gi] = w4[i];
    }
  }
#pragma unroll
  for (int gi = 0; gi < kNormKeep; ++gi)
    if (threadIdx.x + gi * kNormThreads < n4) square_sum(keep[gi]);
  for (int i = threadIdx.x + kNormKeep * kNormThreads; i < n4; i += kNormThreads) square_sum(xr[i]);
  __shared__ float part[kNormThreads / kWave];
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) ss += shfl_xor(ss, off);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kNormThreads / kWave; ++i) tot += part[i];
  const float inv = 1.0f / sqrtf(tot / (float)dim + eps);
  auto write = [&](int i, uint4 v, uint4 g) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
    uint32_t res[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      res[j] = pack_bf16x2(bf16_lo(u[j]) * inv * bf16_lo(gw[j]), bf16_hi(u[j]) * inv * bf16_hi(gw[j]));
    o4[i] = make_uint4(res[0], res[1], res[2], res[3]);
  };
#pragma unroll
  for (int gi = 0; gi < kNormKeep; ++gi) {
    const int i = threadIdx.x + gi * kNormThreads;
    if (i < n4) write(i, keep[gi], wkeep[gi]);
  }
  for (int i = threadIdx.x + kNormKeep * kNormThreads; i < n4; i += kNormThreads) write(i, xr[i], w4[i]);
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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDbWaves = 4;     // waves per workgroup, each 16 of its 64 features
constexpr int kDbN = 64;        // output features per workgroup (four MFMA row blocks)
constexpr int kDbRows = 64;     // decode rows (four MFMA column blocks)
constexpr int kDbStage = 32;    // K per MFMA step
constexpr int kDbSteps = 4;     // MFMA steps per X slice
constexpr int kDbSlice = kDbStage * kDbSteps;   // K per X slice in LDS
constexpr int kXsRow = kDbSlice + 8;            // LDS row pitch (elements): 16 B of padding spreads the rows over the banks
constexpr int kMaxSeg = 3;

// One product of a launch: C[rows][n] (+)= X[rows][k] W[n][k]^T.  Several
// products sharing X and k (the query, key and value projections) go in one
// launch, their 64-feature tiles numbered one after the other.
struct GemmSeg {
  const uint16_t* w;
  uint16_t* c;
  float* part;        // [splits][rows][n] float32 partials when K is split
  int n;              // output features, a multiple of 8
  int tile_begin;     // first tile of this product
  int tile_end;       // one past its last tile
};

struct DecodeGemmArgs {
  GemmSeg seg[kMaxSeg];
  const uint16_t* x;
  int nseg, rows, k, kchunk, splits, accumulate;
  int inter;          // gated mode: W = [gate; up] of 2 inter rows, C = silu(gate) * up [rows][inter]
};

// Decode-batch projection, one workgroup per (64 features, K range, 64-row
// block), each of its four waves one block of 16 features over the whole
// range: C^T[16 n][64 b] as four 16 x 16 tiles of v_mfma_f32_16x16x32_bf16
// (A = the wave's 16 W rows, B = 16 rows of X; 8 k per lane from group
// lane / 16, 16-byte loads; a lane keeps C^T rows 4 (lane / 16) .. + 3 of
// column lane % 16 of each tile).  Each wave streams its 16 rows along K, so
// the workgroup's loads in flight stay within a few DRAM pages per row (a
// wave per K slice over all 64 rows instead keeps every page of the matrix
// open at once and streams at half the rate).  X goes through LDS in slices
// of 128 k (64 rows x 256 B, double-buffered, one barrier per slice), loaded
// once per workgroup; W and X of the next two slices are in flight while the
// current one is multiplied.  Elements past the K range (a K that is not a
// multiple of 128) load as zeros; features past n load the last feature row
// and are not stored.  One K range: the sums (plus C when accumulating) are
// rounded to bf16 into C; several: they go as float32 to the product's
// partials for decode_reduce_kernel.  Gated mode (kGlu): tile t takes gate
// rows 32 t .. + 31 (waves 0, 1) and the matching up rows (waves 2, 3), which
// hand their sums over through LDS; the gate waves write
// silu(bf16(gate)) * bf16(up) for features 32 t .. + 31.
template <bool kGlu>
__global__ __launch_bounds__(kDbWaves * kWave) void decode_gemm_kernel(DecodeGemmArgs args) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // workgroup id = tile x splits + split: ids go to the 8 XCDs in turn, so
  // with 8 splits each XCD (its own L2) takes one K range and fetches only
  // that eighth of X; numbered tile-first, every XCD would fetch all of X
  const int t = blockIdx.x / args.splits;
  const int split = blockIdx.x % args.splits;
  const int row0 = blockIdx.y * kDbRows;
  int si = 0;
  while (si + 1 < args.nseg && t >= args.seg[si].tile_end) ++si;
  const uint16_t* __restrict__ w = args.seg[si].w;
  const int n = args.seg[si].n;
  const int n0 = (t - args.seg[si].tile_begin) * kDbN;
  const int k = args.k;
  const int rows = min(kDbRows, args.rows - row0);  // rows of this block
  const int kbeg = split * args.kchunk;
  const int kc = min(args.kchunk, k - kbeg);        // K range of this workgroup (a multiple of 8)
  const int nfull = kc / kDbSlice;                  // whole 128-wide slices
  const int r16 = lane & 15;
  const int kg = 8 * (lane >> 4);
  int wr = kGlu ? (wv < 2 ? 0 : args.inter) + 32 * t + 16 * (wv & 1) + r16 : n0 + 16 * wv + r16;
  if (!kGlu) wr = min(wr, n - 1);
  const uint16_t* wrow = w + (int64_t)wr * k + kbeg + kg;
  // X slice loads: thread i brings row i / 4's quarter i % 4 of the slice
  // (rows past the block read its first row and store zeros)
  constexpr int kXq = kDbSlice / 4 / 8;           // 16-byte loads per thread and slice
  const int xr = threadIdx.x >> 2, xq = threadIdx.x & 3;
  const bool xok = xr < rows;
  const uint16_t* xsrc = args.x + (int64_t)(row0 + (xok ? xr : 0)) * k + kbeg + (kDbSlice / 4) * xq;
  __shared__ uint16_t xs[2][kDbRows * kXsRow];
  uint16_t* xdst = &xs[0][xr * kXsRow + (kDbSlice / 4) * xq];

  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mul = [&](int buf, const uint4 (&wu)[kDbSteps]) {
    const uint16_t* xb = &xs[buf][r16 * kXsRow + kg];
#pragma unroll
    for (int u = 0; u < kDbSteps; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 bv = *reinterpret_cast<const uint4*>(xb + 16 * j * kXsRow + kDbStage * u);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wu[u]),
                                                         __builtin_bit_cast(bf16x8, bv), acc[j], 0, 0, 0);
      }
  };
  if (nfull > 0) {
    // slices it + 1 and it + 2 are in flight while slice it is multiplied:
    // three register sets for W and X, used in turn (the loop is unrolled by
    // three so every set is named statically); loads past the last whole
    // slice load that one again (in bounds, its lines in L2)
    auto load = [&](int it, uint4 (&wd)[kDbSteps], uint4 (&xd)[kXq]) {
      const int off = (it < nfull ? it : nfull - 1) * kDbSlice;
#pragma unroll
      for (int u = 0; u < kDbSteps; ++u) wd[u] = *reinterpret_cast<const uint4*>(wrow + off + kDbStage * u);
#pragma unroll
      for (int q = 0; q < kXq; ++q) xd[q] = *reinterpret_cast<const uint4*>(xsrc + off + 8 * q);
    };
    auto slice = [&](int it, uint4 (&wu)[kDbSteps], uint4 (&xu)[kXq], uint4 (&wl)[kDbSteps], uint4 (&xl)[kXq]) {
      const int buf = it & 1;
      uint4* xd = reinterpret_cast<uint4*>(xdst + buf * kDbRows * kXsRow);
#pragma unroll
      for (int q = 0; q < kXq; ++q) xd[q] = xok ? xu[q] : make_uint4(0u, 0u, 0u, 0u);
      __syncthreads();
      load(it + 2, wl, xl);
      mul(buf, wu);
    };
    uint4 w0[kDbSteps], w1[kDbSteps], w2[kDbSteps], x0[kXq], x1[kXq], x2[kXq];
    load(0, w0, x0);
    load(1, w1, x1);
    for (int it = 0;; it += 3) {
      slice(it, w0, x0, w2, x2);
      if (it + 1 >= nfull) break;
      slice(it + 1, w1, x1, w0, x0);
      if (it + 2 >= nfull) break;
      slice(it + 2, w2, x2, w1, x1);
      if (it + 3 >= nfull) break;
    }
  }
  if (kc > nfull * kDbSlice) {
    // a short last slice (K not a multiple of 128): elements past the K range
    // read as zeros through buffer descriptors over the whole matrices
    // (under 2^31 bytes, checked on the host): an offset past the
    // descriptor's range reads zeros without touching memory
    constexpr uint32_t kOut = 0x80000000u;
    const int off = nfull * kDbSlice;
    const int w_rows = kGlu ? 2 * args.inter : n;
    const auto wres = buf_rsrc(w, (uint32_t)((int64_t)w_rows * k * 2));
    const auto xres = buf_rsrc(args.x, (uint32_t)((int64_t)args.rows * k * 2));
    const uint32_t woff = (uint32_t)(((int64_t)wr * k + kbeg + off + kg) * 2);
    const uint32_t xoff = (uint32_t)(((int64_t)(row0 + (xok ? xr : 0)) * k + kbeg + off + (kDbSlice / 4) * xq) * 2);
    uint4 wt[kDbSteps], xt[kXq];
#pragma unroll
    for (int u = 0; u < kDbSteps; ++u)
      wt[u] = buf_load16(wres, off + kDbStage * u + kg < kc ? woff + 2u * (kDbStage * u) : kOut);
#pragma unroll
    for (int q = 0; q < kXq; ++q)
      xt[q] = buf_load16(xres, xok && off + (kDbSlice / 4) * xq + 8 * q < kc ? xoff + 16u * q : kOut);
    const int buf = nfull & 1;
    uint4* xd = reinterpret_cast<uint4*>(xdst + buf * kDbRows * kXsRow);
#pragma unroll
    for (int q = 0; q < kXq; ++q) xd[q] = xt[q];
    __syncthreads();
    mul(buf, wt);
  }
  if (kGlu) {   // up waves (2, 3) hand their tiles to gate waves (0, 1)
    __shared__ f32x4 up[2][4][kWave];
    if (wv >= 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) up[wv - 2][j][lane] = acc[j];
    }
    __syncthreads();
    if (wv >= 2) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = 16 * j + r16;
      if (b >= rows) continue;
      const f32x4 u4 = up[wv][j][lane];
      uint32_t o[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float r[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const float g = bf16_lo(pack_bf16x2(acc[j][2 * e + f], 0.f));
          const float u = bf16_lo(pack_bf16x2(u4[2 * e + f], 0.f));
          r[f] = g / (1.0f + expf(-g)) * u;
        }
        o[e] = pack_bf16x2(r[0], r[1]);
      }
      const int f0 = 32 * t + 16 * wv + 4 * (lane >> 4);
      *reinterpret_cast<uint2*>(args.seg[0].c + (int64_t)(row0 + b) * args.inter + f0) = make_uint2(o[0], o[1]);
    }
    return;
  }
  const int nn = n0 + 16 * wv + 4 * (lane >> 4);    // C^T rows nn .. nn + 3 of column b
  if (nn >= n) return;                              // n % 8 == 0: the four columns are in or out together
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = 16 * j + r16;
    if (b >= rows) continue;
    const int64_t gb = row0 + b;
    if (args.splits == 1) {
      uint16_t* crow = args.seg[si].c + gb * n + nn;
      float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
      if (args.accumulate) {
        const uint2 old = *reinterpret_cast<const uint2*>(crow);
        v[0] += bf16_lo(old.x);
        v[1] += bf16_hi(old.x);
        v[2] += bf16_lo(old.y);
        v[3] += bf16_hi(old.y);
      }
      *reinterpret_cast<uint2*>(crow) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    } else {
      *reinterpret_cast<f32x4*>(args.seg[si].part + ((int64_t)split * args.rows + gb) * n + nn) = acc[j];
    }
  }
}

// Narrow-tile variant for products whose feature tiles alone cannot fill the
// chip (the query, key and value projections): one 4-wave workgroup per 16
// output features and 64-row block, the waves taking the four quarters of
// the K slices and their sums added in LDS at the end (quarter 0 + 1 + 2 +
// 3, a fixed order), so no float32 partials leave the workgroup and no
// reduction launch follows.  Each wave streams its 16 W rows (the A operand,
// as in decode_gemm_kernel) and brings its own X slices (64 rows x 128 k)
// through a private LDS tile: 16-byte loads covering four whole rows per
// wave instruction, written to LDS and read back in the B-operand layout.
// X is thus read once per workgroup, four times the weight bytes of a
// 16-feature tile, from L2.  Loads past the K range, the rows or a quarter's
// slices read zeros through the buffer descriptors (an offset with its top
// bit set lies past every range); features past n load the last feature
// row and are not stored.  W and X of the next two slices are in flight
// while one is multiplied.
constexpr int kNwWaves = 4;
constexpr int kNwN = 16;                       // output features per workgroup
constexpr int kNwXq = kDbRows * kDbSlice / 8 / kWave;   // 16-byte X loads per lane and slice (16)
constexpr int kNarrowMaxK = 4096;              // X of a 64-row block at most 512 KB per workgroup

struct NarrowArgs {
  GemmSeg seg[kMaxSeg];         // tile ranges in 16-feature tiles; part unused
  const uint16_t* x;
  int nseg, rows, k, kq;        // kq: 128-wide slices per wave (K quarter)
  int accumulate;
};

__global__ __launch_bounds__(kNwWaves * kWave) void decode_gemm_narrow_kernel(NarrowArgs args) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t = blockIdx.x;
  const int row0 = blockIdx.y * kDbRows;
  int si = 0;
  while (si + 1 < args.nseg && t >= args.seg[si].tile_end) ++si;
  const uint16_t* __restrict__ w = args.seg[si].w;
  const int n = args.seg[si].n;
  const int n0 = (t - args.seg[si].tile_begin) * kNwN;
  const int k = args.k;
  const int rows = min(kDbRows, args.rows - row0);
  const int nsl = (k + kDbSlice - 1) / kDbSlice;
  const int first = wv * args.kq;                       // this wave's first slice
  const int mine = max(0, min(args.kq, nsl - first));   // and how many it has
  const int r16 = lane & 15;
  const int kg = 8 * (lane >> 4);
  const int wr = min(n0 + r16, n - 1);
  const auto wres = buf_rsrc(w, (uint32_t)((int64_t)n * k * 2));
  const auto xres = buf_rsrc(args.x, (uint32_t)((int64_t)args.rows * k * 2));
  constexpr uint32_t kOut = 0x80000000u;
  const uint32_t wbase = (uint32_t)(((int64_t)wr * k + kg) * 2);
  // X load q of this lane: row 4 q + lane / 16 of the block, 16-byte piece lane % 16
  const int xch = lane & 15;
  const int xr0 = lane >> 4;
  const uint32_t xbase = (uint32_t)(((int64_t)(row0 + xr0) * k + 8 * xch) * 2);
  const uint32_t xrow4 = (uint32_t)(4 * k * 2);          // four rows, in bytes
  __shared__ uint16_t xs[kNwWaves][kDbRows * kXsRow];    // one private tile per wave
  uint16_t* xw = &xs[wv][xr0 * kXsRow + 8 * xch];        // + q x 4 rows

  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto load_w = [&](int it, uint4 (&wd)[kDbSteps]) {
    const int off = (first + it) * kDbSlice;
    const uint32_t dead = it < mine ? 0u : kOut;
#pragma unroll
    for (int u = 0; u < kDbSteps; ++u)
      wd[u] = buf_load16(wres, (wbase + 2u * (off + kDbStage * u)) | dead |
                                   (off + kDbStage * u + kg < k ? 0u : kOut));
  };
  auto load_x = [&](int it, uint4 (&xd)[kNwXq]) {
    const int off = (first + it) * kDbSlice;
    const uint32_t dead = (it < mine ? 0u : kOut) | (off + 8 * xch < k ? 0u : kOut);
#pragma unroll
    for (int q = 0; q < kNwXq; ++q)
      xd[q] = buf_load16(xres, (xbase + (uint32_t)q * xrow4 + 2u * off) | dead | (4 * q + xr0 < rows ? 0u : kOut));
  };
  // slice it: its X (in xr) goes to the wave's LDS tile, then slice it + 2's
  // X is requested into the same registers; after the products with its W
  // (in wr_), slice it + 2's W is requested into those: two register sets
  // each, used in turn
  auto slice = [&](int it, uint4 (&wr_)[kDbSteps], uint4 (&xr)[kNwXq]) {
    // the tile is this wave's alone: its earlier reads are done (wave-ordered
    // LDS), so the wave overwrites it and reads it back without a barrier
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < kNwXq; ++q) *reinterpret_cast<uint4*>(xw + q * 4 * kXsRow) = xr[q];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    load_x(it + 2, xr);
    const uint16_t* xb = &xs[wv][r16 * kXsRow + kg];
#pragma unroll
    for (int u = 0; u < kDbSteps; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 bv = *reinterpret_cast<const uint4*>(xb + 16 * j * kXsRow + kDbStage * u);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wr_[u]),
                                                         __builtin_bit_cast(bf16x8, bv), acc[j], 0, 0, 0);
      }
    load_w(it + 2, wr_);
  };
  if (mine > 0) {
    uint4 w0[kDbSteps], w1[kDbSteps], x0[kNwXq], x1[kNwXq];
    load_w(0, w0);
    load_x(0, x0);
    load_w(1, w1);
    load_x(1, x1);
    for (int it = 0;; it += 2) {
      slice(it, w0, x0);
      if (it + 1 >= mine) break;
      slice(it + 1, w1, x1);
      if (it + 2 >= mine) break;
    }
  }
  __shared__ f32x4 hand[kNwWaves - 1][4][kWave];
  if (wv > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) hand[wv - 1][j][lane] = acc[j];
  }
  __syncthreads();
  if (wv > 0) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = ((acc[j] + hand[0][j][lane]) + hand[1][j][lane]) + hand[2][j][lane];
  const int nn = n0 + 4 * (lane >> 4);      // C^T rows nn .. nn + 3 of column b
  if (nn >= n) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = 16 * j + r16;
    if (b >= rows) continue;
    uint16_t* crow = args.seg[si].c + (int64_t)(row0 + b) * n + nn;
    float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
    if (args.accumulate) {
      const uint2 old = *reinterpret_cast<const uint2*>(crow);
      v[0] += bf16_lo(old.x);
      v[1] += bf16_hi(old.x);
      v[2] += bf16_lo(old.y);
      v[3] += bf16_hi(old.y);
    }
    *reinterpret_cast<uint2*>(crow) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
}

struct ReduceSeg {
  uint16_t* c;
  const float* part;
  int n;
  int end;            // one past the last eight-column group of this product, over all products' groups
};

struct ReduceArgs {
  ReduceSeg seg[kMaxSeg];
  int nseg, rows, splits, accumulate;
};

// C[b][8 g .. + 7] = bf16(sum over splits of part[s][b][..] (+ C)), in split
// order; one thread per (row, eight columns), products one after the other.
__global__ __launch_bounds__(256) void decode_reduce_kernel(ReduceArgs args) {
  int gid = blockIdx.x * blockDim.x + threadIdx.x;
  int si = 0;
  while (si + 1 < args.nseg && gid >= args.seg[si].end) ++si;
  if (gid >= args.seg[si].end) return;
  if (si) gid -= args.seg[si - 1].end;
  const int n = args.seg[si].n;
  const int64_t e = (int64_t)gid * 8;           // row gid / (n / 8), columns 8 (gid % (n / 8)) .. + 7
  const int64_t plane = (int64_t)args.rows * n;
  const float* p = args.seg[si].part + e;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = 0; s < args.splits; ++s) {
    const float4 a = reinterpret_cast<const float4*>(p + s * plane)[0];
    const float4 c = reinterpret_cast<const float4*>(p + s * plane)[1];
    v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
    v[4] += c.x; v[5] += c.y; v[6] += c.z; v[7] += c.w;
  }
  uint4* out = reinterpret_cast<uint4*>(args.seg[si].c + e);
  if (args.accumulate) {
    const uint4 old = *out;
    const uint32_t o[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] += bf16_lo(o[q]);
      v[2 * q + 1] += bf16_hi(o[q]);
    }
  }
  *out = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7]));
}

// The attention output projection's finish, one workgroup per row:
// h[b] = bf16(h[b] + sum over splits of part[s][b]) and, from that rounded
// h, m[b] = rmsnorm(h[b]) * w (as rmsnorm_kernel).  A thread's eight
// features at a time: the partials of up to eight splits, h and the norm
// weights are all requested before the first sum (one round trip to memory
// for a row of up to 8 x 256 x 8 features at 8 splits), and the rounded h
// stays in registers for the second pass (up to kRrnKeep groups per thread;
// wider rows re-read what the thread wrote).
constexpr int kRrnKeep = 4;

__global__ __launch_bounds__(kNormThreads) void reduce_residual_norm_kernel(uint16_t* __restrict__ h,
                                                                           uint16_t* __restrict__ m,
                                                                           const float* __restrict__ part,
                                                                           const uint16_t* __restrict__ nw, int rows,
                                                                           int dim, int splits, float eps) {
  const int r = blockIdx.x;
  const int n8 = dim / 8;
  const int64_t plane = (int64_t)rows * dim;
  uint4* hr = reinterpret_cast<uint4*>(h + (int64_t)r * dim);
  const uint4* w4 = reinterpret_cast<const uint4*>(nw);
  float ss = 0.f;
  // h's eight features at group g, summed, rounded, written and returned
  auto finish_h = [&](int g) {
    const float* p = part + (int64_t)r * dim + 8 * g;
    const uint4 old = hr[g];
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < splits; s0 += 8) {
      float4 pa[8], pc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (s0 + i < splits) {
          pa[i] = reinterpret_cast<const float4*>(p + (s0 + i) * plane)[0];
          pc[i] = reinterpret_cast<const float4*>(p + (s0 + i) * plane)[1];
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (s0 + i < splits) {
          v[0] += pa[i].x; v[1] += pa[i].y; v[2] += pa[i].z; v[3] += pa[i].w;
          v[4] += pc[i].x; v[5] += pc[i].y; v[6] += pc[i].z; v[7] += pc[i].w;
        }
      }
    }
    const uint32_t o[4] = {old.x, old.y, old.z, old.w};
    uint32_t res[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      res[q] = pack_bf16x2(v[2 * q] + bf16_lo(o[q]), v[2 * q + 1] + bf16_hi(o[q]));
      const float x0 = bf16_lo(res[q]), x1 = bf16_hi(res[q]);
      ss = __builtin_fmaf(x0, x0, ss);
      ss = __builtin_fmaf(x1, x1, ss);
    }
    const uint4 hv = make_uint4(res[0], res[1], res[2], res[3]);
    hr[g] = hv;
    return hv;
  };
  uint4 keep[kRrnKeep], wkeep[kRrnKeep];
#pragma unroll
  for (int gi = 0; gi < kRrnKeep; ++gi) {
    const int g = threadIdx.x + gi * kNormThreads;
    if (g < n8) {
      wkeep[gi] = w4[g];
      keep[gi] = finish_h(g);
    }
  }
  for (int g = threadIdx.x + kRrnKeep * kNormThreads; g < n8; g += kNormThreads) finish_h(g);
  __shared__ float sh[kNormThreads / kWave];
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) ss += shfl_xor(ss, off);
  if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kNormThreads / kWave; ++i) tot += sh[i];
  const float inv = 1.0f / sqrtf(tot / (float)dim + eps);
  uint4* mr = reinterpret_cast<uint4*>(m + (int64_t)r * dim);
  auto write_m = [&](int g, uint4 v, uint4 gw) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    const uint32_t ww[4] = {gw.x, gw.y, gw.z, gw.w};
    uint32_t res[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      res[q] = pack_bf16x2(bf16_lo(u[q]) * inv * bf16_lo(ww[q]), bf16_hi(u[q]) * inv * bf16_hi(ww[q]));
    mr[g] = make_uint4(res[0], res[1], res[2], res[3]);
  };
#pragma unroll
  for (int gi = 0; gi < kRrnKeep; ++gi) {
    const int g = threadIdx.x + gi * kNormThreads;
    if (g < n8) write_m(g, keep[gi], wkeep[gi]);
  }
  // past the kept groups: each thread re-reads what it wrote
  for (int g = threadIdx.x + kRrnKeep * kNormThreads; g < n8; g += kNormThreads) write_m(g, hr[g], w4[g]);
}

// K splits for a launch of `tiles` 64-feature tiles over `rows` rows: the
// most (a power of two) that keep the workgroups within one round of the
// chip's 256 CUs, each taking whole 128-wide X slices (only the last K range
// may be shorter); 0 if the shape does not fit the kernel (K or rows not
// positive, K not a multiple of 8).  (A second, partial round of workgroups
// costs more than the parallelism it adds: 48 tiles x 8 splits ran 30%
// slower than x 4.)
int decode_gemm_splits(int rows, int tiles, int k) {
  if (rows <= 0 || tiles <= 0 || k <= 0 || k % 8) return 0;
  const int64_t blocks = (int64_t)tiles * ((rows + kDbRows - 1) / kDbRows);
  int s = 1;
  while (blocks * s * 2 <= 256 && k >= kDbSlice * s * 2) s *= 2;
  return s;
}

// K per split for `splits` splits: whole slices, the last range shorter.
int decode_gemm_kchunk(int k, int splits) {
  const int per = (k + splits - 1) / splits;
  return (per + kDbSlice - 1) / kDbSlice * kDbSlice;
}

}  // namespace

size_t decode_gemm_workspace_bytes(int rows, int n, int k) {
  if (n <= 0 || n % 8) return 0;
  int s = decode_gemm_splits(rows, (n + kDbN - 1) / kDbN, k);
  if (s > 1) s = (k + decode_gemm_kchunk(k, s) - 1) / decode_gemm_kchunk(k, s);
  return s > 1 ? (size_t)s * rows * n * sizeof(float) : 0;
}

// Products sharing X [rows][k] (1 to kMaxSeg of them: w[i] [n[i]][k] into
// c[i] [rows][n[i]]) on the projection kernel, K-split partials in `part`
// (part_bytes) when the split pays and they fit (else one K range).
// PKV_ERR_UNSUPPORTED (nothing launched) when the shape does not fit the
// kernel (a feature count or K that is not a multiple of 8).  With reduce ==
// false and K split the partials are left for the caller (the number of
// splits goes to *splits_out when not null).
int decode_gemm(int nseg, uint16_t* const* c, const uint16_t* const* w, const int* n, const uint16_t* x, int rows,
                int k, bool accumulate, void* part, size_t part_bytes, hipStream_t stream, bool reduce = true,
                int* splits_out = nullptr) {
  if (nseg < 1 || nseg > kMaxSeg) return PKV_ERR_INVALID_ARG;
  int tiles = 0;
  int64_t ntot = 0;
  for (int i = 0; i < nseg; ++i) {
    if (n[i] <= 0 || n[i] % 8 || n[i] > (1 << 24)) return PKV_ERR_UNSUPPORTED;
    tiles += (n[i] + kDbN - 1) / kDbN;
    ntot += n[i];
  }
  int splits = decode_gemm_splits(rows, tiles, k);
  if (splits == 0) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)rows * k * 2 > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;     // 31-bit buffer offsets
  for (int i = 0; i < nseg; ++i)
    if ((int64_t)n[i] * k * 2 > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
  const int64_t row_blocks = (rows + kDbRows - 1) / kDbRows;
  if (row_blocks > 65535 || (int64_t)rows * ntot / 8 > 0x7fffff00) return PKV_ERR_INVALID_ARG;
  int kchunk = decode_gemm_kchunk(k, splits);
  splits = (k + kchunk - 1) / kchunk;
  if (splits > 1 && (!part || part_bytes < (size_t)splits * rows * ntot * sizeof(float))) {
    splits = 1;                         // no room for partials: one K range
    kchunk = k;
  }
  if (splits_out) *splits_out = splits;
  DecodeGemmArgs a{};
  ReduceArgs ra{};
  int t0 = 0;
  size_t poff = 0;
  int64_t gend = 0;
  for (int i = 0; i < nseg; ++i) {
    float* pp = splits > 1 ? static_cast<float*>(part) + poff : nullptr;
    const int nt = (n[i] + kDbN - 1) / kDbN;
    a.seg[i] = GemmSeg{w[i], c[i], pp, n[i], t0, t0 + nt};
    t0 += nt;
    poff += (size_t)splits * rows * n[i];
    gend += (int64_t)rows * (n[i] / 8);
    ra.seg[i] = ReduceSeg{c[i], pp, n[i], (int)gend};
  }
  a.x = x;
  a.nseg = nseg;
  a.rows = rows;
  a.k = k;
  a.kchunk = kchunk;
  a.splits = splits;
  a.accumulate = accumulate ? 1 : 0;
  void* args[] = {&a};
  int rc = launch_status(hipLaunchKernel((const void*)decode_gemm_kernel<false>,
                                         dim3(tiles * splits, (unsigned)row_blocks), dim3(kDbWaves * kWave), args, 0,
                                         stream));
  if (rc != PKV_OK || splits == 1 || !reduce) return rc;
  ra.nseg = nseg;
  ra.rows = rows;
  ra.splits = splits;
  ra.accumulate = a.accumulate;
  void* rargs[] = {&ra};
  return launch_status(hipLaunchKernel((const void*)decode_reduce_kernel, dim3((unsigned)((gend + 255) / 256)),
                                       dim3(256), rargs, 0, stream));
}

// act[rows][inter] = silu(bf16(X Wg^T)) * bf16(X Wu^T) for W = [Wg; Wu]
// [2 inter][k], on the projection kernel in gated mode (K never split).
// PKV_ERR_UNSUPPORTED (nothing launched) when the shape does not fit
// (inter % 32, K % 8); the caller then runs the product and the SiLU kernel.
int decode_gemm_glu(uint16_t* act, const uint16_t* x, const uint16_t* w, int rows, int inter, int k,
                    hipStream_t stream) {
  if (rows <= 0 || inter <= 0 || inter % 32 || k <= 0 || k % 8) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)rows * k * 2 > 0x7fffffffLL || (int64_t)2 * inter * k * 2 > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
  const int64_t row_blocks = (rows + kDbRows - 1) / kDbRows;
  if (row_blocks > 65535) return PKV_ERR_INVALID_ARG;
  DecodeGemmArgs a{};
  a.seg[0] = GemmSeg{w, act, nullptr, 2 * inter, 0, inter / 32};
  a.x = x;
  a.nseg = 1;
  a.rows = rows;
  a.k = k;
  a.kchunk = k;
  a.splits = 1;
  a.inter = inter;
  void* args[] = {&a};
  return launch_status(hipLaunchKernel((const void*)decode_gemm_kernel<true>, dim3(inter / 32, (unsigned)row_blocks),
                                       dim3(kDbWaves * kWave), args, 0, stream));
}

// Products sharing X [rows][k] (1 to kMaxSeg of them) on the narrow-tile
// kernel: every output is written (rounded once, plus C when accumulating)
// by the launch itself.  PKV_ERR_UNSUPPORTED (nothing launched) when the
// shape does not fit (a feature count or K that is not a multiple of 8).
int decode_gemm_narrow(int nseg, uint16_t* const* c, const uint16_t* const* w, const int* n, const uint16_t* x,
                       int rows, int k, bool accumulate, hipStream_t stream) {
  if (nseg < 1 || nseg > kMaxSeg) return PKV_ERR_INVALID_ARG;
  if (rows <= 0 || k <= 0 || k % 8) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)rows * k * 2 > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;     // 31-bit buffer offsets
  NarrowArgs a{};
  int t0 = 0;
  for (int i = 0; i < nseg; ++i) {
    if (n[i] <= 0 || n[i] % 8 || n[i] > (1 << 24)) return PKV_ERR_UNSUPPORTED;
    if ((int64_t)n[i] * k * 2 > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
    const int nt = (n[i] + kNwN - 1) / kNwN;
    a.seg[i] = GemmSeg{w[i], c[i], nullptr, n[i], t0, t0 + nt};
    t0 += nt;
  }
  const int64_t row_blocks = (rows + kDbRows - 1) / kDbRows;
  if (row_blocks > 65535) return PKV_ERR_INVALID_ARG;
  const int nsl = (k + kDbSlice - 1) / kDbSlice;
  a.x = x;
  a.nseg = nseg;
  a.rows = rows;
  a.k = k;
  a.kq = (nsl + kNwWaves - 1) / kNwWaves;
  a.accumulate = accumulate ? 1 : 0;
  void* args[] = {&a};
  return launch_status(hipLaunchKernel((const void*)decode_gemm_narrow_kernel, dim3(t0, (unsigned)row_blocks),
                                       dim3(kNwWaves * kWave), args, 0, stream));
}

// h = bf16(h + sum of the output projection's partials), m = rmsnorm(h) * w.
int reduce_residual_norm(uint16_t* h, uint16_t* m, const float* part, const uint16_t* w, int rows, int dim,
                         int splits, float eps, hipStream_t stream) {
  void* args[] = {&h, &m, &part, &w, &rows, &dim, &splits, &eps};
  return launch_status(hipLaunchKernel((const void*)reduce_residual_norm_kernel, dim3(rows), dim3(kNormThreads),
                                       args, 0, stream));
}

}  // namespace pkv

using namespace pkv;

namespace pkv {
namespace {

// Diagnostic: the projection kernels' weight reads alone.  Wave i of the grid
// takes 16-row block i / k_parts of w [n][k] over K part i % k_parts, with the
// projection kernels' lane pattern (row lane % 16, 16 bytes at k 8 (lane /
// 16) + 32 u of each 128-wide slice) and two slices in flight; the data are
// XOR-ed into `sink` under a condition they never meet.
__global__ __launch_bounds__(256) void weight_read_probe_kernel(const uint16_t* __restrict__ w, int k, int k_parts,
                                                                int waves, uint32_t* sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= waves) return;
  const int kw = k / k_parts;                  // a multiple of 128 (checked on the host)
  const int ns = kw / kDbSlice;
  const uint16_t* base = w + (int64_t)(16 * (wave / k_parts) + (lane & 15)) * k + (wave % k_parts) * kw +
                         8 * (lane >> 4);
  uint4 b0[kDbSteps], b1[kDbSteps];
  auto load = [&](int sl, uint4 (&d)[kDbSteps]) {
    const int s = sl < ns ? sl : ns - 1;       // past the last slice: the last one again (in bounds, cached)
#pragma unroll
    for (int u = 0; u < kDbSteps; ++u) d[u] = *reinterpret_cast<const uint4*>(base + s * kDbSlice + kDbStage * u);
  };
  uint32_t acc = 0;
  auto eat = [&](const uint4 (&d)[kDbSteps]) {
#pragma unroll
    for (int u = 0; u < kDbSteps; ++u) acc ^= d[u].x ^ d[u].y ^ d[u].z ^ d[u].w;
  };
  load(0, b0);
  load(1, b1);
  for (int sl = 0; sl < ns; sl += 2) {
    eat(b0);
    load(sl + 2, b0);
    if (sl + 1 < ns) eat(b1);
    load(sl + 3, b1);
  }
  if (acc == 0x9e3779b9u) *sink = acc;
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_weight_read_probe(const pkv_bf16* w, int n, int k, int k_parts, uint32_t* sink, void* stream) {
  if (n <= 0 || k <= 0 || (k_parts != 1 && k_parts != 2 && k_parts != 4 && k_parts != 8)) return PKV_ERR_INVALID_ARG;
  if (n % 16 || k % (128 * k_parts)) return PKV_ERR_UNSUPPORTED;
  if (!w || !sink) return PKV_ERR_NULL;
  if (!aligned16(w) || !aligned4(sink)) return PKV_ERR_MISALIGNED;
  if ((int64_t)n / 16 * k_parts > (int64_t)4 * 0x7fffffff) return PKV_ERR_INVALID_ARG;
  const uint16_t* ww = w;
  int kk = k, kp = k_parts;
  int waves = n / 16 * k_parts;
  uint32_t* sk = sink;
  void* args[] = {&ww, &kk, &kp, &waves, &sk};
  return launch_status(hipLaunchKernel((const void*)weight_read_probe_kernel, dim3((unsigned)((waves + 3) / 4)),
                                       dim3(256), args, 0, (hipStream_t)stream));
}

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

namespace {

// pkv_linear's choice: the narrow-tile kernel where the wide one would split
// K over workgroups (its 64-feature tiles alone leave CUs idle) and X is small
// enough to be read once per 16 features; else the wide kernel.
bool linear_narrow(int rows, int n, int k) {
  if (rows <= 0 || n <= 0 || k <= 0 || k % 8 || n % 8 || k > kNarrowMaxK) return false;
  return decode_gemm_splits(rows, (n + kDbN - 1) / kDbN, k) > 1;
}

}  // namespace

extern "C" size_t pkv_linear_workspace_bytes(int rows, int out_features, int in_features) {
  return linear_narrow(rows, out_features, in_features) ? 0
                                                        : decode_gemm_workspace_bytes(rows, out_features, in_features);
}

extern "C" int pkv_linear(pkv_bf16* out, const pkv_bf16* x, const pkv_bf16* weight, int rows, int out_features,
                          int in_features, int accumulate, void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0 || out_features <= 0 || in_features <= 0) return PKV_ERR_INVALID_ARG;
  if (out_features % 8 || in_features % 8) return PKV_ERR_UNSUPPORTED;
  if (rows == 0) return PKV_OK;
  if (!out || !x || !weight) return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(x) || !aligned16(weight) || (workspace && !aligned16(workspace)))
    return PKV_ERR_MISALIGNED;
  uint16_t* cc[1] = {out};
  const uint16_t* ww[1] = {weight};
  const int nn[1] = {out_features};
  if (linear_narrow(rows, out_features, in_features))
    return decode_gemm_narrow(1, cc, ww, nn, x, rows, in_features, accumulate != 0, static_cast<hipStream_t>(stream));
  return decode_gemm(1, cc, ww, nn, x, rows, in_features, accumulate != 0, workspace, workspace_bytes,
                     static_cast<hipStream_t>(stream));
}

namespace {

// bf16 elements of the float32 K-split partials the layer's projections need
// (the largest over its launches), placed after the activations.
size_t layer_partial_elems(int batch, int hidden, int intermediate, int n_q_heads, int n_kv_heads) {
  const int qd = n_q_heads * kHeadDim, kvd = n_kv_heads * kHeadDim;
  const size_t sizes[] = {decode_gemm_workspace_bytes(batch, qd + 2 * kvd, hidden),
                          decode_gemm_workspace_bytes(batch, hidden, qd),
                          decode_gemm_workspace_bytes(batch, 2 * intermediate, hidden),
                          decode_gemm_workspace_bytes(batch, hidden, intermediate)};
  size_t most = 0;
  for (size_t b : sizes) most = std::max(most, b);
  return (most + 15) / 16 * 8;
}

}  // namespace

extern "C" size_t pkv_decode_layer_scratch_elems(int batch, int hidden, int intermediate, int n_q_heads,
                                                 int n_kv_heads) {
  if (batch <= 0 || hidden <= 0 || intermediate <= 0 || n_q_heads <= 0 || n_kv_heads <= 0) return 0;
  const size_t qd = (size_t)n_q_heads * kHeadDim, kvd = (size_t)n_kv_heads * kHeadDim;
  // a | q | k | v | o | m | gate_up | act, each row-major [batch][width], then the projections' partials
  return (size_t)batch * ((size_t)hidden * 2 + qd * 2 + kvd * 2 + (size_t)intermediate * 3) +
         layer_partial_elems(batch, hidden, intermediate, n_q_heads, n_kv_heads);
}

namespace {

// The scratch regions of one layer (see pkv_decode_layer_scratch_elems).
struct LayerScratch {
  pkv_bf16 *a, *q, *k, *v, *o, *m, *gu, *act;
  void* part;
  size_t part_bytes;
};

LayerScratch layer_scratch(pkv_bf16* scratch, int batch, int hidden, int intermediate, int n_q_heads,
                           int n_kv_heads) {
  const size_t qd = (size_t)n_q_heads * kHeadDim, kvd = (size_t)n_kv_heads * kHeadDim;
  LayerScratch s;
  s.a = scratch;
  s.q = s.a + (size_t)batch * hidden;
  s.k = s.q + (size_t)batch * qd;
  s.v = s.k + (size_t)batch * kvd;
  s.o = s.v + (size_t)batch * kvd;
  s.m = s.o + (size_t)batch * qd;
  s.gu = s.m + (size_t)batch * hidden;
  s.act = s.gu + (size_t)batch * 2 * intermediate;
  s.part = s.act + (size_t)batch * intermediate;   // 16-byte aligned: every region is a multiple of 8 elements
  s.part_bytes = 2 * layer_partial_elems(batch, hidden, intermediate, n_q_heads, n_kv_heads);
  return s;
}

// One layer; `att`: its attention call, checked and planned.  `a_ready`: the
// scratch's a already holds rmsnorm(h, attn_norm) (left there by the previous
// layer).  With `next_norm` the layer ends by leaving a = rmsnorm(h,
// next_norm) for the next layer: where the down projection's K is split, its
// partials, the residual add and that norm are one kernel (as the output
// projection's are with the MLP's norm).  Argument checks are the callers'
// (check_layer_args), so every launch here takes a shape its kernel runs.
int decode_layer_impl(pkv_bf16* h, const pkv_layer_weights* w, int hidden, int intermediate, pkv_bf16* scratch,
                      const DecodeLaunch& att, int batch, int n_q_heads, int n_kv_heads, float eps, void* stream,
                      bool a_ready, const pkv_bf16* next_norm) {
  const int qd = n_q_heads * kHeadDim, kvd = n_kv_heads * kHeadDim;
  const LayerScratch S = layer_scratch(scratch, batch, hidden, intermediate, n_q_heads, n_kv_heads);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  int rc;
  if (!a_ready && (rc = pkv_rmsnorm(S.a, h, w->attn_norm, batch, hidden, eps, stream)) != PKV_OK) return rc;
  // q, k and v in one launch: on the narrow-tile kernel (no partials, no
  // reduction launch) while X is small enough to be read once per 16
  // features, else K split over workgroups plus a reduction
  {
    uint16_t* cs[3] = {S.q, S.k, S.v};
    const uint16_t* ws[3] = {w->wq, w->wk, w->wv};
    const int ns[3] = {qd, kvd, kvd};
    rc = hidden <= kNarrowMaxK ? decode_gemm_narrow(3, cs, ws, ns, S.a, batch, hidden, false, st)
                               : decode_gemm(3, cs, ws, ns, S.a, batch, hidden, false, S.part, S.part_bytes, st);
    if (rc != PKV_OK) return rc;
  }
  if ((rc = decode_enqueue(att, st)) != PKV_OK) return rc;
  // h += x W^T, then (norm_w given) y = rmsnorm(h, norm_w): with K split, the
  // partials' sum, the residual add and the norm are one kernel
  auto residual = [&](const uint16_t* x, const uint16_t* wt, int kdim, const pkv_bf16* norm_w, pkv_bf16* y) {
    uint16_t* cs[1] = {h};
    const uint16_t* ws[1] = {wt};
    const int ns[1] = {hidden};
    int splits = 0;
    int r = decode_gemm(1, cs, ws, ns, x, batch, kdim, true, S.part, S.part_bytes, st, norm_w == nullptr, &splits);
    if (r == PKV_OK && splits > 1 && norm_w)
      return reduce_residual_norm(h, y, static_cast<const float*>(S.part), norm_w, batch, hidden, splits, eps, st);
    if (r == PKV_OK && norm_w) r = pkv_rmsnorm(y, h, norm_w, batch, hidden, eps, stream);
    return r;
  };
  if ((rc = residual(S.o, w->wo, qd, w->mlp_norm, S.m)) != PKV_OK) return rc;
  // act = silu(m Wg^T) * (m Wu^T): one gated launch where it fits, else the
  // product into gate_up and the SiLU kernel
  if (intermediate % 32 == 0) {
    rc = decode_gemm_glu(S.act, S.m, w->w_gate_up, batch, intermediate, hidden, st);
  } else {
    uint16_t* cs[1] = {S.gu};
    const uint16_t* ws[1] = {w->w_gate_up};
    const int ns[1] = {2 * intermediate};
    rc = decode_gemm(1, cs, ws, ns, S.m, batch, hidden, false, S.part, S.part_bytes, st);
    if (rc == PKV_OK) rc = pkv_silu_mul(S.act, S.gu, batch, intermediate, stream);
  }
  if (rc != PKV_OK) return rc;
  return residual(S.act, w->w_down, intermediate, next_norm, S.a);
}

// Everything a layer's launches need, checked before any of them: sizes,
// weights, scratch, and the attention call (planned into `att`, with the
// layer's q, k, v and o in the scratch).
int check_layer_args(pkv_bf16* h, const pkv_layer_weights* w, int hidden, int intermediate, pkv_bf16* scratch,
                     size_t scratch_elems, pkv_bf16* k_pool, pkv_bf16* v_pool, int num_blocks,
                     const int32_t* block_table, int64_t bt_row_stride, int num_slots, int max_blocks_per_seq,
                     const int32_t* slot_ids, const int32_t* context_lens, const int32_t* row_lens_host, int batch,
                     int max_context_len, int n_q_heads, int n_kv_heads, const float* cos_sin, int max_pos,
                     float scale, float eps, void* workspace, size_t workspace_bytes, DecodeLaunch* att,
                     StreamPlan* plan_out = nullptr) {
  if (hidden <= 0 || intermediate <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || !(eps >= 0.f))
    return PKV_ERR_INVALID_ARG;
  if (!h || !w || !scratch || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo || !w->mlp_norm ||
      !w->w_gate_up || !w->w_down)
    return PKV_ERR_NULL;
  if (hidden % 8 || intermediate % 8) return PKV_ERR_INVALID_ARG;
  if ((int64_t)batch > (int64_t)65535 * 64) return PKV_ERR_INVALID_ARG;
  if (scratch_elems < pkv_decode_layer_scratch_elems(batch, hidden, intermediate, n_q_heads, n_kv_heads))
    return PKV_ERR_CAPACITY;
  if (!aligned16(h) || !aligned16(scratch)) return PKV_ERR_MISALIGNED;
  const pkv_bf16* ws[] = {w->attn_norm, w->wq, w->wk, w->wv, w->wo, w->mlp_norm, w->w_gate_up, w->w_down};
  for (const pkv_bf16* p : ws)
    if (!aligned16(p)) return PKV_ERR_MISALIGNED;
  const LayerScratch S = layer_scratch(scratch, batch, hidden, intermediate, n_q_heads, n_kv_heads);
  DecodeCall c{};
  c.fused = true;
  c.out = S.o;
  c.q = S.q;
  c.k_new = S.k;
  c.v_new = S.v;
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
  c.head_dim = kHeadDim;
  c.cos_sin = cos_sin;
  c.max_pos = max_pos;
  c.scale = scale;
  c.workspace = workspace;
  c.workspace_bytes = workspace_bytes;
  c.plan_out = plan_out;
  // att null: the weights and sizes only (the caller derives the attention
  // call from another layer's)
  return att ? decode_prepare(c, att) : PKV_OK;
}

}  // namespace

extern "C" int pkv_decode_layer(pkv_bf16* h, const pkv_layer_weights* w, int hidden, int intermediate,
                                pkv_bf16* scratch, size_t scratch_elems, pkv_bf16* k_pool, pkv_bf16* v_pool,
                                int num_blocks, const int32_t* block_table, int64_t bt_row_stride, int num_slots,
                                int max_blocks_per_seq, const int32_t* slot_ids, const int32_t* context_lens,
                                const int32_t* row_lens_host, int batch, int max_context_len, int n_q_heads,
                                int n_kv_heads, const float* cos_sin, int max_pos, float scale, float eps,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0) return PKV_ERR_INVALID_ARG;
  if (batch == 0) return hidden > 0 && intermediate > 0 && n_q_heads > 0 && n_kv_heads > 0 ? PKV_OK
                                                                                          : PKV_ERR_INVALID_ARG;
  thread_local DecodeLaunch att;
  const int rc = check_layer_args(h, w, hidden, intermediate, scratch, scratch_elems, k_pool, v_pool, num_blocks,
                                  block_table, bt_row_stride, num_slots, max_blocks_per_seq, slot_ids, context_lens,
                                  row_lens_host, batch, max_context_len, n_q_heads, n_kv_heads, cos_sin, max_pos, scale,
                                  eps, workspace, workspace_bytes, &att);
  if (rc != PKV_OK) return rc;
  return decode_layer_impl(h, w, hidden, intermediate, scratch, att, batch, n_q_heads, n_kv_heads, eps, stream, false,
                           nullptr);
}

extern "C" int pkv_decode_layers(pkv_bf16* h, const pkv_layer_weights* layers, int n_layers, int hidden,
                                 int intermediate, pkv_bf16* scratch, size_t scratch_elems, pkv_bf16* k_pool,
                                 pkv_bf16* v_pool, int num_blocks, const int32_t* block_table, int64_t bt_row_stride,
                                 int64_t bt_layer_stride, int num_slots, int max_blocks_per_seq,
                                 const int32_t* slot_ids, const int32_t* context_lens, const int32_t* row_lens_host,
                                 int batch, int max_context_len, int n_q_heads, int n_kv_heads, const float* cos_sin,
                                 int max_pos, float scale, float eps, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (n_layers < 0 || batch < 0 || bt_layer_stride < 0) return PKV_ERR_INVALID_ARG;
  if (n_layers == 0 || batch == 0) return PKV_OK;
  if (!layers || !block_table) return PKV_ERR_NULL;
  thread_local std::vector<DecodeLaunch> att;
  att.resize(n_layers);
  // The layers' attention calls share the rows and their lengths, hence the
  // streaming kernel's plan: the first launch stores it in the workspace and
  // the others read it there (small kernel arguments for them and for their
  // merges; a launch that carries the plan in its arguments waits longer to
  // start).
  const size_t plan_off = decode_plan_offset(n_q_heads);
  StreamPlan* plan_ws = n_layers > 1 && workspace && n_q_heads > 0 && workspace_bytes >= plan_off + kStreamPlanBytes
                            ? reinterpret_cast<StreamPlan*>(static_cast<char*>(workspace) + plan_off)
                            : nullptr;
  // Every layer's arguments are checked before the first launch.  The
  // attention calls differ only in the table view, so the first layer's is
  // planned in full and the others are the same call on their own view (the
  // plan is built once: planning every layer before the first launch would
  // keep the GPU waiting).
  for (int l = 0; l < n_layers; ++l) {
    int rc = check_layer_args(h, &layers[l], hidden, intermediate, scratch, scratch_elems, k_pool, v_pool,
                              num_blocks, block_table + bt_layer_stride * l, bt_row_stride, num_slots,
                              max_blocks_per_seq, slot_ids, context_lens, row_lens_host, batch, max_context_len,
                              n_q_heads, n_kv_heads, cos_sin, max_pos, scale, eps, workspace, workspace_bytes,
                              l == 0 ? &att[0] : nullptr, plan_ws);
    if (rc == PKV_OK && l > 0)
      rc = decode_retarget(att[0], block_table + bt_layer_stride * l, plan_ws && att[0].path == 1 ? plan_ws : nullptr,
                           &att[l]);
    if (rc != PKV_OK) return rc;
  }
  for (int l = 0; l < n_layers; ++l) {
    const int rc = decode_layer_impl(h, &layers[l], hidden, intermediate, scratch, att[l], batch, n_q_heads,
                                     n_kv_heads, eps, stream, l > 0, l + 1 < n_layers ? layers[l + 1].attn_norm : nullptr);
    if (rc != PKV_OK) return rc;
  }
  return PKV_OK;
}

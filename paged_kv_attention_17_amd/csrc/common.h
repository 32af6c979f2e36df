// Shared device/host helpers for the gfx950 kernels of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pagedkv.h"

namespace pkv {

constexpr int kBlock = PKV_BLOCK_SIZE;   // tokens per KV block
constexpr int kHeadDim = PKV_HEAD_DIM;   // compiled head dimension
constexpr int kWave = 64;                // CDNA wavefront width

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- device --

// Widen the low / high bf16 of a packed dword to float32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// Round two float32 to bf16 nearest-even and pack (lo, hi) into one dword;
// gfx950 does this in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
}

// Set bit `bit` of the device error flags (see errors.hip); f may be null.
__device__ __forceinline__ void report_error(uint32_t* f, uint32_t bit) {
  if (f) __hip_atomic_fetch_or(f, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two-term bf16 dot product accumulated in float32: a.lo*b.lo + a.hi*b.hi + c.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                        false);
}

// DPP lane exchanges inside rows of 16 lanes (value from the partner lane).
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF,
                                                               false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each group of 8
constexpr int kDppRowRor8 = 0x128;    // lane i <- (i+8) mod 16 inside a row

// Sum over each aligned group of 8 lanes, result in all 8 lanes.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of lane (self ^ mask) via ds_bpermute (any mask < 64).
__device__ __forceinline__ float shfl_xor(float x, int mask) {
  const int lane = __lane_id();
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Raw buffer access: a scalar descriptor (base, size) and a per-lane 32-bit
// byte offset, so address arithmetic stays on the scalar unit.  Offsets at or
// beyond `bytes` read as zero instead of touching memory.  Word 3 is the gfx9
// family value for untyped dword access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(x[0], x[1], x[2], x[3]);
}
// The same load marked non-temporal (cache policy bit nt): for data read
// once per launch (the K/V stream of a decode call), so that it does not
// push the small, reused data (plans, tables, queries, partial records) out
// of the L2 and last-level caches.
constexpr int kCpolNt = 2;
__device__ __forceinline__ uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCpolNt);
  return make_uint4(x[0], x[1], x[2], x[3]);
}
// Four 16-byte loads of one K/V block (two from each descriptor), marked
// non-temporal when NT is set.  A compile-time choice: loads behind a
// run-time branch make the compiler's wait counting conservative.
template <bool NT>
__device__ __forceinline__ void buf_load_kv4(__amdgpu_buffer_rsrc_t rk, uint32_t ka, uint32_t kb,
                                             __amdgpu_buffer_rsrc_t rv, uint32_t va, uint32_t vb, uint4& k0,
                                             uint4& k1, uint4& v0, uint4& v1) {
  if constexpr (NT) {
    k0 = buf_load16_nt(rk, ka);
    k1 = buf_load16_nt(rk, kb);
    v0 = buf_load16_nt(rv, va);
    v1 = buf_load16_nt(rv, vb);
  } else {
    k0 = buf_load16(rk, ka);
    k1 = buf_load16(rk, kb);
    v0 = buf_load16(rv, va);
    v1 = buf_load16(rv, vb);
  }
}

// Byte permute: result byte k = byte sel[k] of the 8-byte value (hi:lo).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// (lo.bf16[0], hi.bf16[0]) and (lo.bf16[1], hi.bf16[1]) of two packed dwords.
__device__ __forceinline__ uint32_t pack_lo_halves(uint32_t lo, uint32_t hi) { return perm_b32(hi, lo, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi_halves(uint32_t lo, uint32_t hi) { return perm_b32(hi, lo, 0x07060302u); }

// The two halves of a RoPE rotation of the pair (x, y) = (dim i, dim i + d/2)
// by an angle with cosine c and sine s.  Written with explicit fused
// multiply-adds so every kernel that rotates rounds identically.
__device__ __forceinline__ float rope_first(float x, float y, float c, float s) { return __builtin_fmaf(x, c, -(y * s)); }
__device__ __forceinline__ float rope_second(float x, float y, float c, float s) { return __builtin_fmaf(y, c, x * s); }

// ------------------------------------------------------------------ host --

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

inline int launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// The device error flags' address on the current device (errors.hip), or null.
uint32_t* device_errors_ptr();

inline bool ratio_supported(int n_q, int n_kv) {
  if (n_q <= 0 || n_kv <= 0 || n_q % n_kv) return false;
  const int g = n_q / n_kv;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

}  // namespace pkv

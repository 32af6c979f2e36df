// Host-only stand-ins for the library's device calls, so that the host C++
// (block allocator, scheduler) can be built with g++ and the address and
// undefined-behaviour sanitizers: each checks nothing and enqueues nothing.
#include <cstdint>

#include "../../include/pagedkv.h"

namespace pkv {
int patch_distinct(int32_t*, int64_t, const int32_t*, const int32_t*, int, void*) { return PKV_OK; }
int kv_read_override(int policy) {
  static thread_local int current = 0;
  const int prev = current;
  current = policy;
  return prev;
}
}  // namespace pkv

extern "C" {
int pkv_block_table_patch(int32_t*, int64_t, const int32_t*, const int32_t*, int, void*) { return PKV_OK; }
int pkv_rope_decode(pkv_bf16*, pkv_bf16*, const int32_t*, int, int, int, int, const float*, int, void*) {
  return PKV_OK;
}
int pkv_paged_kv_append(pkv_bf16*, pkv_bf16*, int, const pkv_bf16*, const pkv_bf16*, const int32_t*, int64_t, int,
                        int, const int32_t*, const int32_t*, int, int, int, void*) {
  return PKV_OK;
}
int pkv_paged_decode_fused(pkv_bf16*, const pkv_bf16*, const pkv_bf16*, const pkv_bf16*, pkv_bf16*, pkv_bf16*, int,
                           const int32_t*, int64_t, int, int, const int32_t*, const int32_t*, const int32_t*, int, int,
                           int, int, int, const float*, int, float, int, void*, size_t, void*) {
  return PKV_OK;
}
int pkv_paged_attn_prefill(pkv_bf16*, const pkv_bf16*, const int32_t*, const int32_t*, const int32_t*,
                           const pkv_bf16*, const pkv_bf16*, int, const int32_t*, int64_t, int, int, int, int, int, int,
                           int, int, float, const int32_t*, const int32_t*, void*) {
  return PKV_OK;
}
}

// Host interface of the streaming decode kernel (one workgroup per CU, each
// taking an equal share of every block of the batch).  Internal to the library.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pkv {

struct StreamCall {
  uint16_t* out;
  const uint16_t* q;
  const uint16_t* k_new;       // fused only
  const uint16_t* v_new;       // fused only
  uint16_t* k_pool;
  uint16_t* v_pool;
  int num_blocks;
  const int32_t* block_table;
  int64_t bt_row_stride;
  int num_slots;
  int max_blocks;
  const int32_t* slot_ids;     // null = identity
  const int32_t* row_lens_host;
  int batch;
  int n_q, n_kv;
  const float* cos_sin;        // fused only
  int max_pos;
  float scale;
  void* workspace;
  size_t workspace_bytes;
  void* stream;
};

// Workspace bytes the streaming kernel may use for these head counts.
size_t stream_workspace_bytes(int n_q, int n_kv);

// Launch the streaming kernel (and its merge) for `c`.  Returns -1 without
// launching anything when the shapes are outside what it supports (the caller
// then uses the per-partition kernels), else a pkv status.
int stream_decode(bool fused, const StreamCall& c);

}  // namespace pkv

// Host interface of the streaming decode kernel (one workgroup per CU, each
// taking an equal share of every block of the batch).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kStreamMaxSeqs = 256;   // batch rows one launch describes
constexpr int kStreamMaxGrid = 512;   // workgroups (one per CU)
constexpr int kStreamRec = 66;        // record per query head: 64 unnormalised outputs, max, sum

// Kernel arguments (one block of at most 4 KB, passed by value).
struct StreamArgs {
  uint16_t* out;
  const uint16_t* q;
  const uint16_t* k_new;       // fused only
  const uint16_t* v_new;       // fused only
  uint16_t* k_pool;
  uint16_t* v_pool;
  const int32_t* bt;
  const int32_t* slot_ids;     // device slot of each row; null = identity (or slots_in_args)
  const float* rope;           // fused only: [max_pos][32] (cos, sin)
  float* ws;                   // this launch's records [2 * grid][n_q][kStreamRec]
  uint16_t* out_prev;          // prologue merge: output of the previous launch (same rows)
  const float* ws_prev;        // and its records
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
  int grid;
  int slots_in_args;           // row_slot holds each row's slot (0xffff = none)
  int32_t row_start[kStreamMaxSeqs + 1];   // first stream block of each row
  int32_t row_n[kStreamMaxSeqs];           // tokens of each row
  uint16_t row_slot[kStreamMaxSeqs];
  uint16_t wg_rows[kStreamMaxGrid];        // per workgroup: first row << 3 | rows touched
};
static_assert(sizeof(StreamArgs) <= 4096, "kernel argument block");

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
  const int32_t* slot_ids;       // device, null = identity
  const int32_t* slot_ids_host;  // optional host copy of slot_ids (kept in the kernel arguments)
  const int32_t* row_lens_host;
  int batch;
  int n_q, n_kv;
  const float* cos_sin;        // fused only
  int max_pos;
  float scale;
  float* records;              // this launch's records
  size_t records_bytes;
  uint16_t* out_prev;          // non-null: this launch also merges the previous launch's
  const float* records_prev;   //   rows (same rows and lengths), written to out_prev
};

struct StreamLaunch {
  StreamArgs a;
  bool fused;
  bool prev;
  int G;
  int merge;                   // merge launch needed: 0 none, 1 per (row, KV head), 2 per (row, query head)
};

// Bytes of records one streaming launch may write for n_q query heads.
size_t stream_records_bytes(int n_q);

// Build the launch for `c`.  Returns -1 (nothing prepared) when the shapes
// are outside what the kernel supports, PKV_OK otherwise.
int stream_prepare(bool fused, const StreamCall& c, StreamLaunch* L);

// The streaming kernel, then (unless the next launch merges) its merge kernel.
int stream_enqueue(const StreamLaunch& L, hipStream_t st, bool merge);

// The merge kernel alone (for the last launch of a chain).
int stream_merge_enqueue(const StreamLaunch& L, hipStream_t st);

}  // namespace pkv

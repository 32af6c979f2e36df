// Host interface of the streaming decode kernel (one workgroup per CU, each
// taking an equal share of every block of the batch).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kStreamMaxSeqs = 256;   // batch rows one launch describes
constexpr int kStreamMaxGrid = 512;   // workgroups (one per CU)
constexpr int kStreamRec = 68;        // record per query head: 64 unnormalised outputs, max, sum, 2 pad (16-byte rows)

// How the batch's blocks are cut into workgroup shares: rows laid end to end
// (the block stream), each workgroup an equal, contiguous share.  Built on the
// host; travels in the kernel arguments, or (launches captured once and
// replayed as the lengths change) in device memory.
struct StreamPlan {
  int32_t share;               // blocks per workgroup
  int32_t total;               // blocks in the stream
  int32_t grid;                // workgroups with blocks
  int32_t slots_in_args;       // row_slot holds each row's slot (0xffff = none)
  int32_t row_start[kStreamMaxSeqs + 1];   // first stream block of each row
  int32_t row_n[kStreamMaxSeqs];           // tokens of each row
  uint16_t row_slot[kStreamMaxSeqs];
  uint16_t wg_rows[kStreamMaxGrid];        // per workgroup: first row << 3 | rows touched
};

// Kernel arguments: the pointers and sizes (StreamCore, what a launch that
// reads its plan from device memory takes), plus the plan itself for
// launches that carry it (StreamArgs, one block of at most 4 KB, passed by
// value).
struct StreamCore {
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
  const StreamPlan* plan_dev;  // device-plan launches: the plan in device memory
  StreamPlan* plan_out;        // argument-plan launches: workgroup 0 also stores the plan here
  uint32_t* errors;            // device error flags (errors.hip), or null
  int kv_nt;                   // K/V loads marked non-temporal
};
struct StreamArgs : StreamCore {
  StreamPlan plan;             // argument-plan launches: the plan itself
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
  const StreamPlan* plan_dev;  // non-null: the kernels read their plan here (small kernel arguments)
  bool fixed_shape;            // with plan_dev: launch shapes independent of the plan (launches
                               //   captured once and replayed; the plan may change between replays)
  StreamPlan* plan_out;        // non-null: the launch also stores its plan here, in device memory
  bool chain_plan;             // shares sized for chained launches (see stream_plan_build)
  bool kv_nt;                  // K/V loads marked non-temporal (PKV_KV_READ_STREAM)
};

struct StreamLaunch {
  StreamArgs a;
  bool fused;
  bool prev;
  bool devplan;
  bool long_rows;              // a row spans more shares than a chained prologue merges
  int G;
  int grid;                    // workgroups launched
  int merge;                   // merge launch needed: 0 none, 1 per (row, KV head), 2 per (row, query head)
};

// Workgroups of a device-plan launch (one per CU, at most kStreamMaxGrid).
int stream_launch_grid();

// The plan for `batch` rows of host-known lengths (row_lens_host), with the
// rows' slots from slot_ids_host when given (else identity when there are no
// device slot ids).  Shares are equal, ceil(blocks / workgroups); with
// `chain` they are raised, where the rows allow it, until no row spans more
// shares than a chained launch's prologue merges (a few long rows then run on
// fewer workgroups, but every layer's merge rides on the next launch).
// Returns -1 when the streaming kernel cannot serve these rows (a share would
// touch more rows than it stages), 1 when some row spans more shares than a
// chained launch's prologue merges, 0 otherwise; *merge_kind as
// StreamLaunch::merge.
int stream_plan_build(int batch, const int32_t* row_lens_host, int max_blocks, const int32_t* slot_ids_host,
                      bool slot_ids_dev, int num_slots, bool chain, StreamPlan* P, int* merge_kind);

// Bytes of records one streaming launch may write for n_q query heads.
size_t stream_records_bytes(int n_q);

// Bytes a plan takes in device memory (a multiple of 256).
constexpr size_t kStreamPlanBytes = (sizeof(StreamPlan) + 255) / 256 * 256;

// Build the launch for `c`.  Returns -1 (nothing prepared) when the shapes
// are outside what the kernel supports, PKV_OK otherwise.
int stream_prepare(bool fused, const StreamCall& c, StreamLaunch* L);

// The streaming kernel, then (unless the next launch merges) its merge kernel.
int stream_enqueue(const StreamLaunch& L, hipStream_t st, bool merge);

// The merge kernel alone (for the last launch of a chain).
int stream_merge_enqueue(const StreamLaunch& L, hipStream_t st);

// Diagnostic: the streaming kernel's K/V reads alone for the call `c`
// (records are not written).  PKV_ERR_UNSUPPORTED when the kernel cannot
// serve the call or a share exceeds one table window.
int stream_read_probe(const StreamCall& c, uint32_t* sink, hipStream_t st);

}  // namespace pkv

// Internal interface of the decode calls: validation and launch planning
// apart from the launches, so that callers running several launches (a
// decode step over all layers, a decoder layer) find every argument error
// before anything is enqueued.  Internal to the library.
#pragma once

#include "decode_stream.h"

namespace pkv {

// The arguments of pkv_paged_attn_decode / pkv_paged_decode_fused, plus what
// the library's own multi-launch callers know.
struct DecodeCall {
  bool fused;
  uint16_t* out;
  const uint16_t* q;
  const uint16_t* k_new;       // fused
  const uint16_t* v_new;       // fused
  uint16_t* k_pool;
  uint16_t* v_pool;
  int num_blocks;
  const int32_t* block_table;
  int64_t bt_row_stride;
  int num_slots;
  int max_blocks_per_seq;
  const int32_t* slot_ids;
  const int32_t* slot_ids_host;  // optional host copy of slot_ids
  const int32_t* context_lens;
  const int32_t* row_lens_host;
  int batch;
  int max_context_len;
  int n_q_heads;
  int n_kv_heads;
  int head_dim;
  const float* cos_sin;        // fused
  int max_pos;                 // fused
  float scale;
  int partition_size;
  void* workspace;
  size_t workspace_bytes;
  // Chaining of streaming launches over the layers of one step (same rows,
  // same lengths): this launch writes its records at records_half (0 or 1) of
  // the workspace's two record regions and, when out_prev is set, merges the
  // previous launch's cut rows (its records in the other region) into
  // out_prev in its prologue.
  int records_half;
  uint16_t* out_prev;
  bool chain_plan;             // plan the shares for chaining (every launch of a chain sets it)
  // Non-null: the streaming kernel reads its plan from this device copy (the
  // call fails rather than take the per-partition kernels).  The plan built
  // from row_lens_host checks the call.  With fixed_shape the launch shapes
  // do not depend on the plan (launches captured once and replayed).
  const StreamPlan* plan_dev;
  bool fixed_shape;
  // Non-null: the streaming launch also stores its plan here (device memory)
  // for later launches with plan_dev.
  StreamPlan* plan_out;
};

struct DecodeLaunch {
  DecodeCall c;
  int path;                    // 0: nothing to do, 1: streaming kernel, 2: per-partition kernels
  bool kv_nt;                  // K/V loads marked non-temporal (the policy when the call was prepared)
  StreamLaunch s;
};

// Check the call and plan its launches; nothing is enqueued.  PKV_OK or a
// status.  A call that can run chained (streaming path, workspace with two
// record regions and a plan) reports it through decode_chainable.

// The workspace's plan area (after the two record regions) for n_q query heads.
size_t decode_plan_offset(int n_q_heads);
int decode_prepare(const DecodeCall& c, DecodeLaunch* L);
bool decode_chainable(const DecodeLaunch& L);

// A prepared call for the same rows on another table view (another layer's
// entries, same row stride): `out` = `base` with the table replaced, and
// with plan_dev set (streaming path only) the launch reads the plan `base`
// stored there (base.c.plan_out) instead of carrying it.  Checks only what
// differs from `base`; PKV_OK or a status.
int decode_retarget(const DecodeLaunch& base, const int32_t* block_table, const StreamPlan* plan_dev,
                    DecodeLaunch* out);

// Enqueue a prepared call.  merge = false leaves the streaming path's merge
// to the next chained launch (or to decode_finish).
int decode_enqueue(const DecodeLaunch& L, hipStream_t st, bool merge = true);

// The merge a chained streaming launch left for later (no-op otherwise).
int decode_finish(const DecodeLaunch& L, hipStream_t st);

}  // namespace pkv

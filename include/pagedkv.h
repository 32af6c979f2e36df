/*
 * pagedkv.h -- C ABI of libpagedkv, paged KV-cache attention for AMD MI355X (gfx950).
 *
 * The operations follow the engine read in the code series "An Inference Engine
 * in 1,500 Lines of CUDA: The Map" (jaehun.me, English page, and its Korean
 * original): a KV cache that is one pool carved into 16-token blocks, a block
 * table per (sequence slot, layer) whose unassigned entries hold -1 (section
 * "The path of one inference", step (4)), Llama-3-scaled RoPE (same section,
 * step (3)), grouped-query attention with 4 query heads per KV head and an
 * online softmax (Korean page, table in "What is in the box"), and the paired
 * prefill / decode kernels (section "The path of one inference", closing
 * paragraph).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - bf16 values are stored as their 16-bit patterns (pkv_bf16).
 *  - Pointers are DEVICE pointers unless the parameter name ends in _host.
 *    bf16 and float device buffers must be 16-byte aligned, int32 device
 *    arrays 4-byte aligned (PKV_ERR_MISALIGNED otherwise).
 *  - Ownership: the caller allocates and frees every buffer. No call allocates
 *    or frees device memory; the library keeps no state between calls.
 *  - Layouts are row-major with head_dim innermost:
 *      k_pool, v_pool   [num_blocks][16][n_kv_heads][head_dim]   (same block id
 *                        for K and V; a block holds 16 tokens of one layer)
 *      block_table      rows of int32, row s starts at s * bt_row_stride and has
 *                        max_blocks_per_seq entries; entry j names the block that
 *                        holds tokens 16j .. 16j+15 of that row's sequence; -1 = none.
 *                        A caller with a [slots][layers][max_blocks] table passes a
 *                        layer's base pointer and bt_row_stride = layers*max_blocks.
 *      q, out           [tokens][n_q_heads][head_dim];  k_new, v_new [tokens][n_kv_heads][head_dim]
 *  - Query head h reads KV head h / (n_q_heads / n_kv_heads) (contiguous groups).
 *  - Compiled shapes: head_dim == 64, block size 16, n_q_heads / n_kv_heads in
 *    {1, 2, 4, 8}; anything else returns PKV_ERR_UNSUPPORTED.
 *  - Calls that take `stream` (a hipStream_t, NULL = default stream) only
 *    enqueue work and return; argument errors are found on the host before any
 *    launch, and then nothing is enqueued. A failed launch returns PKV_ERR_HIP.
 *  - Device-side data (block ids, context lengths, positions, slot ids) is not
 *    validated by the kernels beyond staying in bounds: a kernel never reads or
 *    writes outside the buffers described by its size arguments, but results for
 *    invalid data are unspecified. pkv_check_block_table validates on the host.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t pkv_bf16;

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,          /* a required pointer is NULL */
  PKV_ERR_MISALIGNED = 2,    /* a device pointer is not suitably aligned */
  PKV_ERR_UNSUPPORTED = 3,   /* head_dim / head ratio outside the compiled set */
  PKV_ERR_INVALID_ARG = 4,   /* negative size, n_q % n_kv != 0, bad partition size, ... */
  PKV_ERR_BAD_BLOCK = 5,     /* host check: -1 or out-of-range block inside a context */
  PKV_ERR_CAPACITY = 6,      /* workspace too small, free list empty, table row too short */
  PKV_ERR_HIP = 7            /* the HIP runtime reported an error */
};

#define PKV_BLOCK_SIZE 16
#define PKV_HEAD_DIM 64

/* Text for a status code (static storage; never NULL). */
const char* pkv_status_str(int status);

/* Version of the library ABI: (major << 16) | minor. */
int pkv_abi_version(void);

/* ------------------------------------------------------------------------ *
 * RoPE (Llama-3 scaling).  Source: "The path of one inference", step (3): a
 * positional-encoding table is built once from head_dim, the maximum length,
 * base 500000 and the scaling numbers 32, 1, 4, 8192; the Korean page's table
 * names the kernel ropeKernel_llama3.  The scaling rule is the public Llama-3
 * one: with f_i = theta^(-2i/d) and wavelength w_i = 2 pi / f_i, pairs with
 * w_i < original_max_pos / high_freq_factor keep f_i, pairs with
 * w_i > original_max_pos / low_freq_factor use f_i / factor, and the rest blend
 * the two linearly in original_max_pos / w_i.
 * ------------------------------------------------------------------------ */

/* Fill the device table cos_sin[max_pos][head_dim/2][2] (float32 cos, sin of
 * p * f_i'), computed in double precision on the host and copied in; the call
 * waits for the copy to finish.  Errors: NULL, max_pos < 1, odd head_dim,
 * non-positive theta/factor, high_freq_factor <= low_freq_factor. */
int pkv_rope_table_init(float* cos_sin, int max_pos, int head_dim, double theta, double factor,
                        double low_freq_factor, double high_freq_factor, int original_max_pos,
                        void* stream);

/* Rotate, in place, q[num_tokens][n_q_heads][head_dim] and k[num_tokens][n_kv_heads][head_dim]
 * of token t by position positions[t]: pair (i, i + head_dim/2) becomes
 * (x cos - y sin, y cos + x sin), computed in float32 and rounded to bf16
 * nearest-even.  Used for the decode step (one token per sequence) and for
 * prefill chunks (many tokens).  k may be NULL (q only).  A position outside
 * [0, max_pos) leaves that token unrotated. */
int pkv_rope_decode(pkv_bf16* q, pkv_bf16* k, const int32_t* positions, int num_tokens,
                    int n_q_heads, int n_kv_heads, int head_dim, const float* cos_sin, int max_pos,
                    void* stream);

/* ------------------------------------------------------------------------ *
 * Paged KV cache.  Source: "The path of one inference", step (4) (pool
 * allocated once and cut into 16-token blocks, free list, block table with -1)
 * and the series' sixth chapter title (reading non-contiguous blocks through
 * the block table).
 * ------------------------------------------------------------------------ */

/* For each token t: s = slot_ids[t], p = positions[t], blk = table[s][p / 16];
 * copy the bits of k_new[t] and v_new[t] into k_pool[blk][p % 16] and
 * v_pool[blk][p % 16].  Tokens whose slot, table entry or block id is out of
 * range are skipped (nothing is written for them). */
int pkv_paged_kv_append(pkv_bf16* k_pool, pkv_bf16* v_pool, int num_blocks,
                        const pkv_bf16* k_new, const pkv_bf16* v_new,
                        const int32_t* block_table, int64_t bt_row_stride, int num_slots,
                        int max_blocks_per_seq, const int32_t* slot_ids, const int32_t* positions,
                        int num_tokens, int n_kv_heads, int head_dim, void* stream);

/* Diagnostic read-back through the same addressing: copy tokens
 * 0 .. context_len-1 of table row `slot` into k_dense/v_dense
 * [context_len][n_kv_heads][head_dim].  Rows whose block id is out of range
 * are written as zeros. */
int pkv_paged_gather(pkv_bf16* k_dense, pkv_bf16* v_dense, const pkv_bf16* k_pool,
                     const pkv_bf16* v_pool, int num_blocks, const int32_t* block_table,
                     int64_t bt_row_stride, int max_blocks_per_seq, int slot, int context_len,
                     int n_kv_heads, int head_dim, void* stream);

/* ------------------------------------------------------------------------ *
 * Device error flags.  Source: "The path of one inference", step (4) (table
 * entries are -1 until a block is assigned; a context must not reach one).
 * The kernels never read outside the pool or the table whatever the device
 * data say: a bad entry is skipped (its tokens count as absent).  They also
 * set a bit in a flag word the library keeps on each device, so that such
 * input is reported rather than silently masked:
 *   PKV_DEVERR_BAD_BLOCK     decode: a table entry inside a context (or the
 *                            new token's entry in the fused step) is -1 or
 *                            not below num_blocks
 *   PKV_DEVERR_BAD_SLOT      decode / prefill: a row's table slot (slot_ids)
 *                            is outside [0, num_slots)
 *   PKV_DEVERR_LONG_CONTEXT  decode: a device context length exceeds
 *                            max_blocks_per_seq x 16 (the rest is not read)
 *   PKV_DEVERR_PREFILL_BLOCK prefill: a table entry a query's keys need is -1
 *                            or not below num_blocks
 * pkv_device_errors copies the current device's word to *flags (host) after
 * the work enqueued on `stream` so far, optionally clears it (clear != 0),
 * and waits for the stream.  The word accumulates over calls until cleared;
 * calls on several streams of one device share it.
 * ------------------------------------------------------------------------ */
#define PKV_DEVERR_BAD_BLOCK 1u
#define PKV_DEVERR_BAD_SLOT 2u
#define PKV_DEVERR_LONG_CONTEXT 4u
#define PKV_DEVERR_PREFILL_BLOCK 8u

int pkv_device_errors(uint32_t* flags, int clear, void* stream);

/* Cache policy of the decode calls' K/V reads (pkv_paged_attn_decode,
 * pkv_paged_decode_fused and its no-allocation form, pkv_decode_step and its
 * two halves, pkv_decode_layer(s), pkv_paged_read_probe).  Source: the
 * chapter-6 title of the category page (each decode step reads all of a
 * sequence's cached K/V again) and its mini-sglang chapter on a radix cache
 * (requests that share a prompt share its cached K/V).
 *   PKV_KV_READ_STREAM (the default): the K/V loads are marked non-temporal.
 *     When every block is listed by one row, a call reads each K/V byte once;
 *     the marking keeps that stream from evicting the small data the calls
 *     reuse (plans, tables, queries, partial records) from the L2 and
 *     last-level caches.
 *   PKV_KV_READ_REUSE: ordinary cached loads, for tables whose rows share
 *     blocks (prefix sharing), so that a block listed by several rows can be
 *     served from the caches.  pkv_sched_run uses it by itself for the
 *     iterations whose decode rows share prefix-cache blocks.
 * Process-wide (every device and thread); a call takes the policy in force
 * when it is enqueued, and a captured graph keeps the one it was captured
 * with.  The policy changes speed only, never results.
 * pkv_set_kv_read_policy: PKV_OK, or PKV_ERR_INVALID_ARG for any other value
 * (nothing changes).  pkv_kv_read_policy: the current setting. */
#define PKV_KV_READ_STREAM 1
#define PKV_KV_READ_REUSE 2
int pkv_set_kv_read_policy(int policy);
int pkv_kv_read_policy(void);

/* Diagnostic, off the attention path: read `bytes` bytes of device memory
 * (16-byte aligned, bytes a multiple of 16) once with wide loads spread over
 * the whole chip, as a reference for the HBM read rate the decode kernels are
 * measured against.  `sink` (device, 4 bytes) is written only when the data
 * XOR to a fixed pattern, so the reads cannot be optimised away. */
int pkv_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Diagnostic, off the attention path: the K/V reads of pkv_paged_attn_decode's
 * streaming kernel alone, for the same arguments (pools, table view, slots,
 * host row lengths): the same plan, per-CU shares, wave split and loads, no
 * arithmetic and no output.  `sink` as pkv_hbm_read_probe.  It measures what
 * reading a batch's blocks in this pattern costs on its own, the floor the
 * decode kernel is compared with.  PKV_ERR_UNSUPPORTED when the streaming
 * kernel cannot serve the arguments or a workgroup's share exceeds 1,024
 * blocks. */
int pkv_paged_read_probe(const pkv_bf16* k_pool, const pkv_bf16* v_pool, int num_blocks,
                         const int32_t* block_table, int64_t bt_row_stride, int num_slots,
                         int max_blocks_per_seq, const int32_t* slot_ids, const int32_t* row_lens_host,
                         int batch, int n_kv_heads, int head_dim, uint32_t* sink, void* stream);

/* Host-side block allocation for one step ("The path of one inference",
 * step (4): blocks come off a free list; -1 marks an unassigned entry).
 * For every token t whose table entry bt_host[slot_ids_host[t]][positions_host[t] / 16]
 * is -1, pop a block from the end of free_list_host (n_free is updated) and
 * store it there; each assignment is also appended to patch_offsets_host /
 * patch_values_host (flat index into the table, block id; room for num_tokens
 * entries) and counted in *n_patch.  All or nothing: if the free list or a
 * table row is too short, nothing changes and PKV_ERR_CAPACITY is returned.
 * Pure host code; no device is touched. */
int pkv_blocks_assign(int32_t* bt_host, int64_t bt_row_stride, int num_slots,
                      int max_blocks_per_seq, int32_t* free_list_host, int* n_free,
                      const int32_t* slot_ids_host, const int32_t* positions_host, int num_tokens,
                      int32_t* patch_offsets_host, int32_t* patch_values_host, int* n_patch);

/* Return every assigned block of table row `slot` to the free list (pushed at
 * the end) and reset the row to -1; the released entries are appended to the
 * patch arrays (room for max_blocks_per_seq entries) with value -1.
 * PKV_ERR_CAPACITY if the free list would exceed free_capacity. Host only. */
int pkv_blocks_release(int32_t* bt_host, int64_t bt_row_stride, int num_slots,
                       int max_blocks_per_seq, int slot, int32_t* free_list_host, int* n_free,
                       int free_capacity, int32_t* patch_offsets_host, int32_t* patch_values_host,
                       int* n_patch);

/* Apply host-side table changes to the device copy: bt_dev[offsets[i]] = values[i]
 * for i < n_patch.  The two arrays are HOST arrays; their contents travel in
 * the kernel arguments, so they may be reused as soon as the call returns.
 * The pairs take effect in list order: when an offset appears more than once
 * the last pair wins (a release followed by a reuse of the same entry may be
 * sent as one list).  Offsets outside [0, bt_elems) are skipped. */
int pkv_block_table_patch(int32_t* bt_dev, int64_t bt_elems, const int32_t* patch_offsets_host,
                          const int32_t* patch_values_host, int n_patch, void* stream);

/* Prefix sharing (host).  Source: the category page "code-series", whose
 * mini-sglang series has a chapter on a radix cache: requests that open with
 * the same prompt reuse that prefix's cached K/V rather than computing it
 * again.  The pages give no mechanism; the one here: a block may be listed by
 * several table entries, refcount_host[b] (one int32 per pool block, kept by
 * the caller, 0 for a free block) counts the entries that list b, and a block
 * is written only through an entry that lists it alone.
 *
 * pkv_blocks_share: row dst_slot takes row src_slot's entries for tokens
 * 0 .. n_tokens-1 (entries 0 .. ceil(n_tokens/16)-1), the same block ids, and
 * each listed block's count grows by one.  Those entries of dst_slot must be
 * -1 and the source's must hold counted blocks of the pool; otherwise nothing
 * changes and PKV_ERR_INVALID_ARG / PKV_ERR_BAD_BLOCK is returned
 * (PKV_ERR_CAPACITY if the row is too short).  Changes are appended to the
 * patch arrays (room for ceil(n_tokens/16) entries). */
int pkv_blocks_share(int32_t* bt_host, int64_t bt_row_stride, int num_slots, int max_blocks_per_seq,
                     int src_slot, int dst_slot, int n_tokens, int32_t* refcount_host, int num_blocks,
                     int32_t* patch_offsets_host, int32_t* patch_values_host, int* n_patch);

/* pkv_blocks_assign with shared blocks.  For every entry that a token
 * (slot_ids_host[t], positions_host[t]) writes into, in token order:
 *   - entry -1: a block is popped from the end of free_list_host, count 1;
 *   - entry listing a block whose count (after the moves earlier in this
 *     call) exceeds 1: copy on write -- a block is popped (count 1), the entry
 *     points to it, the old block's count drops by one and the pair (old, new)
 *     is appended to copy_src_host / copy_dst_host (room for num_tokens pairs;
 *     *n_copy);
 *   - otherwise the entry stays.
 * Every changed entry goes to the patch arrays (room for num_tokens).  The
 * caller copies the listed blocks (pkv_blocks_copy) before the append that
 * writes them.  Popped blocks must have count 0.  All or nothing. Host only. */
int pkv_blocks_assign_shared(int32_t* bt_host, int64_t bt_row_stride, int num_slots, int max_blocks_per_seq,
                             int32_t* free_list_host, int* n_free, int32_t* refcount_host, int num_blocks,
                             const int32_t* slot_ids_host, const int32_t* positions_host, int num_tokens,
                             int32_t* patch_offsets_host, int32_t* patch_values_host, int* n_patch,
                             int32_t* copy_src_host, int32_t* copy_dst_host, int* n_copy);

/* pkv_blocks_release with shared blocks: every assigned entry of row `slot`
 * drops its block's count by one and becomes -1; a block whose count reaches 0
 * is pushed onto the free list.  PKV_ERR_CAPACITY if the free list would
 * exceed free_capacity, PKV_ERR_INVALID_ARG if a count would go negative; a
 * failure changes nothing.  Patch arrays: room for max_blocks_per_seq. */
int pkv_blocks_release_shared(int32_t* bt_host, int64_t bt_row_stride, int num_slots, int max_blocks_per_seq,
                              int slot, int32_t* free_list_host, int* n_free, int free_capacity,
                              int32_t* refcount_host, int num_blocks, int32_t* patch_offsets_host,
                              int32_t* patch_values_host, int* n_patch);

/* Device half of copy on write: for i < n_copy, block dst_host[i] of both
 * pools takes the 16 rows (all KV heads) of block src_host[i].  The id arrays
 * are HOST arrays carried in the kernel arguments (reusable when the call
 * returns).  Every copy reads the pools as they were before the call: ids must
 * lie in [0, num_blocks) (else PKV_ERR_BAD_BLOCK), no block may be written
 * twice or be both written and read (PKV_ERR_INVALID_ARG), checked on the
 * host before anything is enqueued. */
int pkv_blocks_copy(pkv_bf16* k_pool, pkv_bf16* v_pool, int num_blocks, int n_kv_heads, int head_dim,
                    const int32_t* src_host, const int32_t* dst_host, int n_copy, void* stream);

/* Validate tables on the host for rows slot_ids_host[0..batch) (NULL = rows
 * 0..batch-1) and lengths context_lens_host (indexed by row): every entry
 * covering tokens 0 .. len-1 must be in [0, num_blocks), len must fit the row,
 * and no block may appear twice among the checked entries. Returns PKV_OK, or
 * PKV_ERR_BAD_BLOCK with *bad_row / *bad_idx set to the first offending
 * (batch index, table entry); bad_idx = -1 flags a length beyond the row,
 * -2 a slot id out of range. Host only. */
int pkv_check_block_table(const int32_t* bt_host, int64_t bt_row_stride, int num_slots,
                          int max_blocks_per_seq, const int32_t* slot_ids_host,
                          const int32_t* context_lens_host, int batch, int num_blocks,
                          int* bad_row, int* bad_idx);

/* ------------------------------------------------------------------------ *
 * Decode attention.  Source: the Korean page's table ("What is in the box":
 * online softmax and PagedAttention in pagedAttentionKernel, GQA ratio 4) and
 * the chapter-6 title (each decode step re-reads the sequence's cached K/V
 * through the block table).  For batch row b with s = slot_ids[b] (NULL =
 * identity) and n = context_lens[s] (the length includes the token appended
 * this step), query head h with KV head g:
 *     out[b][h] = sum_j softmax_j(scale * <q[b][h], K_j,g>) V_j,g ,  j < n
 * bf16 inputs, float32 accumulation (the softmax weights are rounded to bf16
 * before they multiply V and before they are summed), bf16 output
 * (nearest-even); n == 0 gives a zero row.  Long contexts are split into
 * partitions of partition_size tokens whose partial (max, sum, unnormalised
 * output) a second, small kernel merges.
 * scale must be positive and finite.
 * ------------------------------------------------------------------------ */

/* Bytes of workspace the decode calls need for these sizes: the larger of
 * the per-partition kernels' partials (batch x n_q_heads x partitions records)
 * and the streaming kernel's share: two record regions (two records per
 * workgroup, at most 512 workgroups; a decode step's chained launches
 * alternate between them), each record 68 floats per query head (output, max,
 * sum, two of padding), then 3,840 bytes for the row plan a step's first launch stores for the
 * others.  Returns 0 for invalid arguments.  partition_size 0 = the automatic
 * choice, which depends only on the arguments given here.  A call given less
 * than one record region uses the per-partition kernels; a decode step given
 * less than the whole share runs its layers unchained. */
size_t pkv_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                  int max_context_len, int partition_size);

/* Zero a decode workspace (a kernel on `stream`, no memset node).  Optional:
 * the decode calls need no particular initial contents; provided so that a
 * workspace never holds stale data from other users. */
int pkv_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* The partition size the automatic choice picks for these sizes. */
int pkv_decode_partition_size(int batch, int n_kv_heads, int max_context_len);

/* max_context_len: host-known upper bound of the lengths (sizes the grid);
 * a longer context is still handled correctly, by the last partition, only
 * slower. Contexts are clipped to max_blocks_per_seq * 16.
 * row_lens_host: optional HOST copy of each batch row's length
 * (context_lens[slot_ids[b]]), batch <= 256.  When given, only the partitions
 * that exist are launched, longest first; the kernels still take their lengths
 * from context_lens, and the two must agree (otherwise the result is
 * unspecified).  NULL launches the max_context_len grid.  Either way a row's
 * float32 sums are taken in an order fixed by the row lengths (and the
 * partition size): the same inputs give the same bits from call to call and
 * under any placement of the row's blocks in the pool.
 * partition_size: 0 = automatic, else a positive multiple of 16.
 * workspace: at least pkv_decode_workspace_bytes(...) bytes of device memory,
 * 16-byte aligned, any contents (every value read is written first in the same
 * call); NULL is accepted when no sequence needs more than one partition (the
 * call then uses the per-partition kernels).  Calls sharing one workspace must
 * not run concurrently. */
int pkv_paged_attn_decode(pkv_bf16* out, const pkv_bf16* q, const pkv_bf16* k_pool,
                          const pkv_bf16* v_pool, int num_blocks, const int32_t* block_table,
                          int64_t bt_row_stride, int num_slots, int max_blocks_per_seq,
                          const int32_t* slot_ids, const int32_t* context_lens,
                          const int32_t* row_lens_host, int batch, int max_context_len,
                          int n_q_heads, int n_kv_heads, int head_dim, float scale,
                          int partition_size, void* workspace, size_t workspace_bytes,
                          void* stream);

/* The decode step of one layer in one launch: RoPE + KV append + attention.
 * For batch row b (s = slot_ids[b], n = context_lens[s], new token at
 * p = n - 1): q[b] and k_new[b] are rotated by position p exactly as
 * pkv_rope_decode would (in registers; q and k_new are not modified), the
 * rotated key and v_new[b] are written into pool row p of table row s (the
 * table entry must already hold a block; pkv_blocks_assign), and out[b] is the
 * attention of the rotated query over tokens 0 .. p, the new one included.
 * Same cache contents (bit for bit) and, up to float32 summation order, the
 * same outputs as pkv_rope_decode + pkv_paged_kv_append + pkv_paged_attn_decode.
 * k_new, v_new: [batch][n_kv_heads][64]; cos_sin: pkv_rope_table_init's table. */
int pkv_paged_decode_fused(pkv_bf16* out, const pkv_bf16* q, const pkv_bf16* k_new,
                           const pkv_bf16* v_new, pkv_bf16* k_pool, pkv_bf16* v_pool,
                           int num_blocks, const int32_t* block_table, int64_t bt_row_stride,
                           int num_slots, int max_blocks_per_seq, const int32_t* slot_ids,
                           const int32_t* context_lens, const int32_t* row_lens_host, int batch,
                           int max_context_len, int n_q_heads, int n_kv_heads, int head_dim,
                           const float* cos_sin,
                           int max_pos, float scale, int partition_size, void* workspace,
                           size_t workspace_bytes, void* stream);

/* pkv_paged_decode_fused without a workspace argument, for callers that
 * cannot allocate device memory (code under graph capture, serving loops or
 * harnesses that forbid allocation).  The partial records go to a device
 * array of PKV_NOALLOC_SCRATCH_BYTES inside the library (one per GPU it runs
 * on, held until the process ends; its address is looked up once per device
 * on the first call there).  Arguments and results as pkv_paged_decode_fused;
 * a call whose partials would not fit (pkv_decode_workspace_bytes of its
 * sizes, for the path it takes) returns PKV_ERR_CAPACITY before anything is
 * enqueued.  The call allocates nothing.  Every call on one GPU shares the
 * array: calls that overlap on one GPU (other streams, other host threads)
 * race and must be serialised by the caller.  Nothing in the array needs to
 * start at zero: every value read is written first in the same call. */
#define PKV_NOALLOC_SCRATCH_BYTES (16u << 20)
int pkv_paged_decode_fused_noalloc(pkv_bf16* out, const pkv_bf16* q, const pkv_bf16* k_new,
                                   const pkv_bf16* v_new, pkv_bf16* k_pool, pkv_bf16* v_pool,
                                   int num_blocks, const int32_t* block_table, int64_t bt_row_stride,
                                   int num_slots, int max_blocks_per_seq, const int32_t* slot_ids,
                                   const int32_t* context_lens, const int32_t* row_lens_host, int batch,
                                   int max_context_len, int n_q_heads, int n_kv_heads, int head_dim,
                                   const float* cos_sin, int max_pos, float scale, int partition_size,
                                   void* stream);

/* ------------------------------------------------------------------------ *
 * Chunked causal prefill.  Source: "The path of one inference", closing
 * paragraph (prefill pushes the whole prompt through at once, matrix x
 * matrix) and the category page's chunked-prefill chapter title. Sequence i
 * owns query rows cu_q_lens[i] .. cu_q_lens[i+1]-1; its first query is at
 * absolute position q_start_pos[i]; query row at position a attends keys
 * 0 .. a of table row slot_ids[i] (NULL = i). The chunk's own K/V must already
 * be in the pool (pkv_paged_kv_append). QK^T and PV run on MFMA (bf16 in,
 * float32 accumulate); out is bf16 [total_q][n_q_heads][head_dim].  scale
 * must be positive and finite (PKV_ERR_INVALID_ARG otherwise).
 * max_q_len: host bound on the longest query run (sizes the grid).
 * cu_q_lens_host, q_start_host: optional HOST copies of cu_q_lens and
 * q_start_pos (both or neither).  When given (and the call has at most 768
 * (sequence, query tile) pairs), only real work is launched, the tiles that
 * see the most keys first; the kernels still read the device arrays, and the
 * two must agree (otherwise the result is unspecified).  NULL launches the
 * max_q_len grid.  Either way the output is the same, bit for bit.
 * ------------------------------------------------------------------------ */
int pkv_paged_attn_prefill(pkv_bf16* out, const pkv_bf16* q, const int32_t* cu_q_lens,
                           const int32_t* q_start_pos, const int32_t* slot_ids,
                           const pkv_bf16* k_pool, const pkv_bf16* v_pool, int num_blocks,
                           const int32_t* block_table, int64_t bt_row_stride, int num_slots,
                           int max_blocks_per_seq, int num_seqs, int total_q, int max_q_len,
                           int n_q_heads, int n_kv_heads, int head_dim, float scale,
                           const int32_t* cu_q_lens_host, const int32_t* q_start_host, void* stream);

/* ------------------------------------------------------------------------ *
 * One whole decode step of an n-layer engine, driven natively.  Source: "The
 * path of one inference" (after prefill, every active slot produces one token
 * per decode step; blocks come off the free list as sequences grow).  For each
 * batch row b (slot s = slot_ids_host[b], new token at position
 * p = cached_lens_host[s]):
 *   1. host: for every layer whose table entry bt_host[s][layer][p / 16] is -1,
 *      pop a block from free_list_host (all or nothing: PKV_ERR_CAPACITY and no
 *      change at all if the free list is too short or p / 16 >= max_blocks);
 *   2. cached_lens_host[s] += 1; the new table entries go to bt_dev and the
 *      context lengths, positions and slot ids to meta_dev, carried in kernel
 *      arguments (no host buffer is read after the call returns);
 *   3. per layer l: pkv_paged_decode_fused(out[l], q[l], k[l], v[l]) over the
 *      layer's table view (one launch per layer).
 * q, k, v, out are HOST arrays of n_layers DEVICE pointers ([batch][n_q][64],
 * [batch][n_kv][64], [batch][n_kv][64], [batch][n_q][64]); q and k are not
 * modified.  bt_host / bt_dev: [num_slots][n_layers][max_blocks_per_seq] int32,
 * the device copy mirroring the host one.  meta_dev: device int32
 * [num_slots + 2 * batch] = context lengths (per slot) | positions | slot ids,
 * written by this call; its context-length part must hold cached_lens_host
 * before the first step.  The workspace is pkv_paged_attn_decode's, for
 * (batch, n_q_heads, n_kv_heads, head_dim, max_context_len, partition_size).
 * All launches go to `stream`; the call returns after enqueueing them.
 * ------------------------------------------------------------------------ */
int pkv_decode_step(int n_layers, pkv_bf16* const* q, pkv_bf16* const* k, const pkv_bf16* const* v,
                    pkv_bf16* const* out, pkv_bf16* k_pool, pkv_bf16* v_pool, int num_blocks,
                    int32_t* bt_host, int32_t* bt_dev, int num_slots, int max_blocks_per_seq,
                    int32_t* free_list_host, int* n_free, int32_t* cached_lens_host, int32_t* meta_dev,
                    const int32_t* slot_ids_host, int batch, int n_q_heads, int n_kv_heads, int head_dim,
                    const float* cos_sin, int max_pos, float scale, int max_context_len,
                    int partition_size, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * The same decode step in two halves, for a device half captured once as a
 * HIP graph and replayed every step.  Source: the category page's mini-sglang
 * chapter-7 title (the step's ledger becomes kernel arguments; the launches are
 * captured as a graph) and "The path of one inference" (the step itself).
 * The device half's launch shapes depend only on (n_layers, batch, heads,
 * num_slots), never on the lengths: everything that changes from step to step
 * travels through a staging area that the caller copies to the device inside
 * the captured sequence.
 *
 * pkv_decode_step_staging_bytes: size of the staging area (host and device
 * copies alike) for n_layers, batch and num_slots; 0 for invalid sizes or
 * batch > 256.
 *
 * pkv_decode_step_host: step 1 and 2 of pkv_decode_step on the host (same
 * allocation rule, same all-or-nothing checks, same PKV_ERR_CAPACITY), written
 * into staging_host (any host memory; pinned when it is copied by a captured
 * copy): the table changes, the new metadata (context lengths per slot |
 * positions | slot ids) and the streaming kernel's plan.  Nothing is enqueued.
 * PKV_ERR_UNSUPPORTED, with no change at all, when the rows do not suit the
 * replayed launches (a workgroup share would touch more than 4 rows, or, over
 * several layers, a row spans more than 8 shares: a few long rows beside many
 * short ones); the caller then takes pkv_decode_step for this step.
 *
 * pkv_decode_step_device: enqueues, in a fixed sequence, one small kernel that
 * applies staging_dev (table changes into bt_dev, metadata into meta_dev),
 * then one fused streaming launch per layer (RoPE, append, attention; each
 * merges the previous layer's rows cut by workgroup shares) reading the plan
 * from staging_dev at every launch, then one merge launch (per KV head over
 * several layers, per query head for one layer).  staging_dev must
 * hold a copy of staging_host (made by the caller on `stream` before this
 * call's launches, e.g. an async copy captured in the same graph); the host
 * copy is read only to check the launches when this call is made (capture
 * time).  Replays of a capture serve any later step whose host half used the
 * same n_layers, batch and num_slots.  The caller must not rewrite
 * staging_host while a replay's copy of it may still be pending.  The other
 * arguments are pkv_decode_step's; the workspace must hold the streaming
 * kernel's share (pkv_decode_workspace_bytes for the batch).  Errors: PKV_ERR_UNSUPPORTED
 * when the staged rows or the shapes do not suit the streaming kernel,
 * PKV_ERR_CAPACITY when the workspace is too small, else as pkv_decode_step.
 * ------------------------------------------------------------------------ */
size_t pkv_decode_step_staging_bytes(int n_layers, int batch, int num_slots);

int pkv_decode_step_host(int n_layers, int32_t* bt_host, int num_slots, int max_blocks_per_seq,
                         int32_t* free_list_host, int* n_free, int32_t* cached_lens_host,
                         const int32_t* slot_ids_host, int batch, void* staging_host);

int pkv_decode_step_device(int n_layers, pkv_bf16* const* q, pkv_bf16* const* k, const pkv_bf16* const* v,
                           pkv_bf16* const* out, pkv_bf16* k_pool, pkv_bf16* v_pool, int num_blocks,
                           int32_t* bt_dev, int num_slots, int max_blocks_per_seq, int32_t* meta_dev,
                           int batch, int n_q_heads, int n_kv_heads, int head_dim, const float* cos_sin,
                           int max_pos, float scale, const void* staging_host, const void* staging_dev,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Continuous batching (host scheduler + device iteration).  Source: "The path
 * of one inference" (a fixed set of sequence slots; prompts wait in a queue;
 * a free slot takes the next prompt, which is prefilled; a decode step gives
 * every active slot one token; a finished slot is freed; the loop ends when no
 * slot is active and the queue is empty) and the category page's mini-sglang
 * chapter-3 title (a per-step token budget; long prompts prefilled in chunks).
 *
 * One iteration (pkv_sched_next), in this order:
 *   1. slots whose request produced its last token in the previous iteration
 *      are released (blocks back to the free list, table entries to -1);
 *   2. admission, first come first served: the head of the queue takes the
 *      lowest free slot if the blocks it can ever need, n_layers x
 *      ceil((prompt_len + max_new_tokens - 1) / 16), are not yet reserved by
 *      admitted requests; otherwise the queue waits (no overtaking, no
 *      preemption: an admitted request always finds its blocks);
 *   3. decode rows: every admitted request whose prompt is cached and that
 *      still owes tokens caches one token (row order = admission order);
 *   4. prefill chunks: the rest of the budget goes to requests whose prompt is
 *      not fully cached, admission order, min(uncached tokens, budget left)
 *      each;
 *   5. a block leaves the free list when a token opens a 16-token chunk (the
 *      lowest free block id first on a fresh scheduler).
 * A request yields its first token in the iteration that caches its prompt's
 * last chunk and one more per decode row; it is finished after max_new_tokens
 * tokens (the last one is never cached, so at most prompt_len +
 * max_new_tokens - 1 tokens are cached).
 *
 * The iteration's token rows: rows 0 .. n_decode-1 are the decode rows, rows
 * n_decode .. n_tokens-1 the prefill tokens, chunk by chunk.  All arrays point
 * into the scheduler and stay valid until its next pkv_sched_next/destroy.
 * ------------------------------------------------------------------------ */
typedef struct pkv_sched pkv_sched;

typedef struct {
  int n_tokens;                 /* n_decode + n_prefill_tokens; 0 and no patches: nothing left to do */
  int n_decode;
  const int32_t* decode_slots;  /* [n_decode] slot of each decode row */
  const int32_t* decode_lens;   /* [n_decode] context length with the row's token (its position + 1) */
  const int64_t* decode_ids;    /* [n_decode] request ids */
  int n_chunks;
  const int32_t* chunk_slots;   /* [n_chunks] */
  const int32_t* chunk_start;   /* [n_chunks] position of the chunk's first token */
  const int32_t* cu_chunk;      /* [n_chunks + 1] offsets of the chunks among the prefill tokens */
  const int64_t* chunk_ids;     /* [n_chunks] request ids */
  int n_prefill_tokens;
  const int32_t* token_slots;   /* [n_prefill_tokens] */
  const int32_t* token_pos;     /* [n_prefill_tokens] */
  int n_patch;                  /* table changes of this iteration, in order (flat index, block or -1) */
  const int32_t* patch_off;
  const int32_t* patch_val;
  int n_done;                   /* requests whose last token this iteration produces */
  const int64_t* done_ids;
  int n_admitted;               /* requests admitted in this iteration and their slots */
  const int64_t* admitted_ids;
  const int32_t* admitted_slots;
  const int32_t* admitted_cached;  /* prompt tokens each found in the prefix cache (not prefilled) */
} pkv_sched_iter;

typedef struct {
  int num_slots, n_layers, max_blocks_per_seq, num_blocks, token_budget;
  int n_queued, n_active, n_free, n_reserved;
  const int32_t* table;         /* host table [num_slots][n_layers][max_blocks_per_seq] */
  const int32_t* free_list;     /* [n_free] free blocks (popped from the end) */
  int64_t meta_elems;           /* pkv_sched_meta_elems(num_slots, token_budget) */
  int n_cache_nodes;            /* prefix cache: full prompt blocks held */
  int n_cache_blocks;           /* their pool blocks (n_cache_nodes x n_layers) */
  const int32_t* cache_blocks;  /* [n_cache_blocks] */
  int n_evictable;              /* nodes no active request lists and with no cached continuation */
  int64_t cache_hit_tokens;     /* prompt tokens taken from the cache so far */
} pkv_sched_state;

/* A scheduler with an empty table and all num_blocks blocks free.
 * token_budget >= num_slots (every decode row always fits).
 * PKV_ERR_INVALID_ARG for non-positive sizes or a smaller budget. */
int pkv_sched_create(pkv_sched** sched, int num_slots, int n_layers, int max_blocks_per_seq, int num_blocks,
                     int token_budget);
int pkv_sched_destroy(pkv_sched* sched);

/* Queue a request (ids are the caller's; not checked for uniqueness).
 * prompt_len >= 1, max_new_tokens >= 1.  PKV_ERR_CAPACITY if it could never
 * be admitted (its tokens exceed a table row or its blocks the pool). */
int pkv_sched_submit(pkv_sched* sched, int64_t request_id, int prompt_len, int max_new_tokens);

/* Prefix cache.  Source: the category page's mini-sglang chapter-5 title (a
 * radix cache reuses the cached K/V of prefixes that many requests share, and
 * evicts).  A request queued with its prompt's token ids (copied; HOST array
 * of prompt_len ids) takes part: at admission its table row lists the blocks
 * of the longest run of its prompt's full 16-token blocks already cached
 * (keeping at least one prompt token to prefill), in every layer, and its
 * prefill starts after them; when its whole prompt is cached, its full prompt
 * blocks join the cache (a trie of 16-token keys, one node per block, each
 * holding a pool block per layer) unless an identical block was published
 * first.  Cached blocks are never written (writes start after the listed
 * prefix), stay allocated after their requests finish, and are evicted least
 * recently used first, leaves only and only when no active request lists
 * them, when an admission needs blocks.  K/V of a token must depend only on
 * the tokens before it and its position (true of a model; the caller's duty
 * for synthetic inputs).  pkv_sched_submit is this call with no ids (the
 * request neither reuses nor publishes). */
int pkv_sched_submit_tokens(pkv_sched* sched, int64_t request_id, const int32_t* prompt_tokens_host,
                            int prompt_len, int max_new_tokens);

/* Plan the next iteration (host only; no device is touched). */
int pkv_sched_next(pkv_sched* sched, pkv_sched_iter* iter);

/* Sizes, counters and the host table / free list. */
int pkv_sched_info(const pkv_sched* sched, pkv_sched_state* state);

/* int32 elements of the device metadata array pkv_sched_run needs. */
int64_t pkv_sched_meta_elems(int num_slots, int token_budget);

/* Run an iteration on the device: apply its table patches to bt_dev (device
 * copy of the scheduler's table, all -1 at creation), send the row metadata
 * to meta_dev (device int32 [pkv_sched_meta_elems]; any initial contents) in
 * kernel arguments, then per layer l:
 *   decode rows:    pkv_paged_decode_fused on rows 0 .. n_decode-1 (q, k not modified);
 *   prefill tokens: pkv_rope_decode (in place on those rows of q[l] and k[l]),
 *                   pkv_paged_kv_append, pkv_paged_attn_prefill.
 * q, k, v, out: HOST arrays of n_layers DEVICE pointers, [n_tokens][n_q][64],
 * [n_tokens][n_kv][64], [n_tokens][n_kv][64], [n_tokens][n_q][64] (room for
 * token_budget rows).  Pools, RoPE table and decode workspace as in the calls
 * above (workspace for batch = num_slots).  All launches go to `stream`.
 * Iterations must be run in the order they were planned. */
int pkv_sched_run(const pkv_sched* sched, const pkv_sched_iter* iter, pkv_bf16* const* q, pkv_bf16* const* k,
                  const pkv_bf16* const* v, pkv_bf16* const* out, pkv_bf16* k_pool, pkv_bf16* v_pool,
                  int32_t* bt_dev, int32_t* meta_dev, int n_q_heads, int n_kv_heads, int head_dim,
                  const float* cos_sin, int max_pos, float scale, void* workspace, size_t workspace_bytes,
                  void* stream);

/* ------------------------------------------------------------------------ *
 * The rest of a Llama decode layer.  Source: the opening paragraph of "An
 * Inference Engine in 1,500 Lines of CUDA: The Map" (Llama 3.2 1B; attention,
 * RMSNorm and softmax in the engine's own kernels), the Korean page's "What
 * is in the box" table (rmsNormKernel), the 2048-wide buf_2048_* buffers of
 * "A function with 51 parameters" and the chapter-4 title (projections on the
 * vendor GEMM).  Formulas: the public Llama ones.  All tensors bf16,
 * row-major; weights in the Hugging Face layout [out_features][in_features].
 * ------------------------------------------------------------------------ */

/* out[r] = x[r] / sqrt(mean(x[r]^2) + eps) * weight, float32 math, one
 * nearest-even rounding per output.  dim % 8 == 0. */
int pkv_rmsnorm(pkv_bf16* out, const pkv_bf16* x, const pkv_bf16* weight, int rows, int dim, float eps,
                void* stream);

/* act[r][i] = silu(g) * u with g = gate_up[r][i], u = gate_up[r][intermediate + i]
 * (gate_up [rows][2 * intermediate]), silu(g) = g / (1 + e^-g), float32 math.
 * intermediate % 8 == 0. */
int pkv_silu_mul(pkv_bf16* act, const pkv_bf16* gate_up, int rows, int intermediate, void* stream);

/* Bytes of float32 partials pkv_linear needs for this shape (0: none):
 * nonzero where the product's K is split across workgroups (few output
 * tiles for the chip's 256 CUs and in_features above 4096; at most 4096,
 * such shapes run on the narrow-tile kernel, which needs none). */
size_t pkv_linear_workspace_bytes(int rows, int out_features, int in_features);

/* out[rows][out_features] = x[rows][in_features] weight^T (+ out when
 * accumulate != 0), float32 sums, one rounding per output, on the library's
 * MFMA projection kernels, deterministic (every sum in a fixed order): one
 * workgroup per 64 features and 64-row block, or, where those tiles alone
 * would leave CUs idle and in_features <= 4096, one per 16 features whose
 * four waves split K and add their sums in LDS.  When the 64-feature kernel
 * splits K over workgroups and `workspace` (caller-owned device memory,
 * 16-byte aligned, contents ignored and overwritten) is null or smaller than
 * pkv_linear_workspace_bytes(...), the product runs as one K range.
 * out_features and in_features must be multiples of 8
 * (PKV_ERR_UNSUPPORTED otherwise).  out must not overlap x or weight. */
int pkv_linear(pkv_bf16* out, const pkv_bf16* x, const pkv_bf16* weight, int rows, int out_features,
               int in_features, int accumulate, void* workspace, size_t workspace_bytes, void* stream);

/* Diagnostic, off the layer's path: the projection kernels' weight reads
 * alone over w [n][k] bf16 (n % 16 == 0, k a multiple of 128 x k_parts,
 * else PKV_ERR_UNSUPPORTED; k_parts 1, 2, 4 or 8, else PKV_ERR_INVALID_ARG):
 * one wave per 16-row block and K part, each lane 16-byte loads in the MFMA
 * operand pattern the kernels use (row lane % 16, k 8 (lane / 16) + 32 u of
 * each 128-wide slice), two slices in flight, no arithmetic and no output
 * (the last slice is re-read twice at the end, from cache).  `sink` as
 * pkv_hbm_read_probe.  It gives the rate at which a weight matrix streams in
 * this pattern, the floor the projections are compared with. */
int pkv_weight_read_probe(const pkv_bf16* w, int n, int k, int k_parts, uint32_t* sink, void* stream);

typedef struct {
  const pkv_bf16* attn_norm;    /* [hidden] */
  const pkv_bf16* wq;           /* [n_q_heads * 64][hidden] */
  const pkv_bf16* wk;           /* [n_kv_heads * 64][hidden] */
  const pkv_bf16* wv;           /* [n_kv_heads * 64][hidden] */
  const pkv_bf16* wo;           /* [hidden][n_q_heads * 64] */
  const pkv_bf16* mlp_norm;     /* [hidden] */
  const pkv_bf16* w_gate_up;    /* [2 * intermediate][hidden]: gate rows, then up rows */
  const pkv_bf16* w_down;       /* [hidden][intermediate] */
} pkv_layer_weights;

/* bf16 elements of pkv_decode_layer's scratch: a | q | k | v | o | m |
 * gate_up | act, each [batch][width] (widths hidden, n_q*64, n_kv*64, n_kv*64,
 * n_q*64, hidden, 2*intermediate, intermediate), in that order, then room for
 * the projections' float32 partials (the largest pkv_linear_workspace_bytes
 * over the layer's launches, Q/K/V together as one product of width
 * (n_q + 2 n_kv) * 64); 0 for invalid sizes. */
size_t pkv_decode_layer_scratch_elems(int batch, int hidden, int intermediate, int n_q_heads, int n_kv_heads);

/* One layer's decode step for `batch` rows, in place on the residual stream
 * h [batch][hidden]:
 *   a = rmsnorm(h, attn_norm);  q, k, v = a Wq^T, a Wk^T, a Wv^T;
 *   o = pkv_paged_decode_fused(q, k, v, ...)  (RoPE, append, attention; the
 *       cache arguments as there, head_dim 64);
 *   h += o Wo^T;  m = rmsnorm(h, mlp_norm);  gate_up = m Wgu^T;
 *   act = silu(gate) * up;  h += act Wd^T.
 * scratch: caller-owned device bf16, >= pkv_decode_layer_scratch_elems(...)
 * elements, any contents (the intermediates are left there, except gate_up
 * when the gated launch computes act directly: intermediate % 32 == 0).
 * Q, K and V run as one launch, and the output projection's K-split
 * partials, the residual add and the MLP's RMSNorm are one kernel; the
 * projections are deterministic (partials summed in a fixed order).
 * hidden and intermediate must be multiples of 8.  Every argument, the
 * attention call's included, is checked before anything is launched.
 * All launches go to `stream`. */
int pkv_decode_layer(pkv_bf16* h, const pkv_layer_weights* weights, int hidden, int intermediate,
                     pkv_bf16* scratch, size_t scratch_elems, pkv_bf16* k_pool, pkv_bf16* v_pool,
                     int num_blocks, const int32_t* block_table, int64_t bt_row_stride, int num_slots,
                     int max_blocks_per_seq, const int32_t* slot_ids, const int32_t* context_lens,
                     const int32_t* row_lens_host, int batch, int max_context_len, int n_q_heads,
                     int n_kv_heads, const float* cos_sin, int max_pos, float scale, float eps,
                     void* workspace, size_t workspace_bytes, void* stream);

/* n_layers decode layers in one call, in place on h [batch][hidden]: layer l
 * uses layers[l] and the block table block_table + l * bt_layer_stride (the
 * layer views of a [slots][layers][max_blocks] table: bt_row_stride =
 * layers * max_blocks, bt_layer_stride = max_blocks); every other argument
 * as pkv_decode_layer, shared by the layers (one pool, one scratch, one
 * workspace).  It runs the kernels and roundings of calling
 * pkv_decode_layer for l = 0 .. n_layers - 1, except that between layers
 * the down projection's K-split partials, the residual add and the next
 * layer's attention RMSNorm are one kernel (bit-identical to the separate
 * ones).  Arguments of every layer are checked before anything is launched. */
int pkv_decode_layers(pkv_bf16* h, const pkv_layer_weights* layers, int n_layers, int hidden, int intermediate,
                      pkv_bf16* scratch, size_t scratch_elems, pkv_bf16* k_pool, pkv_bf16* v_pool,
                      int num_blocks, const int32_t* block_table, int64_t bt_row_stride, int64_t bt_layer_stride,
                      int num_slots, int max_blocks_per_seq, const int32_t* slot_ids, const int32_t* context_lens,
                      const int32_t* row_lens_host, int batch, int max_context_len, int n_q_heads,
                      int n_kv_heads, const float* cos_sin, int max_pos, float scale, float eps,
                      void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */

"""paged_kv_attention_17_amd -- paged KV-cache attention for AMD MI355X (gfx950).

The compute lives in libpagedkv.so (HIP kernels behind the C ABI of
include/pagedkv.h); this package is its ctypes binding (``_abi``, re-exported
here under the C names), the in-place build (``build``), a decode-step
driver over the C ABI (``engine``), the continuous-batching
scheduler handle (``Scheduler``) and seeded synthetic workloads
(``workloads``).  Importing the package does not load the library; the first
call does, and raises if it has not been built.
"""
from ._abi import (  # noqa: F401
    PagedKVError, load, header_functions, LIB_PATH,
    pkv_status_str, pkv_abi_version, pkv_rope_table_init, pkv_rope_decode, pkv_paged_kv_append,
    pkv_paged_gather, pkv_hbm_read_probe, pkv_paged_read_probe, pkv_weight_read_probe, pkv_blocks_assign, pkv_blocks_release,
    pkv_block_table_patch,
    pkv_blocks_share, pkv_blocks_assign_shared, pkv_blocks_release_shared, pkv_blocks_copy, pkv_check_block_table,
    pkv_decode_workspace_bytes, pkv_decode_partition_size, pkv_paged_attn_decode, pkv_paged_attn_prefill,
    pkv_decode_step, pkv_decode_workspace_init, pkv_paged_decode_fused, pkv_paged_decode_fused_noalloc,
    pkv_decode_step_staging_bytes, pkv_decode_step_host, pkv_decode_step_device,
    pkv_device_errors, PKV_DEVERR_BAD_BLOCK, PKV_DEVERR_BAD_SLOT, PKV_DEVERR_LONG_CONTEXT, PKV_DEVERR_PREFILL_BLOCK,
    pkv_set_kv_read_policy, pkv_kv_read_policy, PKV_KV_READ_STREAM, PKV_KV_READ_REUSE,
    decode_workspace, Scheduler,
    pkv_rmsnorm, pkv_silu_mul, pkv_linear, pkv_linear_workspace_bytes, pkv_decode_layer,
    pkv_decode_layer_scratch_elems, pkv_decode_layers,
)

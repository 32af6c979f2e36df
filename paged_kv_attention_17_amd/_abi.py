"""ctypes binding of libpagedkv (include/pagedkv.h).

Argument marshalling only: every function here checks the tensors it is
given, turns them into pointers, sizes and the current HIP stream, and calls
the C entry point of the same name.  All arithmetic runs in the library's
HIP kernels; nothing falls back to the host.  Device tensors are torch
tensors on a ROCm device; bf16 tensors may be torch.bfloat16 or int16/uint16
holding the bit patterns.  Host-side calls (block allocation, table checks)
take numpy int32 arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "pagedkv.h")

STATUS = {0: "PKV_OK", 1: "PKV_ERR_NULL", 2: "PKV_ERR_MISALIGNED", 3: "PKV_ERR_UNSUPPORTED",
          4: "PKV_ERR_INVALID_ARG", 5: "PKV_ERR_BAD_BLOCK", 6: "PKV_ERR_CAPACITY", 7: "PKV_ERR_HIP"}
PKV_OK, PKV_ERR_NULL, PKV_ERR_MISALIGNED, PKV_ERR_UNSUPPORTED = 0, 1, 2, 3
PKV_ERR_INVALID_ARG, PKV_ERR_BAD_BLOCK, PKV_ERR_CAPACITY, PKV_ERR_HIP = 4, 5, 6, 7

_lib = None

_p = C.c_void_p
_i = C.c_int
_i64 = C.c_int64
_f = C.c_float
_d = C.c_double
_sz = C.c_size_t
_ip = C.POINTER(C.c_int)

NOALLOC_SCRATCH_BYTES = 16 << 20     # PKV_NOALLOC_SCRATCH_BYTES (include/pagedkv.h)

SIGNATURES = {
    "pkv_status_str": (C.c_char_p, [_i]),
    "pkv_abi_version": (_i, []),
    "pkv_rope_table_init": (_i, [_p, _i, _i, _d, _d, _d, _d, _i, _p]),
    "pkv_rope_decode": (_i, [_p, _p, _p, _i, _i, _i, _i, _p, _i, _p]),
    "pkv_paged_kv_append": (_i, [_p, _p, _i, _p, _p, _p, _i64, _i, _i, _p, _p, _i, _i, _i, _p]),
    "pkv_paged_gather": (_i, [_p, _p, _p, _p, _i, _p, _i64, _i, _i, _i, _i, _i, _p]),
    "pkv_hbm_read_probe": (_i, [_p, _sz, _p, _p]),
    "pkv_weight_read_probe": (_i, [_p, _i, _i, _i, _p, _p]),
    "pkv_paged_read_probe": (_i, [_p, _p, _i, _p, _i64, _i, _i, _p, _p, _i, _i, _i, _p, _p]),
    "pkv_device_errors": (_i, [C.POINTER(C.c_uint32), _i, _p]),
    "pkv_set_kv_read_policy": (_i, [_i]),
    "pkv_kv_read_policy": (_i, []),
    "pkv_blocks_assign": (_i, [_p, _i64, _i, _i, _p, _ip, _p, _p, _i, _p, _p, _ip]),
    "pkv_blocks_release": (_i, [_p, _i64, _i, _i, _i, _p, _ip, _i, _p, _p, _ip]),
    "pkv_block_table_patch": (_i, [_p, _i64, _p, _p, _i, _p]),
    "pkv_blocks_share": (_i, [_p, _i64, _i, _i, _i, _i, _i, _p, _i, _p, _p, _ip]),
    "pkv_blocks_assign_shared": (_i, [_p, _i64, _i, _i, _p, _ip, _p, _i, _p, _p, _i, _p, _p, _ip, _p, _p, _ip]),
    "pkv_blocks_release_shared": (_i, [_p, _i64, _i, _i, _i, _p, _ip, _i, _p, _i, _p, _p, _ip]),
    "pkv_blocks_copy": (_i, [_p, _p, _i, _i, _i, _p, _p, _i, _p]),
    "pkv_check_block_table": (_i, [_p, _i64, _i, _i, _p, _p, _i, _i, _ip, _ip]),
    "pkv_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "pkv_decode_partition_size": (_i, [_i, _i, _i]),
    "pkv_paged_attn_decode": (_i, [_p, _p, _p, _p, _i, _p, _i64, _i, _i, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i,
                                   _p, _sz, _p]),
    "pkv_paged_attn_prefill": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _p, _i64, _i, _i, _i, _i, _i, _i, _i, _i,
                                    _f, _p, _p, _p]),
    "pkv_decode_workspace_init": (_i, [_p, _sz, _p]),
    "pkv_paged_decode_fused": (_i, [_p, _p, _p, _p, _p, _p, _i, _p, _i64, _i, _i, _p, _p, _p, _i, _i, _i, _i, _i, _p,
                                    _i, _f, _i, _p, _sz, _p]),
    "pkv_paged_decode_fused_noalloc": (_i, [_p, _p, _p, _p, _p, _p, _i, _p, _i64, _i, _i, _p, _p, _p, _i, _i, _i,
                                            _i, _i, _p, _i, _f, _i, _p]),
    "pkv_decode_step": (_i, [_i, _p, _p, _p, _p, _p, _p, _i, _p, _p, _i, _i, _p, _ip, _p, _p, _p, _i, _i, _i, _i,
                             _p, _i, _f, _i, _i, _p, _sz, _p]),
    "pkv_decode_step_staging_bytes": (_sz, [_i, _i, _i]),
    "pkv_decode_step_host": (_i, [_i, _p, _i, _i, _p, _ip, _p, _p, _i, _p]),
    "pkv_decode_step_device": (_i, [_i, _p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _p, _i, _i, _i, _i, _p, _i, _f, _p,
                                    _p, _p, _sz, _p]),
    "pkv_sched_create": (_i, [C.POINTER(_p), _i, _i, _i, _i, _i]),
    "pkv_sched_destroy": (_i, [_p]),
    "pkv_sched_submit": (_i, [_p, _i64, _i, _i]),
    "pkv_sched_submit_tokens": (_i, [_p, _i64, _p, _i, _i]),
    "pkv_sched_next": (_i, [_p, _p]),
    "pkv_sched_info": (_i, [_p, _p]),
    "pkv_sched_meta_elems": (_i64, [_i, _i]),
    "pkv_rmsnorm": (_i, [_p, _p, _p, _i, _i, _f, _p]),
    "pkv_silu_mul": (_i, [_p, _p, _i, _i, _p]),
    "pkv_linear_workspace_bytes": (_sz, [_i, _i, _i]),
    "pkv_linear": (_i, [_p, _p, _p, _i, _i, _i, _i, _p, _sz, _p]),
    "pkv_decode_layer_scratch_elems": (_sz, [_i, _i, _i, _i, _i]),
    "pkv_decode_layer": (_i, [_p, _p, _i, _i, _p, _sz, _p, _p, _i, _p, _i64, _i, _i, _p, _p, _p, _i, _i, _i, _i, _p,
                              _i, _f, _f, _p, _sz, _p]),
    "pkv_decode_layers": (_i, [_p, _p, _i, _i, _i, _p, _sz, _p, _p, _i, _p, _i64, _i64, _i, _i, _p, _p, _p, _i, _i, _i,
                               _i, _p, _i, _f, _f, _p, _sz, _p]),
    "pkv_sched_run": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _p, _i, _f, _p, _sz, _p]),
}

_I32P = C.POINTER(C.c_int32)
_I64P = C.POINTER(C.c_int64)


class SchedIter(C.Structure):
    """pkv_sched_iter (include/pagedkv.h)."""
    _fields_ = [("n_tokens", _i), ("n_decode", _i), ("decode_slots", _I32P), ("decode_lens", _I32P),
                ("decode_ids", _I64P), ("n_chunks", _i), ("chunk_slots", _I32P), ("chunk_start", _I32P),
                ("cu_chunk", _I32P), ("chunk_ids", _I64P), ("n_prefill_tokens", _i), ("token_slots", _I32P),
                ("token_pos", _I32P), ("n_patch", _i), ("patch_off", _I32P), ("patch_val", _I32P),
                ("n_done", _i), ("done_ids", _I64P), ("n_admitted", _i), ("admitted_ids", _I64P),
                ("admitted_slots", _I32P), ("admitted_cached", _I32P)]


class SchedState(C.Structure):
    """pkv_sched_state (include/pagedkv.h)."""
    _fields_ = [("num_slots", _i), ("n_layers", _i), ("max_blocks_per_seq", _i), ("num_blocks", _i),
                ("token_budget", _i), ("n_queued", _i), ("n_active", _i), ("n_free", _i), ("n_reserved", _i),
                ("table", _I32P), ("free_list", _I32P), ("meta_elems", _i64), ("n_cache_nodes", _i),
                ("n_cache_blocks", _i), ("cache_blocks", _I32P), ("n_evictable", _i), ("cache_hit_tokens", _i64)]


class PagedKVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = STATUS.get(status, str(status))
        if _lib is not None:
            msg += ": " + _lib.pkv_status_str(status).decode()
        super().__init__(f"{fn} failed with {msg}")


def header_functions() -> list[str]:
    """Names of the functions include/pagedkv.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def load():
    """Load libpagedkv.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with paged_kv_attention_17_amd.build")
    # torch bundles its own libamdhip64 and finds it as "libamdhip64.so"; this
    # library asks for the soname "libamdhip64.so.7".  Loaded first, it would
    # pull in the system runtime and torch would then load a second one, whose
    # streams and allocations this library's kernels cannot use.  Importing
    # torch first makes its runtime the one both resolve to.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != PKV_OK:
        raise PagedKVError(fn, status)


# ------------------------------------------------------------ marshalling --

def _dev_ptr(t, name, dtypes=None):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t.data_ptr()


def _bf16_types():
    import torch
    return (torch.bfloat16, torch.int16, torch.uint16)


def _contig(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _table(bt, name="block_table"):
    """A 2-D table view [rows][max_blocks] whose rows may be strided."""
    import torch
    if bt.dtype != torch.int32 or bt.dim() != 2 or bt.stride(1) != 1:
        raise ValueError(f"{name} must be an int32 [rows, max_blocks] view with unit inner stride")
    return _dev_ptr(bt, name), bt.stride(0), bt.shape[0], bt.shape[1]


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _np_i32(a, name, writable=False):
    if not isinstance(a, np.ndarray) or a.dtype != np.int32:
        raise TypeError(f"{name} must be a numpy int32 array")
    if name in ("free_list", "refcount") and (a.ndim != 1 or not a.flags.c_contiguous):
        raise ValueError(f"{name} must be a contiguous 1-D array")
    if writable and not a.flags.writeable:
        raise ValueError(f"{name} must be writable")
    return a


def _np_table(a, name="bt_host"):
    _np_i32(a, name)
    if a.ndim != 2 or a.strides[1] != 4:
        raise ValueError(f"{name} must be a 2-D int32 view with unit inner stride")
    return a.ctypes.data, a.strides[0] // 4, a.shape[0], a.shape[1]


# -------------------------------------------------------------- entry points --

def pkv_status_str(status: int) -> str:
    return load().pkv_status_str(status).decode()


def pkv_abi_version() -> int:
    return load().pkv_abi_version()


def pkv_rope_table_init(cos_sin, head_dim=64, theta=500000.0, factor=32.0, low_freq_factor=1.0,
                        high_freq_factor=4.0, original_max_pos=8192, stream=None):
    """cos_sin: float32 device tensor [max_pos, head_dim/2, 2]."""
    import torch
    _contig(cos_sin, "cos_sin")
    ptr = _dev_ptr(cos_sin, "cos_sin", (torch.float32,))
    _check("pkv_rope_table_init", load().pkv_rope_table_init(
        ptr, cos_sin.shape[0], head_dim, theta, factor, low_freq_factor, high_freq_factor, original_max_pos,
        _stream(stream)))


def pkv_rope_decode(q, k, positions, cos_sin, stream=None):
    """In-place RoPE on q [T, n_q, 64] and k [T, n_kv, 64] (k may be None)."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (positions, "positions"), (cos_sin, "cos_sin")):
        _contig(t, n)
    T = q.shape[0]
    if positions.shape[0] != T or (k is not None and k.shape[0] != T):
        raise ValueError("q, k and positions disagree on the token count")
    _check("pkv_rope_decode", load().pkv_rope_decode(
        _dev_ptr(q, "q", _bf16_types()), _dev_ptr(k, "k", _bf16_types()),
        _dev_ptr(positions, "positions", (torch.int32,)), T, q.shape[1], 0 if k is None else k.shape[1],
        q.shape[2], _dev_ptr(cos_sin, "cos_sin", (torch.float32,)), cos_sin.shape[0], _stream(stream)))


def pkv_paged_kv_append(k_pool, v_pool, k_new, v_new, block_table, slot_ids, positions, stream=None):
    """Write k_new/v_new [T, n_kv, 64] into their token rows of the pools."""
    import torch
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool"), (k_new, "k_new"), (v_new, "v_new"),
                 (slot_ids, "slot_ids"), (positions, "positions")):
        _contig(t, n)
    if k_pool.shape != v_pool.shape or k_new.shape != v_new.shape:
        raise ValueError("K and V shapes differ")
    if k_pool.shape[2] != k_new.shape[1]:
        raise ValueError("pool and new tokens disagree on n_kv")
    bt, stride, rows, mb = _table(block_table)
    T = k_new.shape[0]
    if slot_ids.shape[0] != T or positions.shape[0] != T:
        raise ValueError("slot_ids / positions must have one entry per token")
    _check("pkv_paged_kv_append", load().pkv_paged_kv_append(
        _dev_ptr(k_pool, "k_pool", _bf16_types()), _dev_ptr(v_pool, "v_pool", _bf16_types()), k_pool.shape[0],
        _dev_ptr(k_new, "k_new", _bf16_types()), _dev_ptr(v_new, "v_new", _bf16_types()), bt, stride, rows, mb,
        _dev_ptr(slot_ids, "slot_ids", (torch.int32,)), _dev_ptr(positions, "positions", (torch.int32,)), T,
        k_new.shape[1], k_new.shape[2], _stream(stream)))


def pkv_paged_gather(k_dense, v_dense, k_pool, v_pool, block_table, slot, context_len, stream=None):
    for t, n in ((k_dense, "k_dense"), (v_dense, "v_dense"), (k_pool, "k_pool"), (v_pool, "v_pool")):
        _contig(t, n)
    bt, stride, rows, mb = _table(block_table)
    if not 0 <= slot < rows:
        raise ValueError("slot outside the table")
    if k_dense.shape[0] < context_len or v_dense.shape[0] < context_len:
        raise ValueError("dense buffers shorter than context_len")
    _check("pkv_paged_gather", load().pkv_paged_gather(
        _dev_ptr(k_dense, "k_dense", _bf16_types()), _dev_ptr(v_dense, "v_dense", _bf16_types()),
        _dev_ptr(k_pool, "k_pool", _bf16_types()), _dev_ptr(v_pool, "v_pool", _bf16_types()), k_pool.shape[0],
        bt + 0, stride, mb, slot, context_len, k_pool.shape[2], k_pool.shape[3], _stream(stream)))


def pkv_weight_read_probe(w, sink, k_parts=1, stream=None):
    """Read weight matrix `w` [n][k] (bf16, contiguous) once in the projection
    kernels' access pattern, K split over `k_parts` waves per 16-row block
    (diagnostic weight-stream rate); `sink` as for pkv_hbm_read_probe."""
    _contig(w, "w")
    n, k = w.shape
    _check("pkv_weight_read_probe", load().pkv_weight_read_probe(
        _dev_ptr(w, "w", _bf16_types()), n, k, k_parts, _dev_ptr(sink, "sink"), _stream(stream)))


def pkv_hbm_read_probe(buf, sink, stream=None):
    """Read the whole of device tensor `buf` once (diagnostic HBM read rate);
    `sink` is a device int32/uint32 tensor of at least one element."""
    _contig(buf, "buf")
    _check("pkv_hbm_read_probe", load().pkv_hbm_read_probe(
        _dev_ptr(buf, "buf"), buf.numel() * buf.element_size(), _dev_ptr(sink, "sink"), _stream(stream)))


PKV_DEVERR_BAD_BLOCK, PKV_DEVERR_BAD_SLOT, PKV_DEVERR_LONG_CONTEXT, PKV_DEVERR_PREFILL_BLOCK = 1, 2, 4, 8


def pkv_device_errors(clear=True, stream=None):
    """The current device's error flags (PKV_DEVERR_* bits) after the work
    enqueued on `stream` so far; cleared unless clear=False."""
    flags = C.c_uint32(0)
    _check("pkv_device_errors", load().pkv_device_errors(C.byref(flags), 1 if clear else 0, _stream(stream)))
    return flags.value


PKV_KV_READ_STREAM, PKV_KV_READ_REUSE = 1, 2


def pkv_set_kv_read_policy(policy):
    """Cache policy of the decode calls' K/V reads, process-wide:
    PKV_KV_READ_STREAM (non-temporal, the default) or PKV_KV_READ_REUSE
    (cached, for tables whose rows share blocks).  Speed only, never
    results."""
    _check("pkv_set_kv_read_policy", load().pkv_set_kv_read_policy(int(policy)))


def pkv_kv_read_policy():
    """The current K/V read policy (PKV_KV_READ_STREAM or PKV_KV_READ_REUSE)."""
    return int(load().pkv_kv_read_policy())


def pkv_paged_read_probe(k_pool, v_pool, block_table, slot_ids, row_lens_host, sink, stream=None):
    """The streaming decode kernel's K/V reads alone (diagnostic): pools
    [NB, 16, n_kv, 64]; block_table [rows, max_blocks] (row-strided view ok);
    slot_ids [B] int32 or None; row_lens_host numpy lengths per batch row;
    sink a device int32/uint32 tensor of at least one element."""
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool"), (slot_ids, "slot_ids"), (sink, "sink")):
        _contig(t, n)
    if k_pool.shape != v_pool.shape:
        raise ValueError("shape mismatch")
    bt, stride, rows, mb = _table(block_table)
    rl = np.ascontiguousarray(row_lens_host, dtype=np.int32)
    B = len(rl)
    if slot_ids is not None and slot_ids.shape[0] != B:
        raise ValueError("slot_ids must have one entry per batch row")
    _check("pkv_paged_read_probe", load().pkv_paged_read_probe(
        _dev_ptr(k_pool, "k_pool", _bf16_types()), _dev_ptr(v_pool, "v_pool", _bf16_types()), k_pool.shape[0], bt,
        stride, rows, mb, None if slot_ids is None else _dev_ptr(slot_ids, "slot_ids"), rl.ctypes.data, B,
        k_pool.shape[2], k_pool.shape[3], _dev_ptr(sink, "sink"), _stream(stream)))


def pkv_blocks_assign(bt_host, free_list, n_free, slot_ids, positions):
    """Host allocation for one step.  Returns (n_free, patch_offsets, patch_values)."""
    ptr, stride, rows, mb = _np_table(bt_host)
    _np_i32(free_list, "free_list", writable=True)
    slot_ids = np.ascontiguousarray(slot_ids, dtype=np.int32)
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    n = len(slot_ids)
    if len(positions) != n:
        raise ValueError("slot_ids / positions lengths differ")
    if not 0 <= n_free <= len(free_list):
        raise ValueError("n_free outside the free list")
    off = np.zeros(max(n, 1), np.int32)
    val = np.zeros(max(n, 1), np.int32)
    nf = C.c_int(n_free)
    npch = C.c_int(0)
    _check("pkv_blocks_assign", load().pkv_blocks_assign(
        ptr, stride, rows, mb, free_list.ctypes.data, C.byref(nf), slot_ids.ctypes.data, positions.ctypes.data, n,
        off.ctypes.data, val.ctypes.data, C.byref(npch)))
    return nf.value, off[:npch.value].copy(), val[:npch.value].copy()


def pkv_blocks_release(bt_host, slot, free_list, n_free):
    """Free table row `slot`.  Returns (n_free, patch_offsets, patch_values)."""
    ptr, stride, rows, mb = _np_table(bt_host)
    _np_i32(free_list, "free_list", writable=True)
    if not 0 <= n_free <= len(free_list):
        raise ValueError("n_free outside the free list")
    off = np.zeros(max(mb, 1), np.int32)
    val = np.zeros(max(mb, 1), np.int32)
    nf = C.c_int(n_free)
    npch = C.c_int(0)
    _check("pkv_blocks_release", load().pkv_blocks_release(
        ptr, stride, rows, mb, slot, free_list.ctypes.data, C.byref(nf), len(free_list), off.ctypes.data,
        val.ctypes.data, C.byref(npch)))
    return nf.value, off[:npch.value].copy(), val[:npch.value].copy()


def pkv_blocks_share(bt_host, src_slot, dst_slot, n_tokens, refcount):
    """Row dst_slot lists row src_slot's blocks for tokens 0..n_tokens-1
    (counts in `refcount` grow).  Returns (patch_offsets, patch_values)."""
    ptr, stride, rows, mb = _np_table(bt_host)
    _np_i32(refcount, "refcount", writable=True)
    nb = -(-int(n_tokens) // 16)
    off = np.zeros(max(nb, 1), np.int32)
    val = np.zeros(max(nb, 1), np.int32)
    npch = C.c_int(0)
    _check("pkv_blocks_share", load().pkv_blocks_share(
        ptr, stride, rows, mb, src_slot, dst_slot, n_tokens, refcount.ctypes.data, len(refcount),
        off.ctypes.data, val.ctypes.data, C.byref(npch)))
    return off[:npch.value].copy(), val[:npch.value].copy()


def pkv_blocks_assign_shared(bt_host, free_list, n_free, refcount, slot_ids, positions):
    """Host allocation with shared blocks (copy on write).  Returns
    (n_free, patch_offsets, patch_values, copy_src, copy_dst)."""
    ptr, stride, rows, mb = _np_table(bt_host)
    _np_i32(free_list, "free_list", writable=True)
    _np_i32(refcount, "refcount", writable=True)
    slot_ids = np.ascontiguousarray(slot_ids, dtype=np.int32)
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    n = len(slot_ids)
    if len(positions) != n:
        raise ValueError("slot_ids / positions lengths differ")
    if not 0 <= n_free <= len(free_list):
        raise ValueError("n_free outside the free list")
    off, val, cs, cd = (np.zeros(max(n, 1), np.int32) for _ in range(4))
    nf, npch, ncp = C.c_int(n_free), C.c_int(0), C.c_int(0)
    _check("pkv_blocks_assign_shared", load().pkv_blocks_assign_shared(
        ptr, stride, rows, mb, free_list.ctypes.data, C.byref(nf), refcount.ctypes.data, len(refcount),
        slot_ids.ctypes.data, positions.ctypes.data, n, off.ctypes.data, val.ctypes.data, C.byref(npch),
        cs.ctypes.data, cd.ctypes.data, C.byref(ncp)))
    k, c = npch.value, ncp.value
    return nf.value, off[:k].copy(), val[:k].copy(), cs[:c].copy(), cd[:c].copy()


def pkv_blocks_release_shared(bt_host, slot, free_list, n_free, refcount):
    """Drop row `slot`'s references; blocks whose count reaches 0 are freed.
    Returns (n_free, patch_offsets, patch_values)."""
    ptr, stride, rows, mb = _np_table(bt_host)
    _np_i32(free_list, "free_list", writable=True)
    _np_i32(refcount, "refcount", writable=True)
    if not 0 <= n_free <= len(free_list):
        raise ValueError("n_free outside the free list")
    off = np.zeros(max(mb, 1), np.int32)
    val = np.zeros(max(mb, 1), np.int32)
    nf, npch = C.c_int(n_free), C.c_int(0)
    _check("pkv_blocks_release_shared", load().pkv_blocks_release_shared(
        ptr, stride, rows, mb, slot, free_list.ctypes.data, C.byref(nf), len(free_list), refcount.ctypes.data,
        len(refcount), off.ctypes.data, val.ctypes.data, C.byref(npch)))
    return nf.value, off[:npch.value].copy(), val[:npch.value].copy()


def pkv_blocks_copy(k_pool, v_pool, copy_src, copy_dst, stream=None):
    """k_pool[dst[i]] = k_pool[src[i]] and the same for v_pool, whole blocks
    (pools [num_blocks][16][n_kv][64], bf16); id lists are host arrays."""
    import torch
    for t, nm in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        _contig(t, nm)
        _dev_ptr(t, nm, _bf16_types())
    if k_pool.shape != v_pool.shape or k_pool.dim() != 4 or k_pool.shape[1] != 16:
        raise ValueError("pools must both be [num_blocks][16][n_kv][head_dim]")
    src = np.ascontiguousarray(copy_src, dtype=np.int32)
    dst = np.ascontiguousarray(copy_dst, dtype=np.int32)
    if src.shape != dst.shape or src.ndim != 1:
        raise ValueError("copy_src / copy_dst must be 1-D of one length")
    st = _stream(stream)
    _check("pkv_blocks_copy", load().pkv_blocks_copy(
        k_pool.data_ptr(), v_pool.data_ptr(), k_pool.shape[0], k_pool.shape[2], k_pool.shape[3],
        src.ctypes.data, dst.ctypes.data, len(src), st))


def pkv_block_table_patch(bt_dev, patch_offsets, patch_values, stream=None):
    """bt_dev.view(-1)[patch_offsets[i]] = patch_values[i] on the device."""
    import torch
    _contig(bt_dev, "bt_dev")
    off = np.ascontiguousarray(patch_offsets, dtype=np.int32)
    val = np.ascontiguousarray(patch_values, dtype=np.int32)
    if len(off) != len(val):
        raise ValueError("patch arrays differ in length")
    _check("pkv_block_table_patch", load().pkv_block_table_patch(
        _dev_ptr(bt_dev, "bt_dev", (torch.int32,)), bt_dev.numel(), off.ctypes.data, val.ctypes.data, len(off),
        _stream(stream)))


def pkv_check_block_table(bt_host, slot_ids, context_lens, num_blocks):
    """Host validation.  Returns (status, bad_row, bad_idx); never raises for BAD_BLOCK."""
    ptr, stride, rows, mb = _np_table(bt_host)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    if len(ctx) < rows:
        raise ValueError("context_lens must have an entry per table row")
    sid = None if slot_ids is None else np.ascontiguousarray(slot_ids, dtype=np.int32)
    batch = rows if sid is None else len(sid)
    br, bi = C.c_int(0), C.c_int(0)
    st = load().pkv_check_block_table(ptr, stride, rows, mb, None if sid is None else sid.ctypes.data,
                                      ctx.ctypes.data, batch, num_blocks, C.byref(br), C.byref(bi))
    if st not in (PKV_OK, PKV_ERR_BAD_BLOCK):
        _check("pkv_check_block_table", st)
    return st, br.value, bi.value


def pkv_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_context_len, partition_size=0):
    return load().pkv_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_context_len,
                                             partition_size)


def pkv_decode_partition_size(batch, n_kv_heads, max_context_len):
    return load().pkv_decode_partition_size(batch, n_kv_heads, max_context_len)


def pkv_decode_workspace_init(workspace, stream=None):
    """Zero a decode workspace (uint8 device tensor) before its first use."""
    _contig(workspace, "workspace")
    _check("pkv_decode_workspace_init", load().pkv_decode_workspace_init(
        _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))


def decode_workspace(batch, n_q_heads, n_kv_heads, max_context_len, partition_size=0, device="cuda", stream=None):
    """Allocate and zero a decode workspace of the size the library asks for."""
    import torch
    n = pkv_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, 64, max_context_len, partition_size)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    pkv_decode_workspace_init(ws, stream=stream)
    return ws


def _row_lens(row_lens_host, B):
    if row_lens_host is None:
        return None, None
    a = np.ascontiguousarray(row_lens_host, dtype=np.int32)
    if a.shape != (B,):
        raise ValueError("row_lens_host must hold one length per batch row")
    return a, a.ctypes.data


def pkv_paged_decode_fused(out, q, k_new, v_new, k_pool, v_pool, block_table, slot_ids, context_lens,
                           max_context_len, cos_sin, scale, partition_size=0, workspace=None, stream=None,
                           row_lens_host=None):
    """RoPE + append + attention for one layer in one launch (q, k_new, v_new not modified).
    row_lens_host: optional numpy copy of each batch row's length (enables the compact schedule)."""
    import torch
    for t, n in ((out, "out"), (q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_pool, "k_pool"), (v_pool, "v_pool"),
                 (slot_ids, "slot_ids"), (context_lens, "context_lens"), (workspace, "workspace"),
                 (cos_sin, "cos_sin")):
        _contig(t, n)
    B, n_q, d = q.shape
    if out.shape != q.shape or k_pool.shape != v_pool.shape or k_new.shape != v_new.shape:
        raise ValueError("shape mismatch")
    if k_new.shape[0] != B or k_new.shape[1] != k_pool.shape[2]:
        raise ValueError("k_new must be [batch, n_kv, 64]")
    bt, stride, rows, mb = _table(block_table)
    if context_lens.shape[0] < rows:
        raise ValueError("context_lens must have an entry per table row")
    if slot_ids is not None and slot_ids.shape[0] != B:
        raise ValueError("slot_ids must have one entry per batch row")
    if slot_ids is None and B > rows:
        raise ValueError("batch larger than the table without slot_ids")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev_ptr(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    keep, rl = _row_lens(row_lens_host, B)
    _check("pkv_paged_decode_fused", load().pkv_paged_decode_fused(
        _dev_ptr(out, "out", _bf16_types()), _dev_ptr(q, "q", _bf16_types()),
        _dev_ptr(k_new, "k_new", _bf16_types()), _dev_ptr(v_new, "v_new", _bf16_types()),
        _dev_ptr(k_pool, "k_pool", _bf16_types()), _dev_ptr(v_pool, "v_pool", _bf16_types()), k_pool.shape[0],
        bt, stride, rows, mb, _dev_ptr(slot_ids, "slot_ids", (torch.int32,)),
        _dev_ptr(context_lens, "context_lens", (torch.int32,)), rl, B, max_context_len, n_q, k_pool.shape[2], d,
        _dev_ptr(cos_sin, "cos_sin", (torch.float32,)), cos_sin.shape[0], float(scale), partition_size, ws_ptr,
        ws_bytes, _stream(stream)))


def pkv_paged_decode_fused_noalloc(out, q, k_new, v_new, k_pool, v_pool, block_table, slot_ids, context_lens,
                                   max_context_len, cos_sin, scale, partition_size=0, stream=None,
                                   row_lens_host=None):
    """pkv_paged_decode_fused with the library's own device scratch array in
    place of a workspace (the call allocates nothing; calls overlapping on one
    GPU must be serialised by the caller)."""
    import torch
    for t, n in ((out, "out"), (q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_pool, "k_pool"), (v_pool, "v_pool"),
                 (slot_ids, "slot_ids"), (context_lens, "context_lens"), (cos_sin, "cos_sin")):
        _contig(t, n)
    B, n_q, d = q.shape
    if out.shape != q.shape or k_pool.shape != v_pool.shape or k_new.shape != v_new.shape:
        raise ValueError("shape mismatch")
    if k_new.shape[0] != B or k_new.shape[1] != k_pool.shape[2]:
        raise ValueError("k_new must be [batch, n_kv, 64]")
    bt, stride, rows, mb = _table(block_table)
    if context_lens.shape[0] < rows:
        raise ValueError("context_lens must have an entry per table row")
    if slot_ids is not None and slot_ids.shape[0] != B:
        raise ValueError("slot_ids must have one entry per batch row")
    if slot_ids is None and B > rows:
        raise ValueError("batch larger than the table without slot_ids")
    keep, rl = _row_lens(row_lens_host, B)
    _check("pkv_paged_decode_fused_noalloc", load().pkv_paged_decode_fused_noalloc(
        _dev_ptr(out, "out", _bf16_types()), _dev_ptr(q, "q", _bf16_types()),
        _dev_ptr(k_new, "k_new", _bf16_types()), _dev_ptr(v_new, "v_new", _bf16_types()),
        _dev_ptr(k_pool, "k_pool", _bf16_types()), _dev_ptr(v_pool, "v_pool", _bf16_types()), k_pool.shape[0],
        bt, stride, rows, mb, _dev_ptr(slot_ids, "slot_ids", (torch.int32,)),
        _dev_ptr(context_lens, "context_lens", (torch.int32,)), rl, B, max_context_len, n_q, k_pool.shape[2], d,
        _dev_ptr(cos_sin, "cos_sin", (torch.float32,)), cos_sin.shape[0], float(scale), partition_size,
        _stream(stream)))


def pkv_paged_attn_decode(out, q, k_pool, v_pool, block_table, slot_ids, context_lens, max_context_len,
                          scale, partition_size=0, workspace=None, stream=None, row_lens_host=None):
    """out/q [B, n_q, 64]; pools [NB, 16, n_kv, 64]; block_table [rows, max_blocks] (row-strided view ok);
    slot_ids [B] int32 or None; context_lens [rows] int32; workspace: zeroed uint8 tensor or None."""
    import torch
    for t, n in ((out, "out"), (q, "q"), (k_pool, "k_pool"), (v_pool, "v_pool"), (slot_ids, "slot_ids"),
                 (context_lens, "context_lens"), (workspace, "workspace")):
        _contig(t, n)
    B, n_q, d = q.shape
    if out.shape != q.shape or k_pool.shape != v_pool.shape:
        raise ValueError("shape mismatch")
    bt, stride, rows, mb = _table(block_table)
    if context_lens.shape[0] < rows:
        raise ValueError("context_lens must have an entry per table row")
    if slot_ids is not None and slot_ids.shape[0] != B:
        raise ValueError("slot_ids must have one entry per batch row")
    if slot_ids is None and B > rows:
        raise ValueError("batch larger than the table without slot_ids")
    ws_ptr = None
    ws_bytes = 0
    if workspace is not None:
        ws_ptr = _dev_ptr(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    keep, rl = _row_lens(row_lens_host, B)
    _check("pkv_paged_attn_decode", load().pkv_paged_attn_decode(
        _dev_ptr(out, "out", _bf16_types()), _dev_ptr(q, "q", _bf16_types()),
        _dev_ptr(k_pool, "k_pool", _bf16_types()), _dev_ptr(v_pool, "v_pool", _bf16_types()), k_pool.shape[0],
        bt, stride, rows, mb, _dev_ptr(slot_ids, "slot_ids", (torch.int32,)),
        _dev_ptr(context_lens, "context_lens", (torch.int32,)), rl, B, max_context_len, n_q, k_pool.shape[2], d,
        float(scale), partition_size, ws_ptr, ws_bytes, _stream(stream)))


def pkv_paged_attn_prefill(out, q, cu_q_lens, q_start_pos, slot_ids, k_pool, v_pool, block_table, max_q_len,
                           scale, stream=None, cu_q_lens_host=None, q_start_host=None):
    """q/out [total_q, n_q, 64]; cu_q_lens [S+1]; q_start_pos [S]; slot_ids [S] or None.
    cu_q_lens_host / q_start_host: optional numpy copies (both or neither) that
    let the library launch only real work, heaviest first."""
    import torch
    for t, n in ((out, "out"), (q, "q"), (cu_q_lens, "cu_q_lens"), (q_start_pos, "q_start_pos"),
                 (slot_ids, "slot_ids"), (k_pool, "k_pool"), (v_pool, "v_pool")):
        _contig(t, n)
    if out.shape != q.shape or k_pool.shape != v_pool.shape:
        raise ValueError("shape mismatch")
    S = q_start_pos.shape[0]
    if cu_q_lens.shape[0] != S + 1 or (slot_ids is not None and slot_ids.shape[0] != S):
        raise ValueError("per-sequence arrays disagree")
    bt, stride, rows, mb = _table(block_table)
    if (cu_q_lens_host is None) != (q_start_host is None):
        raise ValueError("cu_q_lens_host and q_start_host go together")
    cuh = qsh = None
    if cu_q_lens_host is not None:
        cuh = np.ascontiguousarray(cu_q_lens_host, dtype=np.int32)
        qsh = np.ascontiguousarray(q_start_host, dtype=np.int32)
        if cuh.shape != (S + 1,) or qsh.shape != (S,):
            raise ValueError("host copies must match cu_q_lens / q_start_pos")
    _check("pkv_paged_attn_prefill", load().pkv_paged_attn_prefill(
        _dev_ptr(out, "out", _bf16_types()), _dev_ptr(q, "q", _bf16_types()),
        _dev_ptr(cu_q_lens, "cu_q_lens", (torch.int32,)), _dev_ptr(q_start_pos, "q_start_pos", (torch.int32,)),
        _dev_ptr(slot_ids, "slot_ids", (torch.int32,)), _dev_ptr(k_pool, "k_pool", _bf16_types()),
        _dev_ptr(v_pool, "v_pool", _bf16_types()), k_pool.shape[0], bt, stride, rows, mb, S, q.shape[0], max_q_len,
        q.shape[1], k_pool.shape[2], q.shape[2], float(scale), None if cuh is None else cuh.ctypes.data,
        None if qsh is None else qsh.ctypes.data, _stream(stream)))


def pkv_decode_step(q, k, v, out, k_pool, v_pool, bt_host, bt_dev, free_list, n_free, cached_lens, meta_dev,
                    slot_ids, cos_sin, scale, max_context_len, partition_size=0, workspace=None, stream=None):
    """One decode step over all layers (see pkv_decode_step in pagedkv.h).

    q/out [L, B, n_q, 64], k/v [L, B, n_kv, 64] device bf16 (or lists of L
    such tensors); bt_host numpy int32 [slots, L, max_blocks] (updated in
    place) with bt_dev its contiguous device copy; free_list numpy int32
    (popped from index n_free - 1 down); cached_lens numpy int32 [slots]
    (advanced in place); meta_dev device int32 [slots + 2B].  Returns n_free.
    """
    import torch
    L = len(q)
    B = q[0].shape[0]
    _np_i32(bt_host, "bt_host", writable=True)
    _np_i32(free_list, "free_list", writable=True)
    _np_i32(cached_lens, "cached_lens", writable=True)
    if bt_host.ndim != 3 or not bt_host.flags.c_contiguous or bt_host.shape[1] != L:
        raise ValueError("bt_host must be a contiguous [slots, layers, max_blocks] array")
    if not bt_dev.is_contiguous() or tuple(bt_dev.shape) != bt_host.shape or bt_dev.dtype != torch.int32:
        raise ValueError("bt_dev must be the contiguous device copy of bt_host")
    slots, _, mb = bt_host.shape
    sid = np.ascontiguousarray(slot_ids, dtype=np.int32)
    if len(sid) != B or meta_dev.numel() != slots + 2 * B or not meta_dev.is_contiguous():
        raise ValueError("meta_dev must be int32 [slots + 2 * batch]")
    if len(cached_lens) != slots or not 0 <= n_free <= len(free_list):
        raise ValueError("cached_lens / n_free inconsistent")
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        _contig(t, n)
    ptrs = []
    for arr, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        if len(arr) != L:
            raise ValueError(f"{name} needs one tensor per layer")
        for t in arr:
            _contig(t, name)
        ptrs.append((C.c_void_p * L)(*[_dev_ptr(t, name, _bf16_types()) for t in arr]))
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _contig(workspace, "workspace")
        ws_ptr = _dev_ptr(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    nf = C.c_int(n_free)
    _check("pkv_decode_step", load().pkv_decode_step(
        L, ptrs[0], ptrs[1], ptrs[2], ptrs[3], _dev_ptr(k_pool, "k_pool", _bf16_types()),
        _dev_ptr(v_pool, "v_pool", _bf16_types()), k_pool.shape[0], bt_host.ctypes.data,
        _dev_ptr(bt_dev, "bt_dev"), slots, mb, free_list.ctypes.data, C.byref(nf), cached_lens.ctypes.data,
        _dev_ptr(meta_dev, "meta_dev", (torch.int32,)), sid.ctypes.data, B, q[0].shape[1], k_pool.shape[2],
        q[0].shape[2], _dev_ptr(cos_sin, "cos_sin", (torch.float32,)), cos_sin.shape[0], float(scale),
        max_context_len, partition_size, ws_ptr, ws_bytes, _stream(stream)))
    return nf.value


def pkv_decode_step_staging_bytes(n_layers, batch, num_slots):
    """Bytes of the two-half step's staging area (0: sizes not served)."""
    return load().pkv_decode_step_staging_bytes(n_layers, batch, num_slots)


def _host_buffer(buf, name, nbytes):
    """Address of a host buffer: a CPU torch tensor (pinned or not) or a
    writable numpy array, contiguous, at least nbytes long."""
    import torch
    if isinstance(buf, torch.Tensor):
        if buf.is_cuda or not buf.is_contiguous():
            raise ValueError(f"{name} must be a contiguous host tensor")
        have, ptr = buf.numel() * buf.element_size(), buf.data_ptr()
    elif isinstance(buf, np.ndarray):
        if not buf.flags.c_contiguous or not buf.flags.writeable:
            raise ValueError(f"{name} must be a contiguous writable array")
        have, ptr = buf.nbytes, buf.ctypes.data
    else:
        raise TypeError(f"{name} must be a host tensor or numpy array")
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, needs {nbytes}")
    return ptr


def pkv_decode_step_host(bt_host, free_list, n_free, cached_lens, slot_ids, staging_host):
    """Host half of the two-half decode step (see pkv_decode_step_host in
    pagedkv.h): allocation and the step's staging area.  bt_host [slots, L,
    max_blocks], free_list and cached_lens are numpy int32 updated in place;
    staging_host a host buffer of pkv_decode_step_staging_bytes.  Returns
    n_free; raises PagedKVError (status PKV_ERR_UNSUPPORTED: rows the replayed
    launches do not serve, nothing changed)."""
    _np_i32(bt_host, "bt_host", writable=True)
    _np_i32(free_list, "free_list", writable=True)
    _np_i32(cached_lens, "cached_lens", writable=True)
    if bt_host.ndim != 3 or not bt_host.flags.c_contiguous:
        raise ValueError("bt_host must be a contiguous [slots, layers, max_blocks] array")
    slots, L, mb = bt_host.shape
    sid = np.ascontiguousarray(slot_ids, dtype=np.int32)
    if len(cached_lens) != slots or not 0 <= n_free <= len(free_list):
        raise ValueError("cached_lens / n_free inconsistent")
    need = pkv_decode_step_staging_bytes(L, len(sid), slots)
    if need == 0:
        raise ValueError("layers, batch or slots outside what the two-half step serves")
    ptr = _host_buffer(staging_host, "staging_host", need)
    nf = C.c_int(n_free)
    _check("pkv_decode_step_host", load().pkv_decode_step_host(
        L, bt_host.ctypes.data, slots, mb, free_list.ctypes.data, C.byref(nf), cached_lens.ctypes.data,
        sid.ctypes.data, len(sid), ptr))
    return nf.value


def pkv_decode_step_device(q, k, v, out, k_pool, v_pool, bt_dev, meta_dev, cos_sin, scale, staging_host,
                           staging_dev, workspace, stream=None):
    """Device half of the two-half decode step (see pkv_decode_step_device in
    pagedkv.h); enqueues only, so it may be captured in a graph.  q/out
    [L, B, n_q, 64], k/v [L, B, n_kv, 64] device bf16 (or lists of L tensors);
    bt_dev device int32 [slots, L, max_blocks]; meta_dev device int32
    [slots + 2B]; staging_host the host staging area the host half wrote and
    staging_dev its device copy (the caller copies it on the same stream
    first); workspace with two record regions."""
    import torch
    L = len(q)
    B = q[0].shape[0]
    if bt_dev.ndim != 3 or not bt_dev.is_contiguous() or bt_dev.dtype != torch.int32 or bt_dev.shape[1] != L:
        raise ValueError("bt_dev must be a contiguous int32 [slots, layers, max_blocks] device tensor")
    slots, _, mb = bt_dev.shape
    if meta_dev.numel() != slots + 2 * B or not meta_dev.is_contiguous():
        raise ValueError("meta_dev must be int32 [slots + 2 * batch]")
    need = pkv_decode_step_staging_bytes(L, B, slots)
    if need == 0:
        raise ValueError("layers, batch or slots outside what the two-half step serves")
    sh = _host_buffer(staging_host, "staging_host", need)
    _contig(staging_dev, "staging_dev")
    if staging_dev.numel() * staging_dev.element_size() < need:
        raise ValueError(f"staging_dev needs {need} bytes")
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool"), (workspace, "workspace")):
        _contig(t, n)
    ptrs = []
    for arr, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        if len(arr) != L:
            raise ValueError(f"{name} needs one tensor per layer")
        for t in arr:
            _contig(t, name)
        ptrs.append((C.c_void_p * L)(*[_dev_ptr(t, name, _bf16_types()) for t in arr]))
    _check("pkv_decode_step_device", load().pkv_decode_step_device(
        L, ptrs[0], ptrs[1], ptrs[2], ptrs[3], _dev_ptr(k_pool, "k_pool", _bf16_types()),
        _dev_ptr(v_pool, "v_pool", _bf16_types()), k_pool.shape[0], _dev_ptr(bt_dev, "bt_dev", (torch.int32,)),
        slots, mb, _dev_ptr(meta_dev, "meta_dev", (torch.int32,)), B, q[0].shape[1], k_pool.shape[2],
        q[0].shape[2], _dev_ptr(cos_sin, "cos_sin", (torch.float32,)), cos_sin.shape[0], float(scale), sh,
        _dev_ptr(staging_dev, "staging_dev"), _dev_ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


# ------------------------------------------------------ continuous batching --

def _arr(ptr, n, dtype):
    """Copy n elements from a C array into a numpy array."""
    a = np.empty(n, dtype)
    if n:
        C.memmove(a.ctypes.data, ptr, a.nbytes)
    return a


class Scheduler:
    """Handle of a pkv_sched (continuous batching; see pkv_sched_* in
    pagedkv.h).  ``next()`` returns the iteration as a dict of numpy copies
    and keeps the C struct for ``run``."""

    def __init__(self, num_slots, n_layers, max_blocks_per_seq, num_blocks, token_budget):
        h = C.c_void_p()
        _check("pkv_sched_create", load().pkv_sched_create(C.byref(h), num_slots, n_layers, max_blocks_per_seq,
                                                           num_blocks, token_budget))
        self._h = h
        self._it = SchedIter()
        self._sizes = (num_slots, n_layers, max_blocks_per_seq, num_blocks,
                       load().pkv_sched_meta_elems(num_slots, token_budget))

    def close(self):
        if self._h:
            load().pkv_sched_destroy(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def submit(self, request_id, prompt_len, max_new_tokens, tokens=None):
        """Queue a request; with `tokens` (its prompt's ids, int32) it takes
        part in prefix caching (pkv_sched_submit_tokens)."""
        if tokens is None:
            _check("pkv_sched_submit", load().pkv_sched_submit(self._h, int(request_id), int(prompt_len),
                                                               int(max_new_tokens)))
            return
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        if t.shape != (int(prompt_len),):
            raise ValueError("tokens must hold prompt_len ids")
        _check("pkv_sched_submit_tokens", load().pkv_sched_submit_tokens(
            self._h, int(request_id), t.ctypes.data, int(prompt_len), int(max_new_tokens)))

    def next(self):
        _check("pkv_sched_next", load().pkv_sched_next(self._h, C.byref(self._it)))
        it = self._it
        return dict(
            n_tokens=it.n_tokens, n_decode=it.n_decode,
            decode_slots=_arr(it.decode_slots, it.n_decode, np.int32),
            decode_lens=_arr(it.decode_lens, it.n_decode, np.int32),
            decode_ids=_arr(it.decode_ids, it.n_decode, np.int64),
            chunk_slots=_arr(it.chunk_slots, it.n_chunks, np.int32),
            chunk_start=_arr(it.chunk_start, it.n_chunks, np.int32),
            cu_chunk=_arr(it.cu_chunk, it.n_chunks + 1, np.int32),
            chunk_ids=_arr(it.chunk_ids, it.n_chunks, np.int64),
            token_slots=_arr(it.token_slots, it.n_prefill_tokens, np.int32),
            token_pos=_arr(it.token_pos, it.n_prefill_tokens, np.int32),
            patch_off=_arr(it.patch_off, it.n_patch, np.int32),
            patch_val=_arr(it.patch_val, it.n_patch, np.int32),
            done_ids=_arr(it.done_ids, it.n_done, np.int64),
            admitted_ids=_arr(it.admitted_ids, it.n_admitted, np.int64),
            admitted_slots=_arr(it.admitted_slots, it.n_admitted, np.int32),
            admitted_cached=_arr(it.admitted_cached, it.n_admitted, np.int32))

    def info(self):
        st = SchedState()
        _check("pkv_sched_info", load().pkv_sched_info(self._h, C.byref(st)))
        n_tab = st.num_slots * st.n_layers * st.max_blocks_per_seq
        return dict(num_slots=st.num_slots, n_layers=st.n_layers, max_blocks_per_seq=st.max_blocks_per_seq,
                    num_blocks=st.num_blocks, token_budget=st.token_budget, n_queued=st.n_queued,
                    n_active=st.n_active, n_free=st.n_free, n_reserved=st.n_reserved,
                    table=_arr(st.table, n_tab, np.int32).reshape(st.num_slots, st.n_layers,
                                                                  st.max_blocks_per_seq),
                    free_list=_arr(st.free_list, st.n_free, np.int32), meta_elems=st.meta_elems,
                    n_cache_nodes=st.n_cache_nodes, cache_blocks=_arr(st.cache_blocks, st.n_cache_blocks, np.int32),
                    n_evictable=st.n_evictable, cache_hit_tokens=st.cache_hit_tokens)

    def run(self, q, k, v, out, k_pool, v_pool, bt_dev, meta_dev, cos_sin, scale, workspace, stream=None):
        """Run the last planned iteration (pkv_sched_run).  q/k/v/out: one
        device bf16 tensor per layer, [budget rows, heads, 64]; bt_dev:
        contiguous device int32 [slots, layers, max_blocks]; meta_dev: device
        int32 [meta_elems]."""
        import torch
        L = len(q)
        ptrs = []
        for arr, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
            if len(arr) != L:
                raise ValueError(f"{name} needs one tensor per layer")
            for t in arr:
                _contig(t, name)
                if t.shape[0] < self._it.n_tokens:
                    raise ValueError(f"{name} has fewer rows than the iteration's tokens")
            ptrs.append((C.c_void_p * L)(*[_dev_ptr(t, name, _bf16_types()) for t in arr]))
        for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool"), (bt_dev, "bt_dev"), (meta_dev, "meta_dev"),
                     (cos_sin, "cos_sin"), (workspace, "workspace")):
            _contig(t, n)
        slots, layers, mb, nb, meta_elems = self._sizes
        if L != layers or bt_dev.numel() != slots * layers * mb or meta_dev.numel() < meta_elems:
            raise ValueError("layers, bt_dev or meta_dev do not match the scheduler")
        if k_pool.shape[0] != nb:
            raise ValueError("pool size differs from the scheduler's num_blocks")
        _check("pkv_sched_run", load().pkv_sched_run(
            self._h, C.byref(self._it), ptrs[0], ptrs[1], ptrs[2], ptrs[3],
            _dev_ptr(k_pool, "k_pool", _bf16_types()), _dev_ptr(v_pool, "v_pool", _bf16_types()),
            _dev_ptr(bt_dev, "bt_dev", (torch.int32,)), _dev_ptr(meta_dev, "meta_dev", (torch.int32,)),
            q[0].shape[1], k[0].shape[1], q[0].shape[2], _dev_ptr(cos_sin, "cos_sin", (torch.float32,)),
            cos_sin.shape[0], float(scale), _dev_ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream)))


# ------------------------------------------------------- rest of the layer --

def pkv_rmsnorm(out, x, weight, eps=1e-5, stream=None):
    """out[r] = rmsnorm(x[r]) * weight; x/out bf16 [rows, dim], weight [dim]."""
    for t, n in ((out, "out"), (x, "x"), (weight, "weight")):
        _contig(t, n)
    rows, dim = x.shape
    if tuple(out.shape) != (rows, dim) or weight.numel() != dim:
        raise ValueError("out, x and weight disagree")
    bt = _bf16_types()
    _check("pkv_rmsnorm", load().pkv_rmsnorm(_dev_ptr(out, "out", bt), _dev_ptr(x, "x", bt),
                                             _dev_ptr(weight, "weight", bt), rows, dim, float(eps), _stream(stream)))


def pkv_silu_mul(act, gate_up, stream=None):
    """act[r] = silu(gate_up[r, :I]) * gate_up[r, I:]; act [rows, I], gate_up [rows, 2I]."""
    _contig(act, "act")
    _contig(gate_up, "gate_up")
    rows, inter = act.shape
    if tuple(gate_up.shape) != (rows, 2 * inter):
        raise ValueError("gate_up must be [rows, 2 * intermediate]")
    bt = _bf16_types()
    _check("pkv_silu_mul", load().pkv_silu_mul(_dev_ptr(act, "act", bt), _dev_ptr(gate_up, "gate_up", bt), rows,
                                               inter, _stream(stream)))


def pkv_linear_workspace_bytes(rows, out_features, in_features):
    return load().pkv_linear_workspace_bytes(rows, out_features, in_features)


def pkv_linear(out, x, weight, accumulate=False, workspace=None, stream=None):
    """out = x weight^T (+ out when accumulate); x [rows, in], weight [out, in].
    workspace: device tensor of at least pkv_linear_workspace_bytes(...) bytes
    for the K-split partials, allocated here when None and the shape needs
    it; False hands the library a null workspace (the product then runs as
    one K range)."""
    import torch
    for t, n in ((out, "out"), (x, "x"), (weight, "weight")):
        _contig(t, n)
    rows, k = x.shape
    n_out = weight.shape[0]
    if weight.shape[1] != k or tuple(out.shape) != (rows, n_out):
        raise ValueError("out, x and weight disagree")
    bt = _bf16_types()
    if workspace is None:
        nb = pkv_linear_workspace_bytes(rows, n_out, k)
        workspace = torch.empty(nb, dtype=torch.uint8, device=out.device) if nb else False
    if workspace is False:
        ws_ptr, ws_bytes = None, 0
    else:
        _contig(workspace, "workspace")
        ws_ptr, ws_bytes = _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()
    _check("pkv_linear", load().pkv_linear(_dev_ptr(out, "out", bt), _dev_ptr(x, "x", bt),
                                           _dev_ptr(weight, "weight", bt), rows, n_out, k, 1 if accumulate else 0,
                                           ws_ptr, ws_bytes, _stream(stream)))


class LayerWeights(C.Structure):
    """pkv_layer_weights (include/pagedkv.h)."""
    _fields_ = [(n, _p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate_up", "w_down")]


def pkv_decode_layer_scratch_elems(batch, hidden, intermediate, n_q_heads, n_kv_heads):
    return load().pkv_decode_layer_scratch_elems(batch, hidden, intermediate, n_q_heads, n_kv_heads)


def _layer_weights(weights, hidden, n_q_heads, lw=None):
    """Fill a LayerWeights from a dict of device bf16 tensors; returns it
    with the intermediate width."""
    bt16 = _bf16_types()
    lw = LayerWeights() if lw is None else lw
    inter = weights["w_down"].shape[1]
    for name in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate_up", "w_down"):
        _contig(weights[name], name)
        setattr(lw, name, _dev_ptr(weights[name], name, bt16))
    if weights["wq"].shape != (n_q_heads * 64, hidden) or weights["w_gate_up"].shape != (2 * inter, hidden):
        raise ValueError("weight shapes do not match hidden / heads / intermediate")
    return lw, inter


def pkv_decode_layers(h, layers, scratch, k_pool, v_pool, block_table, slot_ids, context_lens, max_context_len,
                      cos_sin, scale, workspace, row_lens_host=None, eps=1e-5, n_q_heads=32, stream=None):
    """len(layers) decode layers in one call, in place on h [B, hidden]
    (pkv_decode_layers).  layers: list of weight dicts as for
    pkv_decode_layer; block_table: int32 [slots, >= len(layers), max_blocks]
    with unit inner stride (layer l uses block_table[:, l, :])."""
    import torch
    bt16 = _bf16_types()
    for t, n in ((h, "h"), (scratch, "scratch"), (k_pool, "k_pool"), (v_pool, "v_pool"), (cos_sin, "cos_sin"),
                 (workspace, "workspace")):
        _contig(t, n)
    B, hidden = h.shape
    L = len(layers)
    if block_table.dtype != torch.int32 or block_table.dim() != 3 or block_table.stride(2) != 1:
        raise ValueError("block_table must be an int32 [slots, layers, max_blocks] tensor with unit inner stride")
    if block_table.shape[1] < L:
        raise ValueError("block_table has fewer layers than weights")
    arr = (LayerWeights * max(L, 1))()
    inter = None
    for l, wd in enumerate(layers):
        _, il = _layer_weights(wd, hidden, n_q_heads, arr[l])
        if inter is not None and il != inter:
            raise ValueError("layers disagree on the intermediate width")
        inter = il
    if inter is None:
        return
    rl, rl_ptr = _row_lens(row_lens_host, B)
    _check("pkv_decode_layers", load().pkv_decode_layers(
        _dev_ptr(h, "h", bt16), arr, L, hidden, inter, _dev_ptr(scratch, "scratch", bt16), scratch.numel(),
        _dev_ptr(k_pool, "k_pool", bt16), _dev_ptr(v_pool, "v_pool", bt16), k_pool.shape[0],
        _dev_ptr(block_table, "block_table"), block_table.stride(0), block_table.stride(1), block_table.shape[0],
        block_table.shape[2], _dev_ptr(slot_ids, "slot_ids", (torch.int32,)),
        _dev_ptr(context_lens, "context_lens", (torch.int32,)), rl_ptr, B, int(max_context_len), n_q_heads,
        k_pool.shape[2], _dev_ptr(cos_sin, "cos_sin", (torch.float32,)), cos_sin.shape[0], float(scale), float(eps),
        _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))


def pkv_decode_layer(h, weights, scratch, k_pool, v_pool, block_table, slot_ids, context_lens, max_context_len,
                     cos_sin, scale, workspace, row_lens_host=None, eps=1e-5, n_q_heads=32, stream=None):
    """One layer's decode step in place on h [B, hidden] (pkv_decode_layer).
    weights: dict of device bf16 tensors attn_norm, wq, wk, wv, wo, mlp_norm,
    w_gate_up, w_down; scratch: device bf16 with at least
    pkv_decode_layer_scratch_elems(...) elements (intermediates left there)."""
    import torch
    bt16 = _bf16_types()
    for t, n in ((h, "h"), (scratch, "scratch"), (k_pool, "k_pool"), (v_pool, "v_pool"), (cos_sin, "cos_sin"),
                 (workspace, "workspace")):
        _contig(t, n)
    B, hidden = h.shape
    inter = weights["w_down"].shape[1]
    n_kv = k_pool.shape[2]
    lw = LayerWeights()
    for name in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate_up", "w_down"):
        _contig(weights[name], name)
        setattr(lw, name, _dev_ptr(weights[name], name, bt16))
    if weights["wq"].shape != (n_q_heads * 64, hidden) or weights["w_gate_up"].shape != (2 * inter, hidden):
        raise ValueError("weight shapes do not match hidden / heads / intermediate")
    ptr, stride, rows, mb = _table(block_table)
    rl, rl_ptr = _row_lens(row_lens_host, B)
    _check("pkv_decode_layer", load().pkv_decode_layer(
        _dev_ptr(h, "h", bt16), C.byref(lw), hidden, inter, _dev_ptr(scratch, "scratch", bt16), scratch.numel(),
        _dev_ptr(k_pool, "k_pool", bt16), _dev_ptr(v_pool, "v_pool", bt16), k_pool.shape[0], ptr, stride, rows, mb,
        _dev_ptr(slot_ids, "slot_ids", (torch.int32,)), _dev_ptr(context_lens, "context_lens", (torch.int32,)),
        rl_ptr, B, int(max_context_len), n_q_heads, n_kv, _dev_ptr(cos_sin, "cos_sin", (torch.float32,)),
        cos_sin.shape[0], float(scale), float(eps), _dev_ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))

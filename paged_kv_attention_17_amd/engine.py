"""Decode-step driver over the C ABI.

One ``DecodeEngine.step`` is one decode step of an n-layer engine for a batch
of sequence slots, in the order "An Inference Engine in 1,500 Lines of CUDA:
The Map" describes (section "The path of one inference": a pool allocated
once, a free list and per-(slot, layer) block tables with -1 for unassigned
entries; decode produces one token per active slot per step):

  a0  host: for every slot whose new token opens a 16-token chunk, pop a free
      block into its table row of every layer (pkv_blocks_assign); the table
      changes, the new context lengths and positions travel to the device in
      the arguments of one pkv_block_table_patch launch (no H2D copy, no sync)
  per layer:
  a1  pkv_rope_decode      rotate the new q (n_q heads) and k (n_kv heads)
  a2  pkv_paged_kv_append  write the rotated k and v into the token's block row
  a3+a4 pkv_paged_attn_decode  attention over the whole context (split into
      partitions and merged when long)

The engine owns no arithmetic: everything on the device is a libpagedkv
kernel, everything on the host is pkv_blocks_assign plus index bookkeeping.
All buffers are allocated once, here, and reused by every step.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import _abi as abi
from .workloads import BLOCK_SIZE


class DecodeEngine:
    def __init__(self, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: np.ndarray,
                 cached_lens: np.ndarray, free_list: np.ndarray, n_q_heads: int = 32,
                 max_pos: int = 131072, scale: float | None = None, partition_size: int = 0,
                 max_context_len: int | None = None, stream=None):
        """k_pool/v_pool: device bf16 [NB, 16, n_kv, 64], already holding each
        slot's cached tokens; block_table: int32 [slots, layers, max_blocks]
        covering those tokens; cached_lens: tokens cached per slot;
        free_list: the blocks not in any table (popped from the end)."""
        self.dev = k_pool.device
        self.k_pool, self.v_pool = k_pool, v_pool
        self.n_slots, self.n_layers, self.max_blocks = block_table.shape
        self.n_kv = k_pool.shape[2]
        self.n_q = n_q_heads
        self.d = k_pool.shape[3]
        self.scale = 1.0 / math.sqrt(self.d) if scale is None else scale
        self.partition_size = partition_size
        self.stream = stream
        self.bt_host = np.ascontiguousarray(block_table, dtype=np.int32).copy()
        self.free = np.ascontiguousarray(free_list, dtype=np.int32).copy()
        self.n_free = len(self.free)
        self.cached = np.ascontiguousarray(cached_lens, dtype=np.int32).copy()
        cap = self.max_blocks * BLOCK_SIZE
        self.max_context_len = cap if max_context_len is None else max_context_len
        # One int32 device buffer: [table | context lengths | positions | slot ids].
        nt = self.bt_host.size
        ns = self.n_slots
        self.meta_host = np.concatenate([self.bt_host.ravel(), self.cached, np.zeros(ns, np.int32),
                                         np.arange(ns, dtype=np.int32)]).astype(np.int32)
        self.meta = torch.from_numpy(self.meta_host).to(self.dev)
        self.bt_dev = self.meta[:nt].view(ns, self.n_layers, self.max_blocks)
        self.ctx_dev = self.meta[nt:nt + ns]
        self.pos_dev = self.meta[nt + ns:nt + 2 * ns]
        self.sid_dev = self.meta[nt + 2 * ns:nt + 3 * ns]
        self._ctx_base = nt
        self._pos_base = nt + ns
        self._sid_base = nt + 2 * ns
        self._last_sids = np.arange(ns, dtype=np.int32)
        self.cos_sin = torch.empty((max_pos, self.d // 2, 2), dtype=torch.float32, device=self.dev)
        abi.pkv_rope_table_init(self.cos_sin, head_dim=self.d, stream=stream)
        ws = abi.pkv_decode_workspace_bytes(self.n_slots, self.n_q, self.n_kv, self.d, self.max_context_len,
                                           partition_size)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=self.dev)

    def plan_step(self, slot_ids: np.ndarray):
        """Host half of a step: allocate blocks, return the patch pairs and
        the per-row positions (0-based position of each new token)."""
        slot_ids = np.asarray(slot_ids, dtype=np.int32)
        positions = self.cached[slot_ids].astype(np.int32)
        offs, vals = [], []
        stride_layer = self.max_blocks
        for layer in range(self.n_layers):
            view = self.bt_host[:, layer, :]
            self.n_free, off, val = abi.pkv_blocks_assign(view, self.free, self.n_free, slot_ids, positions)
            offs.append(off.astype(np.int64) + layer * stride_layer)
            vals.append(val)
        self.cached[slot_ids] += 1
        offs.append(self._ctx_base + slot_ids.astype(np.int64))
        vals.append(self.cached[slot_ids])
        offs.append(self._pos_base + np.arange(len(slot_ids), dtype=np.int64))
        vals.append(positions)
        if not np.array_equal(slot_ids, self._last_sids[:len(slot_ids)]):
            offs.append(self._sid_base + np.arange(len(slot_ids), dtype=np.int64))
            vals.append(slot_ids)
            self._last_sids[:len(slot_ids)] = slot_ids
        return np.concatenate(offs).astype(np.int32), np.concatenate(vals).astype(np.int32), positions

    def step(self, slot_ids, q, k, v, out, layers=None):
        """q/out [L, B, n_q, 64], k/v [L, B, n_kv, 64] device bf16 (q and k are
        rotated in place).  Batch row b is slot slot_ids[b]."""
        slot_ids = np.asarray(slot_ids, dtype=np.int32)
        B = len(slot_ids)
        off, val, _ = self.plan_step(slot_ids)
        abi.pkv_block_table_patch(self.meta, off, val, stream=self.stream)
        sid = self.sid_dev[:B]
        pos = self.pos_dev[:B]
        for layer in (range(self.n_layers) if layers is None else layers):
            bt = self.bt_dev[:, layer, :]
            abi.pkv_rope_decode(q[layer], k[layer], pos, self.cos_sin, stream=self.stream)
            abi.pkv_paged_kv_append(self.k_pool, self.v_pool, k[layer], v[layer], bt, sid, pos,
                                    stream=self.stream)
            abi.pkv_paged_attn_decode(out[layer], q[layer], self.k_pool, self.v_pool, bt, sid, self.ctx_dev,
                                      self.max_context_len, self.scale, self.partition_size, self.workspace,
                                      stream=self.stream)

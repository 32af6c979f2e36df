"""Decode-step driver over the C ABI.

One ``DecodeEngine.step`` is one decode step of an n-layer engine for a batch
of sequence slots, in the order "An Inference Engine in 1,500 Lines of CUDA:
The Map" describes (section "The path of one inference": a pool allocated
once, a free list and per-(slot, layer) block tables with -1 for unassigned
entries; decode produces one token per active slot per step).  The step is
one call of the native ``pkv_decode_step``:

  a0  host: for every slot whose new token opens a 16-token chunk, pop a free
      block into its table row of every layer; the table changes and the new
      context lengths, positions and slot ids reach the device in kernel
      arguments (no H2D copy, no synchronisation)
  per layer:
  a1  RoPE on the new q (n_q heads) and k (n_kv heads)
  a2  append of the rotated k and of v into the token's block row
  a3+a4 paged attention over the whole context (split into partitions and
      merged when long)
  (a1-a4 are one launch per layer: pkv_paged_decode_fused; q and k keep their
  unrotated values)

The engine owns no arithmetic and allocates every buffer once, here.

``GraphStep`` runs the same step as a HIP graph captured once and replayed
(the category page's mini-sglang chapter 7: the step's ledger becomes kernel
arguments, and the launches are captured): the native host half
(``pkv_decode_step_host``) allocates blocks and writes the table changes, the
metadata and the streaming kernel's plan into a pinned staging area; the graph
copies it to the device and runs ``pkv_decode_step_device`` (apply, one fused
launch per layer, one merge), whose launch shapes never depend on the lengths.
A step whose rows the replayed launches do not serve (a few very long rows)
runs eagerly through ``pkv_decode_step`` instead.
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
        self.bt_dev = torch.from_numpy(self.bt_host).to(self.dev)
        # [context lengths (per slot) | positions | slot ids], room for a full batch
        ns = self.n_slots
        self.meta = torch.from_numpy(np.concatenate([self.cached, np.zeros(2 * ns, np.int32)])).to(self.dev)
        self.cos_sin = torch.empty((max_pos, self.d // 2, 2), dtype=torch.float32, device=self.dev)
        abi.pkv_rope_table_init(self.cos_sin, head_dim=self.d, stream=stream)
        self.workspace = abi.decode_workspace(self.n_slots, self.n_q, self.n_kv, self.max_context_len,
                                              partition_size, device=self.dev, stream=stream)

    @property
    def ctx_dev(self):
        return self.meta[:self.n_slots]

    def meta_view(self, batch: int):
        return self.meta[:self.n_slots + 2 * batch]

    def step(self, slot_ids, q, k, v, out):
        """q/out [L, B, n_q, 64], k/v [L, B, n_kv, 64] device bf16 (q, k, v are
        read only).  Batch row b is slot slot_ids[b]."""
        slot_ids = np.asarray(slot_ids, dtype=np.int32)
        self.n_free = abi.pkv_decode_step(
            q, k, v, out, self.k_pool, self.v_pool, self.bt_host, self.bt_dev, self.free, self.n_free,
            self.cached, self.meta_view(len(slot_ids)), slot_ids, self.cos_sin, self.scale,
            self.max_context_len, self.partition_size, self.workspace, stream=self.stream)


class GraphStep:
    """Decode steps of a fixed batch size over one DecodeEngine, replayed from
    captured HIP graphs.  The caller writes each step's q, k, v into
    ``self.q``/``self.k``/``self.v`` ([L, B, n_q|n_kv, 64] bf16) and reads
    ``self.out`` after ``step``; the rows' slots may change from step to step.

    ``depth`` staging areas (each with its own captured graph, whose copy
    reads it) let the host half of the next step run while the previous
    replays execute; a staging area is rewritten only after the replay that
    read it has finished."""

    def __init__(self, engine: DecodeEngine, batch: int, depth: int = 2):
        e = engine
        self.eng, self.batch = e, batch
        L, dev = e.n_layers, e.dev
        n = abi.pkv_decode_step_staging_bytes(L, batch, e.n_slots)
        if n == 0:
            raise ValueError("batch or slots outside what the replayed step serves")
        self.stage_host = [torch.empty(n, dtype=torch.uint8, pin_memory=True) for _ in range(depth)]
        self.stage_dev = torch.empty(n, dtype=torch.uint8, device=dev)
        self.q = torch.zeros((L, batch, e.n_q, e.d), dtype=torch.bfloat16, device=dev)
        self.k = torch.zeros((L, batch, e.n_kv, e.d), dtype=torch.bfloat16, device=dev)
        self.v = torch.zeros_like(self.k)
        self.out = torch.zeros_like(self.q)
        self.graphs = [None] * depth
        self.done = [torch.cuda.Event() for _ in range(depth)]
        self.pending = [False] * depth
        self.next = 0
        self.replays = self.eager_steps = 0

    def capture(self, i: int):
        """Capture the device half reading staging area i, which must hold a
        step that the host half accepted (its rows check the launches); the
        graph runs nothing until replayed."""
        e = self.eng
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.stage_dev.copy_(self.stage_host[i], non_blocking=True)
            abi.pkv_decode_step_device(self.q, self.k, self.v, self.out, e.k_pool, e.v_pool, e.bt_dev,
                                       e.meta_view(self.batch), e.cos_sin, e.scale, self.stage_host[i],
                                       self.stage_dev, e.workspace)
        self.graphs[i] = g

    def step(self, slot_ids):
        """One decode step for batch row b = slot slot_ids[b], enqueued on the
        current stream; returns True when it ran as a replay, False when it
        ran eagerly."""
        e = self.eng
        slot_ids = np.asarray(slot_ids, dtype=np.int32)
        if len(slot_ids) != self.batch:
            raise ValueError("the replayed step serves a fixed batch size")
        i = self.next
        if self.pending[i]:
            self.done[i].synchronize()        # the replay that read staging area i has finished
            self.pending[i] = False
        try:
            e.n_free = abi.pkv_decode_step_host(e.bt_host, e.free, e.n_free, e.cached, slot_ids,
                                                self.stage_host[i])
        except abi.PagedKVError as err:
            if err.status != abi.PKV_ERR_UNSUPPORTED:
                raise
            e.step(slot_ids, self.q, self.k, self.v, self.out)
            self.eager_steps += 1
            return False
        if self.graphs[i] is None:
            self.capture(i)
        self.graphs[i].replay()
        self.done[i].record()
        self.pending[i] = True
        self.next = (i + 1) % len(self.graphs)
        self.replays += 1
        return True

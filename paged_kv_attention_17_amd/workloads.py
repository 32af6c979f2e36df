"""Seeded synthetic inputs for the paged decode / prefill path.

This module is shared by the tests, the bench and the CPU oracle's callers.
It holds none of the attention, RoPE or paging arithmetic: it only draws
random numbers, rounds them to bfloat16 storage bits, and lays out pools,
block tables and context lengths the way the engine in "An Inference Engine
in 1,500 Lines of CUDA: The Map" (section "The path of one inference") sets
them up: one pool carved into 16-token blocks, blocks handed out from a free
list, and a block table whose unassigned entries hold -1.

Everything is numpy on the host (PCG64, seed given by the caller), so a
workload is device independent and reproducible.  The big cache workloads
(tens of thousands of blocks) are filled in slices so that host memory stays
bounded; ``fill_pool_device`` draws the same distribution on a GPU with a
seeded torch generator when the host would be too slow.

bfloat16 values are carried as ``uint16`` bit patterns everywhere.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BLOCK_SIZE = 16          # tokens per KV block
N_Q_HEADS = 32
N_KV_HEADS = 8
HEAD_DIM = 64
UNASSIGNED = -1          # block-table sentinel for "no block yet"

# bf16 quiet NaN with a payload, used to poison pool slots that a correct
# kernel never reads.
BF16_POISON = np.uint16(0x7FC1)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Used only to turn the random draws into bf16 inputs.  NaN stays NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def randn_bf16(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))


def uniform_bf16(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    return f32_to_bf16_bits(rng.uniform(lo, hi, size=shape).astype(np.float32))


def blocks_for(n_tokens: int) -> int:
    return (n_tokens + BLOCK_SIZE - 1) // BLOCK_SIZE


@dataclasses.dataclass
class DecodeWorkload:
    """One decode step's inputs for ``n_layers`` layers.

    Shapes (bf16 as uint16):
      k_pool, v_pool : [num_blocks, 16, n_kv, d]   (one pool shared by all layers)
      block_table    : int32 [n_slots, n_layers, max_blocks], -1 = unassigned
      context_lens   : int32 [n_slots]  -- length INCLUDING the new token
      slot_ids       : int32 [batch]    -- batch row -> slot
      q_new          : [n_layers, batch, n_q, d]   (before RoPE)
      k_new, v_new   : [n_layers, batch, n_kv, d]  (k before RoPE)
      free_list      : int32 blocks not referenced by any table (pop from the end)

    Before the step, each slot's table covers the ``context_lens - 1`` tokens
    already cached; the new token's block is assigned by the step itself
    when its position is a multiple of 16.
    """
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_table: np.ndarray
    context_lens: np.ndarray
    slot_ids: np.ndarray
    q_new: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    free_list: np.ndarray
    scale: float
    seed: int
    n_blocks: int = 0

    @property
    def n_layers(self) -> int:
        return self.block_table.shape[1]

    @property
    def batch(self) -> int:
        return self.slot_ids.shape[0]

    @property
    def num_blocks(self) -> int:
        return self.n_blocks if self.k_pool is None else self.k_pool.shape[0]

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[2]

    @property
    def positions(self) -> np.ndarray:
        return (self.context_lens[self.slot_ids] - 1).astype(np.int32)


def _hand_out_blocks(rng, n_slots, n_layers, prior_tokens, num_blocks, max_blocks,
                     interleave: bool):
    """Build block tables by popping a shuffled free list.

    With ``interleave`` the pops go round-robin over (layer, slot), one block
    at a time, so consecutive blocks of one sequence are far apart in the pool.
    Returns (block_table, remaining_free_list).
    """
    free = rng.permutation(num_blocks).astype(np.int32)
    top = len(free)
    bt = np.full((n_slots, n_layers, max_blocks), UNASSIGNED, dtype=np.int32)
    need = [blocks_for(int(t)) for t in prior_tokens]
    if interleave:
        for j in range(max(need) if need else 0):
            for layer in range(n_layers):
                for s in range(n_slots):
                    if j < need[s]:
                        top -= 1
                        bt[s, layer, j] = free[top]
    else:
        for s in range(n_slots):
            for layer in range(n_layers):
                for j in range(need[s]):
                    top -= 1
                    bt[s, layer, j] = free[top]
    if top < 0:
        raise ValueError("pool too small for the requested contexts")
    return bt, free[:top].copy()


def _fill_pool(rng, pool_shape, kind: str, poison_unused: bool, used_mask=None,
               lo=-1.0, hi=1.0, chunk_blocks: int = 4096):
    pool = np.empty(pool_shape, dtype=np.uint16)
    nb = pool_shape[0]
    for b0 in range(0, nb, chunk_blocks):
        b1 = min(nb, b0 + chunk_blocks)
        shp = (b1 - b0,) + tuple(pool_shape[1:])
        if kind == "normal":
            pool[b0:b1] = randn_bf16(rng, shp)
        else:
            pool[b0:b1] = uniform_bf16(rng, shp, lo, hi)
    if poison_unused and used_mask is not None:
        pool[~used_mask] = BF16_POISON
    return pool


def used_token_mask(block_table: np.ndarray, context_lens: np.ndarray, num_blocks: int,
                    n_cached=None) -> np.ndarray:
    """bool [num_blocks, 16]: token slots that hold live context."""
    mask = np.zeros((num_blocks, BLOCK_SIZE), dtype=bool)
    n_slots, n_layers, _ = block_table.shape
    for s in range(n_slots):
        n = int(context_lens[s] if n_cached is None else n_cached[s])
        for layer in range(n_layers):
            for j in range(blocks_for(n)):
                blk = block_table[s, layer, j]
                cnt = min(BLOCK_SIZE, n - j * BLOCK_SIZE)
                mask[blk, :cnt] = True
    return mask


def make_decode(seed: int, context_lens, n_layers: int = 1, num_blocks: int | None = None,
                pool_slack: float = 1.25, max_blocks: int | None = None,
                interleave: bool = True, k_kind: str = "normal", v_kind: str = "normal",
                poison_unused: bool = False, spikes_per_seq: int = 0, spike_factor: float = 8.0,
                n_q: int = N_Q_HEADS, n_kv: int = N_KV_HEADS, d: int = HEAD_DIM,
                fill_pool: bool = True, extra_steps: int = 0) -> DecodeWorkload:
    """General decode-step generator.

    ``context_lens`` are lengths including the new token.  The pool is sized
    ``num_blocks`` or ``ceil(pool_slack * blocks needed)``; ``extra_steps``
    reserves table room for that many further tokens per slot.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = np.asarray(context_lens, dtype=np.int32)
    n_slots = len(ctx)
    prior = ctx - 1
    if max_blocks is None:
        max_blocks = blocks_for(int(ctx.max()) + extra_steps)
    if num_blocks is None:
        need_total = sum(blocks_for(int(c) + extra_steps) for c in ctx) * n_layers
        num_blocks = int(math.ceil(pool_slack * need_total))
    bt, free = _hand_out_blocks(rng, n_slots, n_layers, prior, num_blocks, max_blocks, interleave)
    shape = (num_blocks, BLOCK_SIZE, n_kv, d)
    if fill_pool:
        mask = used_token_mask(bt, prior, num_blocks) if poison_unused else None
        k_pool = _fill_pool(rng, shape, k_kind, poison_unused, mask)
        v_pool = _fill_pool(rng, shape, v_kind, poison_unused, mask)
        if spikes_per_seq:
            spike_keys(rng, k_pool, bt, prior, spikes_per_seq, spike_factor)
    else:
        k_pool = v_pool = None
    slot_ids = np.arange(n_slots, dtype=np.int32)
    q_new = randn_bf16(rng, (n_layers, n_slots, n_q, d))
    k_new = randn_bf16(rng, (n_layers, n_slots, n_kv, d))
    if v_kind == "normal":
        v_new = randn_bf16(rng, (n_layers, n_slots, n_kv, d))
    else:
        v_new = uniform_bf16(rng, (n_layers, n_slots, n_kv, d), -1.0, 1.0)
    return DecodeWorkload(k_pool, v_pool, bt, ctx, slot_ids, q_new, k_new, v_new, free,
                          scale=1.0 / math.sqrt(d), seed=seed, n_blocks=num_blocks)


def spike_keys(rng, k_pool, bt, n_cached, per_seq: int, factor: float):
    """Multiply ``per_seq`` cached keys of every sequence (all kv heads, all
    layers) by ``factor``.  A power-of-two factor keeps them exact in bf16."""
    assert factor == 2.0 ** round(math.log2(factor))
    n_slots, n_layers, _ = bt.shape
    for s in range(n_slots):
        n = int(n_cached[s])
        if n <= 0:
            continue
        picks = rng.choice(n, size=min(per_seq, n), replace=False)
        for layer in range(n_layers):
            for p in picks:
                blk = bt[s, layer, p // BLOCK_SIZE]
                row = bf16_bits_to_f32(k_pool[blk, p % BLOCK_SIZE]) * np.float32(factor)
                k_pool[blk, p % BLOCK_SIZE] = f32_to_bf16_bits(row)


# ---------------------------------------------------------------------------
# The five workloads the decode path is exercised on.
# ---------------------------------------------------------------------------

def config1(poison_unused: bool = False) -> DecodeWorkload:
    """1 sequence, 1 layer, context 17 (two blocks, the last holding one
    token), 64-block pool, table taken from a seeded permutation."""
    return make_decode(1701, [17], n_layers=1, num_blocks=64, poison_unused=poison_unused)


def config2(poison_unused: bool = False, extra_steps: int = 4) -> DecodeWorkload:
    """4 slots with contexts {17, 14, 300, 1000}, 512-block pool, tables popped
    from a shuffled free list."""
    return make_decode(1702, [17, 14, 300, 1000], n_layers=1, num_blocks=512,
                       poison_unused=poison_unused, extra_steps=extra_steps)


def config3_contexts(seed: int = 1703, batch: int = 64) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(512, 4096, size=batch, endpoint=True).astype(np.int32)


def config3(fill_pool: bool = True, extra_steps: int = 0, batch: int = 64,
            n_layers: int = 16) -> DecodeWorkload:
    """B=64, 16 layers, contexts uniform in [512, 4096], pool = 1.25 x the
    blocks needed, tables interleaved round-robin over (layer, slot)."""
    ctx = config3_contexts(1703, batch)
    return make_decode(1703, ctx, n_layers=n_layers, pool_slack=1.25, interleave=True,
                       fill_pool=fill_pool, extra_steps=extra_steps)


def config4(fill_pool: bool = True, batch: int = 256, ctx: int = 8192) -> DecodeWorkload:
    """B=256, 1 layer, context 8192 each; K ~ N(0,1), V ~ U(-1,1); four keys per
    sequence spiked x8."""
    return make_decode(1704, [ctx] * batch, n_layers=1, pool_slack=1.0, interleave=True,
                       v_kind="uniform", spikes_per_seq=4, fill_pool=fill_pool)


@dataclasses.dataclass
class PrefillWorkload:
    """Chunked prefill inputs: prompts packed along tokens.

      q            : [total_q, n_q, d]   (already positioned: no RoPE applied here)
      k, v         : [total_q, n_kv, d]
      prompt_lens  : int32 [S]
      block_table  : int32 [S, 1, max_blocks] with every prompt block assigned
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    prompt_lens: np.ndarray
    block_table: np.ndarray
    num_blocks: int
    free_list: np.ndarray
    scale: float
    seed: int


def make_prefill(seed: int, prompt_lens, num_blocks: int | None = None, extra_tokens: int = 0,
                 n_q: int = N_Q_HEADS, n_kv: int = N_KV_HEADS, d: int = HEAD_DIM,
                 interleave: bool = True) -> PrefillWorkload:
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(prompt_lens, dtype=np.int32)
    S = len(lens)
    max_blocks = blocks_for(int(lens.max()) + extra_tokens)
    need = sum(blocks_for(int(n) + extra_tokens) for n in lens)
    if num_blocks is None:
        num_blocks = int(math.ceil(1.25 * need))
    bt, free = _hand_out_blocks(rng, S, 1, lens, num_blocks, max_blocks, interleave)
    T = int(lens.sum())
    q = randn_bf16(rng, (T, n_q, d))
    k = randn_bf16(rng, (T, n_kv, d))
    v = randn_bf16(rng, (T, n_kv, d))
    return PrefillWorkload(q, k, v, lens, bt, num_blocks, free, 1.0 / math.sqrt(d), seed)


def config5_prompt_lens(seed: int = 1705, n: int = 8) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(256, 2048, size=n, endpoint=True).astype(np.int32)


def config5(extra_tokens: int = 32) -> PrefillWorkload:
    """8 prompts with lengths uniform in [256, 2048], followed by room for 32
    decode steps per sequence."""
    return make_prefill(1705, config5_prompt_lens(), extra_tokens=extra_tokens)


@dataclasses.dataclass
class SharedPrefixWorkload:
    """Decode inputs where rows open with shared prompts: row b continues
    prompt b % n_prompts (prompt_len tokens, a whole number of blocks, listed
    by every such row) with its own tail.

      k_pool, v_pool : [num_blocks, 16, n_kv, d] or None (fill on the device)
      block_table    : int32 [batch, n_layers, max_blocks], -1 = unassigned
      context_lens   : int32 [batch]  (prompt + tail)
      q              : [batch, n_q, d]
    """
    k_pool: np.ndarray | None
    v_pool: np.ndarray | None
    block_table: np.ndarray
    context_lens: np.ndarray
    q: np.ndarray
    num_blocks: int
    prompt_len: int
    n_prompts: int
    seed: int

    @property
    def listed_blocks(self) -> int:
        return int(np.count_nonzero(self.block_table >= 0))

    @property
    def unique_blocks(self) -> int:
        return int(len(np.unique(self.block_table[self.block_table >= 0])))


def shared_prefix(seed: int = 1706, batch: int = 64, n_prompts: int = 4, prompt_len: int = 2048,
                  tail_lo: int = 64, tail_hi: int = 1024, n_layers: int = 1, fill_pool: bool = True,
                  n_q: int = N_Q_HEADS, n_kv: int = N_KV_HEADS, d: int = HEAD_DIM) -> SharedPrefixWorkload:
    """B rows over a few common prompts (many requests with one system
    prompt), tails uniform in [tail_lo, tail_hi]; each layer's blocks come
    off one shuffled free list, prompts first."""
    if prompt_len % BLOCK_SIZE:
        raise ValueError("prompt_len must be a whole number of blocks")
    rng = np.random.Generator(np.random.PCG64(seed))
    tails = rng.integers(tail_lo, tail_hi, size=batch, endpoint=True).astype(np.int32)
    ctx = (prompt_len + tails).astype(np.int32)
    pb = prompt_len // BLOCK_SIZE
    max_blocks = blocks_for(int(ctx.max()))
    per_layer = n_prompts * pb + sum(blocks_for(int(t)) for t in tails)
    num_blocks = per_layer * n_layers
    free = rng.permutation(num_blocks).astype(np.int32)
    bt = np.full((batch, n_layers, max_blocks), UNASSIGNED, np.int32)
    k = 0
    for layer in range(n_layers):
        prompts = free[k:k + n_prompts * pb].reshape(n_prompts, pb)
        k += n_prompts * pb
        for b in range(batch):
            bt[b, layer, :pb] = prompts[b % n_prompts]
            nt = blocks_for(int(tails[b]))
            bt[b, layer, pb:pb + nt] = free[k:k + nt]
            k += nt
    q = randn_bf16(rng, (batch, n_q, d))
    kp = vp = None
    if fill_pool:
        kp = randn_bf16(rng, (num_blocks, BLOCK_SIZE, n_kv, d))
        vp = randn_bf16(rng, (num_blocks, BLOCK_SIZE, n_kv, d))
    return SharedPrefixWorkload(kp, vp, bt, ctx, q, num_blocks, prompt_len, n_prompts, seed)


def fill_pool_device(pool, seed: int, kind: str = "normal", lo: float = -1.0, hi: float = 1.0,
                     chunk_blocks: int = 8192):
    """Fill a device bf16 tensor [NB, 16, H, D] in place from a seeded torch
    generator on the tensor's device (used for multi-GB caches)."""
    import torch
    g = torch.Generator(device=pool.device)
    g.manual_seed(seed)
    nb = pool.shape[0]
    for b0 in range(0, nb, chunk_blocks):
        b1 = min(nb, b0 + chunk_blocks)
        shp = (b1 - b0,) + tuple(pool.shape[1:])
        if kind == "normal":
            t = torch.randn(shp, generator=g, device=pool.device, dtype=torch.float32)
        else:
            t = torch.rand(shp, generator=g, device=pool.device, dtype=torch.float32)
            t = t * (hi - lo) + lo
        pool[b0:b1].copy_(t.to(torch.bfloat16))
        del t

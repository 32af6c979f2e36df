"""Block-table addressing of the paged KV cache (test infrastructure only).

Source: "An Inference Engine in 1,500 Lines of CUDA: The Map", sections
"What is in the box" and "The path of one inference", step (4): the KV cache
is one pool allocated once and cut into 16-token blocks; a free list numbers
the blocks 0, 1, 2, ...; a block table per (sequence slot, layer) records
which block holds which 16-token chunk of that sequence, and -1 marks an
entry not assigned yet.  The series' sixth chapter title ("Splitting the KV
cache into 16-token blocks -- reading non-contiguous blocks via the block
table") names the read side.

Token p of the sequence in slot s lives in block ``bt[s][p // 16]`` at row
``p % 16``.  Pools are [num_blocks][16][n_kv][d] (K and V alike, same block
id); tables are [n_rows][max_blocks] for one layer.
"""
import numpy as np

BLOCK_SIZE = 16
UNASSIGNED = -1


class BadBlock(ValueError):
    pass


def _entry(bt_row: np.ndarray, p: int, num_blocks: int) -> int:
    j = p // BLOCK_SIZE
    if j >= len(bt_row):
        raise BadBlock(f"position {p} beyond the table ({len(bt_row)} blocks)")
    blk = int(bt_row[j])
    if blk < 0 or blk >= num_blocks:
        raise BadBlock(f"table entry {j} is {blk} (pool has {num_blocks} blocks)")
    return blk


def append(k_pool, v_pool, k_new, v_new, bt, slot_ids, positions):
    """Write token t's k_new[t], v_new[t] ([n_kv][d], bf16 bits) into its
    block row.  Copies bits; returns new (k_pool, v_pool), inputs untouched."""
    k_out, v_out = k_pool.copy(), v_pool.copy()
    nb = k_pool.shape[0]
    for t in range(len(positions)):
        s, p = int(slot_ids[t]), int(positions[t])
        blk = _entry(bt[s], p, nb)
        k_out[blk, p % BLOCK_SIZE] = k_new[t]
        v_out[blk, p % BLOCK_SIZE] = v_new[t]
    return k_out, v_out


def gather(pool, bt_row, context_len):
    """The first ``context_len`` tokens of one sequence, contiguous:
    [context_len][n_kv][d] bits, read through its table row."""
    nb = pool.shape[0]
    out = np.empty((context_len,) + pool.shape[2:], dtype=pool.dtype)
    for p in range(context_len):
        out[p] = pool[_entry(bt_row, p, nb), p % BLOCK_SIZE]
    return out


def allocation_problems(bt_before, bt_after, free_before, free_after, slot_ids, positions):
    """Check one step's block allocation; return a list of problems (empty =
    valid).  Several placements are correct -- any free block will do -- so
    this checks the properties every correct allocation has:

      * a token whose position starts a block (p % 16 == 0) gets a block in
        entry p // 16 that was on the free list before and is not any more;
      * no block is handed out twice, and no other table entry changes;
      * the free list loses exactly the blocks handed out.
    """
    problems = []
    bt_before = np.asarray(bt_before)
    bt_after = np.asarray(bt_after)
    free_before = set(int(b) for b in free_before)
    free_after_l = [int(b) for b in free_after]
    free_after = set(free_after_l)
    if len(free_after) != len(free_after_l):
        problems.append("free list holds a block twice")
    expected_changes = set()
    handed = []
    for s, p in zip(slot_ids, positions):
        s, p = int(s), int(p)
        if p % BLOCK_SIZE != 0:
            continue
        j = p // BLOCK_SIZE
        expected_changes.add((s, j))
        blk = int(bt_after[s, j])
        if bt_before[s, j] != UNASSIGNED:
            problems.append(f"slot {s} entry {j} was already assigned")
        if blk not in free_before:
            problems.append(f"slot {s} entry {j} got block {blk}, not a free block")
        if blk in free_after:
            problems.append(f"block {blk} handed out but still on the free list")
        handed.append(blk)
    if len(set(handed)) != len(handed):
        problems.append("a block was handed out twice")
    diff = np.argwhere(bt_before != bt_after)
    for s, j in diff:
        if (int(s), int(j)) not in expected_changes:
            problems.append(f"unexpected change at slot {s} entry {j}")
    if free_before - set(handed) != free_after:
        problems.append("free list changed by more than the handed-out blocks")
    return problems


# ------------------------------------------------------------------ sharing --
# Prefix reuse.  The category page "code-series" lists, in its mini-sglang
# series, a chapter on a radix cache: when many requests open with the same
# prompt, the cached K/V of that prefix is reused instead of being computed
# again.  The pages give no mechanism.  Reading adopted: a block may be listed
# by several table entries; refcount[b] is the number of entries listing b; a
# block is only written through an entry that lists it alone, so a row that is
# about to append into a shared block first points its entry at a private
# copy of it (copy on write).  Sharing must not change what any sequence
# reads: gather() of every row still returns that sequence's own tokens.


def copy_blocks(k_pool, v_pool, src, dst):
    """Whole-block copies, K and V: block dst[i] takes the 16 rows of block
    src[i].  Returns new (k_pool, v_pool); inputs untouched."""
    k_out, v_out = k_pool.copy(), v_pool.copy()
    for a, b in zip(src, dst):
        k_out[int(b)] = k_pool[int(a)]
        v_out[int(b)] = v_pool[int(a)]
    return k_out, v_out


def refcount_problems(tables, refcount, free_list):
    """Check the sharing bookkeeping over every table view in ``tables``
    (each [rows][max_blocks]); return a list of problems (empty = valid):

      * refcount[b] equals the number of table entries that list b;
      * a block on the free list is listed by no entry and has count 0;
      * no block is on the free list twice;
      * every listed block is a block of the pool.
    """
    problems = []
    nb = len(refcount)
    counts = np.zeros(nb, np.int64)
    for t in tables:
        ids = np.asarray(t).ravel()
        ids = ids[ids != UNASSIGNED]
        bad = ids[(ids < 0) | (ids >= nb)]
        if len(bad):
            problems.append(f"table lists block {int(bad[0])} outside the pool")
            ids = ids[(ids >= 0) & (ids < nb)]
        np.add.at(counts, ids, 1)
    wrong = np.nonzero(counts != np.asarray(refcount))[0]
    for b in wrong[:5]:
        problems.append(f"block {int(b)}: refcount {int(refcount[b])}, listed {int(counts[b])} times")
    free = [int(b) for b in free_list]
    if len(set(free)) != len(free):
        problems.append("free list holds a block twice")
    for b in free:
        if counts[b] or refcount[b]:
            problems.append(f"block {b} is free but listed {int(counts[b])} times (refcount {int(refcount[b])})")
            break
    return problems

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

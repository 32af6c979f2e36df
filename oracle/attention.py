"""Paged attention in float64 with a two-pass softmax (test infrastructure only).

Sources:
  * "An Inference Engine in 1,500 Lines of CUDA: The Map" -- section "The
    path of one inference" (prefill handles the whole prompt as matrix x
    matrix, decode one token per step as vector x matrix; same math) and the
    Korean page's "What is in the box" table: grouped-query attention with
    four query heads per KV head (``GQA_Q_TO_K_RATIO = 4``), online softmax
    and PagedAttention inside ``pagedAttentionKernel``.
  * The series' chapter-6 title: each decode step re-reads all of the
    sequence's cached K/V through the block table.

What is computed (the plain definition the online softmax reaches exactly,
up to rounding order):

  for query head h, KV head g = h // (n_q / n_kv)       (contiguous groups)
  s_j = scale * <q_h, K_j,g>         for every visible key j
  m   = max_j s_j,  p_j = exp(s_j - m),  l = sum_j p_j
  o_h = sum_j p_j V_j,g / l

Decode: the single query of a sequence sees keys 0 .. context_len - 1 (the
length includes the token appended this step, so the query sees itself).
Prefill: the query at absolute position a sees keys 0 .. a (causal).
Keys and values are gathered through the block table first.  An empty
context yields a zero row.
"""
import numpy as np

from . import bf16, paging


def _attend(q, K, V, scale):
    """q [n_q][d], K/V [n][n_kv][d] float64 -> [n_q][d] float64."""
    n_q, d = q.shape
    n, n_kv, _ = K.shape
    out = np.zeros((n_q, d), dtype=np.float64)
    if n == 0:
        return out
    group = n_q // n_kv
    for h in range(n_q):
        g = h // group
        s = scale * (K[:, g, :] @ q[h])          # first pass: scores and their max
        m = s.max()
        p = np.exp(s - m)                        # second pass: weights and sum
        l = p.sum()
        out[h] = (p @ V[:, g, :]) / l
    return out


def decode(q_bits, k_pool, v_pool, bt, slot_ids, context_lens, scale):
    """Single-query attention per batch row.

    q_bits [B][n_q][d] bf16 bits (already rotated); pools [NB][16][n_kv][d];
    bt [n_rows][max_blocks] int32 (one layer); slot_ids [B] -> table row;
    context_lens indexed by table row.  Returns float64 [B][n_q][d].
    """
    q = bf16.to_f64(q_bits)
    B = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(B):
        s = int(slot_ids[b])
        n = int(context_lens[s])
        K = bf16.to_f64(paging.gather(k_pool, bt[s], n))
        V = bf16.to_f64(paging.gather(v_pool, bt[s], n))
        out[b] = _attend(q[b], K, V, scale)
    return out


def prefill(q_bits, cu_q_lens, q_start, slot_ids, k_pool, v_pool, bt, scale):
    """Causal attention for query tokens packed along dimension 0.

    Sequence i owns query rows cu_q_lens[i] .. cu_q_lens[i+1]-1; its first
    query sits at absolute position q_start[i].  Query row r of sequence i
    (absolute position a = q_start[i] + r - cu_q_lens[i]) sees keys 0 .. a of
    table row slot_ids[i].  Returns float64 [total_q][n_q][d].
    """
    q = bf16.to_f64(q_bits)
    out = np.zeros(q.shape, dtype=np.float64)
    for i in range(len(cu_q_lens) - 1):
        r0, r1 = int(cu_q_lens[i]), int(cu_q_lens[i + 1])
        if r1 == r0:
            continue
        s = int(slot_ids[i])
        last = int(q_start[i]) + (r1 - r0)
        K = bf16.to_f64(paging.gather(k_pool, bt[s], last))
        V = bf16.to_f64(paging.gather(v_pool, bt[s], last))
        for r in range(r0, r1):
            a = int(q_start[i]) + (r - r0)
            out[r] = _attend(q[r], K[:a + 1], V[:a + 1], scale)
    return out


def dense_decode(q_bits, K_bits, V_bits, scale):
    """Same softmax as ``decode`` on already-contiguous K/V [n][n_kv][d]."""
    return _attend(bf16.to_f64(q_bits), bf16.to_f64(K_bits), bf16.to_f64(V_bits), scale)

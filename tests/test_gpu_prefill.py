"""GPU parity for chunked causal prefill (MFMA) and the decode steps that
follow it on the same cache."""
import numpy as np
import pytest
import torch

import paged_kv_attention_17_amd as pkv
from paged_kv_attention_17_amd import workloads as W
from paged_kv_attention_17_amd.engine import DecodeEngine
from oracle import attention, paging, rope

from gpu_util import bits, check_attention, dev_bf16, dev_i32, ulp_diff

pytestmark = pytest.mark.gpu


def _setup(lens, n_q=32, n_kv=8, seed=0, poison=True, extra=0):
    rng = np.random.default_rng(seed)
    S = len(lens)
    mb = W.blocks_for(max(lens) + extra) + 1
    nb = sum(W.blocks_for(n + extra) for n in lens) + 5
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((S, mb), -1, np.int32)
    k = 0
    for s, n in enumerate(lens):
        for j in range(W.blocks_for(n + extra)):
            bt[s, j] = perm[k]
            k += 1
    fill = W.BF16_POISON if poison else 0
    kp = np.full((nb, 16, n_kv, 64), fill, np.uint16)
    vp = kp.copy()
    T = int(sum(lens))
    q = W.randn_bf16(rng, (T, n_q, 64))
    kn = W.randn_bf16(rng, (T, n_kv, 64))
    vn = W.randn_bf16(rng, (T, n_kv, 64))
    return q, kn, vn, kp, vp, bt, perm[k:]


def _gpu_chunked(q, kn, vn, kp, vp, bt, lens, chunk, host=False):
    """Append and prefill every sequence chunk by chunk (all sequences'
    i-th chunks in one call); host=True also hands the library host copies of
    the chunk layout (the launch then holds only real work, heaviest first).
    Returns output bits and the device pools."""
    kpd, vpd, btd = dev_bf16(kp), dev_bf16(vp), dev_i32(bt)
    out = torch.zeros((q.shape[0],) + q.shape[1:], dtype=torch.bfloat16, device="cuda")
    qd, knd, vnd = dev_bf16(q), dev_bf16(kn), dev_bf16(vn)
    starts = np.concatenate([[0], np.cumsum(lens)])
    n_chunks = max(-(-n // chunk) for n in lens)
    for c in range(n_chunks):
        rows, sid, pos, cu, qs, seqs = [], [], [], [0], [], []
        for s, n in enumerate(lens):
            a, b = c * chunk, min(n, (c + 1) * chunk)
            if a >= b:
                continue
            r = np.arange(starts[s] + a, starts[s] + b)
            rows.append(r)
            sid += [s] * len(r)
            pos += list(range(a, b))
            cu.append(cu[-1] + len(r))
            qs.append(a)
            seqs.append(s)
        r = torch.from_numpy(np.concatenate(rows)).cuda()
        kc, vc, qc = knd[r].contiguous(), vnd[r].contiguous(), qd[r].contiguous()
        pkv.pkv_paged_kv_append(kpd, vpd, kc, vc, btd, dev_i32(sid), dev_i32(pos))
        oc = torch.empty_like(qc)
        extra = dict(cu_q_lens_host=np.array(cu, np.int32), q_start_host=np.array(qs, np.int32)) if host else {}
        pkv.pkv_paged_attn_prefill(oc, qc, dev_i32(cu), dev_i32(qs), dev_i32(seqs), kpd, vpd, btd,
                                   int(np.diff(cu).max()), 0.125, **extra)
        out[r] = oc
    torch.cuda.synchronize()
    return bits(out), kpd, vpd


def _oracle(q, kn, vn, kp, vp, bt, lens):
    S = len(lens)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    sid = np.repeat(np.arange(S), lens).astype(np.int32)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    kp2, vp2 = paging.append(kp, vp, kn, vn, bt, sid, pos)
    out = attention.prefill(q, starts, np.zeros(S, np.int32), np.arange(S), kp2, vp2, bt, 0.125)
    return out, kp2, vp2


@pytest.mark.parametrize("lens", [[5, 40, 100], [1, 32, 33, 64], [257]])
def test_prefill_whole_prompts(gpu, lens):
    q, kn, vn, kp, vp, bt, _ = _setup(lens, seed=sum(lens))
    got, kpd, vpd = _gpu_chunked(q, kn, vn, kp, vp, bt, lens, chunk=4096)
    ref, kp2, vp2 = _oracle(q, kn, vn, kp, vp, bt, lens)
    np.testing.assert_array_equal(bits(kpd), kp2)
    check_attention(got, ref, f"prefill {lens}")


@pytest.mark.parametrize("n_q,n_kv", [(8, 8), (16, 8), (64, 8)])
def test_prefill_gqa_ratios(gpu, n_q, n_kv):
    lens = [70, 31]
    q, kn, vn, kp, vp, bt, _ = _setup(lens, n_q=n_q, n_kv=n_kv, seed=n_q)
    got, _, _ = _gpu_chunked(q, kn, vn, kp, vp, bt, lens, chunk=4096)
    ref, _, _ = _oracle(q, kn, vn, kp, vp, bt, lens)
    check_attention(got, ref, f"prefill gqa {n_q}/{n_kv}")


@pytest.mark.parametrize("n_q,n_kv", [(8, 8), (16, 8), (64, 8), (16, 4)])
def test_prefill_gqa_long_chunked(gpu, n_q, n_kv):
    """Several query tiles per prompt for every GQA ratio (the workgroup holds
    256 / G queries: 8 query subtiles of one head at G = 1, one subtile of 8
    heads at G = 8), chunked at 160 tokens (chunk starts off the tile grid)
    bit-identical to whole prompts, and the oracle."""
    lens = [700, 300, 1]
    q, kn, vn, kp, vp, bt, _ = _setup(lens, n_q=n_q, n_kv=n_kv, seed=n_q + 7 * n_kv)
    whole, _, _ = _gpu_chunked(q, kn, vn, kp, vp, bt, lens, chunk=4096)
    part, _, _ = _gpu_chunked(q, kn, vn, kp, vp, bt, lens, chunk=160)
    np.testing.assert_array_equal(part, whole)
    for chunk in (160, 4096):
        sched, _, _ = _gpu_chunked(q, kn, vn, kp, vp, bt, lens, chunk=chunk, host=True)
        np.testing.assert_array_equal(sched, whole)
    ref, _, _ = _oracle(q, kn, vn, kp, vp, bt, lens)
    check_attention(whole, ref, f"prefill long gqa {n_q}/{n_kv}")


def test_chunked_equals_whole_bit_identical(gpu):
    lens = [300, 129, 64]
    q, kn, vn, kp, vp, bt, _ = _setup(lens, seed=9)
    whole, _, _ = _gpu_chunked(q, kn, vn, kp, vp, bt, lens, chunk=4096)
    for chunk in (16, 64, 100):
        part, _, _ = _gpu_chunked(q, kn, vn, kp, vp, bt, lens, chunk=chunk)
        np.testing.assert_array_equal(part, whole)
        part, _, _ = _gpu_chunked(q, kn, vn, kp, vp, bt, lens, chunk=chunk, host=True)
        np.testing.assert_array_equal(part, whole)
    ref, _, _ = _oracle(q, kn, vn, kp, vp, bt, lens)
    check_attention(whole, ref, "chunked")


def test_prefill_host_schedule_many_items(gpu):
    """More (sequence, query tile) pairs than the kernel arguments carry: the
    host copies are then ignored and the full grid runs; both agree with the
    oracle and, bit for bit, with each other."""
    lens = [1, 3] * 400 + [70, 200]
    q, kn, vn, kp, vp, bt, _ = _setup(lens, seed=11)
    grid, _, _ = _gpu_chunked(q, kn, vn, kp, vp, bt, lens, chunk=4096)
    sched, _, _ = _gpu_chunked(q, kn, vn, kp, vp, bt, lens, chunk=4096, host=True)
    np.testing.assert_array_equal(sched, grid)
    few = [70, 200, 1, 3]
    q2, kn2, vn2, kp2, vp2, bt2, _ = _setup(few, seed=12)
    a, _, _ = _gpu_chunked(q2, kn2, vn2, kp2, vp2, bt2, few, chunk=64)
    b, _, _ = _gpu_chunked(q2, kn2, vn2, kp2, vp2, bt2, few, chunk=64, host=True)
    np.testing.assert_array_equal(a, b)
    ref, _, _ = _oracle(q, kn, vn, kp, vp, bt, lens)
    check_attention(grid, ref, "prefill many sequences")


@pytest.mark.slow
def test_config5_prefill_then_decode(gpu):
    """8 prompts U[256, 2048] prefilled in 512-token chunks, then 32 decode
    steps per sequence on the same cache.  Sampled prefill rows and the first
    and last decode steps are checked against the oracle."""
    w = W.config5(extra_tokens=32)
    lens = [int(n) for n in w.prompt_lens]
    bt = w.block_table[:, 0, :]
    kp = np.full((w.num_blocks, 16, 8, 64), W.BF16_POISON, np.uint16)
    vp = kp.copy()
    got, kpd, vpd = _gpu_chunked(w.q, w.k, w.v, kp, vp, bt, lens, chunk=512)
    S = len(lens)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    sid = np.repeat(np.arange(S), lens).astype(np.int32)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    kp_o, vp_o = paging.append(kp, vp, w.k, w.v, bt, sid, pos)
    rng = np.random.default_rng(55)
    rows = np.sort(rng.choice(starts[-1], size=96, replace=False))
    rows = np.unique(np.concatenate([rows, starts[1:] - 1, starts[:-1]]))
    refs = []
    for r in rows:
        s = int(np.searchsorted(starts, r, side="right") - 1)
        a = int(r - starts[s])
        refs.append(attention.prefill(w.q[r:r + 1], np.array([0, 1]), np.array([a]), np.array([s]), kp_o, vp_o,
                                      bt, w.scale)[0])
    check_attention(got[rows], np.stack(refs), "config5 prefill sampled rows")

    # decode phase on the same cache
    eng = DecodeEngine(kpd, vpd, w.block_table, w.prompt_lens, w.free_list, max_pos=4096)
    sids = np.arange(S, dtype=np.int32)
    for step in range(32):
        qn = W.randn_bf16(rng, (1, S, 32, 64))
        kn = W.randn_bf16(rng, (1, S, 8, 64))
        vn = W.randn_bf16(rng, (1, S, 8, 64))
        p = eng.cached[sids].copy()
        qd, kd, vd = dev_bf16(qn), dev_bf16(kn), dev_bf16(vn)
        out = torch.empty_like(qd)
        eng.step(sids, qd, kd, vd, out)
        q_rot, k_rot = rope.apply(qn[0], p), rope.apply(kn[0], p)
        kp_o, vp_o = paging.append(kp_o, vp_o, k_rot, vn[0], eng.bt_host[:, 0, :], sids, p)
        if step in (0, 31):
            torch.cuda.synchronize()
            ref = attention.decode(q_rot, kp_o, vp_o, eng.bt_host[:, 0, :], sids, eng.cached, w.scale)
            check_attention(bits(out)[0], ref, f"config5 decode step {step}")
    del kpd, vpd, eng
    torch.cuda.empty_cache()

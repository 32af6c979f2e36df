"""GPU parity for the streaming decode kernel (taken whenever the row lengths
are given on the host and the shapes fit it): the batch's blocks laid end to
end and split into one equal share per CU, so rows start and end anywhere
inside a share, rows cut by share ends are merged from per-share records, and
the fused step appends the new token from the workgroup that owns the row's
last block.  Same bar as the other decode tests: the float64 oracle within
max-abs 2e-2 / mean-abs 2e-3, appends bit-exact, and the device-length path
(per-partition kernels) within the cross-evaluation bound."""
import numpy as np
import pytest
import torch

import paged_kv_attention_17_amd as pkv
from paged_kv_attention_17_amd import workloads as W
from oracle import attention, paging, rope

from gpu_util import (abs_pool, bits, check_attention, check_close_evaluations, cross_bound, dev_bf16, dev_i32,
                      ulp_diff)

pytestmark = pytest.mark.gpu


def _batch(rng, lens, n_kv, spare=3, poison=True, perm_seed=None):
    """Pools with every row's tokens on random blocks; unused slots poisoned."""
    lens = np.asarray(lens, np.int32)
    nb = int(sum(W.blocks_for(int(n)) for n in lens)) + spare
    fill = W.BF16_POISON if poison else 0
    kp = np.full((nb, 16, n_kv, 64), fill, np.uint16)
    vp = kp.copy()
    perm = np.random.default_rng(perm_seed).permutation(nb).astype(np.int32) if perm_seed is not None \
        else rng.permutation(nb).astype(np.int32)
    width = max(W.blocks_for(int(n)) for n in lens) + 2
    bt = np.full((len(lens), width), -1, np.int32)
    k = 0
    for s, n in enumerate(lens):
        m = W.blocks_for(int(n))
        bt[s, :m] = perm[k:k + m]
        k += m
        if n:
            K = W.randn_bf16(rng, (int(n), n_kv, 64))
            V = W.randn_bf16(rng, (int(n), n_kv, 64))
            for p in range(int(n)):
                kp[bt[s, p // 16], p % 16] = K[p]
                vp[bt[s, p // 16], p % 16] = V[p]
    return kp, vp, bt


def _decode(q, kp, vp, bt, sid, lens, row_lens, ps=0):
    """Attention through the C ABI with (row_lens given) or without the host lengths."""
    qd = dev_bf16(q)
    out = torch.empty_like(qd)
    kpd, vpd = (kp, vp) if isinstance(kp, torch.Tensor) else (dev_bf16(kp), dev_bf16(vp))
    mx = int(np.max(lens)) if len(lens) else 0
    ws = pkv.decode_workspace(q.shape[0], q.shape[1], kpd.shape[2], mx, ps)
    pkv.pkv_paged_attn_decode(out, qd, kpd, vpd, dev_i32(bt), None if sid is None else dev_i32(sid),
                              dev_i32(lens), mx, 0.125, ps, ws, row_lens_host=row_lens)
    torch.cuda.synchronize()
    return bits(out)


@pytest.mark.parametrize("n_q,n_kv", [(32, 8), (16, 8), (8, 8), (16, 4), (32, 16), (16, 16)])
def test_stream_mixed_lengths(gpu, n_q, n_kv):
    """Empty, one-token, block-edge and long rows together (rows that start
    and end inside shares, rows spanning several shares)."""
    rng = np.random.default_rng(100 + n_q + n_kv)
    lens = np.array([0, 1, 15, 16, 17, 300, 511, 512, 513, 1030, 2500, 4097, 64, 999, 0, 3333], np.int32)
    kp, vp, bt = _batch(rng, lens, n_kv)
    q = W.randn_bf16(rng, (len(lens), n_q, 64))
    got = _decode(q, kp, vp, bt, None, lens, lens)
    ref = attention.decode(q, kp, vp, bt, np.arange(len(lens)), lens, 0.125)
    check_attention(got, ref, f"stream {n_q}/{n_kv}")
    assert not got[0].any() and not got[14].any()          # empty rows give zeros
    grid = _decode(q, kp, vp, bt, None, lens, None)
    bound = cross_bound(ref, attention.decode(q, kp, abs_pool(vp), bt, np.arange(len(lens)), lens, 0.125))
    check_close_evaluations(grid, got, f"stream vs per-partition {n_q}/{n_kv}", bound)


def test_stream_slot_ids_and_strided_table(gpu):
    """Batch rows reach table rows through slot ids (repeated, permuted) of a
    layer-strided table; an out-of-range slot gives a zero row."""
    rng = np.random.default_rng(7)
    lens_slot = np.array([700, 33, 2049, 1], np.int32)
    kp, vp, bt = _batch(rng, lens_slot, 8)
    bt3 = np.full((4, 3, bt.shape[1]), -1, np.int32)
    bt3[:, 1, :] = bt
    sid = np.array([2, 0, 2, 3, 1, 0], np.int32)
    q = W.randn_bf16(rng, (len(sid), 32, 64))
    row_lens = lens_slot[sid]
    qd = dev_bf16(q)
    out = torch.empty_like(qd)
    ws = pkv.decode_workspace(len(sid), 32, 8, int(lens_slot.max()))
    pkv.pkv_paged_attn_decode(out, qd, dev_bf16(kp), dev_bf16(vp), dev_i32(bt3)[:, 1, :], dev_i32(sid),
                              dev_i32(lens_slot), int(lens_slot.max()), 0.125, 0, ws, row_lens_host=row_lens)
    torch.cuda.synchronize()
    ref = attention.decode(q, kp, vp, bt, sid, lens_slot, 0.125)
    check_attention(bits(out), ref, "stream slot ids")
    # an invalid slot id: zero row, the other rows unchanged
    sid_bad = sid.copy()
    sid_bad[3] = 9
    out2 = torch.empty_like(qd)
    pkv.pkv_paged_attn_decode(out2, qd, dev_bf16(kp), dev_bf16(vp), dev_i32(bt3)[:, 1, :], dev_i32(sid_bad),
                              dev_i32(lens_slot), int(lens_slot.max()), 0.125, 0, ws,
                              row_lens_host=lens_slot[np.clip(sid_bad, 0, 3)])
    torch.cuda.synchronize()
    got2 = bits(out2)
    assert not got2[3].any()
    keep = [0, 1, 2, 4, 5]
    check_attention(got2[keep], ref[keep], "stream slot ids, one invalid")


def test_stream_many_short_rows(gpu):
    """200 one-block rows beside 56 long ones: a share would touch more rows
    than the kernel stages, so the call takes the per-partition kernels; the
    result is the same.  A batch of 256 short rows alone stays on the
    streaming kernel."""
    rng = np.random.default_rng(11)
    lens = np.concatenate([rng.integers(1, 17, size=200), np.full(56, 1024)]).astype(np.int32)
    rng.shuffle(lens)
    kp, vp, bt = _batch(rng, lens, 8, poison=False)
    q = W.randn_bf16(rng, (256, 32, 64))
    got = _decode(q, kp, vp, bt, None, lens, lens)
    ref = attention.decode(q, kp, vp, bt, np.arange(256), lens, 0.125)
    check_attention(got, ref, "short rows beside long ones")
    lens2 = rng.integers(1, 40, size=256).astype(np.int32)
    kp, vp, bt = _batch(rng, lens2, 8)
    got = _decode(q, kp, vp, bt, None, lens2, lens2)
    ref = attention.decode(q, kp, vp, bt, np.arange(256), lens2, 0.125)
    check_attention(got, ref, "256 short rows")


def test_stream_rows_on_share_edges(gpu):
    """Rows whose lengths are whole multiples of a share (on a 256-CU device
    with this total, every share edge falls on a row edge) and rows one token
    past them."""
    rng = np.random.default_rng(12)
    share_tokens = 16 * 4
    lens = np.array([share_tokens] * 40 + [2 * share_tokens] * 40 + [share_tokens + 1] * 4, np.int32)
    kp, vp, bt = _batch(rng, lens, 8)
    q = W.randn_bf16(rng, (len(lens), 32, 64))
    got = _decode(q, kp, vp, bt, None, lens, lens)
    ref = attention.decode(q, kp, vp, bt, np.arange(len(lens)), lens, 0.125)
    check_attention(got, ref, "share edges")


def _scatter(K, V, lens, nb_pool, perm_seed, fill):
    """Rows' tokens K/V [sum(lens)][n_kv][64] placed on a seeded permutation
    of a pool of nb_pool blocks (vectorised); unused slots hold `fill`."""
    n_kv = K.shape[1]
    kp = np.full((nb_pool, 16, n_kv, 64), fill, np.uint16)
    vp = kp.copy()
    perm = np.random.default_rng(perm_seed).permutation(nb_pool).astype(np.int32)
    width = max(W.blocks_for(int(n)) for n in lens) + 1
    bt = np.full((len(lens), width), -1, np.int32)
    k, t = 0, 0
    for s, n in enumerate(lens):
        n = int(n)
        m = W.blocks_for(n)
        bt[s, :m] = perm[k:k + m]
        pos = np.arange(n)
        kp[bt[s, pos // 16], pos % 16] = K[t:t + n]
        vp[bt[s, pos // 16], pos % 16] = V[t:t + n]
        k += m
        t += n
    return kp, vp, bt


def test_stream_permuted_blocks_bit_identical(gpu):
    """Bit-identity under block placement at the step's real size: 64 rows of
    U[512, 4096] tokens (about 9,000 blocks, some 35 per CU share, so every
    wave walks many blocks of several rows) on three seeded placements in the
    pool, two calls each, plain and fused: all outputs identical bit for bit
    (the summation order depends only on logical positions), and the first
    placement's output checked against the oracle on 8 sampled rows."""
    rng = np.random.default_rng(13)
    lens = rng.integers(512, 4097, size=64).astype(np.int32)
    tot = int(lens.sum())
    K = W.randn_bf16(rng, (tot, 8, 64))
    V = W.randn_bf16(rng, (tot, 8, 64))
    q = W.randn_bf16(rng, (64, 32, 64))
    nb_pool = int(sum(W.blocks_for(int(n)) for n in lens)) + 500
    qd = dev_bf16(q)
    ctx = dev_i32(lens)
    mx = int(lens.max())
    ws = pkv.decode_workspace(64, 32, 8, mx)
    tab = torch.empty((8192, 32, 2), dtype=torch.float32, device="cuda")
    pkv.pkv_rope_table_init(tab)
    kn = W.randn_bf16(rng, (64, 8, 64))
    vn = W.randn_bf16(rng, (64, 8, 64))
    kd, vd = dev_bf16(kn), dev_bf16(vn)
    plain, fused = [], []
    first = None
    for seed in (21, 22, 23):
        kp, vp, bt = _scatter(K, V, lens, nb_pool, seed, W.BF16_POISON)
        kpd, vpd, btd = dev_bf16(kp), dev_bf16(vp), dev_i32(bt)
        for _ in range(2):
            out = torch.empty_like(qd)
            pkv.pkv_paged_attn_decode(out, qd, kpd, vpd, btd, None, ctx, mx, 0.125, 0, ws, row_lens_host=lens)
            torch.cuda.synchronize()
            plain.append(bits(out))
        for _ in range(2):
            # fused (after the plain calls, which read the cache as scattered):
            # the row's last token is this step's new one, its pool row
            # rewritten with the same rotated key and value by every call
            out = torch.empty_like(qd)
            pkv.pkv_paged_decode_fused(out, qd, kd, vd, kpd, vpd, btd, None, ctx, mx, tab, 0.125, 0, ws,
                                       row_lens_host=lens)
            torch.cuda.synchronize()
            fused.append(bits(out))
        if first is None:
            first = (kp, vp, bt)
        del kpd, vpd
    for o in plain[1:]:
        np.testing.assert_array_equal(o, plain[0])
    for o in fused[1:]:
        np.testing.assert_array_equal(o, fused[0])
    kp, vp, bt = first
    rows = np.random.default_rng(24).choice(64, size=8, replace=False)
    ref = attention.decode(q[rows], kp, vp, bt, rows, lens, 0.125)
    check_attention(plain[0][rows], ref, "stream, 64 rows, placement 1")


def test_stream_fused_step_equals_separate_calls(gpu):
    """pkv_paged_decode_fused with host lengths = RoPE + append + attention:
    caches bit for bit, outputs within the cross-evaluation bound, and the
    oracle on its own cache."""
    rng = np.random.default_rng(15)
    prior = np.array([13, 0, 15, 16, 700, 2047, 31, 4095], np.int32)    # cached tokens before the step
    lens = prior + 1
    B = len(lens)
    kp, vp, bt = _batch(rng, prior, 8, spare=40)
    # the new tokens' blocks: every row gets the blocks it needs
    free = np.setdiff1d(np.arange(kp.shape[0]), bt[bt >= 0]).astype(np.int32)
    width = max(W.blocks_for(int(n)) for n in lens) + 1      # <= bt's width
    bt2 = bt[:, :width].copy()
    fi = 0
    for b in range(B):
        j = int(prior[b]) // 16
        if bt2[b, j] < 0:
            bt2[b, j] = free[fi]
            fi += 1
    qn = W.randn_bf16(rng, (B, 32, 64))
    kn = W.randn_bf16(rng, (B, 8, 64))
    vn = W.randn_bf16(rng, (B, 8, 64))
    tab = torch.empty((8192, 32, 2), dtype=torch.float32, device="cuda")
    pkv.pkv_rope_table_init(tab)
    mx = int(lens.max())
    btd, ctx = dev_i32(bt2), dev_i32(lens)
    kp1, vp1 = dev_bf16(kp), dev_bf16(vp)
    q, k, v = dev_bf16(qn), dev_bf16(kn), dev_bf16(vn)
    out1 = torch.empty_like(q)
    ws1 = pkv.decode_workspace(B, 32, 8, mx)
    pkv.pkv_paged_decode_fused(out1, q, k, v, kp1, vp1, btd, None, ctx, mx, tab, 0.125, 0, ws1, row_lens_host=lens)
    kp2, vp2 = dev_bf16(kp), dev_bf16(vp)
    q2, k2, v2 = dev_bf16(qn), dev_bf16(kn), dev_bf16(vn)
    pos = dev_i32(prior)
    pkv.pkv_rope_decode(q2, k2, pos, tab)
    pkv.pkv_paged_kv_append(kp2, vp2, k2, v2, btd, dev_i32(np.arange(B)), pos)
    out2 = torch.empty_like(q2)
    ws2 = pkv.decode_workspace(B, 32, 8, mx)
    pkv.pkv_paged_attn_decode(out2, q2, kp2, vp2, btd, None, ctx, mx, 0.125, 0, ws2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(q), qn)                  # inputs are read only
    np.testing.assert_array_equal(bits(k), kn)
    np.testing.assert_array_equal(bits(kp1), bits(kp2))
    np.testing.assert_array_equal(bits(vp1), bits(vp2))
    check_close_evaluations(bits(out1), bits(out2), "stream fused vs separate (per-partition)")
    # the separate calls with host lengths run the same streaming arithmetic:
    # identical bits
    out3 = torch.empty_like(q2)
    pkv.pkv_paged_attn_decode(out3, q2, kp2, vp2, btd, None, ctx, mx, 0.125, 0, ws2, row_lens_host=lens)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out1), bits(out3))
    q_rot = rope.apply(qn, prior)
    k_rot = rope.apply(kn, prior)
    kp_o, vp_o = paging.append(kp, vp, k_rot, vn, bt2, np.arange(B), prior)
    kdev = bits(kp1)
    for b in range(B):
        blk, row = int(bt2[b, prior[b] // 16]), int(prior[b] % 16)
        assert ulp_diff(kdev[blk, row], kp_o[blk, row]).max() <= 1
    ref = attention.decode(q_rot, kp_o, vp_o, bt2, np.arange(B), lens, 0.125)
    check_attention(bits(out1), ref, "stream fused")


def test_stream_workspace_garbage_and_reuse(gpu):
    """The workspace holds no state between calls: refilled with all-ones
    bits (NaN as float) before every call, and calls of different batches
    follow each other, including one whose rows span many shares."""
    rng = np.random.default_rng(16)
    cases = [np.array([4096, 3000, 17, 2500, 1, 4000, 999], np.int32),
             np.array([70000 // 16 * 16, 33], np.int32),
             np.array([1500] * 40, np.int32)]
    ws = pkv.decode_workspace(64, 32, 8, 70000)
    for trial in range(3):
        for lens in cases:
            kp, vp, bt = _batch(rng, lens, 8)
            q = W.randn_bf16(rng, (len(lens), 32, 64))
            ws.fill_(0xFF)
            qd = dev_bf16(q)
            out = torch.empty_like(qd)
            mx = int(lens.max())
            pkv.pkv_paged_attn_decode(out, qd, dev_bf16(kp), dev_bf16(vp), dev_i32(bt), None, dev_i32(lens), mx,
                                      0.125, 0, ws, row_lens_host=lens)
            torch.cuda.synchronize()
            ref = attention.decode(q, kp, vp, bt, np.arange(len(lens)), lens, 0.125)
            check_attention(bits(out), ref, f"garbage workspace trial {trial} B={len(lens)}")


@pytest.mark.slow
def test_stream_long_rows_several_table_slices(gpu):
    """Nine rows of 65536 tokens (36864 blocks): each wave's part of a share
    exceeds one 64-entry table slice; two rows checked against the oracle."""
    n, B = 65536, 9
    nb = B * n // 16
    kpd = torch.empty((nb, 16, 8, 64), dtype=torch.bfloat16, device="cuda")
    vpd = torch.empty_like(kpd)
    W.fill_pool_device(kpd, 51, "normal")
    W.fill_pool_device(vpd, 52, "normal")
    perm = np.random.default_rng(53).permutation(nb).astype(np.int32)
    bt = perm.reshape(B, n // 16)
    lens = np.full(B, n, np.int32)
    lens[4] = n - 5
    rng = np.random.default_rng(54)
    q = W.randn_bf16(rng, (B, 32, 64))
    got = _decode(q, kpd, vpd, bt, None, lens, lens)
    for b in (0, 4):
        idx = torch.from_numpy(bt[b].astype(np.int64)).cuda()
        K = bits(kpd.index_select(0, idx).reshape(-1, 8, 64)[:int(lens[b])])
        V = bits(vpd.index_select(0, idx).reshape(-1, 8, 64)[:int(lens[b])])
        ref = attention.dense_decode(q[b], K, V, 0.125)
        check_attention(got[b], ref, f"long row {b}")
    del kpd, vpd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("lens", [[8192], [3000, 5000], [16 * 256 * 3 + 5]])
def test_stream_few_rows_over_every_share(gpu, lens):
    """One or two rows cut into hundreds of shares: their records are merged
    by four groups of threads combined through LDS."""
    rng = np.random.default_rng(300 + sum(lens))
    lens = np.array(lens, np.int32)
    kp, vp, bt = _batch(rng, lens, 8)
    q = W.randn_bf16(rng, (len(lens), 32, 64))
    got = _decode(q, kp, vp, bt, None, lens, lens)
    ref = attention.decode(q, kp, vp, bt, np.arange(len(lens)), lens, 0.125)
    check_attention(got, ref, f"few rows {lens.tolist()}")
    bound = cross_bound(ref, attention.decode(q, kp, abs_pool(vp), bt, np.arange(len(lens)), lens, 0.125))
    check_close_evaluations(_decode(q, kp, vp, bt, None, lens, None), got, "few rows vs per-partition", bound)


def test_paged_read_probe_reads_without_writing(gpu):
    """The diagnostic read probe runs over the streaming kernel's plan
    (several rows per share, rows over several shares) and writes nothing:
    the pools are unchanged and the sink keeps its value."""
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 700, size=40).astype(np.int32)
    kp, vp, bt = _batch(rng, lens, 8, poison=False)
    kpd, vpd = dev_bf16(kp), dev_bf16(vp)
    sink = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    pkv.pkv_paged_read_probe(kpd, vpd, dev_i32(bt), None, lens, sink)
    pkv.pkv_paged_read_probe(kpd, vpd, dev_i32(bt), dev_i32(np.arange(40)[::-1].copy()), lens[::-1].copy(), sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 5
    np.testing.assert_array_equal(bits(kpd), kp)
    np.testing.assert_array_equal(bits(vpd), vp)


@pytest.mark.parametrize("row_lens", [True, False], ids=["stream", "partitions"])
def test_kv_read_policy_does_not_change_results(gpu, row_lens):
    """Both K/V read policies (non-temporal loads, and ordinary cached loads
    for shared blocks) give the same output bit for bit, on the streaming
    kernel (host lengths) and on the per-partition kernels, over rows that
    share their first blocks (a shared prompt) and rows that do not."""
    rng = np.random.default_rng(31)
    lens = np.array([700, 1500, 33, 2048, 900, 1200], np.int32)
    kp, vp, bt = _batch(rng, lens, 8)
    bt[1, :20] = bt[0, :20]          # rows 0, 1 and 4 share row 0's first 20 blocks
    bt[4, :20] = bt[0, :20]
    q = W.randn_bf16(rng, (len(lens), 32, 64))
    outs = []
    try:
        for policy in (pkv.PKV_KV_READ_REUSE, pkv.PKV_KV_READ_STREAM, pkv.PKV_KV_READ_REUSE):
            pkv.pkv_set_kv_read_policy(policy)
            outs.append(_decode(q, kp, vp, bt, None, lens, lens if row_lens else None))
    finally:
        pkv.pkv_set_kv_read_policy(pkv.PKV_KV_READ_STREAM)
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])
    ref = attention.decode(q, kp, vp, bt, np.arange(len(lens)), lens, 0.125)
    check_attention(outs[0], ref, "both read policies")

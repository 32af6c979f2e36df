"""HIP-graph capture of decode steps.

A multi-layer fused decode step whose lengths live on the device (the launch
then depends on nothing but device memory): every replay, with eager work and
synchronisations between replays, reproduces the eager outputs and caches bit
for bit.  The two-half step (pkv_decode_step_host / pkv_decode_step_device):
one capture replayed as contexts grow, each step against the oracle and the
eager pkv_decode_step."""
import numpy as np
import pytest
import torch

import paged_kv_attention_17_amd as pkv
from paged_kv_attention_17_amd import workloads as W

from oracle import attention, paging, rope

from gpu_util import bits, check_attention, check_close_evaluations, dev_bf16, dev_i32, ulp_diff

pytestmark = pytest.mark.gpu


def test_graph_replay_fused_decode_layers(gpu):
    w = W.config2(poison_unused=True, extra_steps=4)
    bt = w.block_table[:, 0, :].copy()
    free = w.free_list.copy()
    pkv.pkv_blocks_assign(bt, free, len(free), np.arange(4, dtype=np.int32), (w.context_lens - 1).astype(np.int32))
    btd, ctx = dev_i32(bt), dev_i32(w.context_lens)
    tab = torch.empty((4096, 32, 2), dtype=torch.float32, device="cuda")
    pkv.pkv_rope_table_init(tab)
    mx = int(w.context_lens.max())
    rng = np.random.default_rng(21)
    L = 3
    kp0, vp0 = dev_bf16(w.k_pool), dev_bf16(w.v_pool)
    kps = [kp0.clone() for _ in range(L)]
    vps = [vp0.clone() for _ in range(L)]
    qs = [dev_bf16(W.randn_bf16(rng, (4, 32, 64))) for _ in range(L)]
    ks = [dev_bf16(W.randn_bf16(rng, (4, 8, 64))) for _ in range(L)]
    vs = [dev_bf16(W.randn_bf16(rng, (4, 8, 64))) for _ in range(L)]
    outs = [torch.zeros_like(q) for q in qs]
    ws = pkv.decode_workspace(4, 32, 8, mx)

    def step():
        for l in range(L):
            pkv.pkv_paged_decode_fused(outs[l], qs[l], ks[l], vs[l], kps[l], vps[l], btd, None, ctx, mx, tab,
                                       w.scale, 0, ws)

    # eager reference
    step()
    torch.cuda.synchronize()
    ref_out = [bits(o) for o in outs]
    ref_kp = [bits(p) for p in kps]
    ref_vp = [bits(p) for p in vps]

    # capture (the caches start from the same state as the eager step)
    for l in range(L):
        kps[l].copy_(kp0)
        vps[l].copy_(vp0)
        outs[l].zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    scratch = torch.zeros_like(outs[0])
    for r in range(3):
        for o in outs:
            o.zero_()
        # unrelated eager work between replays
        pkv.pkv_paged_attn_decode(scratch, qs[0], kp0, vp0, btd, None, ctx, mx, w.scale, 0,
                                  pkv.decode_workspace(4, 32, 8, mx))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            np.testing.assert_array_equal(bits(outs[l]), ref_out[l], err_msg=f"replay {r} layer {l}")
            np.testing.assert_array_equal(bits(kps[l]), ref_kp[l], err_msg=f"replay {r} layer {l} K")
            np.testing.assert_array_equal(bits(vps[l]), ref_vp[l], err_msg=f"replay {r} layer {l} V")
    del g


# ----------------------------------------------- two-half step, replayed --

def _oracle_step(kp_o, vp_o, bt_host, sids, pos, qn, kn, vn, lens, scale):
    """The step on the oracle's own cache: per layer, its rotation, its append
    and attention over the layer's table view."""
    outs = []
    for l in range(qn.shape[0]):
        bt = bt_host[:, l, :]
        q_rot, k_rot = rope.apply(qn[l], pos), rope.apply(kn[l], pos)
        kp_o, vp_o = paging.append(kp_o, vp_o, k_rot, vn[l], bt, sids, pos)
        outs.append(attention.decode(q_rot, kp_o, vp_o, bt, sids, lens, scale))
    return kp_o, vp_o, outs


# contexts (the first step's lengths, new token included), layers, steps,
# whether the replayed launches serve the rows
GRAPH_CASES = {
    # slots permuted every step; three rows open a block during the walk
    "growing": ([15, 16, 17, 33, 200, 47], 3, 6, True),
    # one block per share, the cut row's (row, head) pairs past what one pass
    # of the prologue merge covers
    "short": ([16, 16, 16, 17], 3, 3, True),
    # few rows, one long: shares grow until every row spans at most 8
    "long": ([17, 14, 300, 1000], 2, 4, True),
    # shares large enough for the long row would touch more than 4 short rows:
    # the step runs eagerly
    "fallback": ([1000] + [9] * 10, 2, 2, False),
    # one layer: equal shares, rows spanning many shares, merged per query
    # head (as the eager step does for these rows)
    "one layer": ([17, 14, 300, 1000], 1, 4, True),
    # one layer, one row over two shares: the eager step merges it per KV
    # head, the replay per query head (the same records in another order of
    # operations: within the bound on two evaluations, not bit for bit)
    "one row": ([17], 1, 3, True),
}


@pytest.mark.parametrize("case", list(GRAPH_CASES))
def test_graph_step_replays_match_oracle_and_eager(gpu, case):
    """The device half captured once and replayed as the contexts grow: every
    step is checked against the oracle on its own cache (per layer) and
    against the eager pkv_decode_step on a second engine, bit for bit (the
    same plan rule, so the same arithmetic)."""
    from paged_kv_attention_17_amd.engine import DecodeEngine, GraphStep
    ctx, L, n_steps, served = GRAPH_CASES[case]
    w = W.make_decode(1800 + len(ctx), ctx, n_layers=L, extra_steps=n_steps, poison_unused=True)
    B = w.batch
    engines = []
    for _ in range(2):
        engines.append(DecodeEngine(dev_bf16(w.k_pool), dev_bf16(w.v_pool), w.block_table, w.context_lens - 1,
                                    w.free_list, max_pos=4096))
    eg, ee = engines
    gs = GraphStep(eg, B)
    kp_o, vp_o = w.k_pool.copy(), w.v_pool.copy()
    fresh = np.zeros(w.k_pool.shape[:2], bool)          # (block, row) written by a step
    rng = np.random.default_rng(7)
    for step in range(n_steps):
        sids = rng.permutation(B).astype(np.int32) if case == "growing" else np.arange(B, dtype=np.int32)
        qn = W.randn_bf16(rng, (L, B, 32, 64))
        kn = W.randn_bf16(rng, (L, B, 8, 64))
        vn = W.randn_bf16(rng, (L, B, 8, 64))
        pos = eg.cached[sids].copy()
        gs.q.copy_(dev_bf16(qn))
        gs.k.copy_(dev_bf16(kn))
        gs.v.copy_(dev_bf16(vn))
        print(f"{case} step {step}: lengths {(pos + 1).tolist()}", flush=True)
        replayed = gs.step(sids)
        assert replayed == served, f"step {step}: replayed {replayed}"
        out_e = torch.empty_like(gs.out)
        ee.step(sids, dev_bf16(qn), dev_bf16(kn), dev_bf16(vn), out_e)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(eg.bt_host, ee.bt_host)
        np.testing.assert_array_equal(eg.cached, ee.cached)
        assert eg.n_free == ee.n_free
        np.testing.assert_array_equal(eg.meta_view(B).cpu().numpy(), ee.meta_view(B).cpu().numpy())
        np.testing.assert_array_equal(eg.bt_dev.cpu().numpy(), eg.bt_host)
        # bit for bit against the eager step
        if case == "one row":
            check_close_evaluations(bits(gs.out), bits(out_e), f"{case} step {step} vs eager")
        else:
            np.testing.assert_array_equal(bits(gs.out), bits(out_e), err_msg=f"step {step} outputs")
        np.testing.assert_array_equal(bits(eg.k_pool), bits(ee.k_pool), err_msg=f"step {step} K pool")
        np.testing.assert_array_equal(bits(eg.v_pool), bits(ee.v_pool), err_msg=f"step {step} V pool")
        # against the oracle on its own cache
        kp_o, vp_o, refs = _oracle_step(kp_o, vp_o, eg.bt_host, sids, pos, qn, kn, vn, eg.cached, w.scale)
        got = bits(gs.out)
        for l in range(L):
            check_attention(got[l], refs[l], f"{case} step {step} layer {l}")
        # the caches: V bit for bit; K bit for bit except the rows the steps
        # rotated and appended, each within one ulp of the oracle's rotation
        np.testing.assert_array_equal(bits(eg.v_pool), vp_o)
        for l in range(L):
            for b, s in enumerate(sids):
                fresh[int(eg.bt_host[s, l, pos[b] // 16]), int(pos[b] % 16)] = True
        kdev = bits(eg.k_pool)
        np.testing.assert_array_equal(kdev[~fresh], kp_o[~fresh])
        assert ulp_diff(kdev[fresh], kp_o[fresh]).max() <= 1
    assert gs.replays == (n_steps if served else 0)

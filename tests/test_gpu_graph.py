"""HIP-graph capture of a multi-layer fused decode step whose lengths live on
the device (the launch then depends on nothing but device memory): every
replay, with eager work and synchronisations between replays, reproduces the
eager outputs and caches bit for bit."""
import numpy as np
import pytest
import torch

import paged_kv_attention_17_amd as pkv
from paged_kv_attention_17_amd import workloads as W

from gpu_util import bits, dev_bf16, dev_i32

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

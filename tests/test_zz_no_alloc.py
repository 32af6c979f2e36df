"""GPU parity of the allocation-free decode entry point
(pkv_paged_decode_fused_noalloc, whose partial records live in the
library's device array) against pkv_paged_decode_fused with a caller
workspace, on the same inputs: two calls in a row, the second with a
smaller batch, through the streaming kernel (host row lengths) and the
per-partition kernels (device lengths only).  Both run the same kernels in
the same order, so outputs and caches must agree bit for bit (stronger than
the attention tolerance); the first call is also checked against the
float64 oracle on sampled rows."""
import numpy as np
import pytest
import torch

import paged_kv_attention_17_amd as pkv
from paged_kv_attention_17_amd import workloads as W
from oracle import attention, paging, rope

from gpu_util import bits, check_attention, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu


def _case(seed, B, lo, hi):
    rng = np.random.default_rng(seed)
    prior = rng.integers(lo, hi, size=B).astype(np.int32)       # cached tokens before the step
    lens = prior + 1
    nbs = [W.blocks_for(int(n)) for n in lens]
    nb = sum(nbs) + 7
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((B, max(nbs) + 1), -1, np.int32)
    k = 0
    for b, m in enumerate(nbs):
        bt[b, :m] = perm[k:k + m]
        k += m
    kp = np.full((nb, 16, 8, 64), W.BF16_POISON, np.uint16)
    vp = kp.copy()
    for b, n in enumerate(prior):
        n = int(n)
        pos = np.arange(n)
        kp[bt[b, pos // 16], pos % 16] = W.randn_bf16(rng, (n, 8, 64))
        vp[bt[b, pos // 16], pos % 16] = W.randn_bf16(rng, (n, 8, 64))
    q = W.randn_bf16(rng, (B, 32, 64))
    kn = W.randn_bf16(rng, (B, 8, 64))
    vn = W.randn_bf16(rng, (B, 8, 64))
    return prior, lens, bt, kp, vp, q, kn, vn


@pytest.mark.parametrize("host_lens", [True, False])
def test_noalloc_matches_workspace_call(gpu, host_lens):
    tab = torch.empty((8192, 32, 2), dtype=torch.float32, device="cuda")
    pkv.pkv_rope_table_init(tab)
    for call, (seed, B, lo, hi) in enumerate(((61, 64, 512, 4096), (62, 8, 10, 700))):
        prior, lens, bt, kp, vp, q, kn, vn = _case(seed, B, lo, hi)
        mx = int(lens.max())
        rl = lens if host_lens else None
        btd, ctx = dev_i32(bt), dev_i32(lens)
        qd, kd, vd = dev_bf16(q), dev_bf16(kn), dev_bf16(vn)
        kp1, vp1, kp2, vp2 = dev_bf16(kp), dev_bf16(vp), dev_bf16(kp), dev_bf16(vp)
        out1, out2 = torch.empty_like(qd), torch.empty_like(qd)
        ws = pkv.decode_workspace(B, 32, 8, mx)
        print(f"call {call}: B={B}, host lengths {host_lens}", flush=True)
        pkv.pkv_paged_decode_fused(out1, qd, kd, vd, kp1, vp1, btd, None, ctx, mx, tab, 0.125, 0, ws,
                                   row_lens_host=rl)
        pkv.pkv_paged_decode_fused_noalloc(out2, qd, kd, vd, kp2, vp2, btd, None, ctx, mx, tab, 0.125,
                                           row_lens_host=rl)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(out1), bits(out2))
        np.testing.assert_array_equal(bits(kp1), bits(kp2))
        np.testing.assert_array_equal(bits(vp1), bits(vp2))
        if call == 0:
            rows = np.random.default_rng(seed).choice(B, size=6, replace=False)
            q_rot = rope.apply(q, prior)
            k_rot = rope.apply(kn, prior)
            kp_o, vp_o = paging.append(kp, vp, k_rot, vn, bt, np.arange(B), prior)
            ref = attention.decode(q_rot[rows], kp_o, vp_o, bt, rows, lens, 0.125)
            check_attention(bits(out2)[rows], ref, f"no-alloc decode, host lengths {host_lens}")
        del kp1, vp1, kp2, vp2

#!/usr/bin/env python3
"""Paged decode attention bench on one MI355X.

Workload: B=64 sequences, 16 layers, contexts uniform in [512, 4096], 32 query
/ 8 KV heads, head_dim 64, bf16 16-token blocks in a pool of 1.25x the blocks
needed with tables interleaved round-robin over (layer, sequence).  One step
= one decode step of all 16 layers through the native pkv_decode_step: host
block allocation, then per layer RoPE on the new q/k, KV append and paged
attention fused into one call: the streaming kernel (one workgroup per CU
over an equal share of all blocks) plus a small kernel that merges the rows
cut by share ends.  Inputs are seeded synthetic
data resident in HBM before timing starts; contexts grow by one token per
step as in a real decode loop.

Prints ONE JSON line:
  value        KV GB/s over the whole step = algorithmic KV bytes of all
               layers / step wall time (2,048 B per context token per layer)
  roofline     the streaming decode launch of the step: algorithmic KV
               bytes per launch / (step time / layers), an upper bound on
               its mean duration (HIP events on its stream around the timed
               steps); the standalone fused call (streaming kernel + its own
               merge, 16 back to back) is reported beside it
  graph_steps  configs 1, 2 and 3: eager pkv_decode_step vs the two-half step
               replayed from captured graphs, us/step
  cpu_baseline the float64 CPU oracle on a bounded sample of the same step
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KV_BYTES_PER_TOKEN = 8 * 64 * 2 * 2          # per layer: 8 KV heads x 64 dims x bf16 x (K and V)
METRIC = "paged decode attn: KV GB/s (% of HBM peak) and us/step at B=64 per layer"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_source_hash() -> str:
    """Hash of the decode kernels' sources with comments and whitespace
    removed, so that a counter summary stays valid across comment edits and
    only a code change invalidates it."""
    h = hashlib.sha256()
    for f in ("decode_stream.hip", "decode.hip", "attn_block.h", "common.h"):
        with open(os.path.join(ROOT, "paged_kv_attention_17_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(src_hash: str):
    """HBM bytes per attention launch from the committed counter summary,
    if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "decode_attn_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != src_hash:
        return None
    return t.get("hbm_bytes_per_launch")


def stream_copy_gbs(torch, nbytes=2 << 30, iters=10):
    """Achievable bandwidth of a plain device-to-device copy (read + write)."""
    a = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(2):
        b.copy_(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(iters):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / 1e3 / iters
    del a, b
    return 2 * nbytes / t / 1e9


def stream_read_gbs(torch, pkv, nbytes=4 << 30, iters=10):
    """Achievable HBM read rate: the library's grid-stride read probe over a
    buffer 16x the 256 MB last-level cache, read once per iteration."""
    a = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        pkv.pkv_hbm_read_probe(a, sink)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(iters):
        pkv.pkv_hbm_read_probe(a, sink)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / 1e3 / iters
    del a, sink
    return nbytes / t / 1e9


def unfused_layer_us(torch, np, pkv, eng, q, k, v, out, stream, iters=3):
    """The unfused decode of one layer at the same point: the RoPE kernel, the
    append kernel and the attention call, each timed over its 16 layers'
    launches back to back (one event pair per kernel and pass, per-launch time
    = interval / 16), queued behind a device-side wait so that the host has
    enqueued them before the GPU starts: the figures are GPU time, not the
    host's launch latency.  Works on copies of q/k so the step's inputs stay
    as they are, and re-appends the tokens of the last step (the cache is
    unchanged)."""
    L = q.shape[0]
    B = q.shape[1]
    pos = torch.from_numpy((eng.cached[:B] - 1).astype(np.int32)).cuda()
    sid = torch.arange(B, dtype=torch.int32, device="cuda")
    ctx_now = eng.cached.copy()
    t = {"rope": [], "append": [], "attention": []}
    for it in range(iters + 1):
        qc, kc = q.clone(), k.clone()
        torch.cuda.synchronize()
        torch.cuda._sleep(10_000_000)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(stream)
        for layer in range(L):
            pkv.pkv_rope_decode(qc[layer], kc[layer], pos, eng.cos_sin, stream=stream)
        ev[1].record(stream)
        for layer in range(L):
            pkv.pkv_paged_kv_append(eng.k_pool, eng.v_pool, kc[layer], v[layer], eng.bt_dev[:, layer, :], sid, pos,
                                    stream=stream)
        ev[2].record(stream)
        for layer in range(L):
            pkv.pkv_paged_attn_decode(out[layer], qc[layer], eng.k_pool, eng.v_pool, eng.bt_dev[:, layer, :], None,
                                      eng.ctx_dev, eng.max_context_len, eng.scale, eng.partition_size,
                                      eng.workspace, stream=stream, row_lens_host=ctx_now)
        ev[3].record(stream)
        torch.cuda.synchronize()
        if it > 0:
            for i, kname in enumerate(("rope", "append", "attention")):
                t[kname].append(ev[i].elapsed_time(ev[i + 1]) * 1e3 / L)
    return {kname: round(float(np.median(v_)), 2) for kname, v_ in t.items()}


def cpu_baseline(eng, q_host, seconds: float, threads: int):
    """Time the float64 oracle (as it stands) on layer-by-layer samples of the
    step: sequences are gathered into a compact host pool (not timed), then
    oracle.attention.decode runs on them until `seconds` have passed, with
    NumPy's BLAS limited to `threads` threads."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    from oracle import attention
    rng = np.random.default_rng(0)
    done_bytes = 0
    t_total = 0.0
    n_rows = 0
    with threadpool_limits(limits=threads):
        while t_total < seconds:
            layer = int(rng.integers(eng.n_layers))
            rows = rng.choice(eng.n_slots, size=4, replace=False).astype(np.int32)
            ctx = eng.cached[rows].astype(np.int32)
            nbs = [-(-int(c) // 16) for c in ctx]
            ids = np.concatenate([eng.bt_host[r, layer, :n] for r, n in zip(rows, nbs)]).astype(np.int64)
            idx = torch.from_numpy(ids).cuda()
            kp = eng.k_pool.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
            vp = eng.v_pool.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
            bt = np.full((4, max(nbs)), -1, np.int32)
            o = 0
            for i, n in enumerate(nbs):
                bt[i, :n] = np.arange(o, o + n)
                o += n
            q = q_host[layer, rows]
            t0 = time.perf_counter()
            attention.decode(q, kp, vp, bt, np.arange(4), ctx, eng.scale)
            t_total += time.perf_counter() - t0
            done_bytes += int(ctx.sum()) * KV_BYTES_PER_TOKEN
            n_rows += 4
    return {"value": done_bytes / t_total / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_rows} (sequence, layer) rows of the B=64 16-layer step, float64 numpy oracle "
                      f"(gather through the block table + two-pass softmax), BLAS limited to {threads} "
                      f"thread(s), {t_total:.1f} s of wall time"}


def prefill_leg(torch, np, pkv, W, iters: int = 5):
    """Chunked causal prefill of the 8-prompt workload (lengths U[256, 2048],
    512-token chunks): every chunk's K/V is appended, then all sequences' i-th
    chunks go through one pkv_paged_attn_prefill call (the 4 calls of a pass
    back to back).  Returns the median time of a pass's prefill calls and the
    causal-triangle flops."""
    w = W.config5(extra_tokens=32)
    lens = [int(n) for n in w.prompt_lens]
    kp = torch.zeros((w.num_blocks, 16, 8, 64), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    btd = torch.from_numpy(w.block_table[:, 0, :].copy()).cuda()
    qd = torch.from_numpy(w.q.view(np.int16)).cuda().view(torch.bfloat16)
    kd = torch.from_numpy(w.k.view(np.int16)).cuda().view(torch.bfloat16)
    vd = torch.from_numpy(w.v.view(np.int16)).cuda().view(torch.bfloat16)
    starts = np.concatenate([[0], np.cumsum(lens)])
    chunk = 512
    calls = []
    for c in range(max(-(-n // chunk) for n in lens)):
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
        i32 = lambda x: torch.tensor(x, dtype=torch.int32, device="cuda")  # noqa: E731
        calls.append(dict(q=qd[r].contiguous(), k=kd[r].contiguous(), v=vd[r].contiguous(), sid=i32(sid),
                          pos=i32(pos), cu=i32(cu), qs=i32(qs), seqs=i32(seqs), mq=int(np.diff(cu).max()),
                          cu_h=np.array(cu, np.int32), qs_h=np.array(qs, np.int32)))
    stream = torch.cuda.current_stream()
    outs = [torch.empty_like(cl["q"]) for cl in calls]
    times = []
    for it in range(iters + 1):
        # the chunks' K/V first (appending the same rows again leaves the
        # cache as it is), then a short device-side wait, so that all chunk
        # calls are already queued when the events around them run: the
        # events then time the prefill kernels back to back, not the host's
        # launch latency
        for cl in calls:
            pkv.pkv_paged_kv_append(kp, vp, cl["k"], cl["v"], btd, cl["sid"], cl["pos"])
        torch.cuda.synchronize()
        torch.cuda._sleep(200000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for cl, out in zip(calls, outs):
            pkv.pkv_paged_attn_prefill(out, cl["q"], cl["cu"], cl["qs"], cl["seqs"], kp, vp, btd, cl["mq"], w.scale,
                                       cu_q_lens_host=cl["cu_h"], q_start_host=cl["qs_h"])
        e1.record(stream)
        torch.cuda.synchronize()
        if it > 0:
            times.append(e0.elapsed_time(e1) / 1e3)
    pairs = sum(n * (n + 1) // 2 for n in lens)
    flops = pairs * 32 * 64 * 2 * 2          # QK and PV, multiply-add = 2 flops
    t = float(np.median(times))
    del kp, vp
    return {"workload": "chunked causal prefill, 8 prompts U[256,2048] (sum %d tokens), 512-token chunks, "
                        "32q/8kv heads, d=64, bf16" % sum(lens),
            "calls": len(calls), "us_per_pass": round(t * 1e6, 2), "flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(flops / t / 1e12, 2), "peak": 2500.0, "unit": "TFLOP/s",
                         "frac": round(flops / t / 1e12 / 2500.0, 4), "traffic": None,
                         "kernel": "pkv_paged_attn_prefill (prefill_kernel<4>)"}}


def long_context_leg(torch, np, pkv, W, iters: int = 10, cpu_seconds: float = 0.0):
    """Split-context decode at B=256 with 8,192 tokens each (4.29 GB of K/V,
    one layer, more than 16x the last-level cache): the streaming kernel and
    its merge (host lengths given) and the per-partition kernels (lengths on
    the device only), each timed with HIP events around back-to-back calls.
    With cpu_seconds > 0 the float64 oracle is also timed on sampled whole
    sequences of the same call (BLAS threads = the host's cores) and its rate
    extrapolated to the call."""
    w = W.config4(fill_pool=False)
    kp = torch.empty((w.num_blocks, 16, 8, 64), dtype=torch.bfloat16, device="cuda").normal_()
    vp = torch.empty_like(kp).uniform_(-1, 1)
    bt = torch.from_numpy(w.block_table[:, 0, :].copy()).cuda()
    ctx = w.context_lens.astype(np.int32)
    ctxd = torch.from_numpy(ctx).cuda()
    q = torch.from_numpy(w.q_new[0].view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty_like(q)
    B, mx = q.shape[0], int(ctx.max())
    ws = torch.empty(pkv.pkv_decode_workspace_bytes(B, 32, 8, 64, mx, 0) // 4 + 64, dtype=torch.int32, device="cuda")
    nbytes = int(ctx.sum()) * KV_BYTES_PER_TOKEN
    res = {"workload": "decode attention, B=256, context 8192 each, 32q/8kv heads, d=64, bf16 16-token blocks, "
                       "one layer", "bytes_per_call": nbytes}
    for name, rl in (("stream", ctx), ("partitions", None)):
        run = lambda: pkv.pkv_paged_attn_decode(out, q, kp, vp, bt, None, ctxd, mx, w.scale, 0, ws,  # noqa: E731
                                                row_lens_host=rl)
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            run()
        e1.record()
        e1.synchronize()
        t = e0.elapsed_time(e1) / 1e3 / iters
        res[name] = {"us_per_call": round(t * 1e6, 1), "GBps": round(nbytes / t / 1e9, 1),
                     "frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
    if cpu_seconds > 0:
        from threadpoolctl import threadpool_limits
        from oracle import attention
        rng = np.random.default_rng(4)
        q_host = w.q_new[0]
        t_cpu, n_seq, done = 0.0, 0, 0
        cores = len(os.sched_getaffinity(0))
        with threadpool_limits(limits=cores):
            while t_cpu < cpu_seconds and n_seq < 64:
                b = int(rng.integers(B))
                n = int(ctx[b])
                ids = torch.from_numpy(w.block_table[b, 0, :-(-n // 16)].astype(np.int64)).cuda()
                kh = kp.index_select(0, ids).view(torch.int16).cpu().numpy().view(np.uint16)
                vh = vp.index_select(0, ids).view(torch.int16).cpu().numpy().view(np.uint16)
                bt1 = np.arange(len(kh), dtype=np.int32)[None]
                t0 = time.perf_counter()
                attention.decode(q_host[b:b + 1], kh, vh, bt1, np.zeros(1, np.int32), np.array([n], np.int32),
                                 w.scale)
                t_cpu += time.perf_counter() - t0
                done += n * KV_BYTES_PER_TOKEN
                n_seq += 1
        res["cpu_oracle"] = {"value": round(done / t_cpu / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                             "sample": f"{n_seq} whole sequences of the call (8,192 tokens each), float64 numpy "
                                       f"oracle, BLAS limited to {cores} threads, {t_cpu:.1f} s of wall time; "
                                       f"extrapolated call time {nbytes / (done / t_cpu):.1f} s"}
    del kp, vp
    torch.cuda.empty_cache()
    return res


def prefix_sharing_leg(torch, np, pkv, W, iters: int = 10):
    """Decode attention where the 64 rows continue 4 shared 2,048-token
    prompts with private tails U[64, 1024] (16 layers, each with its own
    blocks; the rows of one prompt list the same prompt blocks), timed like
    the main step's attention (16 layers back to back, host lengths given).
    Beside it: the same rows with every block private (no sharing), and the
    copy on write of every row's last block in all 16 layers
    (pkv_blocks_copy, 1,024 block pairs)."""
    L = 16
    w = W.shared_prefix(n_layers=L, fill_pool=False)
    B = len(w.context_lens)
    ctx = w.context_lens.astype(np.int32)
    ctxd = torch.from_numpy(ctx).cuda()
    q = torch.from_numpy(w.q.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty_like(q)
    mx = int(ctx.max())
    ws = torch.empty(pkv.pkv_decode_workspace_bytes(B, 32, 8, 64, mx, 0) // 4 + 64, dtype=torch.int32, device="cuda")
    logical = int(ctx.sum()) * KV_BYTES_PER_TOKEN
    tails = ctx - w.prompt_len
    unique = (w.n_prompts * w.prompt_len + int(tails.sum())) * KV_BYTES_PER_TOKEN
    res = {"workload": "decode attention, B=64 rows over 4 shared 2048-token prompts + private tails U[64,1024], "
                       "16 layers, 32q/8kv heads, d=64, bf16 16-token blocks",
           "mean_context": round(float(ctx.mean()), 1), "logical_bytes_per_layer": logical,
           "unique_bytes_per_layer": unique}

    def timed(kp, vp, bts):
        run = lambda: [pkv.pkv_paged_attn_decode(out, q, kp, vp, bt, None, ctxd, mx, 0.125, 0, ws,  # noqa: E731
                                                 row_lens_host=ctx) for bt in bts]
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            run()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / 1e3 / (iters * L)

    extra = B * L                       # destination blocks of the copy-on-write leg
    kp = torch.empty((w.num_blocks + extra, 16, 8, 64), dtype=torch.bfloat16, device="cuda").normal_()
    vp = torch.empty_like(kp).normal_()
    bts = [torch.from_numpy(np.ascontiguousarray(w.block_table[:, l, :])).cuda() for l in range(L)]
    # rows that share blocks read them with cached loads (the default
    # non-temporal loads are for tables without shared blocks)
    t_stream = timed(kp, vp, bts)
    pkv.pkv_set_kv_read_policy(pkv.PKV_KV_READ_REUSE)
    try:
        t = timed(kp, vp, bts)
    finally:
        pkv.pkv_set_kv_read_policy(pkv.PKV_KV_READ_STREAM)
    res["shared"] = {"us_per_layer": round(t * 1e6, 2), "logical_GBps": round(logical / t / 1e9, 1),
                     "unique_GBps": round(unique / t / 1e9, 1), "unique_frac": round(unique / t / 1e9 / HBM_PEAK_GBS, 4),
                     "kv_read_policy": "reuse", "us_per_layer_stream_policy": round(t_stream * 1e6, 2)}

    last = (ctx + 15) // 16 - 1
    src = np.concatenate([w.block_table[np.arange(B), l, last] for l in range(L)]).astype(np.int32)
    dst = np.arange(w.num_blocks, w.num_blocks + extra, dtype=np.int32)
    pkv.pkv_blocks_copy(kp, vp, src, dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        pkv.pkv_blocks_copy(kp, vp, src, dst)
    e1.record()
    e1.synchronize()
    tc = e0.elapsed_time(e1) / 1e3 / iters
    moved = 2 * extra * 2 * 16 * 8 * 64 * 2     # read + write, K and V
    res["copy_on_write"] = {"pairs": extra, "us": round(tc * 1e6, 2), "GBps": round(moved / tc / 1e9, 1)}
    del kp, vp, bts

    # the same rows with private blocks only
    nbp = int(((ctx + 15) // 16).sum())
    perm = np.random.Generator(np.random.PCG64(w.seed)).permutation(nbp * L).astype(np.int32)
    kp = torch.empty((nbp * L, 16, 8, 64), dtype=torch.bfloat16, device="cuda").normal_()
    vp = torch.empty_like(kp).normal_()
    bts, k = [], 0
    for _ in range(L):
        bt = np.full(w.block_table.shape[::2], -1, np.int32)
        for b in range(B):
            n = int((ctx[b] + 15) // 16)
            bt[b, :n] = perm[k:k + n]
            k += n
        bts.append(torch.from_numpy(bt).cuda())
    t = timed(kp, vp, bts)
    res["private"] = {"us_per_layer": round(t * 1e6, 2), "GBps": round(logical / t / 1e9, 1),
                      "frac": round(logical / t / 1e9 / HBM_PEAK_GBS, 4)}
    del kp, vp, bts
    torch.cuda.empty_cache()
    return res


def serving_leg(torch, np, pkv, W, n_req: int = 128, n_slots: int = 64, budget: int = 2048, new_tokens: int = 32):
    """Continuous batching end to end: n_req requests with prompts U[256, 2048]
    (the chunked-prefill workload's distribution) and new_tokens tokens each,
    all queued at the start, served by the native scheduler (pkv_sched_next)
    and run on the device (pkv_sched_run) over 16 layers, n_slots slots and a
    per-iteration token budget.  q/k/v are seeded device tensors reused every
    iteration (inputs resident in HBM).  Timed with HIP events from the first
    iteration to the last."""
    L, NQ, NKV, D = 16, 32, 8, 64
    rng = np.random.default_rng(1707)
    prompts = rng.integers(256, 2049, size=n_req)
    max_blocks = -(-(2048 + new_tokens) // 16)            # longest prompt of either mix + new tokens
    num_blocks = n_slots * L * max_blocks
    dev = torch.device("cuda")
    kp = torch.zeros((num_blocks, 16, NKV, D), dtype=torch.bfloat16, device=dev)
    vp = torch.zeros_like(kp)
    g = torch.Generator(device=dev)
    g.manual_seed(1707)
    mk = lambda h: [torch.randn((budget, h, D), generator=g, device=dev).to(torch.bfloat16)  # noqa: E731
                    for _ in range(L)]
    q, k, v = mk(NQ), mk(NKV), mk(NKV)
    out = [torch.empty_like(t) for t in q]
    cos_sin = torch.empty((4096, D // 2, 2), dtype=torch.float32, device=dev)
    pkv.pkv_rope_table_init(cos_sin)
    ws = pkv.decode_workspace(n_slots, NQ, NKV, max_blocks * 16)
    stream = torch.cuda.current_stream()

    def job(lens, news, tokens=None):
        s = pkv.Scheduler(n_slots, L, max_blocks, num_blocks, budget)
        for i, (p, n) in enumerate(zip(lens, news)):
            s.submit(i, int(p), int(n), tokens=None if tokens is None else tokens[i])
        bt = torch.full((n_slots, L, max_blocks), -1, dtype=torch.int32, device=dev)
        meta = torch.zeros(s.info()["meta_elems"], dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        iters, plan, host, dec_rows, pre_rows = 0, 0.0, 0.0, 0, 0
        while True:
            t0 = time.perf_counter()
            it = s.next()
            t1 = time.perf_counter()
            if it["n_tokens"] == 0 and len(it["patch_off"]) == 0:
                break
            s.run(q, k, v, out, kp, vp, bt, meta, cos_sin, 0.125, ws, stream=stream)
            plan += t1 - t0
            host += time.perf_counter() - t0
            iters += 1
            dec_rows += it["n_decode"]
            pre_rows += it["n_tokens"] - it["n_decode"]
        e1.record(stream)
        torch.cuda.synchronize()
        hits = s.info()["cache_hit_tokens"]
        s.close()
        return e0.elapsed_time(e1) / 1e3, iters, plan, host, dec_rows, pre_rows, hits

    job([300, 40, 1000], [3, 3, 3])                      # warm-up (kernels loaded, caches touched)
    t, iters, plan, host, dec_rows, pre_rows, _ = job(prompts, [new_tokens] * n_req)
    # the same serving run where every prompt opens with one of 4 shared
    # 1,024-token system prompts (then a private part U[64, 1024]): with token
    # ids (prefix cache on) and without (every prompt prefilled in full)
    sys_prompts = rng.integers(0, 128000, size=(4, 1024)).astype(np.int32)
    toks = [np.concatenate([sys_prompts[int(rng.integers(0, 4))],
                            rng.integers(0, 128000, size=int(rng.integers(64, 1025)))]).astype(np.int32)
            for _ in range(n_req)]
    lens_sp = [len(x) for x in toks]
    t_on, it_on, _, _, dec_on, pre_on, hits = job(lens_sp, [new_tokens] * n_req, toks)
    t_off, it_off, _, _, dec_off, pre_off, _ = job(lens_sp, [new_tokens] * n_req)
    del kp, vp
    shared = {"workload": f"{n_req} requests, prompts = one of 4 shared 1024-token system prompts + U[64,1024] "
                          f"private tokens (sum {sum(lens_sp)}), {new_tokens} new tokens each, same slots, budget "
                          "and layers",
              "cache_on": {"seconds": round(t_on, 4), "iterations": it_on, "prefill_tokens": pre_on,
                           "reused_prompt_tokens": int(hits),
                           "output_tokens_per_s": round(n_req * new_tokens / t_on, 1)},
              "cache_off": {"seconds": round(t_off, 4), "iterations": it_off, "prefill_tokens": pre_off,
                            "output_tokens_per_s": round(n_req * new_tokens / t_off, 1)},
              "speedup": round(t_off / t_on, 3)}
    return {"workload": f"continuous batching, {n_req} requests, prompts U[256,2048] (sum {int(prompts.sum())} "
                        f"tokens), {new_tokens} new tokens each, {n_slots} slots, {budget}-token budget, 16 layers, "
                        "32q/8kv heads, d=64, bf16 16-token blocks",
            "seconds": round(t, 4), "iterations": iters,
            "prefill_tokens": pre_rows, "decode_rows": dec_rows,
            "tokens_per_s": round((pre_rows + dec_rows) / t, 1),
            "output_tokens_per_s": round(n_req * new_tokens / t, 1),
            "gpu_us_per_iteration": round(t / max(iters, 1) * 1e6, 1),
            "plan_us_per_iteration": round(plan / max(iters, 1) * 1e6, 1),
            "host_us_per_iteration": round(host / max(iters, 1) * 1e6, 1),
            "shared_prompts": shared}


def graph_leg(torch, np, W, eng3, q3, k3, v3, stream, steps_small: int = 200, steps3: int = 20):
    """Configs 1, 2 and 3: back-to-back decode steps through the eager
    pkv_decode_step against the two-half step (native host half, then the
    replay of a captured graph: staging copy, apply, one fused launch per
    layer, one merge), us/step from HIP events around the steps and host wall
    time.  Configs 1 and 2 (one layer) run on two engines from the same
    start; config 3 runs eager then replayed steps on the main engine (the
    contexts differ by the eager steps' tokens).  The GPU side alone: a few
    eager steps, and replays of the last staged step, queued behind a spin
    kernel (None when the host could not enqueue them before it ended)."""
    from paged_kv_attention_17_amd.engine import DecodeEngine, GraphStep

    def timed(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n, (time.perf_counter() - w0) * 1e6 / n

    # GPU-side time per step: n steps queued behind a spin kernel, so that the
    # host has enqueued them all before the GPU starts on them (checked: the
    # enqueue must end before the spin does)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    torch.cuda._sleep(10_000_000)
    e1.record(stream)
    torch.cuda.synchronize()
    spin_ms_per_cycle = e0.elapsed_time(e1) / 1e7

    def gpu_only(fn, n, spin_ms):
        fn()
        torch.cuda.synchronize()
        torch.cuda._sleep(int(spin_ms / spin_ms_per_cycle))
        w0 = time.perf_counter()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        enq_ms = (time.perf_counter() - w0) * 1e3
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n, enq_ms < 0.8 * spin_ms

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    def gpu_fields(eager_step, gs, n, spin_ms):
        ge, ok_e = gpu_only(eager_step, n, spin_ms)
        g = gs.graphs[(gs.next - 1) % len(gs.graphs)]       # replays of the last staged step (same tokens again)
        gg, ok_g = gpu_only(lambda: g.replay(), n, spin_ms)
        return {"eager_gpu_us_per_step": round(ge, 2) if ok_e else None,
                "graph_gpu_us_per_step": round(gg, 2) if ok_g else None}

    res = {}
    small = (("config1", lambda n: W.make_decode(1701, [17], n_layers=1, num_blocks=64, extra_steps=n),
              "1 sequence, 1 layer, context 17 (+1/step), 64-block pool"),
             ("config2", lambda n: W.config2(extra_steps=n),
              "4 slots, 1 layer, contexts {17,14,300,1000} (+1/step), 512-block pool"))
    for name, make, desc in small:
        w = make(2 * (steps_small + 4))
        engs = [DecodeEngine(dev(w.k_pool), dev(w.v_pool), w.block_table, w.context_lens - 1, w.free_list,
                             max_pos=4096, stream=stream) for _ in range(2)]
        sids = np.arange(w.batch, dtype=np.int32)
        q, k, v = dev(w.q_new), dev(w.k_new), dev(w.v_new)
        out = torch.empty_like(q)
        gs = GraphStep(engs[1], w.batch)
        gs.q.copy_(q)
        gs.k.copy_(k)
        gs.v.copy_(v)
        eager = timed(lambda: engs[0].step(sids, q, k, v, out), steps_small)
        graph = timed(lambda: gs.step(sids), steps_small)
        res[name] = {"workload": desc, "eager_us_per_step": round(eager[0], 2), "graph_us_per_step": round(graph[0], 2),
                     "eager_host_us_per_step": round(eager[1], 2), "graph_host_us_per_step": round(graph[1], 2),
                     "replayed_steps": gs.replays, "eager_fallback_steps": gs.eager_steps}
        res[name].update(gpu_fields(lambda: engs[0].step(sids, q, k, v, out), gs, 8, 20.0))
        del engs, gs
    sids = np.arange(q3.shape[1], dtype=np.int32)
    out3 = torch.empty_like(q3)
    eager = timed(lambda: eng3.step(sids, q3, k3, v3, out3), steps3)
    gs = GraphStep(eng3, q3.shape[1])
    gs.q.copy_(q3)
    gs.k.copy_(k3)
    gs.v.copy_(v3)
    graph = timed(lambda: gs.step(sids), steps3)
    res["config3"] = {"workload": "B=64, 16 layers, ctx U[512,4096] (+1/step), the main workload",
                      "eager_us_per_step": round(eager[0], 2), "graph_us_per_step": round(graph[0], 2),
                      "eager_host_us_per_step": round(eager[1], 2), "graph_host_us_per_step": round(graph[1], 2),
                      "replayed_steps": gs.replays, "eager_fallback_steps": gs.eager_steps}
    res["config3"].update(gpu_fields(lambda: eng3.step(sids, q3, k3, v3, out3), gs, 4, 40.0))
    del gs
    torch.cuda.synchronize()
    return res


def decode_layer_leg(torch, np, pkv, eng, ctx_now, stream, iters: int = 5):
    """Whole Llama-3.2-1B decode layers (pkv_decode_layers: RMSNorm, the
    decode-batch projections, the fused paged attention, the gated MLP; all
    16 layers in one call) for the B=64 rows of the main workload, synthetic
    bf16 weights ~ N(0, 1/fan_in) on the device (121 MB per layer).  Each
    layer's attention re-writes the last token in place, like the attention
    timing.  HIP events around each 16-layer pass, queued behind a device-side
    wait (GPU time; the host's time per pass beside it); the same pass as one
    pkv_decode_layer call per layer is timed too."""
    HID, INTER, NQ, NKV = 2048, 8192, 32, 8
    L = eng.n_layers
    B = len(ctx_now)
    g = torch.Generator(device="cuda")
    g.manual_seed(1708)

    def mat(n, k):
        return (torch.randn((n, k), generator=g, device="cuda") * (1.0 / math.sqrt(k))).to(torch.bfloat16)

    weights = []
    for _ in range(L):
        weights.append({"attn_norm": torch.ones(HID, dtype=torch.bfloat16, device="cuda"),
                        "wq": mat(NQ * 64, HID), "wk": mat(NKV * 64, HID), "wv": mat(NKV * 64, HID),
                        "wo": mat(HID, NQ * 64), "mlp_norm": torch.ones(HID, dtype=torch.bfloat16, device="cuda"),
                        "w_gate_up": mat(2 * INTER, HID), "w_down": mat(HID, INTER)})
    wbytes = sum(t.numel() * 2 for t in weights[0].values())
    h = torch.randn((B, HID), generator=g, device="cuda").to(torch.bfloat16)
    scratch = torch.empty(pkv.pkv_decode_layer_scratch_elems(B, HID, INTER, NQ, NKV), dtype=torch.bfloat16,
                          device="cuda")

    def per_layer_calls():
        for layer in range(L):
            pkv.pkv_decode_layer(h, weights[layer], scratch, eng.k_pool, eng.v_pool, eng.bt_dev[:, layer, :], None,
                                 eng.ctx_dev, eng.max_context_len, eng.cos_sin, eng.scale, eng.workspace,
                                 row_lens_host=ctx_now, stream=stream)

    def one_call():
        pkv.pkv_decode_layers(h, weights, scratch, eng.k_pool, eng.v_pool, eng.bt_dev, None, eng.ctx_dev,
                              eng.max_context_len, eng.cos_sin, eng.scale, eng.workspace, row_lens_host=ctx_now,
                              stream=stream)

    host_s = {}

    def timed(fn, key=None):
        # each pass queued behind a device-side wait, so that the host has
        # enqueued the whole pass (and done its checks and planning) before
        # the GPU starts: the events time the GPU's work, and the host's own
        # time per pass is reported beside it
        fn()
        torch.cuda.synchronize()
        times, walls = [], []
        for _ in range(iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(10_000_000)
            e0.record(stream)
            w0 = time.perf_counter()
            fn()
            walls.append(time.perf_counter() - w0)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / 1e3)
        if key:
            host_s[key] = float(np.median(walls))
        return float(np.median(times))

    t_calls = timed(per_layer_calls, "calls")
    t = timed(one_call, "one")

    # the weight reads alone (pkv_weight_read_probe: the projection kernels'
    # lane pattern, one wave per 16-row block and K part), over the 16
    # layers' matrices back to back (2 GB, so nothing is cached)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def probe(name, parts):
        def run():
            for layer in range(L):
                pkv.pkv_weight_read_probe(weights[layer][name], sink, k_parts=parts, stream=stream)
        us = timed(run) / L * 1e6
        return {"us": round(us, 2), "GBps": round(weights[0][name].numel() * 2 / us / 1e3, 1)}

    read_probe = {"gate_up_one_part": probe("w_gate_up", 1), "gate_up_two_parts": probe("w_gate_up", 2),
                  "down_eight_parts": probe("w_down", 8), "wq_four_parts": probe("wq", 4)}
    del weights
    torch.cuda.empty_cache()
    return {"workload": f"Llama-3.2-1B decode step, B={B}, {L} layers, hidden 2048, intermediate 8192, synthetic "
                        "bf16 weights, the main workload's paged cache (ctx U[512,4096])",
            "ms_per_step": round(t * 1e3, 4), "us_per_layer": round(t / L * 1e6, 2),
            "ms_per_step_layer_calls": round(t_calls * 1e3, 4),
            "host_ms_per_step": round(host_s["one"] * 1e3, 4),
            "host_ms_per_step_layer_calls": round(host_s["calls"] * 1e3, 4),
            "tokens_per_s": round(B / t, 1), "weight_bytes_per_layer": wbytes,
            "kv_bytes_per_layer": int(ctx_now.sum()) * KV_BYTES_PER_TOKEN, "weight_read_probe": read_probe}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--attn-iters", type=int, default=10, help="passes over the 16 layers for kernel timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--leg", choices=["prefill", "decode", "layer"], default=None,
                    help="run one leg alone and print its JSON (for profiling it): prefill, the "
                         "decode step with its roofline, read probe and the plain copy used to scale counters, "
                         "or the whole decode layers after the warm-up steps")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import paged_kv_attention_17_amd as pkv
    from paged_kv_attention_17_amd import workloads as W
    from paged_kv_attention_17_amd.engine import DecodeEngine

    if not os.path.exists(pkv.LIB_PATH):
        from paged_kv_attention_17_amd import build
        build.build()
    pkv.load()
    torch.cuda.set_device(0)
    if args.leg == "prefill":
        print(json.dumps(prefill_leg(torch, np, pkv, W, iters=args.steps)), flush=True)
        return
    steps_total = args.warmup + args.steps
    log(f"building workload (B=64, 16 layers, ctx U[512,4096]) ...")
    w = W.config3(fill_pool=False, extra_steps=steps_total + 64)     # room for the graph leg's steps
    kp = torch.empty((w.num_blocks, 16, 8, 64), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    W.fill_pool_device(kp, 31)
    W.fill_pool_device(vp, 32)
    stream = torch.cuda.current_stream()
    eng = DecodeEngine(kp, vp, w.block_table, w.context_lens - 1, w.free_list, max_pos=8192,
                       partition_size=args.partition_size, stream=stream)
    q = torch.from_numpy(w.q_new.view(np.int16)).cuda().view(torch.bfloat16)
    k = torch.from_numpy(w.k_new.view(np.int16)).cuda().view(torch.bfloat16)
    v = torch.from_numpy(w.v_new.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty_like(q)
    sids = np.arange(w.batch, dtype=np.int32)
    L = w.n_layers
    log(f"pool {w.num_blocks} blocks ({2 * kp.numel() * 2 / 1e9:.2f} GB K+V), mean ctx {w.context_lens.mean():.0f}")

    for _ in range(args.warmup):
        eng.step(sids, q, k, v, out)
    torch.cuda.synchronize()
    if args.leg == "layer":
        print(json.dumps(decode_layer_leg(torch, np, pkv, eng, eng.cached.copy(), stream)), flush=True)
        return

    # ---- timed region: K whole decode steps --------------------------------
    kv_bytes = 0
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # an event after every step as well, for the spread of the step times
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        kv_bytes += (int(eng.cached.sum()) + w.batch) * KV_BYTES_PER_TOKEN * L   # lengths after this step
        eng.step(sids, q, k, v, out)
        step_ev[i].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    t_step = ev0.elapsed_time(ev1) / 1e3 / args.steps
    per_step = np.array([(step_ev[i - 1] if i else ev0).elapsed_time(step_ev[i]) * 1e3 for i in range(args.steps)])
    value = kv_bytes / args.steps / t_step / 1e9
    log(f"step: {t_step * 1e6:.1f} us ({t_step * 1e6 / L:.2f} us/layer), KV {value:.0f} GB/s, "
        f"host wall {wall / args.steps * 1e6:.1f} us/step")

    # ---- dominant kernel: the streaming decode launch of the step.  Its
    # average duration is bounded by the step's own time per layer (16
    # streaming launches, one merge launch and the host allocation inside the
    # timed region above), which is what the roofline uses.  The standalone
    # fused call (streaming kernel + its own merge) is timed too, 16 calls
    # back to back per pass with events around each pass only (each call
    # re-appends the last step's token in place, so the cache does not change).
    ctx_now = eng.cached.copy()
    bytes_per_launch = kv_bytes // (args.steps * L)       # mean over the timed steps
    t_attn = t_step / L
    achieved = bytes_per_launch / t_attn / 1e9
    passes = []
    for it in range(args.attn_iters + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for layer in range(L):
            pkv.pkv_paged_decode_fused(out[layer], q[layer], k[layer], v[layer], kp, vp, eng.bt_dev[:, layer, :],
                                       None, eng.ctx_dev, eng.max_context_len, eng.cos_sin, eng.scale,
                                       eng.partition_size, eng.workspace, stream=stream, row_lens_host=ctx_now)
        e1.record(stream)
        if it > 0:                          # first pass is a warm-up
            passes.append((e0, e1))
    torch.cuda.synchronize()
    durs = np.array([a.elapsed_time(b) / 1e3 / L for a, b in passes])
    t_call = float(durs.mean())
    # the same launches' K/V reads alone (the library's diagnostic read probe:
    # same plan, shares, wave split and loads, no arithmetic), 16 per pass
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    probe = []
    for it in range(args.attn_iters + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for layer in range(L):
            pkv.pkv_paged_read_probe(kp, vp, eng.bt_dev[:, layer, :], None, ctx_now, sink, stream=stream)
        e1.record(stream)
        if it > 0:
            probe.append((e0, e1))
    torch.cuda.synchronize()
    t_probe = float(np.mean([a.elapsed_time(b) / 1e3 / L for a, b in probe]))
    probe_bytes = int(ctx_now.sum()) * KV_BYTES_PER_TOKEN
    log(f"paged read probe (the launch's K/V reads alone): {t_probe * 1e6:.2f} us per launch, "
        f"{probe_bytes / t_probe / 1e9:.0f} GB/s")
    log(f"streaming launch in the step: <= {t_attn * 1e6:.2f} us (step / {L}), {achieved:.0f} GB/s = "
        f"{achieved / HBM_PEAK_GBS:.1%} of peak; standalone fused call {t_call * 1e6:.2f} us "
        f"(16 back to back, p10 {np.percentile(durs, 10) * 1e6:.2f}, p90 {np.percentile(durs, 90) * 1e6:.2f})")

    if args.leg == "decode":
        copy_gbs = stream_copy_gbs(torch)
        print(json.dumps({"metric": METRIC, "ms_per_step": round(t_step * 1e3, 4),
                          "us_per_layer": round(t_step * 1e6 / L, 3), "value": round(value, 2), "unit": "GB/s",
                          "roofline_us_per_launch": round(t_attn * 1e6, 3), "bytes_per_launch": bytes_per_launch,
                          "standalone_call_us": round(t_call * 1e6, 3), "probe_us": round(t_probe * 1e6, 3),
                          "copy_kernel_GBps": round(copy_gbs, 1), "source_hash": decode_source_hash()}),
              flush=True)
        return

    dl = decode_layer_leg(torch, np, pkv, eng, ctx_now, stream)
    bytes_layer = dl["weight_bytes_per_layer"] + dl["kv_bytes_per_layer"]
    dl["attention_us_per_layer"] = round(t_call * 1e6, 2)
    dl["rest_us_per_layer"] = round(dl["us_per_layer"] - t_call * 1e6, 2)
    dl["GBps"] = round(bytes_layer / (dl["us_per_layer"] * 1e-6) / 1e9, 1)
    log(f"decode layer (B={w.batch}, weights + paged attention): {dl['us_per_layer']:.1f} us/layer "
        f"({dl['attention_us_per_layer']:.1f} us attention, {dl['rest_us_per_layer']:.1f} us norms, projections "
        f"and MLP), {dl['tokens_per_s']:.0f} tokens/s, {dl['GBps']:.0f} GB/s of weights + K/V")

    unf = unfused_layer_us(torch, np, pkv, eng, q, k, v, out, stream)
    log(f"unfused layer: rope {unf['rope']:.2f} us, append {unf['append']:.2f} us, "
        f"attention {unf['attention']:.2f} us (fused call: {t_call * 1e6:.2f} us)")

    gl = graph_leg(torch, np, W, eng, q, k, v, stream)
    for name, r in gl.items():
        log(f"{name} eager vs graph: {r['eager_us_per_step']:.1f} vs {r['graph_us_per_step']:.1f} us/step "
            f"(host {r['eager_host_us_per_step']:.1f} vs {r['graph_host_us_per_step']:.1f} us/step; "
            f"{r['replayed_steps']} replays, {r['eager_fallback_steps']} eager fallbacks); GPU side alone "
            f"{r['eager_gpu_us_per_step']} vs {r['graph_gpu_us_per_step']} us/step")

    pre = prefill_leg(torch, np, pkv, W)
    log(f"prefill: {pre['us_per_pass']:.1f} us per pass over {pre['calls']} chunk calls, "
        f"{pre['roofline']['achieved']:.1f} TFLOP/s = {pre['roofline']['frac']:.2%} of bf16 MFMA peak")

    lc = long_context_leg(torch, np, pkv, W, cpu_seconds=0.0 if args.no_cpu_baseline else 3.0)
    log(f"long context (B=256 x 8192): stream {lc['stream']['us_per_call']:.1f} us = {lc['stream']['GBps']:.0f} GB/s "
        f"({lc['stream']['frac']:.1%}); per-partition {lc['partitions']['us_per_call']:.1f} us = "
        f"{lc['partitions']['GBps']:.0f} GB/s ({lc['partitions']['frac']:.1%})")
    if "cpu_oracle" in lc:
        log(f"long context, cpu oracle: {lc['cpu_oracle']['value']:.3f} GB/s ({lc['cpu_oracle']['sample']})")

    ps = prefix_sharing_leg(torch, np, pkv, W)
    log(f"prefix sharing (B=64 over 4 shared 2048-token prompts): {ps['shared']['us_per_layer']:.1f} us/layer "
        f"({ps['shared']['logical_GBps']:.0f} GB/s of rows' K/V, {ps['shared']['unique_GBps']:.0f} GB/s of distinct "
        f"blocks) vs {ps['private']['us_per_layer']:.1f} us/layer with private blocks; copy on write of "
        f"{ps['copy_on_write']['pairs']} blocks {ps['copy_on_write']['us']:.1f} us = {ps['copy_on_write']['GBps']:.0f} GB/s")

    sv = serving_leg(torch, np, pkv, W)
    log(f"serving: {sv['iterations']} iterations in {sv['seconds'] * 1e3:.1f} ms, {sv['tokens_per_s']:.0f} tokens/s "
        f"({sv['prefill_tokens']} prompt tokens, {sv['decode_rows']} decode rows), "
        f"{sv['output_tokens_per_s']:.0f} output tokens/s; per iteration: plan {sv['plan_us_per_iteration']:.0f} us, "
        f"plan + enqueue {sv['host_us_per_iteration']:.0f} us (includes waits for a full launch queue)")
    sp = sv["shared_prompts"]
    log(f"serving over shared system prompts: prefix cache on {sp['cache_on']['seconds'] * 1e3:.1f} ms "
        f"({sp['cache_on']['prefill_tokens']} prompt tokens prefilled, {sp['cache_on']['reused_prompt_tokens']} "
        f"reused), off {sp['cache_off']['seconds'] * 1e3:.1f} ms ({sp['cache_off']['prefill_tokens']} prefilled): "
        f"{sp['speedup']:.2f}x")

    copy_gbs = stream_copy_gbs(torch)
    read_gbs = stream_read_gbs(torch, pkv)
    log(f"plain copy kernel: {copy_gbs:.0f} GB/s (read + write); streaming read of 4 GiB: {read_gbs:.0f} GB/s")

    src_hash = decode_source_hash()
    traffic = traffic_from_profile(src_hash)
    cpu = None
    if not args.no_cpu_baseline:
        # the host's cores (BLAS threads set to match), and one thread beside it
        cores = len(os.sched_getaffinity(0))
        cpu = cpu_baseline(eng, w.q_new, args.cpu_seconds / 2, cores)
        one = cpu_baseline(eng, w.q_new, args.cpu_seconds / 2, 1)
        cpu["value_1_thread"] = one["value"]
        log(f"cpu oracle: {cpu['value']:.3f} GB/s on {cores} cores ({cpu['sample']}); "
            f"{one['value']:.3f} GB/s on one thread")

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode step, B=64, 16 layers, ctx U[512,4096] (+1/step), 32q/8kv heads, d=64, "
                               "bf16 16-token blocks, pool 1.25x, interleaved tables",
                   "batch": w.batch, "layers": L, "mean_context": round(float(ctx_now.mean()), 1),
                   "partition_size": pkv.pkv_decode_partition_size(w.batch, 8, eng.max_context_len)
                   if args.partition_size == 0 else args.partition_size},
        "us_per_layer": round(t_step * 1e6 / L, 3),
        "step_us_p10_p50_p90": [round(float(np.percentile(per_step, x)), 1) for x in (10, 50, 90)],
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "stream_kernel<4, fused, chained> (one per layer of the step)",
                     "bytes_per_launch": bytes_per_launch,
                     "touched_bytes_per_launch": int(((ctx_now + 15) // 16).sum()) * 16 * KV_BYTES_PER_TOKEN,
                     "us_per_launch": round(t_attn * 1e6, 3),
                     "timing": "step time / layers, from the timed region (streaming launches, one merge, host "
                               "allocation and launch gaps included)",
                     "standalone_call_us": round(t_call * 1e6, 3),
                     "standalone_call_us_p10": round(float(np.percentile(durs, 10)) * 1e6, 3),
                     "standalone_call_us_p90": round(float(np.percentile(durs, 90)) * 1e6, 3),
                     "source_hash": src_hash},
        "paged_read_probe": {"us_per_launch": round(t_probe * 1e6, 3),
                             "GBps": round(probe_bytes / t_probe / 1e9, 1),
                             "what": "pkv_paged_read_probe over each layer's table view, 16 back to back per pass: "
                                     "the streaming launch's K/V reads alone"},
        "copy_kernel_GBps": round(copy_gbs, 1),
        "read_kernel_GBps": round(read_gbs, 1),
        "unfused_layer_us": unf,
        "graph_steps": gl,
        "prefill": pre,
        "long_context": lc,
        "prefix_sharing": ps,
        "serving": sv,
        "decode_layer": dl,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

"""GPU parity for the rest of the Llama decode layer: RMSNorm, the gated
SiLU product, the projections (the library's MFMA kernel for every
shape) and pkv_decode_layer (Llama-3.2-1B
shapes: hidden 2048, 32 / 8 heads of 64, intermediate 8192, synthetic bf16
weights ~ N(0, 1/fan_in)) against the float64 oracle with bf16 rounding where
the engine keeps a buffer.

Tolerances, from the arithmetic.  Every buffer is one nearest-even rounding
of a float32 (GPU) or float64 (oracle) value.  RMSNorm and the SiLU product
have no cancellation: the two pre-rounding values agree to a few float32
ulps, so the outputs agree within 1 bf16 ulp.  A projection's float32 sum of
K products, in whatever order the library takes them, is within the standard
a-priori bound K 2^-24 sum_k |x_k w_k| of the exact sum; after rounding the
output is within that bound plus 1 ulp of the oracle (a near-cancelling sum
has a tiny value whose ulp is below the float32 error of its large terms).
Through the whole layer each stage's input already differs from the
oracle's (the attention output by up to the attention bar, max-abs 2e-2 and
mean-abs 2e-3, which it is held to), so each stage is held to what its
measured input difference allows: a projection to |dx| |W|^T plus the
float32 bound plus 1 ulp, RMSNorm and silu(g) * u to their first-order
(mean-value) sensitivity to their inputs' differences plus 1 ulp.  The
layer leaves its intermediates in the scratch buffer, so every stage but
the attention residual (bounded through the output projection) is checked
on the kernels' own inputs."""
import numpy as np
import pytest
import torch

import paged_kv_attention_17_amd as pkv
from paged_kv_attention_17_amd import workloads as W
from oracle import bf16, layer, paging

from gpu_util import ATOL_MAX, ATOL_MEAN, bits, dev_bf16, dev_i32, f64, ulp_diff

pytestmark = pytest.mark.gpu

HID, NQ, NKV, INTER = 2048, 32, 8, 8192


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (normal range)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -126)))
    return 2.0 ** (np.maximum(e, -126) - 7)


def assert_within(got_bits, ref, bound, what):
    """|got - ref| <= bound plus the two sides' roundings (half an ulp each,
    at most one ulp of the larger of the two)."""
    got = f64(got_bits)
    err = np.abs(got - ref)
    bound = bound + bf16_ulp(np.maximum(np.abs(got), np.abs(ref)))
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} outside, worst {np.max(err - bound):.3e} over the bound"


def _weights(rng):
    s = layer.init_scale
    w = {"attn_norm": W.f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(HID)).astype(np.float32)),
         "wq": W.randn_bf16(rng, (NQ * 64, HID), s(HID)), "wk": W.randn_bf16(rng, (NKV * 64, HID), s(HID)),
         "wv": W.randn_bf16(rng, (NKV * 64, HID), s(HID)), "wo": W.randn_bf16(rng, (HID, NQ * 64), s(NQ * 64)),
         "mlp_norm": W.f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(HID)).astype(np.float32)),
         "w_gate_up": W.randn_bf16(rng, (2 * INTER, HID), s(HID)), "w_down": W.randn_bf16(rng, (HID, INTER), s(INTER))}
    return w


def test_rmsnorm_within_one_ulp(gpu):
    rng = np.random.default_rng(1)
    x = W.randn_bf16(rng, (7, HID), 2.0)
    w = W.f32_to_bf16_bits((1.0 + 0.3 * rng.standard_normal(HID)).astype(np.float32))
    out = torch.empty((7, HID), dtype=torch.bfloat16, device="cuda")
    pkv.pkv_rmsnorm(out, dev_bf16(x), dev_bf16(w))
    torch.cuda.synchronize()
    ref = bf16.from_f64(layer.rmsnorm(f64(x), f64(w)))
    d = ulp_diff(bits(out), ref)
    assert d.max() <= 1 and (d == 0).mean() > 0.95


def test_silu_mul_within_one_ulp(gpu):
    rng = np.random.default_rng(2)
    gu = W.randn_bf16(rng, (5, 2 * INTER), 2.0)
    act = torch.empty((5, INTER), dtype=torch.bfloat16, device="cuda")
    pkv.pkv_silu_mul(act, dev_bf16(gu))
    torch.cuda.synchronize()
    g, u = f64(gu[:, :INTER]), f64(gu[:, INTER:])
    ref = bf16.from_f64(layer.silu(g) * u)
    d = ulp_diff(bits(act), ref)
    assert d.max() <= 1 and (d == 0).mean() > 0.95


# the projections of a decode batch (K split over 1 to 16 workgroups, ragged
# rows, one to three 128-wide X slices per workgroup), wider batches (two and
# three 64-row blocks), K that is not a multiple of 128 (a short last slice,
# a short last K range), feature counts that are not a multiple of 64, and a
# split shape handed a null workspace (one K range)
@pytest.mark.parametrize("rows,n,k,ws", [(64, 3072, 2048, None), (1, 512, 2048, None), (13, 2048, 8192, None),
                                         (64, 16384, 2048, None), (64, 2048, 2048, None), (64, 2048, 8192, None),
                                         (37, 192, 384, None), (100, 512, 2048, None), (8, 64, 104, None),
                                         (5, 64, 128, None), (8, 64, 96, None), (150, 200, 520, None),
                                         (65, 2048, 2056, None), (3, 24, 8, None),
                                         (64, 2048, 8192, False)])
def test_linear_within_one_ulp(gpu, rows, n, k, ws):
    rng = np.random.default_rng(rows + n + k)
    x = W.randn_bf16(rng, (rows, k))
    w = W.randn_bf16(rng, (n, k), layer.init_scale(k))
    c0 = W.randn_bf16(rng, (rows, n))
    out = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")
    pkv.pkv_linear(out, dev_bf16(x), dev_bf16(w), workspace=ws)
    acc = dev_bf16(c0)
    pkv.pkv_linear(acc, dev_bf16(x), dev_bf16(w), accumulate=True, workspace=ws)
    torch.cuda.synchronize()
    prod = layer.linear(f64(x), f64(w))
    fp32_sum = k * 2.0 ** -24 * layer.linear(np.abs(f64(x)), np.abs(f64(w)))
    assert_within(bits(out), prod, fp32_sum, "linear")
    ref_acc = f64(c0) + prod
    assert_within(bits(acc), ref_acc, fp32_sum, "linear, accumulate")
    assert (ulp_diff(bits(out), bf16.from_f64(prod)) == 0).mean() > 0.95


def test_linear_decode_batch_is_deterministic(gpu):
    """The K-split partials are summed in a fixed order: repeated calls, with
    the workspace refilled with garbage in between, give the same bits."""
    rng = np.random.default_rng(77)
    rows, n, k = 64, 2048, 8192
    assert pkv.pkv_linear_workspace_bytes(rows, n, k) > 0
    assert pkv.pkv_linear_workspace_bytes(64, 2048, 8012) == 0          # K % 8: not a shape the kernel takes
    assert pkv.pkv_linear_workspace_bytes(65, n, k) > 0
    x, w = dev_bf16(W.randn_bf16(rng, (rows, k))), dev_bf16(W.randn_bf16(rng, (n, k), layer.init_scale(k)))
    ws = torch.empty(pkv.pkv_linear_workspace_bytes(rows, n, k), dtype=torch.uint8, device="cuda")
    outs = []
    for fill in (0, 255, 0x7f):
        ws.fill_(fill)
        out = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")
        pkv.pkv_linear(out, x, w, workspace=ws)
        outs.append(bits(out))
    torch.cuda.synchronize()
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


# 4 rows, 64 rows (one full 64-row block; with host lengths this is the
# bench's combination: streaming attention and the decode-batch projections)
# and 65 rows (two row blocks, one holding a single row), all with q, k, v in
# one launch and the gated gate/up launch that leaves the gate_up buffer
# unwritten
@pytest.mark.parametrize("host_lens,extra_rows", [(True, 0), (False, 0), (False, 60), (True, 60), (True, 61)])
def test_decode_layer_matches_oracle(gpu, host_lens, extra_rows):
    rng = np.random.default_rng(5)
    wts = _weights(rng)
    pos = np.array([16, 1, 299, 1000], np.int32)           # new token positions (cached tokens before it)
    pos = np.concatenate([pos, rng.integers(0, 40, extra_rows).astype(np.int32)])
    gated = True                                            # intermediate % 32 == 0
    B = len(pos)
    nbs = [-(-(int(p) + 1) // 16) for p in pos]
    nb = sum(nbs) + 3
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((B, max(nbs) + 1), -1, np.int32)
    o_ = 0
    for b, n in enumerate(nbs):
        bt[b, :n] = perm[o_:o_ + n]
        o_ += n
    kp = np.full((nb, 16, NKV, 64), W.BF16_POISON, np.uint16)
    vp = kp.copy()
    hist_k, hist_v = [], []
    for b, p in enumerate(pos):
        K = W.randn_bf16(rng, (int(p), NKV, 64))
        V = W.randn_bf16(rng, (int(p), NKV, 64))
        if p:
            kp, vp = paging.append(kp, vp, K, V, bt, np.full(int(p), b, np.int32), np.arange(int(p), dtype=np.int32))
        hist_k.append(f64(K))
        hist_v.append(f64(V))
    h = W.randn_bf16(rng, (B, HID))
    ref = layer.decode_layer(f64(h), {k: f64(v) for k, v in wts.items() if k not in ("w_gate_up", "w_down")} | {
        "wg": f64(wts["w_gate_up"][:INTER]), "wu": f64(wts["w_gate_up"][INTER:]), "wd": f64(wts["w_down"])},
        hist_k, hist_v, pos, NQ, NKV, scale=0.125)

    dw = {k: dev_bf16(v) for k, v in wts.items()}
    hd = dev_bf16(h)
    kpd, vpd = dev_bf16(kp), dev_bf16(vp)
    n_scr = pkv.pkv_decode_layer_scratch_elems(B, HID, INTER, NQ, NKV)
    scr = torch.empty(n_scr, dtype=torch.bfloat16, device="cuda")
    cos_sin = torch.empty((4096, 32, 2), dtype=torch.float32, device="cuda")
    pkv.pkv_rope_table_init(cos_sin)
    ctx = pos + 1
    ws = pkv.decode_workspace(B, NQ, NKV, int(ctx.max()))
    pkv.pkv_decode_layer(hd, dw, scr, kpd, vpd, dev_i32(bt), dev_i32(np.arange(B)), dev_i32(ctx), int(ctx.max()),
                         cos_sin, 0.125, ws, row_lens_host=ctx if host_lens else None)
    torch.cuda.synchronize()
    s = bits(scr)
    off = 0

    def take(width):
        nonlocal off
        x = s[off:off + B * width].reshape(B, width)
        off += B * width
        return x

    a, q, k, v, o, m, gu, act = (take(HID), take(NQ * 64), take(NKV * 64), take(NKV * 64), take(NQ * 64), take(HID),
                                 take(2 * INTER), take(INTER))
    Wf = {name: f64(wts[name]) for name in ("wq", "wk", "wv", "wo", "w_gate_up", "w_down")}
    a_, o_, m_, gu_, act_ = f64(a), f64(o), f64(m), f64(gu), f64(act)

    def lin_bound(x_gpu, x_ref, w):
        """How far x_gpu W^T, summed in float32, can be from x_ref W^T."""
        aw = np.abs(w).T
        return np.abs(x_gpu - x_ref) @ aw + w.shape[1] * 2.0 ** -24 * (np.abs(x_gpu) @ aw)

    assert ulp_diff(a, bf16.from_f64(ref["a"])).max() <= 1
    for name, got, w in (("q", q, Wf["wq"]), ("k", k, Wf["wk"]), ("v", v, Wf["wv"])):
        want = ref[name].reshape(B, -1)
        assert_within(got, want, lin_bound(a_, ref["a"], w), name)
    err = np.abs(o_ - ref["o"])
    assert err.max() <= ATOL_MAX and err.mean() <= ATOL_MEAN, (err.max(), err.mean())
    # h after the attention residual is not kept: its bound comes from o's difference
    b_mid = lin_bound(o_, ref["o"], Wf["wo"]) + 2 * bf16_ulp(ref["h_mid"])
    # rmsnorm: m = h w / r moves by |w| (|dh| / r + |h| |dr| / r^2), |dr| <= rms(dh)
    r = np.sqrt(np.mean(np.square(ref["h_mid"]), axis=1, keepdims=True))
    dr = np.sqrt(np.mean(np.square(b_mid), axis=1, keepdims=True))
    wn = np.abs(f64(wts["mlp_norm"]))
    assert_within(m, ref["m"], wn * (b_mid / r + np.abs(ref["h_mid"]) * dr / r ** 2) * 1.01, "m")
    bg = lin_bound(m_, ref["m"], Wf["w_gate_up"][:INTER])
    bu = lin_bound(m_, ref["m"], Wf["w_gate_up"][INTER:])
    if gated:
        # g and u stay in registers: |g_gpu - g| <= bg plus the two sides'
        # roundings (1 ulp of the larger), likewise u; |silu'| <= 1.1
        dg = bg + bf16_ulp(np.abs(ref["g"]) + bg)
        du = bu + bf16_ulp(np.abs(ref["u"]) + bu)
        act_bound = 1.1 * dg * (np.abs(ref["u"]) + du) + np.abs(layer.silu(ref["g"])) * du
    else:
        g_gpu, u_gpu = gu_[:, :INTER], gu_[:, INTER:]
        assert_within(gu[:, :INTER], ref["g"], bg, "g")
        assert_within(gu[:, INTER:], ref["u"], bu, "u")
        # silu(g) u from the kernel's own g, u: |silu'| <= 1.1, so it moves by
        # at most 1.1 |dg| |u| + |silu(g)| |du|, plus its rounding
        dg, du = np.abs(g_gpu - ref["g"]), np.abs(u_gpu - ref["u"])
        act_bound = 1.1 * dg * np.abs(u_gpu) + np.abs(layer.silu(ref["g"])) * du
    assert_within(act, ref["act"], act_bound, "act")
    assert_within(bits(hd), ref["h"], b_mid + lin_bound(act_, ref["act"], Wf["w_down"]), "h")
    eh = np.abs(f64(bits(hd)) - ref["h"])
    print(f"decode layer: h max-abs {eh.max():.3e} mean-abs {eh.mean():.3e}, "
          f"bit-equal {(bits(hd) == bf16.from_f64(ref['h'])).mean():.3f}", flush=True)
    # the new token's cache rows: the rotated k, and v exactly as the layer's v buffer
    for b, p in enumerate(pos):
        blk = int(bt[b, p // 16])
        kb = (lin_bound(a_, ref["a"], Wf["wk"]) + bf16_ulp(ref["k"].reshape(B, -1)))[b].reshape(NKV, 64)
        # the rotation mixes pairs (|cos| + |sin| <= sqrt 2) and rounds once more
        assert_within(bits(kpd[blk, p % 16]), ref["k_rot"][b], 1.5 * (kb + np.roll(kb, 32, axis=1))
                      , "cached k")
        np.testing.assert_array_equal(bits(vpd[blk, p % 16]), v[b].reshape(NKV, 64))


def _device_layer_weights(gen, inter=INTER):
    def rnd(shape, fan_in):
        return (torch.randn(shape, device="cuda", generator=gen) * fan_in ** -0.5).to(torch.bfloat16)
    return {"attn_norm": (1.0 + 0.1 * torch.randn(HID, device="cuda", generator=gen)).to(torch.bfloat16),
            "wq": rnd((NQ * 64, HID), HID), "wk": rnd((NKV * 64, HID), HID), "wv": rnd((NKV * 64, HID), HID),
            "wo": rnd((HID, NQ * 64), NQ * 64),
            "mlp_norm": (1.0 + 0.1 * torch.randn(HID, device="cuda", generator=gen)).to(torch.bfloat16),
            "w_gate_up": rnd((2 * inter, HID), HID), "w_down": rnd((HID, inter), inter)}


# the multi-layer call against one call per layer, bit for bit: h after the
# last layer and every cache row.  Both run the same kernels except the
# fused down-partials / residual / next-norm kernel between layers, which
# is what this checks (every kernel's summation order is fixed, so the two
# forms must agree exactly).  Rows of up to 16 tokens or up to 300, with
# host lengths (streaming attention) or without (per-partition attention);
# 4 and 64 rows are one row block of the projections, 65 rows two.
@pytest.mark.parametrize("B,short,host", [(4, True, True), (64, True, True), (65, True, True), (64, False, True),
                                          (64, False, False)])
def test_decode_layers_match_per_layer_calls(gpu, B, short, host):
    L = 3
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234 + B)
    layers = [_device_layer_weights(gen) for _ in range(L)]
    rng = np.random.default_rng(B)
    pos = rng.integers(0, 16 if short else 300, B).astype(np.int32)
    ctx = pos + 1
    nbs = -(-ctx // 16)
    mb = int(nbs.max()) + 1
    nb = int(nbs.sum()) * L + 5
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((B, L, mb), -1, np.int32)
    o_ = 0
    for b in range(B):
        for l in range(L):
            bt[b, l, :nbs[b]] = perm[o_:o_ + nbs[b]]
            o_ += nbs[b]
    kp = torch.randn((nb, 16, NKV, 64), device="cuda", generator=gen).to(torch.bfloat16)
    vp = torch.randn((nb, 16, NKV, 64), device="cuda", generator=gen).to(torch.bfloat16)
    h0 = torch.randn((B, HID), device="cuda", generator=gen).to(torch.bfloat16)
    cos_sin = torch.empty((4096, 32, 2), dtype=torch.float32, device="cuda")
    pkv.pkv_rope_table_init(cos_sin)
    btd = dev_i32(bt)
    slots, ctxd = dev_i32(np.arange(B)), dev_i32(ctx)
    ws = pkv.decode_workspace(B, NQ, NKV, int(ctx.max()))
    n_scr = pkv.pkv_decode_layer_scratch_elems(B, HID, INTER, NQ, NKV)

    lens = ctx if host else None
    h1, kp1, vp1 = h0.clone(), kp.clone(), vp.clone()
    scr1 = torch.empty(n_scr, dtype=torch.bfloat16, device="cuda")
    for l in range(L):
        pkv.pkv_decode_layer(h1, layers[l], scr1, kp1, vp1, btd[:, l, :], slots, ctxd, int(ctx.max()), cos_sin,
                             0.125, ws, row_lens_host=lens)
    h2, kp2, vp2 = h0.clone(), kp.clone(), vp.clone()
    scr2 = torch.empty(n_scr, dtype=torch.bfloat16, device="cuda")
    pkv.pkv_decode_layers(h2, layers, scr2, kp2, vp2, btd, slots, ctxd, int(ctx.max()), cos_sin, 0.125, ws,
                          row_lens_host=lens)
    torch.cuda.synchronize()
    assert torch.isfinite(h2.float()).all()
    assert not torch.equal(h1.view(torch.int16), h0.view(torch.int16))
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(kp1.view(torch.int16), kp2.view(torch.int16))
    assert torch.equal(vp1.view(torch.int16), vp2.view(torch.int16))


@pytest.mark.parametrize("n,k,parts", [(64, 2048, 1), (48, 512, 2), (16, 512, 4), (32, 128, 1), (16, 2048, 8)])
def test_weight_read_probe_reads_without_writing(gpu, n, k, parts):
    """The diagnostic weight-stream probe reads the matrix (one to eight K
    parts per 16-row block, one slice and several) and writes nothing: the
    matrix is unchanged and the sink keeps its value."""
    rng = np.random.default_rng(n + k + parts)
    w = W.randn_bf16(rng, (n, k))
    wd = dev_bf16(w)
    sink = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    pkv.pkv_weight_read_probe(wd, sink, k_parts=parts)
    torch.cuda.synchronize()
    assert int(sink.item()) == 5
    np.testing.assert_array_equal(bits(wd), w)

"""Pins for the oracle's Llama decode layer (CPU only): RMSNorm, SiLU, the
gated MLP and the whole layer (with rounding switched off) against the
float64 modules of transformers' Llama implementation, fed the same weights
and the same cached keys and values; closed-form special cases (zero output
projections leave the residual stream unchanged); and planted mistakes in
the oracle that these pins must catch."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import layer, rope

D_SMALL, NQ, NKV, INTER = 256, 4, 2, 512


def _cfg():
    from transformers import LlamaConfig
    return LlamaConfig(hidden_size=D_SMALL, intermediate_size=INTER, num_attention_heads=NQ,
                       num_key_value_heads=NKV, head_dim=64, rms_norm_eps=layer.EPS, max_position_embeddings=131072,
                       rope_parameters={"rope_type": "llama3", "rope_theta": rope.ROPE_THETA,
                                        "factor": rope.ROPE_FACTOR, "low_freq_factor": rope.LOW_FREQ_FACTOR,
                                        "high_freq_factor": rope.HIGH_FREQ_FACTOR,
                                        "original_max_position_embeddings": rope.ORIGINAL_MAX_POS},
                       attention_bias=False, mlp_bias=False, attn_implementation="eager")


def _weights(rng, D=D_SMALL, nq=NQ, nkv=NKV, inter=INTER):
    s = layer.init_scale
    return {"attn_norm": 1.0 + 0.1 * rng.standard_normal(D),
            "wq": rng.standard_normal((nq * 64, D)) * s(D), "wk": rng.standard_normal((nkv * 64, D)) * s(D),
            "wv": rng.standard_normal((nkv * 64, D)) * s(D), "wo": rng.standard_normal((D, nq * 64)) * s(nq * 64),
            "mlp_norm": 1.0 + 0.1 * rng.standard_normal(D),
            "wg": rng.standard_normal((inter, D)) * s(D), "wu": rng.standard_normal((inter, D)) * s(D),
            "wd": rng.standard_normal((D, inter)) * s(inter)}


def test_rmsnorm_matches_transformers():
    from transformers.models.llama.modeling_llama import LlamaRMSNorm
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, D_SMALL)) * 3.0
    w = rng.standard_normal(D_SMALL)
    m = LlamaRMSNorm(D_SMALL, eps=layer.EPS).double()
    with torch.no_grad():
        m.weight.copy_(torch.from_numpy(w))
        ref = m(torch.from_numpy(x)).numpy()
    # transformers' RMSNorm takes the mean square in float32 even in a float64 module
    np.testing.assert_allclose(layer.rmsnorm(x, w), ref, rtol=1e-6, atol=1e-6)
    # closed forms: a constant row c becomes sign(c) * w (up to eps); scale invariance
    c = np.full((1, D_SMALL), 7.0)
    np.testing.assert_allclose(layer.rmsnorm(c, w)[0], w * 7.0 / np.sqrt(49.0 + layer.EPS), rtol=1e-14)
    np.testing.assert_allclose(layer.rmsnorm(1000 * x, w), layer.rmsnorm(x, w), rtol=1e-6)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(layer.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-300)
    assert layer.silu(np.array([0.0]))[0] == 0.0


def test_mlp_matches_transformers():
    from transformers.models.llama.modeling_llama import LlamaMLP
    rng = np.random.default_rng(2)
    W = _weights(rng)
    m = rng.standard_normal((3, D_SMALL))
    mod = LlamaMLP(_cfg()).double()
    with torch.no_grad():
        mod.gate_proj.weight.copy_(torch.from_numpy(W["wg"]))
        mod.up_proj.weight.copy_(torch.from_numpy(W["wu"]))
        mod.down_proj.weight.copy_(torch.from_numpy(W["wd"]))
        ref = mod(torch.from_numpy(m)).numpy()
    np.testing.assert_allclose(layer.mlp(m, W["wg"], W["wu"], W["wd"], rnd=None), ref, rtol=1e-11, atol=1e-12)


def _transformers_layer(W, h, hist_k, hist_v, pos):
    """transformers' LlamaDecoderLayer in float64 for rows that share the
    history length `pos` (cache pre-filled with the rotated history)."""
    from transformers import DynamicCache
    from transformers.models.llama.modeling_llama import LlamaDecoderLayer, LlamaRotaryEmbedding
    cfg = _cfg()
    lay = LlamaDecoderLayer(cfg, layer_idx=0).double()
    with torch.no_grad():
        lay.input_layernorm.weight.copy_(torch.from_numpy(W["attn_norm"]))
        lay.post_attention_layernorm.weight.copy_(torch.from_numpy(W["mlp_norm"]))
        for name, key in (("q_proj", "wq"), ("k_proj", "wk"), ("v_proj", "wv"), ("o_proj", "wo")):
            getattr(lay.self_attn, name).weight.copy_(torch.from_numpy(W[key]))
        for name, key in (("gate_proj", "wg"), ("up_proj", "wu"), ("down_proj", "wd")):
            getattr(lay.mlp, name).weight.copy_(torch.from_numpy(W[key]))
    B = h.shape[0]
    cache = DynamicCache(config=cfg)
    if pos > 0:
        # cache layout [batch, kv heads, tokens, dim]
        ks = torch.from_numpy(np.stack(hist_k)).permute(0, 2, 1, 3).contiguous()
        vs = torch.from_numpy(np.stack(hist_v)).permute(0, 2, 1, 3).contiguous()
        cache.update(ks, vs, 0)
    x = torch.from_numpy(h).reshape(B, 1, D_SMALL)
    pid = torch.full((B, 1), pos, dtype=torch.long)
    rot = LlamaRotaryEmbedding(cfg).double()
    cos, sin = rot(x, pid)
    with torch.no_grad():
        out = lay(x, attention_mask=None, position_ids=pid, past_key_values=cache, use_cache=True,
                  cache_position=torch.tensor([pos]), position_embeddings=(cos.double(), sin.double()))
    out = out[0] if isinstance(out, tuple) else out
    return out.reshape(B, D_SMALL).numpy()


@pytest.mark.parametrize("pos", [0, 1, 37])
def test_decode_layer_matches_transformers(pos):
    rng = np.random.default_rng(10 + pos)
    W = _weights(rng)
    B = 3
    h = rng.standard_normal((B, D_SMALL))
    hist_k = [rng.standard_normal((pos, NKV, 64)) for _ in range(B)]
    hist_v = [rng.standard_normal((pos, NKV, 64)) for _ in range(B)]
    got = layer.decode_layer(h, W, hist_k, hist_v, [pos] * B, NQ, NKV, scale=0.125, rnd=None)["h"]
    ref = _transformers_layer(W, h, hist_k, hist_v, pos)
    # float32 inside transformers' RMSNorm (twice per layer) sets the tolerance
    np.testing.assert_allclose(got, ref, rtol=5e-6, atol=5e-6)


def test_zero_output_projections_keep_the_residual_stream():
    rng = np.random.default_rng(3)
    W = _weights(rng)
    h = rng.standard_normal((2, D_SMALL))
    hk = [rng.standard_normal((5, NKV, 64)) for _ in range(2)]
    W0 = dict(W, wo=np.zeros_like(W["wo"]), wd=np.zeros_like(W["wd"]))
    np.testing.assert_array_equal(layer.decode_layer(h, W0, hk, hk, [5, 5], NQ, NKV, rnd=None)["h"], h)
    Wg0 = dict(W, wg=np.zeros_like(W["wg"]))          # silu(0) = 0: the MLP adds nothing
    r = layer.decode_layer(h, Wg0, hk, hk, [5, 5], NQ, NKV, rnd=None)
    np.testing.assert_array_equal(r["h"], r["h_mid"])


def test_planted_mistakes_fail_the_transformers_pins(monkeypatch):
    rng = np.random.default_rng(4)
    W = _weights(rng)
    h = rng.standard_normal((2, D_SMALL))
    hk = [rng.standard_normal((4, NKV, 64)) for _ in range(2)]
    hv = [rng.standard_normal((4, NKV, 64)) for _ in range(2)]
    ref = _transformers_layer(W, h, hk, hv, 4)
    # a norm over mean |x| instead of the root mean square
    monkeypatch.setattr(layer, "rmsnorm", lambda x, w, eps=layer.EPS: np.asarray(x) / (
        np.mean(np.abs(x), axis=-1, keepdims=True) + eps) * w)
    assert not np.allclose(layer.decode_layer(h, W, hk, hv, [4, 4], NQ, NKV, rnd=None)["h"], ref, atol=1e-6)
    monkeypatch.undo()
    # the gate without its SiLU
    monkeypatch.setattr(layer, "silu", lambda x: np.asarray(x, dtype=np.float64))
    assert not np.allclose(layer.decode_layer(h, W, hk, hv, [4, 4], NQ, NKV, rnd=None)["h"], ref, atol=1e-6)
    monkeypatch.undo()
    # the query rotated at the wrong position
    bad = layer.decode_layer(h, W, hk, hv, [5, 5], NQ, NKV, rnd=None)["h"]
    assert not np.allclose(bad, ref, atol=1e-6)
    np.testing.assert_allclose(layer.decode_layer(h, W, hk, hv, [4, 4], NQ, NKV, rnd=None)["h"], ref,
                               rtol=5e-6, atol=5e-6)

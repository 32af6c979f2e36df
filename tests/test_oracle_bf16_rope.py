"""Pins for the oracle's bf16 rounding and Llama-3 RoPE (CPU only).

Each check ties the oracle to something other than itself: torch's own
float32 -> bfloat16 conversion, transformers' Llama-3 RoPE parameters and
rotate-half rotation, the constants printed on the pages, closed forms.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import bf16, rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def golden():
    with open(GOLDEN) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


# ---------------------------------------------------------------- bf16 ------

def test_bf16_matches_torch_on_float32_inputs():
    # For inputs exactly representable in float32 a single rounding from
    # float64 equals torch's float32 -> bfloat16 rounding (RNE).
    rng = np.random.default_rng(0)
    x32 = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # bf16 subnormal range
        (rng.uniform(-1, 1, 2000) * 3.3e38).astype(np.float32),     # near overflow
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 3.4e38], dtype=np.float32),
    ])
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16.from_f64(x32.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_ties_and_single_rounding():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even (1.0).
    assert bf16.from_f64(np.array([1 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: even is 1+2^-6.
    assert bf16.from_f64(np.array([1 + 3 * 2.0 ** -8]))[0] == 0x3F82
    # Just above the tie rounds up; a float32 intermediate would lose the 2^-30.
    assert bf16.from_f64(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 0x3F81
    assert bf16.from_f64(np.array([-(1 + 2.0 ** -8 + 2.0 ** -30)]))[0] == 0xBF81
    # Overflow and specials.
    assert bf16.from_f64(np.array([1e39]))[0] == 0x7F80
    assert bf16.from_f64(np.array([-np.inf]))[0] == 0xFF80
    assert np.isnan(bf16.to_f64(bf16.from_f64(np.array([np.nan]))))[0]
    # Smallest subnormal 2^-133 and half of it (ties to even -> 0).
    assert bf16.from_f64(np.array([2.0 ** -133]))[0] == 0x0001
    assert bf16.from_f64(np.array([2.0 ** -134]))[0] == 0x0000
    assert bf16.from_f64(np.array([1.5 * 2.0 ** -133]))[0] == 0x0002


def test_bf16_roundtrip_all_finite_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16.to_f64(bits)
    fin = np.isfinite(vals)
    back = bf16.from_f64(vals[fin])
    # -0.0 and +0.0 both round-trip to their own sign
    np.testing.assert_array_equal(back, bits[fin])


# ---------------------------------------------------------------- RoPE ------

def test_rope_constants_are_the_pages():
    g = golden()
    assert rope.ROPE_THETA == g["rope_theta"]
    assert rope.ROPE_FACTOR == g["rope_factor"]
    assert rope.LOW_FREQ_FACTOR == g["rope_low_freq_factor"]
    assert rope.HIGH_FREQ_FACTOR == g["rope_high_freq_factor"]
    assert rope.ORIGINAL_MAX_POS == g["rope_original_max_pos"]


def _hf_llama3_inv_freq(theta, factor, low, high, orig, head_dim=64):
    from transformers import LlamaConfig
    from transformers import modeling_rope_utils as mru
    cfg = LlamaConfig(hidden_size=2048, num_attention_heads=32, num_key_value_heads=8,
                      head_dim=head_dim, max_position_embeddings=131072,
                      rope_parameters={"rope_type": "llama3", "rope_theta": theta,
                                       "factor": factor, "low_freq_factor": low,
                                       "high_freq_factor": high,
                                       "original_max_position_embeddings": orig})
    inv, _ = mru._compute_llama3_parameters(cfg, device="cpu")
    return inv.double().numpy()


def test_rope_inv_freq_matches_transformers_llama3():
    ref = _hf_llama3_inv_freq(500000.0, 32.0, 1.0, 4.0, 8192)
    got = rope.inv_freq(64)
    # transformers computes in float32
    np.testing.assert_allclose(got, ref, rtol=3e-6, atol=0)


@pytest.mark.parametrize("params", [(10000.0, 8.0, 1.0, 4.0, 8192), (500000.0, 16.0, 2.0, 8.0, 4096)])
def test_rope_inv_freq_matches_transformers_other_params(params):
    ref = _hf_llama3_inv_freq(*params)
    theta, factor, low, high, orig = params
    got = rope.inv_freq(64, theta, factor, low, high, orig)
    np.testing.assert_allclose(got, ref, rtol=3e-6, atol=0)


def test_rope_factor_one_is_plain_rope():
    # With factor 1 every branch of the scaling leaves f_i alone: the table
    # must be transformers' default (unscaled) RoPE.
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding
    cfg = LlamaConfig(hidden_size=2048, num_attention_heads=32, num_key_value_heads=8,
                      head_dim=64, rope_parameters={"rope_type": "default", "rope_theta": 500000.0})
    ref, _ = LlamaRotaryEmbedding.compute_default_rope_parameters(cfg, device="cpu")
    got = rope.inv_freq(64, 500000.0, 1.0, 1.0, 4.0, 8192)
    np.testing.assert_allclose(got, ref.double().numpy(), rtol=3e-6)


def test_rope_band_structure():
    # Fast pairs untouched, slow pairs divided by the factor, a smooth ramp
    # between (each ramp value lies strictly between f/32 and f).
    plain = rope.inv_freq(64, 500000.0, 1.0, 1.0, 4.0, 8192)
    f = rope.inv_freq(64)
    wl = 2 * math.pi / plain
    keep = wl < 8192 / 4
    slow = wl > 8192 / 1
    ramp = ~keep & ~slow
    np.testing.assert_array_equal(f[keep], plain[keep])
    np.testing.assert_allclose(f[slow], plain[slow] / 32, rtol=1e-15)
    assert ramp.sum() >= 1
    assert np.all(f[ramp] < plain[ramp]) and np.all(f[ramp] > plain[ramp] / 32)
    assert keep.sum() == 15 and ramp.sum() == 3 and slow.sum() == 14


def test_rope_rotation_matches_transformers_rotate_half():
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    rng = np.random.default_rng(1)
    T, Hq, Hk, d = 7, 4, 2, 64
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hk, d))
    pos = np.array([0, 1, 5, 16, 1000, 8191, 100000])
    f = rope.inv_freq(d)
    ang = pos[:, None] * f[None, :]
    emb = np.concatenate([ang, ang], axis=-1)                 # [T, d]
    cos = torch.from_numpy(np.cos(emb))[None]                 # [1, T, d]
    sin = torch.from_numpy(np.sin(emb))[None]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]           # [1, H, T, d]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    rq, rk = apply_rotary_pos_emb(qt, kt, cos, sin)
    np.testing.assert_allclose(rope.rotate_f64(q, pos, f), rq[0].permute(1, 0, 2).numpy(), atol=1e-12)
    np.testing.assert_allclose(rope.rotate_f64(k, pos, f), rk[0].permute(1, 0, 2).numpy(), atol=1e-12)


def test_rope_position_zero_is_identity_bitwise():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((3, 8, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(rope.apply(x, np.zeros(3, dtype=np.int64)), x)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(3)
    d = 64
    f = rope.inv_freq(d)
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    # each (i, i + d/2) pair keeps its length
    for p in [1, 17, 4095, 70000]:
        r = rope.rotate_f64(q, np.array([p]), f)[0, 0]
        np.testing.assert_allclose(r[:32] ** 2 + r[32:] ** 2, q[0, 0, :32] ** 2 + q[0, 0, 32:] ** 2, rtol=1e-12)
    # <R(m) q, R(n) k> depends only on m - n
    dots = []
    for m, n in [(10, 3), (107, 100), (5007, 5000)]:
        rq = rope.rotate_f64(q, np.array([m]), f)[0, 0]
        rk = rope.rotate_f64(k, np.array([n]), f)[0, 0]
        dots.append(rq @ rk)
    np.testing.assert_allclose(dots, dots[0], rtol=1e-9)


def test_rope_unit_vector_turns_by_the_angle():
    # e_0 at position p moves to (cos p f_0, sin p f_0) in the (0, 32) pair;
    # f_0 = 1 so the angle is p radians.  A sign or pairing slip fails this.
    d = 64
    x = np.zeros((1, 1, d))
    x[0, 0, 0] = 1.0
    r = rope.rotate_f64(x, np.array([2]), rope.inv_freq(d))[0, 0]
    assert abs(r[0] - math.cos(2.0)) < 1e-15 and abs(r[32] - math.sin(2.0)) < 1e-15
    assert np.count_nonzero(r) == 2

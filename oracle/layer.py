"""One Llama decode layer around the paged attention, float64 (test
infrastructure only).

Source: "An Inference Engine in 1,500 Lines of CUDA: The Map" -- the engine
runs Llama 3.2 1B Instruct (opening paragraph), computes RMSNorm in its own
kernel (``rmsNormKernel``, Korean page, "What is in the box" table, which
cites Zhang & Sennrich 2019 for it), keeps a 2048-wide hidden state
(``buf_2048_*`` buffers in "A function with 51 parameters") and does the
projections with a vendor GEMM (chapter-4 title).  The pages do not print
the layer's formulas; they are the public Llama definitions, restated:

  rmsnorm(x, w) = x / sqrt(mean(x^2) + eps) * w          (eps = 1e-5)
  a    = rmsnorm(h, w_attn)
  q, k, v = a Wq^T, a Wk^T, a Wv^T                       (n_q*64, n_kv*64, n_kv*64 wide)
  o    = attention(rope(q), rope(k), v)                  (the decode step: the new
                                                          token's k, v join the history)
  h    = h + o Wo^T
  m    = rmsnorm(h, w_mlp)
  g, u = m Wg^T, m Wu^T
  h    = h + (silu(g) * u) Wd^T,   silu(x) = x / (1 + e^-x)

Reading adopted for where values are rounded: every buffer the engine keeps
is bf16 (its buffers are nv_bfloat16), so with ``rnd = round_bf16`` the
oracle rounds to bf16 (nearest even) exactly where a buffer is written --
a, q, k, v, the rotated q and k, o, h after each residual add, m, g, u and
the activation -- and computes everything between in float64.  With
``rnd = None`` nothing is rounded (the form the library pins compare).
"""
import math

import numpy as np

from . import attention, bf16, rope

EPS = 1e-5


def round_bf16(x):
    """float64 -> nearest-even bf16 -> float64."""
    return bf16.to_f64(bf16.from_f64(np.asarray(x, dtype=np.float64)))


def _ident(x):
    return np.asarray(x, dtype=np.float64)


def rmsnorm(x, w, eps=EPS):
    """Rows of x (float64 [rows][dim]) scaled to unit root mean square, times
    the gain w [dim]."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def linear(x, W):
    """x [rows][k] times W^T, W [n][k] (a projection in the Hugging Face
    weight layout)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def mlp(m, Wg, Wu, Wd, rnd=round_bf16):
    """The gated MLP on the normalised hidden state m."""
    rnd = rnd or _ident
    g = rnd(linear(m, Wg))
    u = rnd(linear(m, Wu))
    act = rnd(silu(g) * u)
    return linear(act, Wd)


def decode_layer(h, W, hist_k, hist_v, positions, n_q, n_kv, scale=0.125, eps=EPS, rnd=round_bf16):
    """One decode step of one layer for a batch of rows.

    h: float64 [B][n_q*64], the residual stream before the layer.
    W: float64 weights -- attn_norm [D], wq [n_q*64][D], wk and wv
      [n_kv*64][D], wo [D][n_q*64], mlp_norm [D], wg and wu [I][D], wd [D][I].
    hist_k[b], hist_v[b]: float64 [positions[b]][n_kv][64], row b's cached
      (rotated) keys and values of tokens 0 .. positions[b] - 1.
    Returns dict: h (after the layer) and the intermediate buffers a, q, k
    (before RoPE), q_rot, k_rot, v, o, h_mid (after the attention residual),
    m, g, u (gate and up projections), act.
    """
    rnd = rnd or _ident
    h = np.asarray(h, dtype=np.float64)
    B = h.shape[0]
    d = 64
    pos = np.asarray(positions)
    a = rnd(rmsnorm(h, W["attn_norm"], eps))
    q = rnd(linear(a, W["wq"])).reshape(B, n_q, d)
    k = rnd(linear(a, W["wk"])).reshape(B, n_kv, d)
    v = rnd(linear(a, W["wv"])).reshape(B, n_kv, d)
    f = rope.inv_freq(d)
    q_rot = rnd(rope.rotate_f64(q, pos, f))
    k_rot = rnd(rope.rotate_f64(k, pos, f))
    o = np.zeros((B, n_q, d))
    for b in range(B):
        K = np.concatenate([np.asarray(hist_k[b], dtype=np.float64).reshape(-1, n_kv, d), k_rot[b][None]])
        V = np.concatenate([np.asarray(hist_v[b], dtype=np.float64).reshape(-1, n_kv, d), v[b][None]])
        o[b] = attention._attend(q_rot[b], K, V, scale)
    o = rnd(o.reshape(B, n_q * d))
    h_mid = rnd(h + linear(o, W["wo"]))
    m = rnd(rmsnorm(h_mid, W["mlp_norm"], eps))
    g = rnd(linear(m, W["wg"]))
    u = rnd(linear(m, W["wu"]))
    act = rnd(silu(g) * u)
    h_out = rnd(h_mid + linear(act, W["wd"]))
    return dict(h=h_out, a=a, q=q, k=k, q_rot=q_rot, k_rot=k_rot, v=v, o=o, h_mid=h_mid, m=m, g=g, u=u, act=act)


def init_scale(fan_in):
    """Standard deviation of the synthetic weights: 1 / sqrt(fan_in), so each
    projection keeps unit-variance inputs at unit variance."""
    return 1.0 / math.sqrt(fan_in)

"""Llama-3-scaled rotary position embedding, float64 (test infrastructure only).

Source: "An Inference Engine in 1,500 Lines of CUDA: The Map", section "The
path of one inference", step (3): the engine builds a positional-encoding
table from head_dim, the maximum sequence length and five numbers -- base
500000, factor 32, low-frequency factor 1, high-frequency factor 4 and an
original context of 8192 -- and the Korean page's "What is in the box"
table names the kernel ``ropeKernel_llama3``.  The pages do not print the
rule that uses the five numbers; it is the public Llama 3 ``rope_scaling``
definition, restated here:

  f_i   = base ** (-2 i / d),  i = 0 .. d/2 - 1        (plain RoPE frequency)
  w_i   = 2 pi / f_i                                   (its wavelength)
  w_hi  = orig / high_freq_factor,  w_lo = orig / low_freq_factor
  f_i'  = f_i                     if w_i < w_hi        (fast dims kept)
        = f_i / factor            if w_i > w_lo        (slow dims slowed)
        = (1 - s) f_i / factor + s f_i  otherwise,
          s = (orig / w_i - low_freq_factor) / (high_freq_factor - low_freq_factor)

Rotation (reading adopted where the pages are silent): dimension i is paired
with i + d/2 ("rotate half", the layout of Hugging Face Llama checkpoints,
which the engine loads), and at position p the pair (x, y) becomes
(x cos a - y sin a, y cos a + x sin a) with a = p * f_i'.  The rotated bf16
buffer holds the result rounded to nearest-even.
"""
import math

import numpy as np

from . import bf16

ROPE_THETA = 500000.0
ROPE_FACTOR = 32.0
LOW_FREQ_FACTOR = 1.0
HIGH_FREQ_FACTOR = 4.0
ORIGINAL_MAX_POS = 8192


def inv_freq(head_dim: int = 64, theta: float = ROPE_THETA, factor: float = ROPE_FACTOR,
             low_freq_factor: float = LOW_FREQ_FACTOR, high_freq_factor: float = HIGH_FREQ_FACTOR,
             original_max_pos: int = ORIGINAL_MAX_POS) -> np.ndarray:
    """The d/2 scaled frequencies f_i' in float64, one per rotated pair."""
    half = head_dim // 2
    out = np.empty(half, dtype=np.float64)
    w_hi = original_max_pos / high_freq_factor
    w_lo = original_max_pos / low_freq_factor
    for i in range(half):
        f = theta ** (-(2.0 * i) / head_dim)
        w = 2.0 * math.pi / f
        if w < w_hi:
            out[i] = f
        elif w > w_lo:
            out[i] = f / factor
        else:
            s = (original_max_pos / w - low_freq_factor) / (high_freq_factor - low_freq_factor)
            out[i] = (1.0 - s) * f / factor + s * f
    return out


def rotate_f64(x: np.ndarray, positions: np.ndarray, freqs: np.ndarray) -> np.ndarray:
    """Rotate float64 vectors x[T, H, d] by their token's position, unrounded."""
    x = np.asarray(x, dtype=np.float64)
    T, H, d = x.shape
    half = d // 2
    out = np.empty_like(x)
    for t in range(T):
        a = float(positions[t]) * freqs            # [half]
        c, s = np.cos(a), np.sin(a)
        lo, hi = x[t, :, :half], x[t, :, half:]
        out[t, :, :half] = lo * c - hi * s
        out[t, :, half:] = hi * c + lo * s
    return out


def apply(x_bits: np.ndarray, positions: np.ndarray, freqs: np.ndarray | None = None) -> np.ndarray:
    """RoPE on bf16 vectors x_bits[T, H, d]: float64 rotation, then bf16 RNE."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if freqs is None:
        freqs = inv_freq(x_bits.shape[-1])
    return bf16.from_f64(rotate_f64(bf16.to_f64(x_bits), np.asarray(positions), freqs))

"""bfloat16 storage for the oracle (test infrastructure only).

The engine's activations and KV cache are bf16 buffers ("An Inference Engine
in 1,500 Lines of CUDA: The Map", sections "The path of one inference" and
"A function with 51 parameters": ``__nv_bfloat16 *kv_cache``,
``nv_bfloat16 *buf_2048_1``).  bf16 is the top half of an IEEE binary32:
1 sign bit, 8 exponent bits, 7 stored significand bits.
"""
import numpy as np


def to_f64(bits) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns (uint16)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):        # NaN patterns stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def from_f64(x) -> np.ndarray:
    """Round float64 values straight to bf16, nearest with ties to even.

    Rounds once, from float64 (no float32 intermediate).  A finite x has the
    form m * 2**e with 0.5 <= |m| < 1; bf16 keeps 8 significant bits, so the
    spacing of representable values near x is 2**(e-8), never finer than the
    subnormal spacing 2**-133.  Results of magnitude 2**128 or more overflow
    to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.round(xf / quantum) * quantum          # numpy rounds halves to even
    big = np.abs(r) >= 2.0 ** 128
    r = np.where(big, np.copysign(np.inf, xf), r)
    out[...] = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    out[nan] = 0x7FC0
    inf = np.isinf(x)
    out[inf] = np.where(x[inf] > 0, 0x7F80, 0xFF80)
    return out

"""Helpers shared by the GPU parity tests (host/device transfers, tolerances)."""
import numpy as np

ATOL_MAX = 2e-2      # max-abs error vs the float64 oracle (attention outputs)
ATOL_MEAN = 2e-3     # mean-abs error vs the float64 oracle


def dev_bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).cuda()


def dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def bits(t):
    """Device bf16 tensor -> numpy uint16 bit patterns."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits_u16):
    return (np.asarray(bits_u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_attention(got_bits, ref, what=""):
    got = f64(got_bits)
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    err = np.abs(got - ref)
    print(f"{what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}", flush=True)
    assert err.max() <= ATOL_MAX, f"{what}: max-abs error {err.max():.3e}"
    assert err.mean() <= ATOL_MEAN, f"{what}: mean-abs error {err.mean():.3e}"
    return err


def ulp_diff(a_bits, b_bits):
    """Distance in bf16 units in the last place (same-sign finite values)."""
    a = np.asarray(a_bits, np.uint16).astype(np.int32)
    b = np.asarray(b_bits, np.uint16).astype(np.int32)
    # map sign-magnitude bit patterns onto a monotone integer line
    a = np.where(a & 0x8000, -(a & 0x7FFF), a)
    b = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(a - b)


# Two correct float32 evaluations of the same attention may differ: the
# softmax weights are rounded to bf16 (relative error <= 2^-9 each) after
# subtracting a running max whose value depends on the evaluation order, so
# each weight can round differently; the output moves by at most about
# 2 * 2^-9 * max|V| plus one bf16 output ulp (2^-8 relative).
CROSS_MAX = 2.0 ** -7 * 2      # |V| <= ~4 in the tests' data
CROSS_MEAN = 2e-4


def check_close_evaluations(a_bits, b_bits, what=""):
    a, b = f64(a_bits), f64(b_bits)
    d = np.abs(a - b)
    print(f"{what}: cross max {d.max():.3e} mean {d.mean():.3e}", flush=True)
    assert d.max() <= CROSS_MAX, f"{what}: evaluations differ by {d.max():.3e}"
    assert d.mean() <= CROSS_MEAN, f"{what}: evaluations differ on average by {d.mean():.3e}"

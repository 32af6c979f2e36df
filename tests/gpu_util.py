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


# Two correct float32 evaluations of the same attention may differ: each
# softmax weight is rounded to bf16 (relative error <= u = 2^-8) after
# subtracting a running max whose value depends on the evaluation order, so
# each weight can round differently.  With o = sum_j p_j V_j / sum_j p_j, a
# relative change e_j of weight j moves o by sum_j p_j e_j (V_j - o) / sum_j p_j,
# at most u (A + |o|) per evaluation, where A = sum_j p_j |V_j| / sum_j p_j;
# each output is then rounded to bf16 once more (at most u |o|).  Two
# evaluations differ by at most 2u (A + |o|) + 2u |o| (first order), checked
# element by element where the oracle's A and o are given (cross_bound), and
# by CROSS_MAX (|V| <= ~4 in the tests' data) otherwise.
U_BF16 = 2.0 ** -8
CROSS_MAX = 2.0 ** -6
CROSS_MEAN = 2e-4


def cross_bound(ref, ref_abs_v):
    """Per-element bound on the difference of two correct evaluations, from
    the float64 oracle's output (ref) and its output with |V| in place of V
    (ref_abs_v = A, the same softmax weights)."""
    return 2 * U_BF16 * (ref_abs_v + np.abs(ref)) + 2 * U_BF16 * np.abs(ref) + 1e-6


def abs_pool(pool_bits):
    """bf16 pool with every value's sign cleared (the oracle then returns A)."""
    return np.asarray(pool_bits, np.uint16) & np.uint16(0x7FFF)


def check_close_evaluations(a_bits, b_bits, what="", bound=None):
    a, b = f64(a_bits), f64(b_bits)
    d = np.abs(a - b)
    print(f"{what}: cross max {d.max():.3e} mean {d.mean():.3e}", flush=True)
    if bound is not None:
        worst = np.max(d - bound)
        assert worst <= 0, f"{what}: evaluations differ beyond the per-element bound by {worst:.3e}"
    assert d.max() <= CROSS_MAX, f"{what}: evaluations differ by {d.max():.3e}"
    assert d.mean() <= CROSS_MEAN, f"{what}: evaluations differ on average by {d.mean():.3e}"

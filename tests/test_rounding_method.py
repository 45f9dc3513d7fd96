"""The rounding method the RoPE / QK-norm kernels use for fp64 -> bf16, checked on the host.

The kernels round a binary64 value y to bfloat16 as: RNE to binary32, then RNE to bfloat16,
except when the binary32 value lies exactly on a bfloat16 midpoint (low 16 bits 0x8000) or in
the binary32 subnormal range, where they use an exact one-step rounding.  This test applies the
same two steps with numpy's (RNE) casts and compares with the oracle's correctly rounded
fp64 -> bf16 on random values, exact midpoints and values a few fp64 ulps around them, and the
zero / subnormal / overflow / inf edges: the two-step form must equal one rounding everywhere.
(It pins the argument, not the device code; the GPU parity tests pin the kernels.)"""
import numpy as np

import oracle


def _bits_bf16_exact(y):
    return (oracle.round_bf16(y).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bits_bf16_two_step(y):
    with np.errstate(over="ignore"):
        f = y.astype(np.float32)                       # RNE binary64 -> binary32
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)   # RNE binary32 -> bfloat16
    u32 = f.view(np.uint32)
    slow = ((u32 & 0xFFFF) == 0x8000) | ((u32 & 0x7F800000) == 0)
    r[slow] = _bits_bf16_exact(y[slow])
    return r, slow


def test_two_step_rounding_equals_one_rounding():
    rng = np.random.default_rng(20261202)
    parts = [rng.standard_normal(400_000) * np.exp2(rng.integers(-140, 128, 400_000))]
    b = rng.integers(0, 0x7F7F, 100_000).astype(np.uint32)
    mid = ((b << 16) | 0x8000).view(np.float32).astype(np.float64)
    sgn = np.where(rng.random(mid.size) < 0.5, -1.0, 1.0)
    for k in (0, 1, -1, 3, -3, 1 << 20, -(1 << 20), 1 << 28, -(1 << 28)):
        parts.append(sgn * (mid + k * np.spacing(mid)))
    parts.append(np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-40, 2.0 ** -126, 2.0 ** -127,
                           1.5 * 2.0 ** -133, 3.3895313892515355e38, 3.4e38, 3.5e38, 1e300, 5e-324]))
    y = np.concatenate(parts)
    got, slow = _bits_bf16_two_step(y)
    ref = _bits_bf16_exact(y)
    assert slow.any() and not slow.all()
    assert np.array_equal(got, ref)


def test_two_step_rounding_needs_the_midpoint_fallback():
    """Without the fallback the two steps round wrongly just above / below a midpoint."""
    one_plus_mid = 1.0 + 2.0 ** -8                 # a bfloat16 midpoint (tie between 1 and 1+2^-7)
    y = np.array([one_plus_mid + 2.0 ** -40, one_plus_mid - 2.0 ** -40])
    f = y.astype(np.float32)                       # both land exactly on the midpoint
    assert np.all((f.view(np.uint32) & 0xFFFF) == 0x8000)
    u = f.view(np.uint32).astype(np.uint64)
    naive = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    exact = _bits_bf16_exact(y)
    assert naive[0] != exact[0]                    # tie-to-even went down, the value is above
    assert np.array_equal(_bits_bf16_two_step(y)[0], exact)

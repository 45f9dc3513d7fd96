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


# ---------------------------------------------------------------------------------------------
# The QK-norm kernel's bfloat16 path: y32 = x * r32 * w in binary32 (r32 = r rounded to
# binary32), RNE to bfloat16, except for lanes whose y32 lies within 4 binary32 ulps of a
# bfloat16 midpoint (or is subnormal), which round x * r * w from binary64 exactly.
# ---------------------------------------------------------------------------------------------

def _norm_fast_path(x, r, w):
    """numpy float32 emulation of the kernel's fast path -> (bf16 bits, slow mask)."""
    r32 = np.float32(r)
    y = (x.astype(np.float32) * r32) * w.astype(np.float32)        # two binary32 roundings
    u = y.view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    u32 = y.view(np.uint32)
    slow = (((u32 - np.uint32(0x7FFC)) & np.uint32(0xFFFF)) <= 8) | ((u32 & 0x7F800000) == 0)
    return bits, slow


def test_norm_fast_path_is_correctly_rounded_outside_the_window():
    """Wherever the kernel keeps its binary32 result, that result rounds to the same bfloat16 as
    the correctly rounded binary64 product x * r * w: on random tokens, and on inputs crafted so
    that x * r * w falls within a few binary32 ulps of a bfloat16 midpoint."""
    rng = np.random.default_rng(7)
    n = 200_000
    x = oracle.round_bf16(rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n)))
    w = (1.0 + 0.3 * rng.standard_normal(n)).astype(np.float32).astype(np.float64)
    r = 1.0 / np.sqrt(rng.uniform(0.01, 100.0) + 1e-6)
    # crafted: choose w so that x * r * w is a midpoint plus k binary64 units of 2^-30 relative
    b = rng.integers(0x3F00, 0x4100, 50_000).astype(np.uint32)
    mid = ((b << 16) | 0x8000).view(np.float32).astype(np.float64)
    xc = oracle.round_bf16(rng.uniform(0.5, 2.0, mid.size))
    k = rng.integers(-64, 65, mid.size)
    wc = (mid * (1.0 + k * 2.0 ** -30) / (xc * r)).astype(np.float32).astype(np.float64)
    x, w = np.concatenate([x, xc]), np.concatenate([w, wc])
    bits, slow = _norm_fast_path(x, r, w)
    exact = _bits_bf16_exact(x * np.float64(np.float32(r)) * w)   # reference with r32's value
    exact_r = _bits_bf16_exact(x * r * w)                        # ... and with r itself
    keep = ~slow
    assert slow.any() and keep.mean() > 0.5
    assert np.array_equal(bits[keep], exact_r[keep])
    assert np.array_equal(bits[keep], exact[keep])


def test_norm_fast_path_needs_the_window():
    """Without the window the binary32 product rounds to the wrong side of a midpoint."""
    rng = np.random.default_rng(8)
    b = rng.integers(0x3F00, 0x4100, 200_000).astype(np.uint32)
    mid = ((b << 16) | 0x8000).view(np.float32).astype(np.float64)
    x = oracle.round_bf16(rng.uniform(0.5, 2.0, mid.size))
    r = 0.7390851332151607
    k = rng.integers(-40, 41, mid.size)
    w = (mid * (1.0 + k * 2.0 ** -30) / (x * r)).astype(np.float32).astype(np.float64)
    bits, slow = _norm_fast_path(x, r, w)
    exact = _bits_bf16_exact(x * r * w)
    assert (bits != exact).any()                       # some land on the wrong side ...
    assert slow[bits != exact].all()                   # ... and the window catches every one

"""Pins of the fp64 oracle against what the mathematics and the pages fix.

Every test here runs on the CPU.  None compares the oracle with itself through
a retyped formula: each checks a closed form, an invariant, a library route
(torch / numpy in fp64) or a value printed on the pages.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, video_grid

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


# --------------------------------------------------------------------------------------
# Workload geometry: the pages' worked example
# --------------------------------------------------------------------------------------

def test_geometry_worked_example():
    with open(os.path.join(GOLDEN, "geometry.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        grid = video_grid(c["frames"], c["height"], c["width"])
        assert list(grid) == c["grid"]
        assert grid[0] * grid[1] * grid[2] == c["S"]
        if "S_mod_8" in c:
            assert c["S"] % 8 == c["S_mod_8"]


def test_workload_table():
    sizes = {w.name: (w.Nv, w.S, w.n_chunks) for w in WORKLOADS}
    assert sizes["tiny"] == (240, 256, 4)
    assert sizes["lite-clip"] == (3024, 3216, 7)
    assert sizes["image-dit"] == (4096, 4352, 1)
    assert sizes["pro-clip"] == (51840, 52608, 13)
    assert sizes["long-video"] == (118800, 119056, 15)
    for w in WORKLOADS:
        assert sum(w.split) == w.D


# --------------------------------------------------------------------------------------
# Rounding to storage formats
# --------------------------------------------------------------------------------------

def test_round_bf16_matches_torch_on_fp32_values():
    # Values exactly representable in fp32: a single RNE step to bf16, which
    # torch's fp32 -> bf16 conversion performs.
    x32 = np.concatenate([
        RNG.standard_normal(20000).astype(np.float32),
        (RNG.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormal range
        (RNG.standard_normal(2000) * 1e38).astype(np.float32),
        np.array([3.3895314e38, -3.3895314e38, 3.4e38], dtype=np.float32),
    ])
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(x32.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_bf16_ties_to_even():
    one = 1.0
    assert oracle.round_bf16(one + 2.0 ** -8)[()] == 1.0              # tie -> even (down)
    assert oracle.round_bf16(one + 3 * 2.0 ** -8)[()] == 1.0 + 2.0 ** -6  # tie -> even (up)
    assert oracle.round_bf16(one + 2.0 ** -8 + 2.0 ** -40)[()] == 1.0 + 2.0 ** -7
    assert oracle.round_bf16(2.0 ** -134)[()] == 0.0                   # half the min subnormal
    assert oracle.round_bf16(3 * 2.0 ** -134)[()] == 2.0 ** -132
    assert np.isinf(oracle.round_bf16(3.5e38)[()])


# --------------------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------------------

SPLIT = (16, 24, 24)
THETA = 10000.0


def _rand(*shape):
    return RNG.standard_normal(shape)


def test_rope_identity_at_origin():
    x = _rand(64)
    assert np.array_equal(oracle.rope_vec(x, (0, 0, 0), SPLIT, THETA), x)


def test_rope_preserves_pair_norms():
    x = _rand(64)
    y = oracle.rope_vec(x, (3, 7, 11), SPLIT, THETA)
    nx = x.reshape(32, 2)
    ny = y.reshape(32, 2)
    np.testing.assert_allclose(np.hypot(ny[:, 0], ny[:, 1]), np.hypot(nx[:, 0], nx[:, 1]),
                               rtol=1e-14)


def test_rope_inverse():
    x = _rand(128)
    sp = (32, 48, 48)
    y = oracle.rope_vec(oracle.rope_vec(x, (5, 9, 33), sp, THETA), (-5, -9, -33), sp, THETA)
    np.testing.assert_allclose(y, x, atol=1e-13)


def test_rope_relative_position():
    q, k = _rand(64), _rand(64)
    p, pp, delta = np.array([1, 4, 9]), np.array([0, 7, 2]), np.array([6, -3, 13])
    a = oracle.rope_vec(q, p, SPLIT, THETA) @ oracle.rope_vec(k, pp, SPLIT, THETA)
    b = oracle.rope_vec(q, p + delta, SPLIT, THETA) @ oracle.rope_vec(k, pp + delta, SPLIT, THETA)
    assert abs(a - b) < 1e-12
    # and it does depend on p - p'
    c = oracle.rope_vec(q, p + np.array([1, 0, 0]), SPLIT, THETA) @ oracle.rope_vec(k, pp, SPLIT,
                                                                                     THETA)
    assert abs(a - c) > 1e-3


def test_rope_first_pair_of_each_axis_rotates_by_position():
    # The first pair of every axis segment has frequency theta^0 = 1, so a unit
    # vector on it turns by exactly p_axis radians, counter-clockwise.
    pos = (2, 5, 11)
    for axis, off in enumerate((0, 16, 40)):
        x = np.zeros(64)
        x[off] = 1.0
        y = oracle.rope_vec(x, pos, SPLIT, THETA)
        want = np.zeros(64)
        want[off], want[off + 1] = math.cos(pos[axis]), math.sin(pos[axis])
        np.testing.assert_allclose(y, want, atol=1e-15)


def test_rope_matches_complex_multiplication():
    # Library route for the rotation itself: pairs as complex numbers times
    # e^{i phi}, with phi from the per-axis frequency ladder.
    sp = (32, 48, 48)
    x = _rand(128)
    pos = (7, 13, 40)
    phis = []
    for a, d in enumerate(sp):
        j = torch.arange(d // 2, dtype=torch.float64)
        phis.append(pos[a] * torch.pow(torch.tensor(THETA, dtype=torch.float64), -2 * j / d))
    phi = torch.cat(phis)
    z = torch.view_as_complex(torch.from_numpy(x).reshape(64, 2).contiguous())
    want = torch.view_as_real(z * torch.polar(torch.ones_like(phi), phi)).reshape(128).numpy()
    np.testing.assert_allclose(oracle.rope_vec(x, pos, sp, THETA), want, atol=1e-13)


def test_rope3d_token_positions_row_major():
    grid = (2, 3, 5)
    x = _rand(1, 30, 2, 64)
    y = oracle.rope3d(x, grid, SPLIT, THETA)
    for n in (0, 1, 4, 5, 14, 15, 29):
        t, h, w = np.unravel_index(n, grid)
        for hd in range(2):
            np.testing.assert_array_equal(y[0, n, hd],
                                          oracle.rope_vec(x[0, n, hd], (t, h, w), SPLIT, THETA))


def test_rope_2d_and_single_frame():
    x = _rand(1, 16, 1, 128)
    y2d = oracle.rope3d(x, (1, 4, 4), (0, 64, 64), THETA)
    y3d = oracle.rope3d(x, (1, 4, 4), (32, 48, 48), THETA)
    # t = 0 for every token: the t segment of the 3-D split is untouched
    np.testing.assert_array_equal(y3d[..., :32], x[..., :32])
    assert not np.allclose(y2d[..., 64:], x[..., 64:])
    with pytest.raises(ValueError):
        oracle.rope3d(x, (1, 4, 5), (32, 48, 48), THETA)


# --------------------------------------------------------------------------------------
# Joint concat + permute
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [np.uint16, np.float32, np.float64])
def test_permute_matches_numpy(dtype):
    segs = [(RNG.integers(0, 65535, size=(2, n, 3, 8))).astype(dtype) for n in (17, 5, 0, 9)]
    out = oracle.joint_concat_permute(segs)
    want = np.concatenate(segs, axis=1).transpose(0, 2, 1, 3)
    assert out.dtype == want.dtype and np.array_equal(out, want)


def test_permute_inverse():
    segs = [RNG.standard_normal((1, n, 4, 16)) for n in (11, 3)]
    out = oracle.joint_concat_permute(segs)
    back = out.transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(back[:, :11], segs[0])
    np.testing.assert_array_equal(back[:, 11:], segs[1])


# --------------------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------------------

def _qkv(B, H, Sq, Skv, D):
    return _rand(B, H, Sq, D), _rand(B, H, Skv, D), _rand(B, H, Skv, D)


def test_attention_single_key_returns_value():
    q, k, v = _qkv(1, 2, 5, 1, 16)
    out, lse = oracle.attention(q, k, v, 0.25)
    np.testing.assert_array_equal(out, np.broadcast_to(v, out.shape))
    np.testing.assert_allclose(lse, 0.25 * np.einsum("bhqd,bhkd->bhq", q, k), rtol=1e-15)


def test_attention_identical_keys_give_mean_value():
    q, k, v = _qkv(1, 2, 7, 13, 32)
    k[:] = k[:, :, :1]
    out, lse = oracle.attention(q, k, v, 0.3)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=2, keepdims=True), out.shape),
                               atol=1e-14)
    s = 0.3 * np.einsum("bhqd,bhd->bhq", q, k[:, :, 0])
    np.testing.assert_allclose(lse, s + math.log(13), rtol=1e-14)


def test_attention_zero_query_is_uniform():
    q, k, v = _qkv(1, 1, 3, 40, 8)
    q[:] = 0
    out, lse = oracle.attention(q, k, v, 1.0)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(v[0, 0].mean(0), (3, 8)), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(40), rtol=1e-15)


@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 4), (1, 2, 9, 17, 8), (2, 3, 33, 64, 64),
                                   (1, 1, 64, 48, 128)])
def test_attention_matches_torch_softmax(shape):
    B, H, Sq, Skv, D = shape
    q, k, v = _qkv(B, H, Sq, Skv, D)
    scale = 1.0 / math.sqrt(D)
    out, lse = oracle.attention(q, k, v, scale)
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    logits = (tq @ tk.transpose(-1, -2)) * scale
    want = torch.softmax(logits, dim=-1) @ tv
    np.testing.assert_allclose(out, want.numpy(), atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=-1).numpy(), atol=1e-13)


def test_attention_hard_max_limit():
    q, k, v = _qkv(1, 1, 4, 30, 16)
    out, _ = oracle.attention(q, k, v, 1e5)
    amax = np.argmax(np.einsum("qd,kd->qk", q[0, 0], k[0, 0]), axis=1)
    np.testing.assert_allclose(out[0, 0], v[0, 0][amax], atol=1e-12)


def test_attention_kv_permutation_invariance():
    q, k, v = _qkv(1, 2, 11, 37, 16)
    perm = RNG.permutation(37)
    a = oracle.attention(q, k, v, 0.25)
    b = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.25)
    np.testing.assert_allclose(a[0], b[0], atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13)


def test_attention_query_rows_independent():
    q, k, v = _qkv(2, 3, 19, 23, 16)
    out, lse = oracle.attention(q, k, v, 0.25)
    rows = np.array([0, 5, 18, 19, 40, 113, 2 * 3 * 19 - 1])
    o_r, l_r = oracle.attention_rows(q, k, v, rows, 0.25)
    np.testing.assert_array_equal(o_r, out.reshape(-1, 16)[rows])
    np.testing.assert_array_equal(l_r, lse.reshape(-1)[rows])


@pytest.mark.parametrize("kv_chunk", [1, 3, 7, 16, 50, 51, 0, 1000])
def test_chunked_plus_merge_equals_unchunked(kv_chunk):
    q, k, v = _qkv(1, 2, 9, 51, 16)
    q *= 3.0  # sharper softmax: partial maxima differ between chunks
    a_out, a_lse = oracle.attention(q, k, v, 0.25)
    b_out, b_lse = oracle.attention_chunked(q, k, v, 0.25, kv_chunk)
    np.testing.assert_allclose(b_out, a_out, atol=1e-12)
    np.testing.assert_allclose(b_lse, a_lse, atol=1e-12)


# --------------------------------------------------------------------------------------
# LSE merge
# --------------------------------------------------------------------------------------

def test_lse_merge_equal_weights():
    parts = _rand(2, 5, 8)
    lse = np.full((2, 5), 1.7)
    out, L = oracle.lse_merge(parts, lse)
    np.testing.assert_allclose(out, parts.mean(0), atol=1e-15)
    np.testing.assert_allclose(L, 1.7 + math.log(2), atol=1e-15)


def test_lse_merge_ignores_empty_parts():
    parts = _rand(3, 4, 8)
    lse = RNG.standard_normal((3, 4))
    lse[1] = -np.inf
    parts[1] = 1e300  # weight exactly zero
    out, L = oracle.lse_merge(parts, lse)
    o2, L2 = oracle.lse_merge(parts[[0, 2]], lse[[0, 2]])
    np.testing.assert_allclose(out, o2, atol=1e-14)
    np.testing.assert_allclose(L, L2, atol=1e-14)
    out3, L3 = oracle.lse_merge(parts[:1] * 0 + 5, np.full((1, 4), -np.inf))
    assert np.all(out3 == 0) and np.all(np.isneginf(L3))


@pytest.mark.parametrize("cuts", [(0, 20, 51), (0, 1, 2, 30, 51), (0, 51)])
def test_lse_merge_of_kv_slices_equals_full_attention(cuts):
    q, k, v = _qkv(1, 2, 6, 51, 16)
    q *= 2.0
    full_out, full_lse = oracle.attention(q, k, v, 0.25)
    outs, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l_ = oracle.attention(q, k[:, :, a:b], v[:, :, a:b], 0.25)
        outs.append(o)
        lses.append(l_)
    out, L = oracle.lse_merge(np.stack(outs), np.stack(lses))
    np.testing.assert_allclose(out, full_out, atol=1e-12)
    np.testing.assert_allclose(L, full_lse, atol=1e-12)


# --------------------------------------------------------------------------------------
# Whole pipeline on a tiny joint sequence
# --------------------------------------------------------------------------------------

def test_pipeline_against_torch_route():
    """prepare_qkv + attention against a torch fp64 route built from library
    pieces (complex rotation, cat, permute, softmax) on a tiny joint sequence."""
    grid, sp = (2, 2, 3), (16, 24, 24)
    B, H, D = 1, 2, 64
    segs = {n: [RNG.standard_normal((B, 12, H, D)), RNG.standard_normal((B, 5, H, D))]
            for n in "qkv"}
    q, k, v = oracle.prepare_qkv(segs["q"], segs["k"], segs["v"], grid, sp, THETA, "f32")
    out, lse = oracle.attention(q, k, v, 0.125)

    def rot(x):
        t = torch.from_numpy(x)
        pos = torch.stack(torch.meshgrid(*[torch.arange(g) for g in grid], indexing="ij"),
                          -1).reshape(-1, 3).to(torch.float64)
        phis = []
        for a, d in enumerate(sp):
            j = torch.arange(d // 2, dtype=torch.float64)
            phis.append(pos[:, a:a + 1] * torch.pow(torch.tensor(THETA, dtype=torch.float64),
                                                     -2 * j / d))
        phi = torch.cat(phis, dim=1)[None, :, None, :]
        z = torch.view_as_complex(t.reshape(B, 12, H, D // 2, 2).contiguous())
        r = torch.view_as_real(z * torch.polar(torch.ones_like(phi), phi)).reshape(B, 12, H, D)
        return r.to(torch.float32).to(torch.float64)

    def joint(segs_, rope):
        first = rot(segs_[0]) if rope else torch.from_numpy(segs_[0])
        return torch.cat([first, torch.from_numpy(segs_[1])], dim=1).transpose(1, 2)

    tq, tk, tv = joint(segs["q"], True), joint(segs["k"], True), joint(segs["v"], False)
    logits = (tq @ tk.transpose(-1, -2)) * 0.125
    want = torch.softmax(logits, -1) @ tv
    np.testing.assert_allclose(out, want.numpy(), atol=1e-6)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, -1).numpy(), atol=1e-6)


# ---------------------------------------------------------------------------------------------
# QK-norm (RMS over a token's whole hidden vector, "Context Parallelism in vLLM Omni Neuron",
# §Self-Attention with Context Parallelism: norm_q / norm_k before unflatten and RoPE)
# ---------------------------------------------------------------------------------------------

def test_rms_norm_worked_example():
    # mean of squares of (1, 2, 3, 4) is 30/4 = 7.5
    y = oracle.rms_norm(np.array([[1.0, 2.0, 3.0, 4.0]]), np.ones(4), 0.0)
    np.testing.assert_allclose(y, np.array([[1.0, 2.0, 3.0, 4.0]]) / math.sqrt(7.5), rtol=1e-15)


def test_rms_norm_constant_row_and_eps():
    # a row of a's: mean square a^2, so y = a / sqrt(a^2 + eps) * w exactly in the formula
    a, eps = -3.0, 0.5
    w = RNG.standard_normal(6)
    y = oracle.rms_norm(np.full((1, 6), a), w, eps)
    np.testing.assert_allclose(y[0], a / math.sqrt(a * a + eps) * w, rtol=1e-15)


def test_rms_norm_output_has_unit_rms_and_is_scale_free():
    x = RNG.standard_normal((5, 384)) * RNG.uniform(0.1, 10.0, (5, 1))
    y = oracle.rms_norm(x, np.ones(384), 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(axis=1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.rms_norm(-7.5 * x, np.ones(384), 0.0), -y, rtol=1e-14)


def test_rms_norm_weight_is_per_channel():
    x = RNG.standard_normal((3, 64))
    w = np.zeros(64)
    w[17] = 2.5
    y = oracle.rms_norm(x, w, 1e-6)
    assert (y[:, :17] == 0).all() and (y[:, 18:] == 0).all()
    np.testing.assert_allclose(y[:, 17], 2.5 * x[:, 17] / np.sqrt((x * x).mean(1) + 1e-6), rtol=1e-14)


def test_rms_norm_matches_torch():
    x = RNG.standard_normal((7, 3 * 128))
    w = RNG.standard_normal(3 * 128)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (3 * 128,), weight=torch.from_numpy(w),
                                        eps=1e-6)
    np.testing.assert_allclose(oracle.rms_norm(x, w, 1e-6), want.numpy(), rtol=1e-13, atol=1e-15)


def test_qknorm_then_rope_keeps_unit_rms_per_token():
    # RoPE rotates pairs, so after an RMS norm with w = 1, eps = 0 every token's hidden
    # vector (all heads) still has RMS 1; the other segments are normalised and not rotated.
    grid, sp = (2, 3, 4), (16, 24, 24)
    B, H, D = 2, 3, 64
    segs = [RNG.standard_normal((B, 24, H, D)) * 3.0, RNG.standard_normal((B, 5, H, D))]
    v = [np.zeros_like(s) for s in segs]
    ones = np.ones(H * D)
    q, _, _ = oracle.prepare_qkv(segs, segs, v, grid, sp, THETA, "f32", norm_q=[ones, ones],
                                 norm_k=None, eps=0.0)
    rms = np.sqrt((q.transpose(0, 2, 1, 3) ** 2).reshape(B, 29, H * D).mean(-1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-6)       # f32 storage rounding only
    _, k, _ = oracle.prepare_qkv(segs, segs, v, grid, sp, THETA, "f32", norm_q=[ones, ones])
    # no norm on K: segment 1 is copied exactly
    np.testing.assert_array_equal(k[:, :, 24:], segs[1].transpose(0, 2, 1, 3))


def test_qknorm_segment_without_weights_is_untouched():
    grid, sp = (1, 2, 2), (0, 32, 32)
    B, H, D = 1, 2, 64
    segs = [RNG.standard_normal((B, 4, H, D)), RNG.standard_normal((B, 3, H, D))]
    v = [np.zeros_like(s) for s in segs]
    w = RNG.standard_normal(H * D)
    q1, _, _ = oracle.prepare_qkv(segs, segs, v, grid, sp, THETA, "f32", norm_q=[w, None])
    q0, _, _ = oracle.prepare_qkv(segs, segs, v, grid, sp, THETA, "f32")
    np.testing.assert_array_equal(q1[:, :, 4:], q0[:, :, 4:])
    assert not np.array_equal(q1[:, :, :4], q0[:, :, :4])


def _torch_route_qknorm_rope(x, w, eps, grid, split, theta, *, order="norm_first", weight_after=False,
                             per_head=False, round_between=True):
    """prepare_qkv's segment-0 Q, built only from torch library pieces: rms_norm over the token's
    H*D values with the weight, a stored bf16 tensor, RoPE as multiplication of (x_2j + i x_2j+1)
    by e^(i phi) (torch.polar), a stored bf16 tensor.  The keyword arguments build the plausible
    wrong compositions the pin must reject."""
    B, S, H, D = x.shape
    t = torch.from_numpy(x)
    wt = torch.from_numpy(w)
    st = lambda a: a.to(torch.float32).to(torch.bfloat16).to(torch.float64)  # noqa: E731  stored bf16

    def norm(a):
        if per_head:
            return torch.nn.functional.rms_norm(a, (D,), eps=eps) * wt.reshape(H, D)
        return torch.nn.functional.rms_norm(a.reshape(B, S, H * D), (H * D,), weight=None if weight_after else wt,
                                            eps=eps).reshape(B, S, H, D)

    pos = np.stack(np.unravel_index(np.arange(S), grid), -1)       # (t, h, w) of each token
    phi = []
    for a, d in enumerate(split):
        j = np.arange(d // 2)
        phi.append(pos[:, a:a + 1] * theta ** (-2.0 * j / d))
    phi = torch.from_numpy(np.concatenate(phi, -1))                 # [S, D/2]
    rot = torch.polar(torch.ones_like(phi), phi)

    def rope(a):
        z = torch.view_as_complex(a.reshape(B, S, H, D // 2, 2).contiguous()) * rot[None, :, None, :]
        return torch.view_as_real(z).reshape(B, S, H, D)

    if order == "norm_first":
        y = norm(t)
        if round_between:
            y = st(y)
        y = rope(y)
        if weight_after:
            y = y * wt.reshape(H, D)
    else:                                                            # RoPE, then the norm
        y = norm(st(rope(t)))
    return st(y).numpy()


def _bf16_ulp(x):
    ax = np.abs(x)
    return np.exp2(np.maximum(np.floor(np.log2(np.where(ax > 0, ax, 1.0))), -126) - 7)


def test_prepare_qkv_qknorm_matches_torch_route():
    """Pins the QK-norm composition of prepare_qkv (norm with per-channel weights over the token's
    H*D values, stored in bf16, then RoPE, stored again) against an independent torch route, on
    non-unit weights, heads of different scales and a grid with every axis moving.  The bar is the
    GPU's (within 1 bf16 ulp, >= 99.9% equal: torch's fp64 -> bf16 cast rounds twice).  Each
    plausible mistake -- RoPE before the norm, the weight applied after the rotation, a per-head
    statistic, or one rounding of the whole composition -- is shown to fail that bar."""
    grid, sp = (3, 4, 5), (16, 24, 24)
    B, H, D = 2, 3, 64
    S = grid[0] * grid[1] * grid[2]
    x = RNG.standard_normal((B, S, H, D)) * np.array([0.5, 2.0, 7.0])[None, None, :, None]
    x = oracle.round_bf16(x)                                         # stored bf16 inputs
    w = 1.0 + 0.5 * RNG.standard_normal(H * D)
    joint = oracle.round_bf16(RNG.standard_normal((B, 7, H, D)))
    eps = 1e-6
    q, _, _ = oracle.prepare_qkv([x, joint], [x, joint], [x, joint], grid, sp, THETA, "bf16",
                                 norm_q=[w, None], eps=eps)
    got = q[:, :, :S].transpose(0, 2, 1, 3)

    def meets_bar(want):
        d = np.abs(got - want)
        return bool((d <= _bf16_ulp(want)).all() and (d == 0).mean() >= 0.999)

    assert meets_bar(_torch_route_qknorm_rope(x, w, eps, grid, sp, THETA))
    for wrong in (dict(order="rope_first"), dict(weight_after=True), dict(per_head=True),
                  dict(round_between=False)):
        assert not meets_bar(_torch_route_qknorm_rope(x, w, eps, grid, sp, THETA, **wrong)), wrong
    # the joint segment without weights is a bit-exact copy
    np.testing.assert_array_equal(q[:, :, S:], joint.transpose(0, 2, 1, 3))


def test_prepare_qkv_qknorm_joint_segment_single_rounding():
    """A weighted joint segment (not rotated) is the norm's stored output: torch's rms_norm of the
    token's H*D values, cast to bf16 once."""
    grid, sp = (1, 2, 3), (0, 32, 32)
    B, H, D = 1, 4, 64
    vid = oracle.round_bf16(RNG.standard_normal((B, 6, H, D)))
    txt = oracle.round_bf16(RNG.standard_normal((B, 9, H, D)) * 3.0)
    w = 1.0 + 0.3 * RNG.standard_normal(H * D)
    q, _, _ = oracle.prepare_qkv([vid, txt], [vid, txt], [vid, txt], grid, sp, THETA, "bf16",
                                 norm_q=[None, w], eps=1e-6)
    want = torch.nn.functional.rms_norm(torch.from_numpy(txt).reshape(B, 9, H * D), (H * D,),
                                        weight=torch.from_numpy(w), eps=1e-6)
    want = want.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy().reshape(B, 9, H, D)
    got = q[:, :, 6:].transpose(0, 2, 1, 3)
    d = np.abs(got - want)
    assert (d <= _bf16_ulp(want)).all() and (d == 0).mean() >= 0.999

"""GPU parity on tensors of more than 2^31 elements (4.3-9 GB each): the 64-bit element
offsets of every entry point, through the C ABI, against the fp64 oracle on sampled rows.

Each case puts sampled rows on both sides of the point where a flat element offset
crosses 2^31 (for the query/output rows, the key/value rows, the permute's source and
destination, the merge's partials), plus the first and last rows and seeded random ones.
Inputs are drawn N(0, 1) on the GPU from a seeded generator; only the sampled rows (and
the heads of K and V they attend) are copied to the host for the oracle.  Each output row
depends on its own query row and its head's keys only, so a sampled row is exact, not an
approximation.  Bars as in test_gpu_parity.
"""
import math
import sys

import numpy as np
import pytest
import torch

import long_sequence_attention_rope3d_amd as r3d
import oracle
from workloads.inputs import to_f64

pytestmark = pytest.mark.gpu

BF16_MAX_ABS, BF16_MEAN_ABS, LSE_ABS = 2e-2, 2e-3, 1e-3
I31 = 2 ** 31


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _randn(shape, seed, dev, dtype=torch.bfloat16):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=dev, dtype=dtype)


def _rows_around(n_rows: int, per_row: int, extra, rng, n_random: int = 12):
    """Flat row ids: both sides of the row holding element 2^31 (per_row elements per
    row), the first and last rows, `extra`, and n_random seeded random rows."""
    cross = I31 // per_row
    rows = {0, 1, n_rows - 1, n_rows - 2, cross - 1, cross, cross + 1, *extra}
    rows |= set(int(x) for x in rng.integers(0, n_rows, n_random))
    return np.array(sorted(r for r in rows if 0 <= r < n_rows), dtype=np.int64)


def _check_rows(got_out, got_lse, ref_out, ref_lse, what):
    d = np.abs(got_out - ref_out)
    dl = np.abs(got_lse - ref_lse)
    say(f"[{what}] {got_out.shape[0]} rows: max-abs {d.max():.3e} mean-abs {d.mean():.3e} "
        f"lse max-abs {dl.max():.3e}")
    assert np.isfinite(got_out).all(), what
    assert d.max() <= BF16_MAX_ABS, what
    assert d.mean() <= BF16_MEAN_ABS, what
    assert dl.max() <= LSE_ABS, what


def _oracle_rows(q, k, v, rows, Sq, scale):
    """The oracle on flat rows (b*H + h)*Sq + i of q [B,H,Sq,D] (device), head by head:
    only the sampled query rows and the K/V of their heads go to the host."""
    B, H, _, D = q.shape
    out = np.empty((rows.size, D))
    lse = np.empty(rows.size)
    qf = q.reshape(-1, D)
    for bh in np.unique(rows // Sq):
        sel = np.nonzero(rows // Sq == bh)[0]
        b, h = divmod(int(bh), H)
        qh = to_f64(qf[torch.from_numpy(rows[sel]).to(q.device)].cpu()).reshape(1, 1, sel.size, D)
        kh = to_f64(k[b, h].cpu()).reshape(1, 1, -1, D)
        vh = to_f64(v[b, h].cpu()).reshape(1, 1, -1, D)
        o, l = oracle.attention(qh, kh, vh, scale)
        out[sel] = o.reshape(sel.size, D)
        lse[sel] = l.reshape(sel.size)
        del kh, vh
    return out, lse


def _gather(out, lse, rows, D):
    idx = torch.from_numpy(rows).to(out.device)
    return to_f64(out.reshape(-1, D)[idx].cpu()), lse.reshape(-1)[idx].double().cpu().numpy()


def test_attn_query_rows_past_2g_elements(gpu):
    """Q and out of 2.28e9 elements (17 heads x 1049000 rows x 128): query and output rows
    past element 2^31, 2732 query tiles per head, a ragged last tile; 300 keys (a ragged
    key tile), one chunk."""
    B, H, Sq, Skv, D = 1, 17, 1_049_000, 300, 128
    assert B * H * Sq * D > I31
    scale = 1.0 / math.sqrt(D)
    say(f"large Q: B={B} H={H} Sq={Sq} Skv={Skv} D={D}")
    q = _randn((B, H, Sq, D), 31, gpu)
    k = _randn((B, H, Skv, D), 32, gpu)
    v = _randn((B, H, Skv, D), 33, gpu)
    out, lse = r3d.attn_fwd(q, k, v, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    rows = _rows_around(B * H * Sq, D, [(H - 1) * Sq, (H - 1) * Sq + 383, (H - 1) * Sq + 384], rng)
    got_out, got_lse = _gather(out, lse, rows, D)
    ref_out, ref_lse = _oracle_rows(q, k, v, rows, Sq, scale)
    _check_rows(got_out, got_lse, ref_out, ref_lse, "Q/out past 2^31 elements")
    del q, k, v, out, lse
    torch.cuda.empty_cache()


def test_attn_key_rows_past_2g_elements(gpu):
    """K and V of 2.18e9 elements (17 heads x 1000003 keys x 128): the last heads' key
    tiles lie past element 2^31; 400 query rows per head (a 384-row tile and a 16-row one,
    so the planner splits the keys of this small grid into ranges merged afterwards);
    kv_chunk 131072 (8 chunks, the last ragged)."""
    B, H, Sq, Skv, D = 1, 17, 400, 1_000_003, 128
    assert B * H * Skv * D > I31
    scale = 1.0 / math.sqrt(D)
    say(f"large K/V: B={B} H={H} Sq={Sq} Skv={Skv} D={D} kv_chunk=131072")
    q = _randn((B, H, Sq, D), 41, gpu)
    k = _randn((B, H, Skv, D), 42, gpu)
    v = _randn((B, H, Skv, D), 43, gpu)
    out, lse = r3d.attn_fwd(q, k, v, scale=scale, kv_chunk=131072)
    torch.cuda.synchronize()
    # Heads 0 (offsets below 2^31), 16 (wholly past it) and 15 (K rows crossing it:
    # element 2^31 is key 2^31/128 - 15*Skv of head 15).
    rows = np.array([h * Sq + i for h in (0, 15, 16) for i in (0, 1, 200, 383, 384, 399)], dtype=np.int64)
    got_out, got_lse = _gather(out, lse, rows, D)
    ref_out, ref_lse = _oracle_rows(q, k, v, rows, Sq, scale)
    _check_rows(got_out, got_lse, ref_out, ref_lse, "K/V past 2^31 elements")
    del q, k, v, out, lse
    torch.cuda.empty_cache()


def test_permute_rope_past_2g_elements(gpu):
    """joint_concat_permute with RoPE of 2.18e9 elements (video grid 61x128x128 = 999424
    tokens, 256 audio and 512 text tokens, 17 heads x 128): source and destination
    offsets past 2^31.  Joint tokens must be bit-exact copies; video tokens the oracle's
    rotation rounded to bf16 within 1 ulp and equal on >= 99.9% of the sampled values."""
    grid, split, theta = (61, 128, 128), (32, 48, 48), 10000.0
    H, D = 17, 128
    Nv = grid[0] * grid[1] * grid[2]
    lens = (Nv, 256, 512)
    S = sum(lens)
    assert H * S * D > I31
    say(f"large permute: grid={grid} lens={lens} H={H} D={D}")
    segs = [_randn((1, n, H, D), 51 + i, gpu) for i, n in enumerate(lens)]
    out = r3d.joint_concat_permute(segs, r3d.Rope3D(grid, split, theta))
    torch.cuda.synchronize()
    # (h, s) pairs: the destination element 2^31 is at h*S + s = 2^24; the source element
    # 2^31 at video token s with s*H + h = 2^24.
    dst_cross = I31 // D
    src_cross = I31 // D // H
    pairs = {(dst_cross // S, dst_cross % S + d) for d in (-1, 0, 1)}
    pairs |= {(h, src_cross + d) for h in (0, H - 1) for d in (-1, 0, 1)}
    pairs |= {(0, 0), (H - 1, Nv - 1), (H - 1, Nv), (H - 1, S - 1), (3, Nv + 255), (3, Nv + 256)}
    rng = np.random.default_rng(51)
    pairs |= {(int(h), int(s)) for h, s in zip(rng.integers(0, H, 24), rng.integers(0, S, 24))}
    offs = np.cumsum((0,) + lens)
    ref, got = [], []
    for h, s in sorted(pairs):
        got.append(to_f64(out[0, h, s].cpu()))
        seg = int(np.searchsorted(offs, s, side="right")) - 1
        x = to_f64(segs[seg][0, s - offs[seg], h].cpu())
        if seg == 0:
            t, rem = divmod(s, grid[1] * grid[2])
            hh, w = divmod(rem, grid[2])
            ref.append(oracle.round_bf16(oracle.rope_vec(x, (t, hh, w), split, theta)))
        else:
            ref.append(x)
    got, ref = np.array(got), np.array(ref)
    d = np.abs(got - ref)
    ax = np.abs(ref)
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.where(ax > 0, ax, 1.0))), -126) - 7)
    joint = np.array([s >= Nv for _, s in sorted(pairs)])
    say(f"[permute past 2^31] {len(pairs)} (head, token) rows: exact fraction {(d == 0).mean():.6f}, "
        f"max ulps {(d / ulp).max():.2f}")
    assert (d[joint] == 0).all()
    assert (d <= ulp).all()
    assert (d == 0).mean() >= 0.999
    del segs, out
    torch.cuda.empty_cache()


def test_lse_merge_past_2g_elements(gpu):
    """lse_merge of two fp32 partials [2, 1, 17, 500000, 128] (2.18e9 elements, 8.7 GB):
    the second partial's rows lie past element 2^31; bf16 output.  Sampled rows against the
    oracle's merge of the same rows, within one bf16 ulp of its value (+1e-5)."""
    n, B, H, S, D = 2, 1, 17, 500_000, 128
    assert n * B * H * S * D > I31
    say(f"large lse_merge: n={n} B={B} H={H} S={S} D={D}")
    parts = _randn((n, B, H, S, D), 61, gpu, torch.float32)
    lse_parts = 3.0 * _randn((n, B, H, S), 62, gpu, torch.float32)
    out, lse = r3d.lse_merge(parts, lse_parts, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(61)
    rows = _rows_around(B * H * S, D, [], rng)
    rows = np.unique(np.concatenate([rows, (I31 // D - B * H * S) + np.arange(-1, 2)]))
    idx = torch.from_numpy(rows).to(gpu)
    p = to_f64(parts.reshape(n, -1, D)[:, idx].cpu())
    lp = lse_parts.reshape(n, -1)[:, idx].double().cpu().numpy()
    ref_out, ref_lse = oracle.lse_merge(p, lp)
    got_out, got_lse = _gather(out, lse, rows, D)
    ref_r = oracle.round_bf16(ref_out)
    ax = np.abs(ref_r)
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.where(ax > 0, ax, 1.0))), -126) - 7)
    d = np.abs(got_out - ref_out)
    dl = np.abs(got_lse - ref_lse)
    say(f"[lse_merge past 2^31] {rows.size} rows: max-abs {d.max():.3e}, max ulps "
        f"{(d / ulp).max():.2f}, lse max-abs {dl.max():.3e}")
    assert (d <= ulp + 1e-5).all()
    assert (dl <= 1e-5 * np.maximum(1.0, np.abs(ref_lse))).all()
    del parts, lse_parts, out, lse
    torch.cuda.empty_cache()


def test_rope3d_apply_in_place_past_2g_elements(gpu):
    """rope3d_apply in place on [1, 999424, 17, 128] bf16 video tokens (2.18e9 elements, grid
    61x128x128): sampled (token, head) rows on both sides of element 2^31 and at the ends equal
    the oracle's rotation of the saved input rows, rounded to bf16 (within 1 ulp, >= 99.9% equal)."""
    grid, split, theta = (61, 128, 128), (32, 48, 48), 10000.0
    H, D = 17, 128
    Nv = grid[0] * grid[1] * grid[2]
    assert Nv * H * D > I31
    say(f"large rope3d_apply in place: grid={grid} H={H} D={D}")
    x = _randn((1, Nv, H, D), 71, gpu)
    cross = I31 // D                       # flat (token, head) row holding element 2^31
    pairs = {divmod(cross + d, H) for d in (-1, 0, 1)}
    pairs |= {(0, 0), (Nv - 1, H - 1), (Nv // 2, 3)}
    rng = np.random.default_rng(71)
    pairs |= {(int(s), int(h)) for s, h in zip(rng.integers(0, Nv, 24), rng.integers(0, H, 24))}
    pairs = sorted(pairs)
    saved = [to_f64(x[0, s, h].cpu()) for s, h in pairs]
    y = r3d.rope3d_apply(x, grid, split, theta, out=x)
    torch.cuda.synchronize()
    assert y.data_ptr() == x.data_ptr()
    got = np.array([to_f64(x[0, s, h].cpu()) for s, h in pairs])
    ref = []
    for (s, h), v in zip(pairs, saved):
        t, rem = divmod(s, grid[1] * grid[2])
        hh, w = divmod(rem, grid[2])
        ref.append(oracle.round_bf16(oracle.rope_vec(v, (t, hh, w), split, theta)))
    ref = np.array(ref)
    d = np.abs(got - ref)
    ax = np.abs(ref)
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.where(ax > 0, ax, 1.0))), -126) - 7)
    say(f"[rope3d_apply past 2^31] {len(pairs)} rows: exact fraction {(d == 0).mean():.6f}, "
        f"max ulps {(d / ulp).max():.2f}")
    assert (d <= ulp).all() and (d == 0).mean() >= 0.999
    del x
    torch.cuda.empty_cache()


def test_permute_qknorm_rope_past_2g_elements(gpu):
    """joint_concat_permute with the RMS QK-norm (weights on the video and text segments) and
    RoPE, 2.18e9 elements (the 61x128x128 video grid + 256 audio + 512 text tokens, 17 heads x
    128): sampled tokens on both sides of each 2^31 crossing against the oracle's norm over the
    token's H*D values (stored in bf16), then its rotation (stored in bf16); within 1 ulp and
    >= 99.9% equal; the audio segment (no weights) bit-exact."""
    grid, split, theta, eps = (61, 128, 128), (32, 48, 48), 10000.0, 1e-6
    H, D = 17, 128
    Nv = grid[0] * grid[1] * grid[2]
    lens = (Nv, 256, 512)
    S = sum(lens)
    assert H * S * D > I31
    say(f"large permute + QK-norm + RoPE: grid={grid} lens={lens} H={H} D={D}")
    segs = [_randn((1, n, H, D), 81 + i, gpu) for i, n in enumerate(lens)]
    g = torch.Generator().manual_seed(81)
    wts = [1.0 + 0.3 * torch.randn(H * D, generator=g), None, 0.5 + torch.rand(H * D, generator=g)]
    out = r3d.joint_concat_permute(segs, r3d.Rope3D(grid, split, theta),
                                   norm=[w.to(gpu) if w is not None else None for w in wts], eps=eps)
    torch.cuda.synchronize()
    dst_cross = I31 // D                    # h*S + s of destination element 2^31
    src_cross = I31 // D // H               # video token holding source element 2^31
    toks = {dst_cross % S + d for d in (-1, 0, 1)} | {src_cross + d for d in (-1, 0, 1)}
    toks |= {0, Nv - 1, Nv, Nv + 255, Nv + 256, S - 1}
    rng = np.random.default_rng(81)
    toks |= {int(s) for s in rng.integers(0, S, 12)}
    offs = np.cumsum((0,) + lens)
    got, ref, exact_seg = [], [], []
    for s in sorted(toks):
        seg = int(np.searchsorted(offs, s, side="right")) - 1
        x = to_f64(segs[seg][0, s - offs[seg]].cpu())          # [H, D]: the whole token
        y = x
        if wts[seg] is not None:
            y = oracle.round_bf16(oracle.rms_norm(x.reshape(1, H * D), wts[seg].double().numpy(), eps)).reshape(H, D)
        if seg == 0:
            t, rem = divmod(s, grid[1] * grid[2])
            hh, w = divmod(rem, grid[2])
            y = np.stack([oracle.round_bf16(oracle.rope_vec(y[h], (t, hh, w), split, theta)) for h in range(H)])
        got.append(to_f64(out[0, :, s].cpu()))
        ref.append(y)
        exact_seg.append(wts[seg] is None and seg != 0)
    got, ref = np.array(got), np.array(ref)
    d = np.abs(got - ref)
    ax = np.abs(ref)
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.where(ax > 0, ax, 1.0))), -126) - 7)
    say(f"[QK-norm past 2^31] {len(toks)} tokens x {H} heads: exact fraction {(d == 0).mean():.6f}, "
        f"max ulps {(d / ulp).max():.2f}")
    assert (d[np.array(exact_seg)] == 0).all()
    assert (d <= ulp).all() and (d == 0).mean() >= 0.999
    del segs, out
    torch.cuda.empty_cache()

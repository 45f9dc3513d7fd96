"""The entry points under HIP graph capture: the library allocates nothing and issues no
memset, so a call with caller-owned buffers records into a graph.  Each test captures the
calls once, replays the graph several times with eager work between the replays, and checks
every replay against the eager result, bit for bit."""
import math

import pytest
import torch

import long_sequence_attention_rope3d_amd as r3d

pytestmark = pytest.mark.gpu


def _rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


def _replay_and_check(graph, outputs, want, perturb):
    for r in range(3):
        for o in outputs:
            o.fill_(float("nan"))              # eager work between replays, and no stale result
        torch.cuda.synchronize()
        perturb()
        graph.replay()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert torch.equal(o, w), f"replay {r}"


@pytest.mark.parametrize("shape,layout", [
    ((1, 24, 4352, 4352, 128, 0), "bhsd"),   # 256 whole 12-wave tiles + 32 split 7 ways: pre-pass, attention, merge
    ((1, 24, 4352, 4352, 128, 0), "bshd"),   # the same with token-major output (the merge writes token-major rows)
    ((1, 4, 300, 9000, 128, 0), "bhsd"),     # few tiles: 8-wave blocks, every tile split
    ((1, 2, 700, 1300, 64, 1024), "bhsd"),   # D = 64, two chunks
])
def test_attn_fwd_graph_replay(gpu, shape, layout):
    B, H, Sq, Skv, D, kv_chunk = shape
    q, k, v = (_rand((B, H, S, D), torch.bfloat16, 40 + i).to(gpu) for i, S in enumerate((Sq, Skv, Skv)))
    scale = 1.0 / math.sqrt(D)
    ws = torch.empty(max(1, r3d.attn_fwd_workspace_size(B, H, Sq, Skv, D, kv_chunk, torch.bfloat16)),
                     dtype=torch.uint8, device=gpu)
    oshape = (B, H, Sq, D) if layout == "bhsd" else (B, Sq, H, D)
    out = torch.empty(oshape, dtype=torch.bfloat16, device=gpu)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=gpu)
    call = lambda o, l: r3d.attn_fwd(q, k, v, scale=scale, kv_chunk=kv_chunk, out=o, lse=l,  # noqa: E731
                                     workspace=ws, out_layout=layout)
    want_out, want_lse = call(None, None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out, lse)  # warm-up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, lse)
    # between replays, an eager call of its own overwrites the workspace
    other_out = torch.empty(oshape, dtype=torch.bfloat16, device=gpu)
    _replay_and_check(g, [out, lse], [want_out, want_lse], lambda: call(other_out, None))


def test_permute_and_merge_graph_replay(gpu):
    B, H, D = 1, 6, 128
    grid, split = (3, 6, 7), (32, 48, 48)
    lens = (126, 19, 5)
    segs = [_rand((B, n, H, D), torch.bfloat16, 60 + i).to(gpu) for i, n in enumerate(lens)]
    wts = [(1.0 + 0.1 * _rand((H * D,), torch.float32, 70 + i)).to(gpu) for i in range(3)]
    parts = _rand((5, B, H, 150, D), torch.float32, 80).to(gpu)
    lp = (3.0 * _rand((5, B, H, 150), torch.float32, 81)).to(gpu)
    rope = r3d.Rope3D(grid, split)
    want_p = r3d.joint_concat_permute(segs, rope, norm=wts, eps=1e-6)
    want_m, want_l = r3d.lse_merge(parts, lp, out_dtype=torch.bfloat16)
    out_p = torch.empty_like(want_p)
    out_m, out_l = torch.empty_like(want_m), torch.empty_like(want_l)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r3d.joint_concat_permute(segs, rope, norm=wts, eps=1e-6, out=out_p)
        r3d.lse_merge(parts, lp, out=out_m, lse_out=out_l)
    _replay_and_check(g, [out_p, out_m, out_l], [want_p, want_m, want_l], lambda: None)


def test_attn_constmax_graph_replay(gpu):
    """The constant-max call records three kernels (pre-pass, constant-max pass, recompute
    of flagged tiles); the flags live in the workspace.  One key of heads 0 and 2 is scaled
    x64, so their bound overshoots most rows' maxima past fp32's range and those tiles are
    recomputed, while heads 1 and 3 are not.  Between replays an eager call on inputs
    without the outlier rewrites the workspace's statistics and flags."""
    B, H, Sq, Skv, D = 1, 4, 900, 1500, 128
    q, k, v = (_rand((B, H, S, D), torch.bfloat16, 90 + i).to(gpu) for i, S in enumerate((Sq, Skv, Skv)))
    k_plain = k.clone()
    k[:, 0::2, 7, :] *= 64
    scale = 1.0 / math.sqrt(D)
    ws = torch.empty(r3d.attn_fwd_constmax_workspace_size(B, H, Sq, Skv, D, torch.bfloat16),
                     dtype=torch.uint8, device=gpu)
    want_out, want_lse = r3d.attn_fwd_constmax(q, k, v, scale=scale, workspace=ws)
    ref_out, ref_lse = r3d.attn_fwd(q, k, v, scale=scale)
    torch.cuda.synchronize()
    # the recompute made the flagged tiles equal to the online kernel's result
    assert torch.isfinite(want_out.float()).all() and torch.isfinite(want_lse).all()
    assert (want_out.float() - ref_out.float()).abs().max().item() <= 2e-2
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=gpu)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        r3d.attn_fwd_constmax(q, k, v, scale=scale, out=out, lse=lse, workspace=ws)  # warm-up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r3d.attn_fwd_constmax(q, k, v, scale=scale, out=out, lse=lse, workspace=ws)
    other_out = torch.empty_like(q)
    _replay_and_check(g, [out, lse], [want_out, want_lse],
                      lambda: r3d.attn_fwd_constmax(q, k_plain, v, scale=scale, out=other_out, workspace=ws))

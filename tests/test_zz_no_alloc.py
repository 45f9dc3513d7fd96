"""r3d_attn_fwd_noalloc (the allocation-free form of r3d_attn_fwd, for callers that cannot
allocate) against r3d_attn_fwd, through the C ABI, on two calls in a row -- the second with a
smaller input -- so the second reuses the fixed per-GPU scratch the first one filled."""
import math
import sys

import numpy as np
import pytest
import torch

import long_sequence_attention_rope3d_amd as r3d

pytestmark = pytest.mark.gpu


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16)


def _case(gpu, B, H, Sq, Skv, D, kv_chunk, seed):
    q, k, v = (_rand((B, H, S, D), seed + i).to(gpu) for i, S in enumerate((Sq, Skv, Skv)))
    scale = 1.0 / math.sqrt(D)
    ref, ref_lse = r3d.attn_fwd(q, k, v, scale=scale, kv_chunk=kv_chunk)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=gpu)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(gpu)
    r3d.attn_fwd_noalloc(q, k, v, scale=scale, kv_chunk=kv_chunk, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated(gpu) == before        # nothing allocated through torch
    d = (out.float() - ref.float()).abs()
    dl = (lse - ref_lse).abs().max().item()
    print(f"noalloc B={B} H={H} Sq={Sq} Skv={Skv} chunk={kv_chunk}: max-abs {d.max().item():.3e} "
          f"mean-abs {d.mean().item():.3e} lse {dl:.3e} equal {torch.equal(out, ref)}", file=sys.stderr, flush=True)
    assert torch.isfinite(out.float()).all()
    assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3 and dl <= 1e-3
    return out, ref


def test_noalloc_matches_attn_fwd_two_calls(gpu):
    # 1st: 24 heads x 4352 rows: r3d_attn_fwd key-splits this grid, and the split's partials do
    # not fit the scratch, so the no-alloc call runs it unsplit (equal up to rounding).
    _case(gpu, 1, 24, 4352, 4352, 128, 0, 301)
    # 2nd, smaller: the same key split as r3d_attn_fwd (its partials fit): bit for bit equal.
    out, ref = _case(gpu, 1, 2, 300, 9000, 128, 0, 311)
    assert torch.equal(out, ref)

"""Seeded host inputs for a workload.

Recipe (stated once, used by both the HIP path and the oracle):
  * torch CPU generator seeded with 20261202 + workload index;
  * draw Q, then K, then V as fp32 N(0, 1), each segment by segment
    (video, then the joint segments in order) in [B, S_i, H, D] layout;
  * Q and K draws are multiplied by ``qk_mult`` (sqrt(3) for the image
    workload, giving scaled logits of std ~3);
  * cast to the storage dtype with round-to-nearest-even (fp32 stays fp32);
  * outlier keys: floor(outlier_frac * S) token indices of the joint
    sequence, drawn without replacement from the same generator, have K
    multiplied by ``outlier_mult`` for every head, after the cast (x8 is exact
    in bf16);
Nothing here computes any part of the method.
"""
from __future__ import annotations

import hashlib
from typing import Dict, List

import numpy as np
import torch

from .configs import Workload


def _storage_dtype(w: Workload):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def make_inputs(w: Workload) -> Dict[str, List[torch.Tensor]]:
    """Returns {"q": [seg...], "k": [...], "v": [...]} of CPU tensors [B,S_i,H,D]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    dt = _storage_dtype(w)
    out = {}
    for name in ("q", "k", "v"):
        segs = []
        for n in w.seg_lens:
            x = torch.randn((w.B, n, w.H, w.D), generator=g, dtype=torch.float32)
            if name in ("q", "k") and w.qk_mult != 1.0:
                x.mul_(w.qk_mult)
            segs.append(x.to(dt).contiguous())
            del x
        out[name] = segs
    if w.outlier_frac > 0.0:
        n_out = int(w.outlier_frac * w.S)
        idx = torch.randperm(w.S, generator=g)[:n_out]
        offs = np.cumsum((0,) + w.seg_lens)
        for i, seg in enumerate(out["k"]):
            sel = idx[(idx >= int(offs[i])) & (idx < int(offs[i + 1]))] - int(offs[i])
            if sel.numel():
                seg[:, sel] = seg[:, sel] * w.outlier_mult
        out["outlier_tokens"] = [idx.sort().values]
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a stored bf16/fp32 tensor."""
    return t.to(torch.float64).numpy()


def digest(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()[:16]


def sample_rows(w: Workload, n_random: int = 16, seed_offset: int = 0, heads=None) -> np.ndarray:
    """Query rows for row-sampled parity at full size, as flat (b*H + h)*S + i.

    Per head: the first and last video token, the first, middle and last
    token of each joint segment, the rows on both sides of every kv_chunk
    boundary (kv_chunk 0: every 1024th row), the last row, and ``n_random``
    seeded random rows."""
    rng = np.random.default_rng(w.seed + 1000 + seed_offset)
    S = w.S
    base = {0, w.Nv - 1, S - 1}
    offs = np.cumsum((0,) + w.seg_lens)
    for i in range(1, len(w.seg_lens)):
        lo, hi = int(offs[i]), int(offs[i + 1])
        if hi > lo:
            base.update({lo, (lo + hi) // 2, hi - 1})
    step = w.kv_chunk if 0 < w.kv_chunk < S else 1024
    for b in range(step, S, step):
        base.update({b - 1, b})
    rows = []
    heads = range(w.H) if heads is None else heads
    for b in range(w.B):
        for h in heads:
            picks = set(base)
            picks.update(rng.integers(0, S, size=n_random).tolist())
            rows.extend(((b * w.H + h) * S + np.array(sorted(picks), dtype=np.int64)).tolist())
    return np.array(rows, dtype=np.int64)

"""The five synthetic workloads, shaped like the pages' video / image DiTs.

Video grids follow the latent-size rule printed in "Context Parallelism in
vLLM Omni Neuron", §Sequence Length Constraints / §Problem:
  latent_frames = (frames - 1) // 4 + 1
  post_patch_h  = (height // 8) // 2
  post_patch_w  = (width  // 8) // 2
applied to the pages' geometries: Kandinsky 6 Lite 432x256x25 (diffusers
issue "Kandinsky 6: add context-parallel (_cp_plan) support ..."), Kandinsky 6
Pro 864x480x125 (vLLM-Omni recipe "Kandinsky 6 TI2VA"), HunyuanVideo
1280x720x129 and Flux 1024x1024 (xDiT PR "Adds support for KV-cache and joint
tensors to USP method").  Joint (audio/text) token counts, head geometry,
dtype, RoPE split/theta and kv_chunk are those of the benchmark problem
statement.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Tuple


def video_grid(frames: int, height: int, width: int) -> Tuple[int, int, int]:
    """Latent (t, h, w) token grid of a clip, per the rule quoted above."""
    return ((frames - 1) // 4 + 1, (height // 8) // 2, (width // 8) // 2)


@dataclass(frozen=True)
class Workload:
    index: int                      # 1..5; seed = 20261202 + index
    name: str
    B: int
    H: int
    D: int
    grid: Tuple[int, int, int]      # video token grid (t, h, w)
    joint: Tuple[Tuple[str, int], ...]  # joint segments after the video, in order
    dtype: str                      # "f32" or "bf16" (storage and MFMA operand type)
    split: Tuple[int, int, int]     # RoPE dims per axis (d_t, d_h, d_w)
    kv_chunk: int                   # 0 = one chunk
    theta: float = 10000.0
    qk_mult: float = 1.0            # multiplies the fp32 Q and K draws before the cast
    outlier_frac: float = 0.0       # fraction of key tokens scaled by outlier_mult
    outlier_mult: float = 1.0
    note: str = field(default="", compare=False)

    @property
    def seed(self) -> int:
        return 20261202 + self.index

    @property
    def Nv(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def seg_lens(self) -> Tuple[int, ...]:
        return (self.Nv,) + tuple(n for _, n in self.joint)

    @property
    def S(self) -> int:
        return sum(self.seg_lens)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def n_chunks(self) -> int:
        c = self.kv_chunk if 0 < self.kv_chunk < self.S else self.S
        return -(-self.S // c)

    @property
    def attn_flops(self) -> int:
        """Algorithmic QK^T + PV flops, 4*B*H*Sq*Skv*D."""
        return 4 * self.B * self.H * self.S * self.S * self.D

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = (
    Workload(1, "tiny", 1, 2, 64, (2, 8, 15), (("text", 16),), "f32", (16, 24, 24), 64,
             note="fp32 oracle check"),
    Workload(2, "lite-clip", 1, 16, 128, video_grid(25, 256, 432), (("audio", 64), ("text", 128)),
             "bf16", (32, 48, 48), 512, note="Kandinsky 6 Lite 432x256, 25 frames"),
    Workload(3, "image-dit", 1, 24, 128, video_grid(1, 1024, 1024), (("text", 256),), "bf16",
             (0, 64, 64), 0, qk_mult=math.sqrt(3.0),
             note="Flux-like 1024x1024 image + 256 text tokens, 2-D RoPE, logit std ~3"),
    Workload(4, "pro-clip", 1, 24, 128, video_grid(125, 480, 864), (("audio", 256), ("text", 512)),
             "bf16", (32, 48, 48), 4096, note="Kandinsky 6 Pro 864x480, 125 frames"),
    Workload(5, "long-video", 1, 24, 128, video_grid(129, 720, 1280), (("text", 256),), "bf16",
             (32, 48, 48), 8192, outlier_frac=0.01, outlier_mult=8.0,
             note="HunyuanVideo-like 1280x720, 129 frames, 1% outlier keys at 8x"),
)


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name or str(w.index) == str(name) or f"C{w.index}" == name:
            return w
    raise KeyError(name)

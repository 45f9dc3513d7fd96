"""Joint-sequence attention with 3-D RoPE on one AMD MI355X (gfx950).

Thin ctypes binding over ``lib/librope3d_attn.so`` (C ABI in
``include/r3d_attn.h``).  This module only marshals arguments: it takes
torch tensors that already live on the GPU, passes their device pointers,
sizes and torch's current HIP stream to the library, and maps error codes to
exceptions.  Every step of the computation runs in the library's HIP
kernels; there is no fallback.  If the library is missing, importing this
package raises ImportError (build it with ``python
long_sequence_attention_rope3d_amd/build.py``).

Calls (same names as the C entry points without the ``r3d_`` prefix):
  rope3d_apply(x, grid, split, theta=10000.0, out=None)
  joint_concat_permute(segs, rope=None, out=None, norm=None, eps=1e-6)
  attn_fwd(q, k, v, scale=None, kv_chunk=0, out=None, lse=None, return_lse=True,
           out_layout="bhsd", workspace=None)
  attn_fwd_workspace_size(B, H, Sq, Skv, D, kv_chunk, dtype)
  attn_fwd_plan(B, H, Sq, Skv, D, kv_chunk, n_cus)
  attn_fwd_constmax(q, k, v, scale=None, out=None, lse=None, workspace=None)
  attn_fwd_constmax_workspace_size(B, H, Sq, Skv, D, dtype)
  lse_merge(o_parts, lse_parts, out_dtype=None, out=None, lse_out=None)
The attention calls take the device scratch the library needs as a
caller-owned ``workspace`` (a uint8 device tensor of at least the queried
size); when none is given the binding allocates one with torch (its caching
allocator, in the call's stream order).
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import torch

__all__ = ["rope3d_apply", "joint_concat_permute", "attn_fwd", "attn_fwd_workspace_size", "attn_fwd_plan",
           "attn_fwd_noalloc",
           "attn_fwd_constmax",
           "attn_fwd_constmax_workspace_size", "lse_merge", "joint_attention", "Rope3D", "library_path", "R3D_OK",
           "R3D_EINVAL", "R3D_EUNSUPPORTED", "R3D_EHIP"]

_PKG = os.path.dirname(os.path.abspath(__file__))
# R3D_LIBRARY names another build of the same library (the host-sanitizer
# build of tests/sanitize.py); by default the in-tree one.
_LIB_PATH = os.environ.get("R3D_LIBRARY") or os.path.join(_PKG, "lib", "librope3d_attn.so")

R3D_OK, R3D_EINVAL, R3D_EUNSUPPORTED, R3D_EHIP = 0, -1, -2, -3
_F32, _BF16 = 0, 1


def library_path() -> str:
    return _LIB_PATH


class _RopeDesc(ctypes.Structure):
    _fields_ = [("grid_t", ctypes.c_int64), ("grid_h", ctypes.c_int64), ("grid_w", ctypes.c_int64),
                ("d_t", ctypes.c_int32), ("d_h", ctypes.c_int32), ("d_w", ctypes.c_int32),
                ("theta", ctypes.c_double)]


class _AttnPlan(ctypes.Structure):
    _fields_ = [("waves", ctypes.c_int32), ("n_split", ctypes.c_int32), ("n_tiles", ctypes.c_int64),
                ("n_bulk", ctypes.c_int64), ("split_len", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python long_sequence_attention_rope3d_amd/build.py` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.r3d_rope3d_apply.argtypes = [P, P, I32, I64, I64, I64, I64, ctypes.POINTER(_RopeDesc), P]
    lib.r3d_joint_concat_permute.argtypes = [P, P, I32, P, I32, I64, I64, I64,
                                             ctypes.POINTER(_RopeDesc), P]
    lib.r3d_joint_concat_permute_qknorm.argtypes = [P, P, I32, P, ctypes.c_double, P, I32, I64, I64, I64,
                                                    ctypes.POINTER(_RopeDesc), P]
    SZ = ctypes.c_size_t
    lib.r3d_attn_fwd.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, ctypes.c_float, I64, I32, P, SZ, P]
    lib.r3d_attn_fwd_bshd.argtypes = lib.r3d_attn_fwd.argtypes
    lib.r3d_attn_fwd_noalloc.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, ctypes.c_float, I64, I32, P]
    lib.r3d_attn_fwd_workspace_size.argtypes = [I64, I64, I64, I64, I64, I64, I32, ctypes.POINTER(SZ)]
    lib.r3d_attn_fwd_constmax.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, ctypes.c_float, I32, P, SZ, P]
    lib.r3d_attn_fwd_constmax_workspace_size.argtypes = [I64, I64, I64, I64, I64, I32, ctypes.POINTER(SZ)]
    lib.r3d_attn_fwd_plan.argtypes = [I64, I64, I64, I64, I64, I64, I32, ctypes.POINTER(_AttnPlan)]
    lib.r3d_lse_merge.argtypes = [P, P, I32, I32, P, P, I32, I64, I64, I64, I64, P]
    for f in ("r3d_rope3d_apply", "r3d_joint_concat_permute", "r3d_joint_concat_permute_qknorm",
              "r3d_attn_fwd", "r3d_attn_fwd_bshd", "r3d_attn_fwd_noalloc", "r3d_attn_fwd_workspace_size",
              "r3d_attn_fwd_constmax", "r3d_attn_fwd_plan",
              "r3d_attn_fwd_constmax_workspace_size", "r3d_lse_merge"):
        getattr(lib, f).restype = ctypes.c_int
    lib.r3d_last_error.restype = ctypes.c_char_p
    lib.r3d_last_error.argtypes = []
    lib.r3d_version.restype = ctypes.c_char_p
    lib.r3d_version.argtypes = []
    return lib


_lib = _load()


@dataclass(frozen=True)
class Rope3D:
    """Video token grid (t, h, w) and the split of D over the three axes."""
    grid: Tuple[int, int, int]
    split: Tuple[int, int, int]
    theta: float = 10000.0

    def desc(self) -> _RopeDesc:
        return _RopeDesc(int(self.grid[0]), int(self.grid[1]), int(self.grid[2]), int(self.split[0]),
                         int(self.split[1]), int(self.split[2]), float(self.theta))


def _check(status: int, what: str) -> None:
    if status == R3D_OK:
        return
    msg = (_lib.r3d_last_error() or b"").decode(errors="replace")
    if status in (R3D_EINVAL, R3D_EUNSUPPORTED):
        raise ValueError(f"{what}: {msg}")
    raise RuntimeError(f"{what}: {msg} (status {status})")


_DTYPES = {torch.float32: _F32, torch.bfloat16: _BF16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _F32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


# torch's current stream of a device as a raw handle, without building a
# torch.cuda.Stream object per call (~0.2 instead of ~2 us on the host);
# the public route where that query is not available.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor) -> int:
    if _raw_stream is not None:
        return _raw_stream(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


def _one_device(first: torch.Tensor, first_name: str, **others: Optional[torch.Tensor]) -> torch.device:
    """The device of ``first``; every other tensor given must be on it.  The
    library plans and launches on the current device, so each call runs with
    this device made current (_on)."""
    if not isinstance(first, torch.Tensor) or not first.is_cuda:
        raise ValueError(f"{first_name} must be a GPU tensor (got {getattr(first, 'device', type(first))})")
    for name, t in others.items():
        if t is not None and isinstance(t, torch.Tensor) and t.device != first.device:
            raise ValueError(f"{name} is on {t.device}, the call's tensors on {first.device}")
    return first.device


def _on(dev: torch.device):
    """Context making ``dev`` the current device; free when it already is (the usual case)."""
    return contextlib.nullcontext() if dev.index == torch.cuda.current_device() else torch.cuda.device(dev)


def rope3d_apply(x: torch.Tensor, grid, split, theta: float = 10000.0,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rotate video tokens x [B, Nv, H, D] by their (t, h, w) grid position.
    ``out`` may be ``x`` itself (in place)."""
    if x.dim() != 4:
        raise ValueError("x must be [B, Nv, H, D]")
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    B, Nv, H, D = x.shape
    desc = Rope3D(tuple(grid), tuple(split), theta).desc()
    with _on(_one_device(x, "x", out=out)):
        _check(_lib.r3d_rope3d_apply(_dev(x, "x"), _dev(out, "out"), _dtype_code(x), B, Nv, H, D,
                                     ctypes.byref(desc), _stream(x)), "rope3d_apply")
    return out


def joint_concat_permute(segs: Sequence[torch.Tensor], rope: Optional[Rope3D] = None,
                         out: Optional[torch.Tensor] = None,
                         norm: Optional[Sequence[Optional[torch.Tensor]]] = None,
                         eps: float = 1e-6) -> torch.Tensor:
    """segs: [B, S_i, H, D] tensors (video first) -> [B, H, sum S_i, D].
    With ``rope``, segment 0 is rotated while it is copied.  With ``norm`` (one
    entry per segment: None or a float32 [H*D] weight vector on the device),
    each token of a weighted segment is first RMS-normalised over its H*D
    values (QK-norm, r3d_joint_concat_permute_qknorm)."""
    segs = list(segs)
    if not segs:
        raise ValueError("need at least one segment")
    B, _, H, D = segs[0].shape
    dt = segs[0].dtype
    for s in segs:
        if s.dim() != 4 or s.shape[0] != B or s.shape[2] != H or s.shape[3] != D or s.dtype != dt:
            raise ValueError("segments must be [B, S_i, H, D] with equal B, H, D and dtype")
        if s.device != segs[0].device:
            raise ValueError("segments must be on one device")
    S = sum(int(s.shape[1]) for s in segs)
    if out is None:
        out = torch.empty((B, H, S, D), dtype=dt, device=segs[0].device)
    if tuple(out.shape) != (B, H, S, D) or out.dtype != dt:
        raise ValueError("out must be [B, H, S, D] of the segments' dtype")
    dev = _one_device(segs[0], "segment", out=out)
    ptrs = (ctypes.c_void_p * len(segs))(
        *[(_dev(s, "segment") if s.shape[1] > 0 else None) for s in segs])
    lens = (ctypes.c_int64 * len(segs))(*[int(s.shape[1]) for s in segs])
    desc = rope.desc() if rope is not None else None
    rope_arg = ctypes.byref(desc) if desc is not None else None
    if norm is None:
        with _on(dev):
            _check(_lib.r3d_joint_concat_permute(ctypes.cast(ptrs, ctypes.c_void_p),
                                                 ctypes.cast(lens, ctypes.c_void_p), len(segs),
                                                 _dev(out, "out"), _dtype_code(out), B, H, D, rope_arg,
                                                 _stream(out)), "joint_concat_permute")
        return out
    norm = list(norm)
    if len(norm) != len(segs):
        raise ValueError("norm needs one entry (None or a weight vector) per segment")
    for w in norm:
        if w is not None and (w.dtype != torch.float32 or w.numel() != H * D or not w.is_contiguous()):
            raise ValueError("norm weights must be contiguous float32 vectors of H*D values")
        _one_device(segs[0], "segment", norm_weight=w)
    wptrs = (ctypes.c_void_p * len(segs))(*[(_dev(w, "norm weight") if w is not None else None)
                                             for w in norm])
    with _on(dev):
        _check(_lib.r3d_joint_concat_permute_qknorm(ctypes.cast(ptrs, ctypes.c_void_p),
                                                    ctypes.cast(lens, ctypes.c_void_p), len(segs),
                                                    ctypes.cast(wptrs, ctypes.c_void_p), float(eps),
                                                    _dev(out, "out"), _dtype_code(out), B, H, D, rope_arg,
                                                    _stream(out)), "joint_concat_permute_qknorm")
    return out


def _workspace(ws: Optional[torch.Tensor], need: int, device) -> Tuple[Optional[int], int]:
    """(pointer, bytes) of the call's workspace: the caller's tensor, or a new
    uint8 tensor from torch's caching allocator (stream-ordered reuse)."""
    if ws is None:
        if need == 0:
            return None, 0
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def attn_fwd_workspace_size(B: int, H: int, Sq: int, Skv: int, D: int, kv_chunk: int,
                            dtype: torch.dtype) -> int:
    """Bytes of workspace attn_fwd needs on the current device (r3d_attn_fwd_workspace_size)."""
    n = ctypes.c_size_t(0)
    _check(_lib.r3d_attn_fwd_workspace_size(B, H, Sq, Skv, D, kv_chunk, _DTYPES[dtype], ctypes.byref(n)),
           "attn_fwd_workspace_size")
    return int(n.value)


def attn_fwd_constmax_workspace_size(B: int, H: int, Sq: int, Skv: int, D: int, dtype: torch.dtype) -> int:
    """Bytes of workspace attn_fwd_constmax needs (r3d_attn_fwd_constmax_workspace_size)."""
    n = ctypes.c_size_t(0)
    _check(_lib.r3d_attn_fwd_constmax_workspace_size(B, H, Sq, Skv, D, _DTYPES[dtype], ctypes.byref(n)),
           "attn_fwd_constmax_workspace_size")
    return int(n.value)


def attn_fwd_plan(B: int, H: int, Sq: int, Skv: int, D: int, kv_chunk: int, n_cus: int) -> dict:
    """The bf16 launch plan attn_fwd would use on a device with n_cus compute units
    (r3d_attn_fwd_plan): waves per block, query tiles, whole tiles, key ranges per split
    tile, keys per range and the workspace bytes."""
    p = _AttnPlan()
    _check(_lib.r3d_attn_fwd_plan(B, H, Sq, Skv, D, kv_chunk, n_cus, ctypes.byref(p)), "attn_fwd_plan")
    return {f: getattr(p, f) for f, _ in _AttnPlan._fields_}


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
             kv_chunk: int = 0, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             return_lse: bool = True, out_layout: str = "bhsd", workspace: Optional[torch.Tensor] = None):
    """Blockwise non-causal attention. q [B,H,Sq,D], k/v [B,H,Skv,D] ->
    (out, lse [B,H,Sq] fp32 natural log) — or out alone if return_lse is False
    and no lse buffer is given.  out is [B,H,Sq,D] (out_layout="bhsd") or
    token-major [B,Sq,H,D] (out_layout="bshd", r3d_attn_fwd_bshd).
    ``workspace``: device scratch of at least attn_fwd_workspace_size(...)
    bytes (allocated through torch if None)."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    if out_layout not in ("bhsd", "bshd"):
        raise ValueError(f"out_layout must be 'bhsd' or 'bshd', got {out_layout!r}")
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if tuple(k.shape) != (B, H, Skv, D) or tuple(v.shape) != (B, H, Skv, D):
        raise ValueError("k and v must be [B, H, Skv, D] matching q")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    oshape = (B, H, Sq, D) if out_layout == "bhsd" else (B, Sq, H, D)
    if out is None:
        out = torch.empty(oshape, dtype=q.dtype, device=q.device)
    if tuple(out.shape) != oshape or out.dtype != q.dtype:
        raise ValueError(f"out must be {list(oshape)} of q's dtype")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if lse is not None and (tuple(lse.shape) != (B, H, Sq) or lse.dtype != torch.float32):
        raise ValueError("lse must be [B, H, Sq] float32")
    fn = _lib.r3d_attn_fwd if out_layout == "bhsd" else _lib.r3d_attn_fwd_bshd
    with _on(_one_device(q, "q", k=k, v=v, out=out, lse=lse, workspace=workspace)):
        need = attn_fwd_workspace_size(B, H, Sq, Skv, D, int(kv_chunk), q.dtype) if workspace is None else 0
        ws_ptr, ws_bytes = _workspace(workspace, need, q.device)
        _check(fn(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                  _dev(lse, "lse") if lse is not None else None, B, H, Sq, Skv, D,
                  float(scale), int(kv_chunk), _dtype_code(q), ws_ptr, ws_bytes, _stream(q)), "attn_fwd")
    return (out, lse) if lse is not None else out


def attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
                     kv_chunk: int = 0, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     return_lse: bool = True):
    """attn_fwd ([B,H,Sq,D] output) through r3d_attn_fwd_noalloc: the library's fixed
    per-GPU scratch instead of a workspace (no allocation beyond out/lse when the
    caller passes those)."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if tuple(k.shape) != (B, H, Skv, D) or tuple(v.shape) != (B, H, Skv, D):
        raise ValueError("k and v must be [B, H, Skv, D] matching q")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if tuple(out.shape) != (B, H, Sq, D) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if lse is not None and (tuple(lse.shape) != (B, H, Sq) or lse.dtype != torch.float32):
        raise ValueError("lse must be [B, H, Sq] float32")
    with _on(_one_device(q, "q", k=k, v=v, out=out, lse=lse)):
        _check(_lib.r3d_attn_fwd_noalloc(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                                         _dev(lse, "lse") if lse is not None else None, B, H, Sq, Skv, D,
                                         float(scale), int(kv_chunk), _dtype_code(q), _stream(q)),
               "attn_fwd_noalloc")
    return (out, lse) if lse is not None else out


def attn_fwd_constmax(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, return_lse: bool = True):
    """attn_fwd (bf16, [B,H,Sq,D]) with the softmax reference fixed per row at the
    Cauchy-Schwarz bound |scale| |q_i| max_j |k_j| (r3d_attn_fwd_constmax); rows
    the bound leaves underflowed are recomputed with the running max inside the
    call.  ``workspace``: device scratch of at least
    attn_fwd_constmax_workspace_size(...) bytes (allocated through torch if None)."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if tuple(k.shape) != (B, H, Skv, D) or tuple(v.shape) != (B, H, Skv, D):
        raise ValueError("k and v must be [B, H, Skv, D] matching q")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if tuple(out.shape) != (B, H, Sq, D) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if lse is not None and (tuple(lse.shape) != (B, H, Sq) or lse.dtype != torch.float32):
        raise ValueError("lse must be [B, H, Sq] float32")
    with _on(_one_device(q, "q", k=k, v=v, out=out, lse=lse, workspace=workspace)):
        need = attn_fwd_constmax_workspace_size(B, H, Sq, Skv, D, q.dtype) if workspace is None else 0
        ws_ptr, ws_bytes = _workspace(workspace, need, q.device)
        _check(_lib.r3d_attn_fwd_constmax(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                                          _dev(lse, "lse") if lse is not None else None, B, H, Sq, Skv, D,
                                          float(scale), _dtype_code(q), ws_ptr, ws_bytes, _stream(q)),
               "attn_fwd_constmax")
    return (out, lse) if lse is not None else out


def lse_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
              out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
              return_lse: bool = True):
    """o_parts [n,B,H,S,D], lse_parts [n,B,H,S] fp32 -> (out [B,H,S,D], lse [B,H,S])."""
    if o_parts.dim() != 5 or lse_parts.dim() != 4:
        raise ValueError("o_parts must be [n,B,H,S,D] and lse_parts [n,B,H,S]")
    n, B, H, S, D = o_parts.shape
    if tuple(lse_parts.shape) != (n, B, H, S) or lse_parts.dtype != torch.float32:
        raise ValueError("lse_parts must be float32 [n, B, H, S]")
    out_dtype = out_dtype or o_parts.dtype
    if out is None:
        out = torch.empty((B, H, S, D), dtype=out_dtype, device=o_parts.device)
    if tuple(out.shape) != (B, H, S, D):
        raise ValueError("out must be [B, H, S, D]")
    if lse_out is None and return_lse:
        lse_out = torch.empty((B, H, S), dtype=torch.float32, device=o_parts.device)
    if lse_out is not None and (tuple(lse_out.shape) != (B, H, S) or lse_out.dtype != torch.float32):
        raise ValueError("lse_out must be [B, H, S] float32")
    with _on(_one_device(o_parts, "o_parts", lse_parts=lse_parts, out=out, lse_out=lse_out)):
        _check(_lib.r3d_lse_merge(_dev(o_parts, "o_parts"), _dev(lse_parts, "lse_parts"), n,
                                  _dtype_code(o_parts), _dev(out, "out"),
                                  _dev(lse_out, "lse_out") if lse_out is not None else None,
                                  _dtype_code(out), B, H, S, D, _stream(out)), "lse_merge")
    return (out, lse_out) if lse_out is not None else out


def joint_attention(q_segs: Sequence[torch.Tensor], k_segs: Sequence[torch.Tensor],
                    v_segs: Sequence[torch.Tensor], rope: Optional[Rope3D], scale: Optional[float] = None,
                    kv_chunk: int = 0, return_lse: bool = True):
    """The whole path for one attention call: per-segment [B, S_i, H, D] Q/K/V
    (video first) -> RoPE on the video part of Q and K fused into the joint
    concat + [B, H, S, D] re-layout -> blockwise attention.  Returns
    attn_fwd's result in [B, H, S, D]."""
    q = joint_concat_permute(q_segs, rope)
    k = joint_concat_permute(k_segs, rope)
    v = joint_concat_permute(v_segs, None)
    return attn_fwd(q, k, v, scale=scale, kv_chunk=kv_chunk, return_lse=return_lse)

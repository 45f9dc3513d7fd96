"""Reference oracle — TEST INFRASTRUCTURE ONLY.

A plain fp64 CPU implementation (``oracle.c``, plain C + OpenMP) of what the
library computes, with a thin ctypes wrapper over numpy arrays.  Only the
tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  It shares no code with the HIP path and never
imports it.

Composition of the full joint-attention pipeline (``reference_forward``):
  0. (optional, ``prepare_qkv``) RMS QK-norm of each token's H*D values in
     fp64, rounded to the storage dtype: the norm's output is a stored tensor.
  1. RoPE in fp64 on the video segment of Q and K ("Context Parallelism in
     vLLM Omni Neuron", §Self-Attention with Context Parallelism: RoPE on
     query and key, never on value).
  2. Round the rotated Q/K to the storage dtype (RNE).  The pages' module
     materialises apply_rotary_emb_wan's output in the model dtype before the
     transpose and the attention call, so the attention inputs are that
     rounded value.
  3. Concatenate video | audio | text and move to [B, H, S, D] (xDiT PR
     "Adds support for KV-cache and joint tensors to USP method"; Ulysses
     input all-to-all + transpose(1, 2)).
  4. Full softmax attention in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# R3D_ORACLE_LIBRARY names another build of oracle.c (the host-sanitizer
# build of tests/sanitize.py), used as is; by default liboracle.so here.
_LIB_OVERRIDE = os.environ.get("R3D_ORACLE_LIBRARY")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, OpenMP, IEEE semantics)."""
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    D = ctypes.c_double
    lib.oracle_num_threads.restype = I
    lib.oracle_round_bf16.argtypes = [D]
    lib.oracle_round_bf16.restype = D
    lib.oracle_round_bf16_array.argtypes = [P, P, I64]
    lib.oracle_round_f32_array.argtypes = [P, P, I64]
    lib.oracle_rope_vec.argtypes = [P, P, I64, I64, I64, I64, I, I, I, D]
    lib.oracle_rope3d.argtypes = [P, P, I64, I64, I64, I64, I64, I64, I64, I, I, I, D]
    lib.oracle_rope3d.restype = I
    lib.oracle_rms_norm.argtypes = [P, P, I64, I64, P, D]
    lib.oracle_rms_norm.restype = I
    lib.oracle_joint_concat_permute.argtypes = [P, P, I, P, I64, I64, I64, I64]
    lib.oracle_joint_concat_permute.restype = I
    lib.oracle_attention.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, D]
    lib.oracle_attention.restype = I
    lib.oracle_attention_rows.argtypes = [P, P, P, P, I64, P, P, I64, I64, I64, I64, I64, D]
    lib.oracle_attention_rows.restype = I
    lib.oracle_attention_chunked.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, D, I64]
    lib.oracle_attention_chunked.restype = I
    lib.oracle_lse_merge.argtypes = [P, P, I64, I64, I64, P, P]
    lib.oracle_lse_merge.restype = I
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


# --- rounding ---------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """fp64 -> nearest bfloat16 value (ties to even), returned as fp64."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().oracle_round_bf16_array(_ptr(x), _ptr(y), x.size)
    return y


def round_f32(x) -> np.ndarray:
    x = _f64(x)
    y = np.empty_like(x)
    _load().oracle_round_f32_array(_ptr(x), _ptr(y), x.size)
    return y


def round_to(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    raise ValueError(dtype)


# --- RoPE -------------------------------------------------------------------

def rope_vec(x, pos, split, theta: float) -> np.ndarray:
    """Rotate one head vector x[D] at grid position pos=(t,h,w) (any integers)."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().oracle_rope_vec(_ptr(x), _ptr(y), x.size, int(pos[0]), int(pos[1]), int(pos[2]),
                            int(split[0]), int(split[1]), int(split[2]), float(theta))
    return y


def rope3d(x, grid, split, theta: float) -> np.ndarray:
    """x: [B, Nv, H, D] video tokens in (t,h,w) row-major order -> rotated copy."""
    x = _f64(x)
    B, Nv, H, D = x.shape
    y = np.empty_like(x)
    rc = _load().oracle_rope3d(_ptr(x), _ptr(y), B, Nv, H, D, int(grid[0]), int(grid[1]),
                               int(grid[2]), int(split[0]), int(split[1]), int(split[2]),
                               float(theta))
    if rc != 0:
        raise ValueError("oracle_rope3d: grid/split do not match the tensor")
    return y


# --- QK-norm --------------------------------------------------------------------

def rms_norm(x, w, eps: float) -> np.ndarray:
    """x: [..., n] -> x / sqrt(mean(x^2 over the last axis) + eps) * w[n] (fp64)."""
    x = _f64(x)
    w = _f64(w).reshape(-1)
    n = x.shape[-1]
    if w.size != n:
        raise ValueError("rms_norm: weight length must equal the last axis")
    y = np.empty_like(x)
    rc = _load().oracle_rms_norm(_ptr(x), _ptr(y), x.size // n, n, _ptr(w), float(eps))
    if rc != 0:
        raise ValueError("oracle_rms_norm: n <= 0 or eps < 0")
    return y


# --- joint concat + permute ---------------------------------------------------

def joint_concat_permute(segs) -> np.ndarray:
    """segs: list of [B, S_i, H, D] arrays of one dtype -> [B, H, S, D] (byte copy)."""
    segs = [np.ascontiguousarray(s) for s in segs]
    B, _, H, D = segs[0].shape
    dt = segs[0].dtype
    for s in segs:
        if s.dtype != dt or s.shape[0] != B or s.shape[2] != H or s.shape[3] != D:
            raise ValueError("segments disagree in dtype or B/H/D")
    lens = np.array([s.shape[1] for s in segs], dtype=np.int64)
    S = int(lens.sum())
    out = np.empty((B, H, S, D), dtype=dt)
    ptrs = (ctypes.c_void_p * len(segs))(*[s.ctypes.data for s in segs])
    rc = _load().oracle_joint_concat_permute(ctypes.cast(ptrs, ctypes.c_void_p), _ptr(lens),
                                             len(segs), _ptr(out), dt.itemsize, B, H, D)
    if rc != 0:
        raise ValueError("oracle_joint_concat_permute failed")
    return out


# --- attention ----------------------------------------------------------------

def attention(q, k, v, scale: float):
    """q [B,H,Sq,D], k/v [B,H,Skv,D] -> (out [B,H,Sq,D], lse [B,H,Sq]) in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    out = np.empty_like(q)
    lse = np.empty((B, H, Sq), dtype=np.float64)
    rc = _load().oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Sq, Skv,
                                  D, float(scale))
    if rc != 0:
        raise ValueError("oracle_attention failed")
    return out, lse


def attention_rows(q, k, v, rows, scale: float):
    """Rows given as flat indices (b*H + h)*Sq + i -> (out [n, D], lse [n])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, D), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    rc = _load().oracle_attention_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(rows), rows.size,
                                       _ptr(out), _ptr(lse), B, H, Sq, Skv, D, float(scale))
    if rc != 0:
        raise ValueError("oracle_attention_rows failed")
    return out, lse


def attention_chunked(q, k, v, scale: float, kv_chunk: int):
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    out = np.empty_like(q)
    lse = np.empty((B, H, Sq), dtype=np.float64)
    rc = _load().oracle_attention_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H,
                                          Sq, Skv, D, float(scale), int(kv_chunk))
    if rc != 0:
        raise ValueError("oracle_attention_chunked failed")
    return out, lse


def lse_merge(parts, lse_parts):
    """parts [n, ..., D], lse_parts [n, ...] -> (out [..., D], lse [...])."""
    parts = _f64(parts)
    lse_parts = _f64(lse_parts)
    n = parts.shape[0]
    D = parts.shape[-1]
    rows = int(np.prod(parts.shape[1:-1], dtype=np.int64))
    if lse_parts.shape != parts.shape[:-1]:
        raise ValueError("lse_parts shape mismatch")
    out = np.empty(parts.shape[1:], dtype=np.float64)
    lse = np.empty(parts.shape[1:-1], dtype=np.float64)
    rc = _load().oracle_lse_merge(_ptr(parts), _ptr(lse_parts), n, rows, D, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_lse_merge failed")
    return out, lse


# --- the whole path -------------------------------------------------------------

def prepare_qkv(q_segs, k_segs, v_segs, grid, split, theta, io_dtype, norm_q=None, norm_k=None,
                eps: float = 1e-6):
    """Steps 1-3 of the pipeline, one stored tensor after each of the page's ops
    ("Context Parallelism in vLLM Omni Neuron", §Self-Attention with Context
    Parallelism: q = norm_q(q), then unflatten into heads, then
    apply_rotary_emb_wan(q, ...), each producing a tensor in the model dtype):
      * optional RMS QK-norm (norm_q / norm_k: None, or one entry per segment,
        None or the segment's [H*D] weight vector; the statistic is over each
        token's H*D values), computed in fp64 and rounded to ``io_dtype``
        ("bf16" or "f32") -- the stored norm output;
      * fp64 RoPE of segment 0 of Q and K (from the stored values), rounded
        to ``io_dtype`` -- the stored rotary output;
      * the joint concat + [B,S,H,D] -> [B,H,S,D] re-layout.
    Inputs are fp64 arrays holding the exact values of the stored inputs, one
    [B,S_i,H,D] array per segment, video first.  Returns fp64 q, k, v in
    [B,H,S,D]."""
    def prepared(segs, norms):
        out = []
        for i, s in enumerate(segs):
            x = _f64(s)
            if norms is not None and norms[i] is not None:
                B, S, H, D = x.shape
                x = round_to(rms_norm(x.reshape(B, S, H * D), norms[i], eps).reshape(B, S, H, D), io_dtype)
            if i == 0:
                x = round_to(rope3d(x, grid, split, theta), io_dtype)
            out.append(x)
        return out
    q = joint_concat_permute(prepared(q_segs, norm_q))
    k = joint_concat_permute(prepared(k_segs, norm_k))
    v = joint_concat_permute([_f64(s) for s in v_segs])
    return q, k, v


def reference_forward(q_segs, k_segs, v_segs, grid, split, theta, io_dtype, scale, rows=None):
    """Full pipeline.  rows=None: every query row, returns (out [B,H,S,D], lse
    [B,H,S]); otherwise rows are flat indices and (out [n,D], lse [n])."""
    q, k, v = prepare_qkv(q_segs, k_segs, v_segs, grid, split, theta, io_dtype)
    if rows is None:
        return attention(q, k, v, scale)
    return attention_rows(q, k, v, rows, scale)

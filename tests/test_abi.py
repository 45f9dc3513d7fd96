"""C-ABI checks that need no GPU: the library loads, exports every entry
point declared in include/*.h (and nothing else), and rejects bad arguments on
the host before anything is launched.

The error-path calls pass fake, aligned, never-dereferenced addresses: every
case below fails validation, which happens before any HIP call.
"""
import ctypes
import glob
import os
import re
import subprocess

import pytest

import long_sequence_attention_rope3d_amd as r3d

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = ctypes.CDLL(r3d.library_path())


def _declared():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        names += re.findall(r"R3D_API\s+[\w\s\*]+?\b(r3d_\w+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    assert _declared() == sorted(["r3d_rope3d_apply", "r3d_joint_concat_permute",
                                  "r3d_joint_concat_permute_qknorm", "r3d_attn_fwd", "r3d_attn_fwd_bshd",
                                  "r3d_attn_fwd_noalloc", "r3d_attn_fwd_workspace_size", "r3d_attn_fwd_constmax",
                                  "r3d_attn_fwd_constmax_workspace_size", "r3d_attn_fwd_plan", "r3d_lse_merge",
                                  "r3d_last_error", "r3d_version"])


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", r3d.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in _declared():
        assert name in exported, name
        assert getattr(LIB, name) is not None
    ours = {n for n in exported if n.startswith("r3d_")}
    assert ours == set(_declared())


def test_version_string():
    LIB.r3d_version.restype = ctypes.c_char_p
    assert b"gfx950" in LIB.r3d_version()


# ---------------------------------------------------------------------------------------------
# Host-side validation (no launch happens in any of these)
# ---------------------------------------------------------------------------------------------
P = ctypes.c_void_p
I32, I64 = ctypes.c_int32, ctypes.c_int64
F = ctypes.c_float
SZ = ctypes.c_size_t
LIB.r3d_attn_fwd.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, F, I64, I32, P, SZ, P]
LIB.r3d_attn_fwd_bshd.argtypes = LIB.r3d_attn_fwd.argtypes
LIB.r3d_attn_fwd_noalloc.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, F, I64, I32, P]
LIB.r3d_attn_fwd_workspace_size.argtypes = [I64, I64, I64, I64, I64, I64, I32, ctypes.POINTER(SZ)]
LIB.r3d_attn_fwd_constmax.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, F, I32, P, SZ, P]
LIB.r3d_attn_fwd_constmax_workspace_size.argtypes = [I64, I64, I64, I64, I64, I32, ctypes.POINTER(SZ)]
LIB.r3d_rope3d_apply.argtypes = [P, P, I32, I64, I64, I64, I64, P, P]
LIB.r3d_joint_concat_permute.argtypes = [P, P, I32, P, I32, I64, I64, I64, P, P]
LIB.r3d_joint_concat_permute_qknorm.argtypes = [P, P, I32, P, ctypes.c_double, P, I32, I64, I64, I64, P, P]
LIB.r3d_lse_merge.argtypes = [P, P, I32, I32, P, P, I32, I64, I64, I64, I64, P]
LIB.r3d_last_error.restype = ctypes.c_char_p

A, B_, C, O, L_, W = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000, 0x70000000


def _attn(fn="r3d_attn_fwd", **kw):
    a = dict(q=A, k=B_, v=C, out=O, lse=L_, B=1, H=2, Sq=64, Skv=64, D=128, scale=0.125,
             kv_chunk=0, dtype=1, ws=W, ws_bytes=1 << 24)
    a.update(kw)
    return getattr(LIB, fn)(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Sq"],
                            a["Skv"], a["D"], a["scale"], a["kv_chunk"], a["dtype"], a["ws"], a["ws_bytes"],
                            None)


def _ws_size(fn="r3d_attn_fwd_workspace_size", **kw):
    a = dict(B=1, H=2, Sq=64, Skv=64, D=128, kv_chunk=0, dtype=1)
    a.update(kw)
    n = SZ(12345)
    args = [a["B"], a["H"], a["Sq"], a["Skv"], a["D"]]
    if fn == "r3d_attn_fwd_workspace_size":
        args.append(a["kv_chunk"])
    st = getattr(LIB, fn)(*args, a["dtype"], ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status,needle", [
    (dict(D=96), -2, "D=96"),
    (dict(dtype=7), -2, "dtype"),
    (dict(q=None), -1, "NULL"),
    (dict(k=B_ + 8), -1, "aligned"),
    (dict(Sq=0), -1, "> 0"),
    (dict(Skv=-3), -1, "> 0"),
    (dict(kv_chunk=-1), -1, "kv_chunk"),
    (dict(scale=float("nan")), -1, "finite"),
    (dict(scale=float("inf")), -1, "finite"),
    (dict(out=A), -1, "overlaps"),
    (dict(lse=O + 1024), -1, "overlaps"),
    (dict(B=1 << 40, H=1 << 20), -1, "too large"),
    # small tensors, but 2^19 heads: the key-norm pre-pass grid would pass 2^32 work-items
    (dict(B=1 << 10, H=1 << 9, Sq=1, Skv=1), -1, "one launch"),
    # bf16 rows are indexed in 32 bits: at most 2^31 - 1024 query or key rows
    (dict(H=1, Sq=(1 << 31) - 1023, D=64), -2, "at most 2147482624"),
    (dict(H=1, Skv=(1 << 31) - 1023, D=64), -2, "at most 2147482624"),
])
@pytest.mark.parametrize("fn", ["r3d_attn_fwd", "r3d_attn_fwd_bshd"])
def test_attn_fwd_rejects(fn, kw, status, needle):
    assert _attn(fn, **kw) == status
    assert needle in LIB.r3d_last_error().decode()


def test_attn_fwd_workspace_size():
    """The bf16 path needs the per-head statistics (2*B*H*64 floats, rounded up to 256
    bytes); without a GPU no key split is planned, so that is all.  fp32 needs nothing."""
    st, n = _ws_size(B=3, H=5)
    assert st == 0 and n == -(-2 * 15 * 64 * 4 // 256) * 256
    st, n = _ws_size(dtype=0)
    assert st == 0 and n == 0
    assert _ws_size(dtype=5)[0] == -2
    assert _ws_size(Sq=0)[0] == -1 and "> 0" in LIB.r3d_last_error().decode()
    assert _ws_size(kv_chunk=-1)[0] == -1
    assert _ws_size(B=1 << 40, H=1 << 20)[0] == -1 and "too large" in LIB.r3d_last_error().decode()
    assert LIB.r3d_attn_fwd_workspace_size(1, 2, 64, 64, 128, 0, 1, None) == -1
    # constant-max: statistics + one int flag per wave (12) of every 384-row tile
    st, n = _ws_size("r3d_attn_fwd_constmax_workspace_size", B=2, H=3, Sq=1000)
    assert st == 0 and n == -(-2 * 6 * 64 * 4 // 256) * 256 + -(-6 * 3 * 12 * 4 // 256) * 256
    assert _ws_size("r3d_attn_fwd_constmax_workspace_size", dtype=0)[0] == -2


@pytest.mark.parametrize("fn", ["r3d_attn_fwd", "r3d_attn_fwd_bshd"])
def test_attn_fwd_rejects_bad_workspace(fn):
    need = _ws_size()[1]
    assert _attn(fn, ws=None) == -1 and "NULL workspace" in LIB.r3d_last_error().decode()
    assert _attn(fn, ws_bytes=need - 1) == -1 and f"needs {need}" in LIB.r3d_last_error().decode()
    assert _attn(fn, ws=W + 8) == -1 and "aligned" in LIB.r3d_last_error().decode()
    assert _attn(fn, ws=O + 4096) == -1 and "workspace overlaps" in LIB.r3d_last_error().decode()
    assert _attn(fn, ws=L_ - 64) == -1 and "workspace overlaps" in LIB.r3d_last_error().decode()
    # argument errors are reported before workspace errors
    assert _attn(fn, ws=None, D=96) == -2


def test_attn_fwd_noalloc_rejects():
    def call(**kw):
        a = dict(q=A, k=B_, v=C, out=O, lse=L_, B=1, H=2, Sq=64, Skv=64, D=128, kv_chunk=0, dtype=1)
        a.update(kw)
        return LIB.r3d_attn_fwd_noalloc(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Sq"],
                                        a["Skv"], a["D"], 0.125, a["kv_chunk"], a["dtype"], None)
    # the fixed scratch holds the statistics of at most 32768 heads (512 bytes each)
    assert call(B=2, H=16385, Sq=1, Skv=1) == -1
    msg = LIB.r3d_last_error().decode()
    assert "attn_fwd_noalloc" in msg and "scratch" in msg and "16777216" in msg
    assert call(D=96) == -2
    assert call(q=None) == -1 and "NULL" in LIB.r3d_last_error().decode()
    assert call(out=A) == -1 and "overlaps" in LIB.r3d_last_error().decode()
    assert call(kv_chunk=-2) == -1


def test_attn_fwd_constmax_rejects():
    def call(ws=W, ws_bytes=1 << 24, dtype=1, D=128, out=O, Sq=64, Skv=64):
        return LIB.r3d_attn_fwd_constmax(A, B_, C, out, L_, 1, 2, Sq, Skv, D, 0.125, dtype, ws, ws_bytes, None)
    assert call(dtype=0) == -2 and "bf16" in LIB.r3d_last_error().decode()
    assert call(ws=None) == -1 and "workspace" in LIB.r3d_last_error().decode()
    assert call(ws=W + 2) == -1
    assert call(ws_bytes=100) == -1 and "needs" in LIB.r3d_last_error().decode()
    assert call(ws=O + 64) == -1 and "overlaps" in LIB.r3d_last_error().decode()
    assert call(D=96) == -2
    assert call(out=A) == -1
    assert call(Sq=(1 << 31) - 1023, D=64) == -2 and "at most" in LIB.r3d_last_error().decode()
    assert call(Skv=(1 << 31) - 1023, D=64) == -2


class Rope(ctypes.Structure):
    _fields_ = [("grid_t", I64), ("grid_h", I64), ("grid_w", I64), ("d_t", I32), ("d_h", I32),
                ("d_w", I32), ("theta", ctypes.c_double)]


@pytest.mark.parametrize("rope,Nv,D,status,needle", [
    (Rope(2, 8, 15, 16, 24, 24, 1e4), 241, 64, -1, "grid product"),
    (Rope(2, 8, 15, 16, 24, 26, 1e4), 240, 64, -1, "sum to D"),
    (Rope(2, 8, 15, 15, 25, 24, 1e4), 240, 64, -1, "even"),
    (Rope(2, 8, 15, 16, 24, 24, -1.0), 240, 64, -1, "theta"),
    (Rope(0, 8, 15, 16, 24, 24, 1e4), 0, 64, -1, "> 0"),
    (Rope(2, 8, 15, 32, 48, 16, 1e4), 240, 96, -2, "D=96"),
])
def test_rope3d_apply_rejects(rope, Nv, D, status, needle):
    assert LIB.r3d_rope3d_apply(A, O, 1, 1, Nv, 2, D, ctypes.byref(rope), None) == status
    assert needle in LIB.r3d_last_error().decode()


def test_rope3d_apply_rejects_partial_overlap_and_null_desc():
    r = Rope(2, 8, 15, 16, 24, 24, 1e4)
    assert LIB.r3d_rope3d_apply(A, A + 64, 1, 1, 240, 2, 64, ctypes.byref(r), None) == -1
    assert "overlap" in LIB.r3d_last_error().decode()
    assert LIB.r3d_rope3d_apply(A, O, 1, 1, 240, 2, 64, None, None) == -1
    assert "NULL" in LIB.r3d_last_error().decode()


def _perm(ptrs, lens, out=O, D=128, dtype=1, rope=None):
    arr = (P * len(ptrs))(*ptrs)
    ln = (I64 * len(lens))(*lens)
    return LIB.r3d_joint_concat_permute(ctypes.cast(arr, P), ctypes.cast(ln, P), len(ptrs), out,
                                        dtype, 1, 2, D, ctypes.byref(rope) if rope else None, None)


def test_permute_rejects():
    assert _perm([A, B_], [10, -1]) == -1
    assert _perm([A, None], [10, 5]) == -1 and "segment 1" in LIB.r3d_last_error().decode()
    assert _perm([A], [0]) == -1 and "is 0" in LIB.r3d_last_error().decode()
    assert _perm([A, B_], [10, 5], out=A + 256) == -1 and "overlaps" in LIB.r3d_last_error().decode()
    assert _perm([A], [10], D=12) == -2          # 24-byte rows
    assert _perm([A] * 9, [1] * 9) == -1         # too many segments
    assert _perm([A], [240], D=64, rope=Rope(2, 8, 14, 16, 24, 24, 1e4)) == -1
    assert _perm([A], [240], D=48, dtype=1, rope=Rope(2, 8, 15, 16, 16, 16, 1e4)) == -2


def _permn(ptrs, lens, wts, eps=1e-6, out=O, D=128, dtype=1, rope=None, null_w=False):
    arr = (P * len(ptrs))(*ptrs)
    ln = (I64 * len(lens))(*lens)
    w = (P * len(wts))(*wts)
    return LIB.r3d_joint_concat_permute_qknorm(ctypes.cast(arr, P), ctypes.cast(ln, P), len(ptrs),
                                               None if null_w else ctypes.cast(w, P), eps, out, dtype, 1,
                                               2, D, ctypes.byref(rope) if rope else None, None)


def test_permute_qknorm_rejects():
    W = 0x60000000
    assert _permn([A, B_], [10, 5], [W, None], null_w=True) == -1
    assert "norm weight array" in LIB.r3d_last_error().decode()
    assert _permn([A, B_], [10, 5], [W, None], eps=-1.0) == -1 and "eps" in LIB.r3d_last_error().decode()
    assert _permn([A, B_], [10, 5], [W, None], eps=float("nan")) == -1
    assert _permn([A, B_], [10, 5], [W + 4, None]) == -1 and "aligned" in LIB.r3d_last_error().decode()
    assert _permn([A, B_], [10, 5], [None, W], D=96) == -2 and "QK-norm" in LIB.r3d_last_error().decode()
    assert _permn([A, B_], [10, 5], [None, O + 64]) == -1 and "norm weights" in LIB.r3d_last_error().decode()
    # every plain-permute check still applies
    assert _permn([A, None], [10, 5], [W, None]) == -1 and "segment 1" in LIB.r3d_last_error().decode()
    # 2^26 tokens: the norm's 4-token blocks would pass 2^32 work-items (8-token blocks would not)
    assert _permn([1 << 40], [1 << 26], [1 << 42], out=1 << 41) == -1
    assert "one launch" in LIB.r3d_last_error().decode()


def test_lse_merge_rejects():
    def call(n=2, D=128, pdt=0, odt=1, out=O, lse_out=L_):
        return LIB.r3d_lse_merge(A, B_, n, pdt, out, lse_out, odt, 1, 2, 64, D, None)
    assert call(n=0) == -1
    assert call(n=65) == -1
    assert call(D=12) == -2
    assert call(pdt=3) == -2
    assert call(out=A + 4096) == -1 and "overlap" in LIB.r3d_last_error().decode()
    assert call(lse_out=O + 16) == -1


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 240, 2, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        r3d.rope3d_apply(x, (2, 8, 15), (16, 24, 24))
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        r3d.attn_fwd(q, q, q)
    with pytest.raises(ValueError, match="out_layout"):
        r3d.attn_fwd(q, q, q, out_layout="sbhd")


class _Plan(ctypes.Structure):
    _fields_ = [("waves", ctypes.c_int32), ("n_split", ctypes.c_int32), ("n_tiles", ctypes.c_int64),
                ("n_bulk", ctypes.c_int64), ("split_len", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64)]


LIB.r3d_attn_fwd_plan.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int32, ctypes.POINTER(_Plan)]
LIB.r3d_attn_fwd_plan.restype = ctypes.c_int


def _plan(B, H, Sq, Skv, D, kv_chunk, n_cus):
    p = _Plan()
    st = LIB.r3d_attn_fwd_plan(B, H, Sq, Skv, D, kv_chunk, n_cus, ctypes.byref(p))
    return st, p


@pytest.mark.parametrize("name,args,want", [
    # (B, H, Sq, Skv, D, kv_chunk) -> (waves, n_tiles, n_bulk, n_split, split_len) on 256 CUs
    ("pro-clip", (1, 24, 52608, 52608, 128, 4096), (12, 3288, 3288, 1, 52608)),     # last round 84% full
    ("image-dit", (1, 24, 4352, 4352, 128, 0), (12, 288, 256, 7, 640)),
    ("long-video", (1, 24, 119056, 119056, 128, 8192), (12, 7464, 7424, 5, 24576)),  # 3 chunks a range
    ("lite-clip", (1, 16, 3216, 3216, 128, 512), (8, 208, 208, 1, 3216)),           # 8-wave tiles, one round
    ("Ulysses rank", (1, 3, 52608, 52608, 128, 4096), (12, 411, 256, 13, 4096)),    # one chunk a range
    ("CP rank", (1, 24, 6576, 52608, 128, 6576), (12, 432, 256, 4, 13152)),         # two chunks a range
])
def test_attn_fwd_plan_on_256_cus(name, args, want):
    """The key-split planner's choice for each workload and shard shape on the MI355X's
    256 CUs (host logic; the GPU tests run these plans): a thin last round of query
    tiles is split into key ranges of whole chunks, a grid of few tiles takes 8-wave
    blocks, and the workspace holds the statistics plus the split tiles' partials."""
    st, p = _plan(*args, 256)
    assert st == 0, LIB.r3d_last_error()
    assert (p.waves, p.n_tiles, p.n_bulk, p.n_split, p.split_len) == want, name
    B, H, Sq, Skv, D, _ = args
    stats = -(-2 * B * H * 64 * 4 // 256) * 256
    if p.n_split == 1:
        assert p.workspace_bytes == stats
    else:
        rows_per_tile = 32 * p.waves
        first_row = (p.n_bulk // (p.n_tiles // (B * H))) * Sq + (p.n_bulk % (p.n_tiles // (B * H))) * rows_per_tile
        rows = B * H * Sq - first_row
        assert p.workspace_bytes == stats + -(-p.n_split * rows * (D + 1) * 4 // 256) * 256


def test_attn_fwd_plan_without_a_device_count_and_rejects():
    """n_cus = 0 (unknown device) plans no split, which is what the workspace query gives
    on a host without a GPU; bad arguments are refused."""
    st, p = _plan(1, 24, 4352, 4352, 128, 0, 0)
    assert st == 0 and p.waves == 12 and p.n_split == 1 and p.n_bulk == p.n_tiles == 288
    n = ctypes.c_size_t(0)
    assert LIB.r3d_attn_fwd_workspace_size(1, 24, 4352, 4352, 128, 0, 1, ctypes.byref(n)) == 0
    assert n.value == p.workspace_bytes
    assert _plan(1, 24, 4352, 4352, 128, 0, -1)[0] == -1
    assert _plan(1, 24, 4352, 4352, 96, 0, 256)[0] == -2
    assert LIB.r3d_attn_fwd_plan(1, 2, 64, 64, 128, 0, 256, None) == -1
    assert "NULL" in LIB.r3d_last_error().decode()


def test_binding_attn_fwd_plan():
    p = r3d.attn_fwd_plan(1, 24, 4352, 4352, 128, 0, 256)
    assert (p["waves"], p["n_tiles"], p["n_bulk"], p["n_split"], p["split_len"]) == (12, 288, 256, 7, 640)
    with pytest.raises(ValueError, match="n_cus"):
        r3d.attn_fwd_plan(1, 24, 4352, 4352, 128, 0, -1)

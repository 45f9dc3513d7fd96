"""The oracle's pins catch planted mistakes.

Each case copies the oracle (oracle/oracle.c, oracle/__init__.py), the workload
definitions and the pin suite (tests/test_oracle.py) into a scratch directory, plants
ONE plausible mistake in the copied oracle -- a dropped term, a wrong sign, a wrong or
transposed index, a misplaced rounding -- builds the copy's library, and runs the pin
suite against it in a child process.  The suite must fail (exit status 1: a test
failed, not a build or collection error).  A control case with no mistake must pass.
Nothing here touches the real oracle or the HIP library.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C, PY = "oracle/oracle.c", "oracle/__init__.py"
# (file, text, replacement, what the mistake is)
MUTANTS = [
    (C, "double y = rint(x / q) * q;", "double y = round(x / q) * q;",
     "bf16 rounding: ties away from zero instead of to even"),
    (C, "double q = ldexp(1.0, exp2_floor - 7);", "double q = ldexp(1.0, exp2_floor - 8);",
     "bf16 rounding: one significant bit too many"),
    (C, "if (exp2_floor < -126) exp2_floor = -126;", "if (exp2_floor < -133) exp2_floor = -133;",
     "bf16 rounding: subnormal spacing"),
    (C, "const double omega = pow(theta, -2.0 * (double)j / (double)da);",
     "const double omega = pow(theta, -1.0 * (double)j / (double)da);",
     "RoPE: frequency exponent -j/d instead of -2j/d"),
    (C, "y[off + 2 * j] = x0 * c - x1 * s;", "y[off + 2 * j] = x0 * c + x1 * s;",
     "RoPE: sign of the rotation's first row"),
    (C, "y[off + 2 * j + 1] = x0 * s + x1 * c;", "y[off + 2 * j + 1] = x0 * c + x1 * s;",
     "RoPE: sin and cos exchanged in the second row"),
    (C, "const int64_t pos[3] = {pt, ph, pw};", "const int64_t pos[3] = {pt, pw, ph};",
     "RoPE: h and w positions exchanged"),
    (C, "const int64_t h = (n / grid_w) % grid_h;", "const int64_t h = (n / grid_h) % grid_w;",
     "RoPE: token -> grid row index transposed"),
    (C, "const double inv = 1.0 / sqrt(ss / (double)n + eps);",
     "const double inv = 1.0 / (sqrt(ss / (double)n) + eps);",
     "QK-norm: eps added outside the square root"),
    (C, "const double inv = 1.0 / sqrt(ss / (double)n + eps);",
     "const double inv = 1.0 / sqrt(ss + eps);",
     "QK-norm: sum of squares instead of mean"),
    (C, "y[r * n + i] = xr[i] * inv * w[i];", "y[r * n + i] = xr[i] * inv * w[n - 1 - i];",
     "QK-norm: weight channel index reversed"),
    (C, "memcpy(o + (((b * H + h) * S) + off + s) * row, src + ((b * Si + s) * H + h) * row,",
     "memcpy(o + (((b * H + h) * S) + s) * row, src + ((b * Si + s) * H + h) * row,",
     "permute: segment offset dropped"),
    (C, "memcpy(o + (((b * H + h) * S) + off + s) * row, src + ((b * Si + s) * H + h) * row,",
     "memcpy(o + (((b * H + h) * S) + off + s) * row, src + ((b * H + h) * Si + s) * row,",
     "permute: source read as [B, H, S, D]"),
    (C, "s[j] = scale * dot;", "s[j] = dot;", "attention: scale dropped"),
    (C, "dot += q[d] * k[j * D + d];", "dot += q[d] * k[d * Skv + j];",
     "attention: K read transposed"),
    (C, "*lse = m + log(l);", "*lse = log(l);", "attention: max dropped from lse"),
    (C, "const double p = exp(s[j] - m);", "const double p = exp(s[j]);",
     "attention: max not subtracted"),
    (C, "for (int64_t d = 0; d < D; ++d) out[d] /= l;",
     "for (int64_t d = 0; d < D; ++d) out[d] /= (double)Skv;",
     "attention: mean of the weighted values instead of the softmax normalisation"),
    (C, "const double wa = exp(L - Lnew), wb = exp(lse_c - Lnew);",
     "const double wa = exp(lse_c - Lnew), wb = exp(L - Lnew);",
     "chunked attention: merge weights exchanged"),
    (C, "const int64_t n = (Skv - c0 < kv_chunk) ? (Skv - c0) : kv_chunk;",
     "const int64_t n = (Skv - c0 < kv_chunk) ? (Skv - c0) : kv_chunk - 1;",
     "chunked attention: one key per chunk skipped"),
    (C, "const double w = exp(lse_parts[i * rows + r] - L);",
     "const double w = exp(L - lse_parts[i * rows + r]);",
     "lse_merge: weight exponent negated"),
    (C, "const double L = hi + log(sum);", "const double L = hi;",
     "lse_merge: log-sum replaced by the max"),
    (PY, "x = round_to(rms_norm(x.reshape(B, S, H * D), norms[i], eps).reshape(B, S, H, D), io_dtype)",
     "x = rms_norm(x.reshape(B, S, H * D), norms[i], eps).reshape(B, S, H, D)",
     "pipeline: the norm's output not stored (one rounding for norm + RoPE)"),
    (PY, "x = round_to(rope3d(x, grid, split, theta), io_dtype)", "x = rope3d(x, grid, split, theta)",
     "pipeline: the RoPE output not rounded to the storage type"),
    (PY, "v = joint_concat_permute([_f64(s) for s in v_segs])",
     "v = joint_concat_permute(prepared(v_segs, None))",
     "pipeline: V rotated as well"),
]

_FILES = [C, PY, "workloads/__init__.py", "workloads/configs.py", "workloads/inputs.py",
          "tests/conftest.py", "tests/test_oracle.py"]


def _copy_tree(dst):
    for rel in _FILES:
        os.makedirs(os.path.join(dst, os.path.dirname(rel)), exist_ok=True)
        shutil.copy2(os.path.join(ROOT, rel), os.path.join(dst, rel))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))


def _run_pins(dst):
    env = {k: v for k, v in os.environ.items() if k not in ("R3D_ORACLE_LIBRARY", "PYTEST_ADDOPTS")}
    env["OMP_NUM_THREADS"] = "4"
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    p = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle.py", "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=dst, env=env, capture_output=True, text=True, timeout=600)
    return p.returncode, p.stdout[-3000:] + p.stderr[-2000:]


def test_unmutated_copy_passes(tmp_path):
    dst = str(tmp_path / "tree")
    _copy_tree(dst)
    rc, log = _run_pins(dst)
    assert rc == 0, log


@pytest.mark.parametrize("path,old,new,what", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(tmp_path, path, old, new, what):
    dst = str(tmp_path / "tree")
    _copy_tree(dst)
    f = os.path.join(dst, path)
    src = open(f).read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    open(f, "w").write(src.replace(old, new))
    rc, log = _run_pins(dst)
    assert rc == 1, f"{what}: the pin suite did not fail (exit {rc})\n{log}"

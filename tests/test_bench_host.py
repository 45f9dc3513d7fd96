"""Host-side logic of bench.py (no GPU): the kernel-code hash that decides whether the
committed HBM-traffic profile still describes the current attention kernel."""
import importlib.util
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    argv = sys.argv
    try:
        sys.argv = ["bench.py"]
        spec.loader.exec_module(mod)
    finally:
        sys.argv = argv
    return mod


def test_kernel_code_hash_ignores_comments_but_not_code(tmp_path):
    b = _bench()
    base = "int f(int x) {\n  return x + 1;  // add one\n}\n"
    p = tmp_path / "k.hip"
    p.write_text(base)
    h0 = b.kernel_code_sha256(str(p))
    p.write_text("// a new header comment\n\n" + base.replace("// add one", "// increment"))
    assert b.kernel_code_sha256(str(p)) == h0
    p.write_text(base.replace("x + 1", "x + 2"))
    assert b.kernel_code_sha256(str(p)) != h0


def test_traffic_is_null_when_the_recorded_hash_differs(tmp_path, monkeypatch):
    b = _bench()
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; }\n")
    prof = tmp_path / "traffic.md"
    prof.write_text(f"kernel_code_sha256: {b.kernel_code_sha256(str(src))}\nhbm_bytes_per_launch: 1.5e+09\n")
    monkeypatch.setattr(b, "ATTN_SRC", str(src))
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(prof))
    assert b._traffic_for_current_kernel() == 1.5e9
    src.write_text("int f() { return 2; }\n")
    assert b._traffic_for_current_kernel() is None


def test_mfma_counters_follow_the_kernel_hash(tmp_path, monkeypatch):
    b = _bench()
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; }\n")
    prof = tmp_path / "mfma.md"
    prof.write_text(f"kernel_code_sha256: {b.kernel_code_sha256(str(src))}\n"
                    "mfma_busy_frac: 0.628\nsclk_ghz_under_load: 1.869\n")
    monkeypatch.setattr(b, "ATTN_SRC", str(src))
    monkeypatch.setattr(b, "MFMA_FILE", str(prof))
    c = b._mfma_counters_for_current_kernel()
    assert c["mfma_busy_frac"] == 0.628 and c["sclk_ghz_under_load"] == 1.869
    src.write_text("int f() { return 2; }\n")
    assert b._mfma_counters_for_current_kernel() is None



def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    """bench.py --gpus N with N != 1 exits with status 2 and says why (one GPU only)."""
    import subprocess
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert p.returncode == 2
    assert "exactly one GPU" in (p.stdout + p.stderr)


def test_power_figures_follow_the_kernel_hash(tmp_path, monkeypatch):
    b = _bench()
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; }\n")
    h = b.kernel_code_sha256(str(src))
    mfma = tmp_path / "mfma.md"
    mfma.write_text(f"kernel_code_sha256: {h}\nmfma_busy_frac: 0.67\nsclk_ghz_under_load: 1.77\n")
    power = tmp_path / "power.md"
    power.write_text(f"kernel_code_sha256: {h}\npackage_power_w_under_load: 1349\npower_cap_w: 1400\n")
    monkeypatch.setattr(b, "ATTN_SRC", str(src))
    monkeypatch.setattr(b, "MFMA_FILE", str(mfma))
    monkeypatch.setattr(b, "POWER_FILE", str(power))
    c = b._mfma_counters_for_current_kernel()
    assert c["package_power_w_under_load"] == 1349 and c["power_cap_w"] == 1400
    power.write_text("kernel_code_sha256: " + "0" * 64 + "\npackage_power_w_under_load: 1349\npower_cap_w: 1400\n")
    c = b._mfma_counters_for_current_kernel()
    assert "package_power_w_under_load" not in c and c["mfma_busy_frac"] == 0.67


def test_power_cap_query_parses_the_smi_line(monkeypatch):
    """The bench records the board's power cap from `rocm-smi --showmaxpower`; a host
    without the tool (or with other output) gives None."""
    import subprocess as sp
    import bench

    class _Done:
        stdout = "GPU[0]\t\t: Max Graphics Package Power (W): 1400.0\n"
    monkeypatch.setattr(sp, "run", lambda *a, **k: _Done())
    assert bench.power_cap_watts() == 1400.0

    def _missing(*a, **k):
        raise FileNotFoundError("rocm-smi")
    monkeypatch.setattr(sp, "run", _missing)
    assert bench.power_cap_watts() is None

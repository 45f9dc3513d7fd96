"""Host-sanitizer run of the C ABI and the oracle (CPU only; not a pytest module).

    python tests/sanitize.py

Builds, into _build/sanitize/:
  * librope3d_attn.so from the same sources as build.py, its HOST code compiled with
    AddressSanitizer and UndefinedBehaviorSanitizer (each -fsanitize= sits behind
    -Xarch_host, so no device code is instrumented);
  * liboracle.so from oracle/oracle.c with the same sanitizers, by ROCm's clang, so that
    both libraries share clang's sanitizer runtime (OpenMP left out: the oracle's loops run
    serially);
then runs the CPU tests that exercise them -- tests/test_abi.py (export list and every host
validation path of the C ABI), tests/test_oracle.py and tests/test_rounding_method.py -- in a
child process with that runtime preloaded and R3D_LIBRARY / R3D_ORACLE_LIBRARY pointing at
the sanitized builds.  Any sanitizer report aborts the run with a non-zero status."""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
LLVM = "/opt/rocm/llvm"
sys.path.insert(0, os.path.join(ROOT, "long_sequence_attention_rope3d_amd"))
import build as B  # noqa: E402  (build.py, loaded as a file: the package would load the library)

SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def run(cmd, **kw):
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, **kw)


def main() -> int:
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in B.SOURCES:
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        run([B._hipcc(), *B.CFLAGS, *SAN_HOST, "-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", obj])
        objs.append(obj)
    lib = os.path.join(OUT, "librope3d_attn.so")
    run([B._hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libsan", *SAN_HOST, "-o", lib, *objs])
    olib = os.path.join(OUT, "liboracle.so")
    run([os.path.join(LLVM, "bin", "clang"), "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-shared-libsan",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         "-fno-fast-math", "-ffp-contract=off", "-Wno-unknown-pragmas", "-o", olib,
         os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    rt = glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not rt:
        print("clang's shared ASan runtime not found", file=sys.stderr)
        return 2
    env = dict(os.environ, LD_PRELOAD=rt[0], R3D_LIBRARY=lib, R3D_ORACLE_LIBRARY=olib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    tests = [os.path.join(ROOT, "tests", t) for t in ("test_abi.py", "test_oracle.py", "test_rounding_method.py")]
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *tests],
                          env=env).returncode


if __name__ == "__main__":
    sys.exit(main())

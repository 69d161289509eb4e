"""The host-side code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two instrumented builds go to a temporary directory: the fp64 oracle (plain C, clang) and
libkda.so with the sanitizers on its host half only (argument validation, path selection,
workspace sizing, launch set-up; the gfx950 device code is built as usual and never runs here,
no GPU is touched).  The oracle pins
(tests/test_oracle.py) and the ABI validation tests (tests/test_abi.py) then run against them in a
child process with the sanitizer runtime preloaded; any report fails the run."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunked_gated_delta_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = "/opt/rocm/bin/hipcc"


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(not (os.path.exists(CLANG) and os.path.exists(HIPCC) and _asan_runtime()),
                    reason="ROCm clang, hipcc or the ASan runtime is missing")
def test_oracle_and_host_validation_under_asan_ubsan(tmp_path):
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
    oracle = tmp_path / "liboracle_san.so"
    subprocess.run([CLANG, *san, "-std=c99", "-fPIC", "-shared", "-o", str(oracle),
                    os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm", "-lpthread"], check=True)
    lib = tmp_path / "libkda_san.so"
    # every sanitizer flag goes to the host compiler only
    host_san = [x for f in san[:4] for x in ("-Xarch_host", f)]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                        "-shared", "-fvisibility=hidden", *host_san, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                        "-o", str(lib), *srcs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), KDA_ORACLE_LIB=str(oracle), KDA_LIB_PATH=str(lib),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py"), os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    summary = [ln for ln in out.splitlines() if " passed" in ln]
    print("sanitized run:", summary[-1] if summary else "?")
    assert summary and "skipped" not in summary[-1]

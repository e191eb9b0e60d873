"""The host code under AddressSanitizer (CPU only): libmla's host side (the
planner, argument checks and C ABI; device code is built as usual) and the
C oracle are built with -fsanitize=address into a temporary folder, and the
host-ABI and oracle test files run against those builds in a child process
that preloads the sanitizer runtime.  Any sanitizer report fails the test.
The oracle's sanitizer build takes clang's OpenMP runtime."""
import glob
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
LLVM = Path(os.environ.get("ROCM_PATH", "/opt/rocm")) / "llvm"
HIPCC = Path(os.environ.get("ROCM_PATH", "/opt/rocm")) / "bin" / "hipcc"


def _asan_runtime():
    hits = sorted(glob.glob(str(LLVM / "lib" / "clang" / "*" / "lib" / "linux" / "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


@pytest.mark.timeout(900)
def test_host_code_under_address_sanitizer(tmp_path):
    rt = _asan_runtime()
    if rt is None or not HIPCC.exists():
        pytest.skip("no clang sanitizer runtime or hipcc in this image")
    sys.path.insert(0, str(ROOT))
    from mla_latent_kv_07_amd import build as B

    lib = tmp_path / "libmla_asan.so"
    cmd = [str(HIPCC), *B.HIPCC_FLAGS, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", str(ROOT / "include"), "-o", str(lib), *B.sources()]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    orc = tmp_path / "liboracle_asan.so"
    subprocess.run([str(LLVM / "bin" / "clang"), "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
                    "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(orc), str(ROOT / "oracle" / "mla_oracle.c"),
                    "-L" + str(LLVM / "lib"), "-Wl,-rpath," + str(LLVM / "lib"), "-lm"],
                   check=True, capture_output=True, text=True)

    env = dict(os.environ)
    env.update({"LD_PRELOAD": rt, "MLA_LIB": str(lib), "MLA_ORACLE_LIB": str(orc),
                # the interpreter and the ROCm runtime are not instrumented:
                # their allocations are not leak-checked
                "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=97",
                "PYTHONDONTWRITEBYTECODE": "1"})
    # the child loads the sanitizer builds, not the in-tree ones
    probe = ("import oracle, mla_latent_kv_07_amd._lib as L; L.load(); oracle.lib(); "
             "m = open('/proc/self/maps').read(); print('libmla_asan' in m, 'liboracle_asan' in m)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.split() == ["True", "True"], r.stdout + r.stderr[-2000:]
    tests = ["tests/test_host_abi.py", "tests/test_f8w8_layout_model.py",
             *sorted(str(p.relative_to(ROOT)) for p in (ROOT / "tests").glob("test_oracle_*.py"))]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        "-p", "no:xdist", *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=840)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out

"""The library's host code under AddressSanitizer + UndefinedBehaviorSanitizer.

libddt.so and the split checker are rebuilt with every host-pass option behind
-Xarch_host (the device code is compiled as usual), and the CPU suites that
drive their host code run again in a child process with clang's ASan runtime
loaded first: every entry point's argument validation and error reporting
(test_abi.py) and the attention work split for every workgroup of the swept
launches (test_split_plan.py).  Out-of-bounds or freed-memory accesses and
undefined behaviour (signed overflow, bad shifts, misaligned loads) abort the
child.  A planted overflow shows that the sanitizers are live in such a build."""
import glob
import os
import subprocess
import sys

import pytest

from tree_verify_mla_ddt_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["test_abi.py", "test_split_plan.py"]


def _asan_runtime():
    try:
        r = subprocess.run(["/opt/rocm/llvm/bin/clang", "-print-resource-dir"],
                           capture_output=True, text=True, timeout=60)
    except (OSError, subprocess.TimeoutExpired):
        return None
    res = r.stdout.strip()
    for pat in ("lib/linux/libclang_rt.asan-x86_64.so", "lib/*/libclang_rt.asan.so"):
        hits = sorted(glob.glob(os.path.join(res, pat)))
        if hits:
            return hits[0]
    return None


def _env(runtime, **extra):
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(p for p in (runtime, os.environ.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra)
    return env


@pytest.fixture(scope="module")
def runtime():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    return rt


def test_planted_overflow_is_caught(runtime, tmp_path):
    src = tmp_path / "plant.hip"
    src.write_text("#include <hip/hip_runtime.h>\n"
                   'extern "C" int plant(int a) { return a + 2147483600; }\n')
    out = tmp_path / "libplant.so"
    cmd = ["hipcc", f"--offload-arch={libbuild.ARCH}", "-std=c++17", "-fPIC", "-shared"]
    cmd += libbuild.SAN_HOST_FLAGS + [str(src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    code = f"import ctypes; print(ctypes.CDLL({str(out)!r}).plant(100))"
    r = subprocess.run([sys.executable, "-c", code], env=_env(runtime), capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0 and "signed integer overflow" in r.stderr, r.stderr[-2000:]


def test_host_code_under_asan_ubsan(runtime, tmp_path):
    lib, check = libbuild.build_sanitized(str(tmp_path))
    env = _env(runtime, DDT_LIB=lib, DDT_SPLIT_CHECK_LIB=check)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
    cmd += [os.path.join(ROOT, "tests", t) for t in SUITES]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "skipped" not in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail

"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU: the oracle (oracle.cpp, g++) runs its pin tests, and the C ABI's
host side (every csrc/*.hip, with the sanitizers on the host pass only and
the gfx950 device code built as usual) runs the argument-validation tests.
Each build goes to a temporary directory and is loaded in a child Python
through GS_ORACLE_LIB / GS_LIB_PATH with the matching sanitizer runtime
preloaded; any report ends the child with a non-zero status. A planted
heap overrun, built with the same flags, shows that each runtime is live.
No GPU is used: the validation tests make no compute call."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=23",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=23"}

OVERRUN = r"""
#include <stdlib.h>
#include <string.h>
extern "C" int planted_overrun(int n) {
    int* a = (int*)malloc(sizeof(int) * n);
    memset(a, 0, sizeof(int) * n);
    int s = a[n];  // one past the end
    free(a);
    return s;
}
"""


def _gcc_runtimes():
    out = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
        if not os.path.isabs(p) or not os.path.exists(p):
            pytest.skip(f"g++ has no {name}")
        out.append(p)
    return out


def _clang_runtime():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not hits:
        pytest.skip("the ROCm clang AddressSanitizer runtime is not installed")
    return [hits[0]]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not found")


def _child(code_or_args, preload, extra_env, timeout=600):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(extra_env)
    env["LD_PRELOAD"] = " ".join(preload)
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    args = code_or_args if isinstance(code_or_args, list) else ["-c", code_or_args]
    return subprocess.run([sys.executable] + args, cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def _check_planted(lib, preload):
    r = _child(f"import ctypes; ctypes.CDLL({lib!r}).planted_overrun(5)", preload, {})
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]


def test_oracle_under_sanitizers(tmp_path):
    preload = _gcc_runtimes()
    flags = ["-O1", "-g", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["g++"] + flags + ["-o", lib, os.path.join(ROOT, "oracle", "oracle.cpp")], check=True)
    planted = str(tmp_path / "planted.so")
    (tmp_path / "planted.cpp").write_text(OVERRUN)
    subprocess.run(["g++"] + flags + ["-o", planted, str(tmp_path / "planted.cpp")], check=True)
    _check_planted(planted, preload)

    env = {"GS_ORACLE_LIB": lib}
    r = _child("import oracle; oracle.lib(); maps = open('/proc/self/maps').read(); "
               f"assert {lib!r} in maps and 'libasan' in maps, 'sanitized oracle not loaded'", preload, env)
    assert r.returncode == 0, r.stderr[-2000:]
    pins = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    assert pins
    r = _child(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"] + pins, preload, env, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "failed" not in r.stdout


def test_abi_host_code_under_sanitizers(tmp_path):
    preload = _clang_runtime()
    hipcc = _hipcc()
    host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-shared",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "gaussian_splatting_tile_amd", "csrc")]
    lib = str(tmp_path / "libgs_san.so")
    srcs = sorted(glob.glob(os.path.join(ROOT, "gaussian_splatting_tile_amd", "csrc", "*.hip")))
    subprocess.run([hipcc] + common + host + ["-o", lib] + srcs, check=True, capture_output=True)
    planted = str(tmp_path / "planted.so")
    (tmp_path / "planted.hip").write_text(OVERRUN)
    subprocess.run([hipcc] + common + host + ["-o", planted, str(tmp_path / "planted.hip")], check=True,
                   capture_output=True)
    _check_planted(planted, preload)

    env = {"GS_LIB_PATH": lib}
    r = _child("from gaussian_splatting_tile_amd import _lib; _lib.load(); maps = open('/proc/self/maps').read(); "
               f"assert {lib!r} in maps and 'libclang_rt.asan' in maps, 'sanitized library not loaded'",
               preload, env)
    assert r.returncode == 0, r.stderr[-2000:]
    r = _child(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi_host.py")],
               preload, env, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "failed" not in r.stdout

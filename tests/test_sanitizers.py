"""CPU runs under AddressSanitizer and UndefinedBehaviorSanitizer.

* The C ABI's host code (kda_api.hip: argument checks, size functions, buffer
  layouts, the static workspace limit) is built with both sanitizers on its
  host pass only, linked with launcher stubs (tests/sanitize/launch_stubs.cpp)
  and driven by tests/sanitize/abi_checks.c, which expects every call to fail
  its checks before any HIP call.  Leak detection is on.
* The fp64 oracle (oracle/kda_oracle.c) is built with gcc's sanitizers and the
  oracle pins (tests/test_oracle_pins.py) run against that build in a child
  process with the sanitizer runtime preloaded.

No GPU is used; a sanitizer report fails the run (-fno-sanitize-recover).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout[-3000:]}\n{res.stderr[-3000:]}"
    return res


def test_abi_host_code_under_asan_ubsan(tmp_path):
    for tool in (HIPCC, CLANG, CLANGXX):
        if not os.path.exists(tool):
            pytest.skip(f"{tool} not found")
    host_san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"):
        host_san += ["-Xarch_host", f]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
    api = str(tmp_path / "api.o")
    stubs = str(tmp_path / "stubs.o")
    checks = str(tmp_path / "checks.o")
    exe = str(tmp_path / "abi_san")
    _run([HIPCC] + common + host_san + ["-c", os.path.join(ROOT, "gated_delta_rule_41_amd", "csrc", "kda_api.hip"),
                                        "-o", api])
    _run([HIPCC, "-x", "hip", "--offload-host-only"] + common + host_san +
         ["-c", os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), "-o", stubs])
    _run([CLANG, "-O1", "-g"] + SAN + ["-c", os.path.join(ROOT, "tests", "sanitize", "abi_checks.c"), "-o", checks])
    _run([CLANGXX] + SAN + [checks, api, stubs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                            "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    res = _run([exe], env=env, timeout=120)
    assert "abi checks ok" in res.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    lib = str(tmp_path / "libkda_oracle_san.so")
    _run([gcc, "-O1", "-g"] + SAN + ["-fPIC", "-shared", "-std=c99", "-o", lib,
                                     os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lpthread", "-lm"])
    asan = _run([gcc, "-print-file-name=libasan.so"]).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
               KDA_ORACLE_LIB=lib)
    probe = _run([sys.executable, "-c", "import oracle; print(oracle._load()._name)"], env=env, cwd=ROOT, timeout=120)
    assert probe.stdout.strip() == lib
    _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
          os.path.join(ROOT, "tests", "test_oracle_pins.py")], env=env, cwd=ROOT, timeout=600)

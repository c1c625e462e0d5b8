"""CPU-tier sanitizer runs (no GPU needed).

* The fp64 oracle (oracle/kda_oracle.c) is rebuilt with AddressSanitizer and
  UndefinedBehaviorSanitizer (gcc), and its pins and the finite-difference
  checks of its adjoint run against that build.
* The host side of the HIP library (argument validation, size arithmetic,
  the C ABI) is rebuilt with the same sanitizers on the host pass only
  (clang via hipcc; the device code is compiled as usual), and the C-ABI tests
  run against that build -- every invalid and edge argument they pass goes
  through the sanitized checks.

Each run is a separate Python process with the sanitizer runtime preloaded;
any report makes it exit non-zero.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["kda_api", "kda_prepare", "kda_scan", "kda_scan_wave", "kda_decode", "kda_combine", "kda_backward"]


def _run(cmd, env=None, timeout=900):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    out = r.stdout + r.stderr
    # a sanitizer report first, where there is one
    reports = [l for l in out.splitlines() if "runtime error" in l or "Sanitizer" in l]
    return r.returncode, "\n".join(reports[:20]) + "\n" + out


def _env(preload, **extra):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:symbolize=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra)
    return env


def test_oracle_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libkda_oracle_san.so")
    rc, msg = _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-std=c11", "-fPIC", "-shared", "-pthread",
                    os.path.join(ROOT, "oracle", "kda_oracle.c"), "-o", lib, "-lm"])
    assert rc == 0, msg
    rt = [subprocess.check_output(["gcc", f"-print-file-name={n}"], text=True).strip()
          for n in ("libasan.so", "libubsan.so")]
    rc, msg = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                    os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                    os.path.join(ROOT, "tests", "test_oracle_grad.py")],
                   env=_env(":".join(rt), KDA_ORACLE_LIB=lib))
    assert rc == 0 and "passed" in msg, msg[:3000]
    assert "ERROR: AddressSanitizer" not in msg and "runtime error" not in msg, msg[:3000]


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(_clang_asan_runtime() is None or not os.path.exists(HIPCC), reason="needs hipcc and clang's ASan")
def test_library_host_code_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    csrc = os.path.join(ROOT, "gated_delta_rule_91_amd", "csrc")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
             # sanitizers on the host pass only
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(name):
        return _run([HIPCC, *flags, "-c", os.path.join(csrc, name + ".hip"), "-o", os.path.join(OUT, name + ".o")])

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        for rc, msg in ex.map(compile_one, SOURCES):
            assert rc == 0, msg
    lib = os.path.join(OUT, "libkda_san.so")
    rc, msg = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                    *[os.path.join(OUT, n + ".o") for n in SOURCES], "-o", lib])
    assert rc == 0, msg
    rc, msg = _run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                    os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                   env=_env(_clang_asan_runtime(), KDA_LIB=lib))
    assert rc == 0 and "passed" in msg, msg[:3000]
    assert "ERROR: AddressSanitizer" not in msg and "runtime error" not in msg, msg[:3000]

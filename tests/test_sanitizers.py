"""CPU sanitizer runs (AddressSanitizer + UndefinedBehaviorSanitizer, every
finding fatal), each in a subprocess:

* the oracle, built by gcc with the sanitizers, under its whole pin suite;
* the host side of the C ABI: the library's host code (argument checks,
  workspace arithmetic, status strings, error-word setting) built by clang
  with the sanitizers and linked with the unchanged device objects, under
  the host ABI tests (no kernel runs; there is no GPU here).

The device code is never built with a sanitizer.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_OPTIONS = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
               "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_pytest(test_file, env_extra, lib, prelude=""):
    code = (prelude + "import sys, pytest\n"
            f"rc = pytest.main([{test_file!r}, '-q', '-x', '-s', '-p', 'no:cacheprovider'])\n"
            "import ctypes\n"
            "assert hasattr(ctypes.CDLL(None), '__asan_init'), 'sanitizer runtime not loaded'\n"
            f"assert {lib!r} in open('/proc/self/maps').read(), 'sanitized library not loaded'\n"
            "sys.exit(rc)\n")
    env = dict(os.environ)
    env.update(SAN_OPTIONS)
    env.update(env_extra)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, out
    return out


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    from oracle import build as oracle_build
    lib = oracle_build.build(out=str(tmp_path / "liboracle_san.so"),
                             extra_flags=("-g", "-fno-omit-frame-pointer",
                                          "-fsanitize=address,undefined",
                                          "-fno-sanitize-recover=all"))
    rt = [subprocess.check_output(["gcc", f"-print-file-name={n}"], text=True).strip()
          for n in ("libasan.so", "libubsan.so")]
    if not all(os.path.isabs(p) and os.path.exists(p) for p in rt):
        pytest.skip("gcc sanitizer runtimes not installed")
    out = _run_pytest("tests/test_oracle_pins.py",
                      {"PKV_ORACLE_LIB": lib, "LD_PRELOAD": ":".join(rt)}, lib)
    assert " passed" in out


def test_host_abi_checks_under_asan_and_ubsan(tmp_path):
    dev_objs = sorted(glob.glob(os.path.join(ROOT, "_build", "pkv", "*.hip.o")))
    if not dev_objs:
        from paged_kv_decode_store_amd import build as pkv_build
        pkv_build.build()
        dev_objs = sorted(glob.glob(os.path.join(ROOT, "_build", "pkv", "*.hip.o")))
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt or not os.path.exists(HIPCC):
        pytest.skip("clang sanitizer runtime or hipcc not installed")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    obj = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libpkv_san.so")
    subprocess.run([HIPCC, "-c", "-O1", "-g", "-std=c++17", "-fPIC", "-Wall",
                    "-I" + os.path.join(ROOT, "include"), *san,
                    os.path.join(ROOT, "paged_kv_decode_store_amd", "csrc", "api.cpp"), "-o", obj],
                   check=True, capture_output=True)
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *san[:4],
                    "-shared-libasan", *dev_objs, obj, "-o", lib],
                   check=True, capture_output=True)
    prelude = ("import paged_kv_decode_store_amd._lib as L\n"
               f"L.LIB_PATH = {lib!r}\n")
    out = _run_pytest("tests/test_abi_host.py", {"LD_PRELOAD": rt[-1]}, lib, prelude)
    assert " passed" in out

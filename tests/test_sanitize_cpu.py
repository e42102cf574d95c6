"""Sanitizer builds of the CPU-side code, run on the host (no GPU involved).

- The fp64 oracle (oracle/gdn_oracle.c) under AddressSanitizer + UndefinedBehaviorSanitizer
  (leak detection on), and under ThreadSanitizer (its worker threads share a job counter),
  driven by tests/sanitize/oracle_driver.c.
- The library's host code (argument validation and size arithmetic of the C ABI, in
  gdn_api.cpp and the host functions of the kernel files) under AddressSanitizer +
  UndefinedBehaviorSanitizer, driven by tests/sanitize/abi_driver.cpp: every call it makes is
  refused before any device work, including sizes and strides whose products would overflow.
  Device code is built without sanitizers (the flags go to the host compilation only).
Each driver exits 0 only if every check passed; any sanitizer report aborts it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_streaming_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
           TSAN_OPTIONS="halt_on_error=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
@pytest.mark.parametrize("kind", ["address,undefined", "thread"])
def test_oracle_under_sanitizers(tmp_path, kind):
    exe = str(tmp_path / "oracle_driver")
    flags = ["-fsanitize=" + kind, "-O1", "-g", "-fno-omit-frame-pointer", "-std=c11"]
    if kind != "thread":
        flags.append("-fno-sanitize-recover=all")
    _run(["gcc", *flags, "-o", exe, os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "gdn_oracle.c"),
          "-lpthread", "-lm"])
    res = _run([exe], env=ENV, timeout=300)
    assert "ok: 0 failures" in res.stdout
    assert "Sanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not found")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    host_san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer"):
        host_san += ["-Xarch_host", f]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    objs, procs = [], []
    for src in ("gdn_kernels.hip", "gdn_backward.hip", "gdn_attention.hip", "gdn_lowp.hip", "gdn_api.cpp"):
        obj = str(tmp_path / (src + ".o"))
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        procs.append((src, subprocess.Popen([HIPCC, *common, *host_san, *lang, "-c", os.path.join(CSRC, src), "-o", obj],
                                            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    for src, p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{src}: {err}"
    drv = str(tmp_path / "abi_driver.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]   # host-only objects and link
    _run([CLANGXX, "-O1", "-g", "-std=c++17", *san, "-I", INCLUDE, "-c", os.path.join(SAN, "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([CLANGXX, *san, "-o", exe, drv, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
          "-lpthread"])
    # the HIP runtime keeps allocations alive to process exit; leaks are checked on the oracle build
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    res = _run([exe], env=env, timeout=300)
    assert "ok: 0 failures" in res.stdout, res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr

"""Build the gfx950 libraries in-tree with hipcc: ``libgdn_stream.so`` (the GDN path and its
C ABI) and ``libgdn_peaks.so`` (copy and MFMA probes that measure the machine's peaks for the
roofline; measurement support, not part of the path)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdn_stream.so")
SOURCES = [os.path.join(CSRC, "gdn_kernels.hip"), os.path.join(CSRC, "gdn_backward.hip"),
           os.path.join(CSRC, "gdn_attention.hip"), os.path.join(CSRC, "gdn_api.cpp")]
PEAKS_LIB = os.path.join(PKG, "libgdn_peaks.so")
PEAKS_SOURCES = [os.path.join(CSRC, "gdn_peaks.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results and accumulators in ordinary VGPRs: the scan scales and converts its
    # accumulators every step, which with accumulation registers costs a copy per value
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result",
]


def command(out: str = LIB, sources=None) -> list:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    return [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", out, *(sources or SOURCES)]


def _build_one(lib: str, sources, verbose: bool) -> str:
    tmp = lib + ".tmp"
    res = subprocess.run(command(tmp, sources), capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(res.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Builds both libraries; returns the path of the GDN library."""
    _build_one(PEAKS_LIB, PEAKS_SOURCES, verbose)
    return _build_one(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))

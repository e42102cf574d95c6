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
           os.path.join(CSRC, "gdn_attention.hip"), os.path.join(CSRC, "gdn_lowp.hip"), os.path.join(CSRC, "gdn_api.cpp")]
PEAKS_LIB = os.path.join(PKG, "libgdn_peaks.so")
PEAKS_SOURCES = [os.path.join(CSRC, "gdn_peaks.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
# MFMA results and accumulators in ordinary VGPRs: the scan scales and converts its accumulators every step,
# which with accumulation registers costs a copy per value.  Not for the FP8 GEMM, whose 144 accumulators per
# wavefront live in the accumulation registers (one wavefront per SIMD, 512 registers).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
NO_VGPR_FORM = {"gdn_lowp.hip"}


def _flags(src: str) -> list:
    return HIPCC_FLAGS + ([] if os.path.basename(src) in NO_VGPR_FORM else VGPR_FORM)


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def command(out: str = LIB, sources=None) -> list:
    """The link command of a library from its sources' objects (object of s: out + '.' + basename(s) + '.o')."""
    objs = [out + "." + os.path.basename(s) + ".o" for s in (sources or SOURCES)]
    return [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out, *objs]


def _build_one(lib: str, sources, verbose: bool) -> str:
    tmp = lib + ".tmp"
    procs = []
    for src in sources:
        obj = tmp + "." + os.path.basename(src) + ".o"
        cmd = [_hipcc(), *_flags(src), "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    errors, objs = [], []
    for src, obj, p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            errors.append(f"{src}:\n{out}{err}")
        elif verbose:
            print(err)
        objs.append(obj)
    try:
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        res = subprocess.run(command(tmp, sources), capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + res.stdout + res.stderr)
        os.replace(tmp, lib)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return lib


def build(verbose: bool = False) -> str:
    """Builds both libraries; returns the path of the GDN library."""
    _build_one(PEAKS_LIB, PEAKS_SOURCES, verbose)
    return _build_one(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))

"""Builds libcpattn.so (the gfx950 HIP kernels plus the C ABI) in-tree with hipcc.

Usage: python -m context_long_sequence_amd.build [--report]
  --report  also prints hipcc's per-kernel register / LDS / spill report.
"""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libcpattn.so")
ARCH = "gfx950"

HIP_SOURCES = ["partial_fwd.hip", "partial_bwd.hip", "partial_bwd_f32.hip", "merge_lse.hip"]
HOST_SOURCES = ["api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall"]
# Packed fp32 VALU ops are kept out of the device code on purpose.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def build(report=False, verbose=False):
    cc = hipcc()
    with tempfile.TemporaryDirectory() as tmp:
        objs = []
        for src in HIP_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc, *COMMON, *DEVICE, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
            if report:
                cmd.append("-Rpass-analysis=kernel-resource-usage")
            _run(cmd, verbose or report)
            objs.append(obj)
        for src in HOST_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            _run([cc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        tmp_lib = LIB + ".tmp"
        _run([cc, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp_lib], verbose)
        os.replace(tmp_lib, LIB)
    return LIB


def _run(cmd, show):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), out))
    if show and out:
        print(out)


if __name__ == "__main__":
    print(build(report="--report" in sys.argv, verbose="-v" in sys.argv))

"""Build libspecverify.so (host C ABI + gfx950 HIP kernels) in place.

    python -m lossless_draft_verification_verify_amd.build

Always recompiles.  Uses hipcc from ROCM_PATH (default /opt/rocm).
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libspecverify.so")
SOURCES = ["capi.cpp", "verify_kernels.hip", "schedule_kernel.hip", "acceptance_kernel.hip",
           "calibration_kernel.hip", "noalloc.hip"]
ARCH = "gfx950"

# -ffp-contract=off: every fp expression is evaluated as written (the final
# draw re-scan must reproduce the tile masses bit for bit).
# packed fp32 ops are disabled for all device code.
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    f"--offload-arch={ARCH}", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    if os.path.exists(path):
        return path
    found = shutil.which("hipcc")
    if not found:
        raise RuntimeError("hipcc not found; set ROCM_PATH")
    return found


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [l for l in proc.stdout.splitlines() if "is not a recognized feature for this target" not in l]
    if proc.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    out = "\n".join(l for l in lines if l.strip() and "(ignoring feature)" not in l)
    if out:
        sys.stderr.write(out + "\n")


def build(verbose=False):
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        _run(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

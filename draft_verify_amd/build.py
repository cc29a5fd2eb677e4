"""Compile libspecv.so (gfx950 HIP kernels + host runtime + proposer) in-tree.

    python -m draft_verify_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Packed fp32 instructions are
disabled in device code (-packed-fp32-ops); the host pass warns that it does
not know the feature, which is harmless.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspecv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["kernels.hip", "runtime.hip", "ngram.cpp", "governor.cpp"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
         "-Wno-unused-command-line-argument"]


def build(out: str = LIB, extra=()) -> str:
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libspecv")
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS, *extra, *srcs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())

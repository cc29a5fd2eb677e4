"""Build the CPU oracle (test infrastructure only) with gcc.

    python oracle/build.py            -> oracle/liboracle.so
    build(plant=k, out=path)          -> a copy with deliberate mistake k,
                                         used by the tests that check the
                                         oracle's pins catch mistakes.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# x86-64-v3 (AVX2) runs on every host this is used on; no -ffast-math and no
# FMA contraction, so every sum keeps the order written in the source.
CFLAGS = ["-O3", "-march=x86-64-v3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-fvisibility=hidden", "-std=c11", "-Wall"]


def build(plant: int = 0, out: str = LIB) -> str:
    cmd = ["gcc", *CFLAGS, f"-DORC_PLANT={int(plant)}", SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else 0))

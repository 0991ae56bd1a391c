"""Compiles the C oracle (oracle/dspark_ref.c) into oracle/_lib/libdspark_ref.so.

Test infrastructure only: called by the entry script's build() so that the
checker is compiled with everything else (building it is not using it).  Plain
IEEE fp64/fp32 arithmetic: no fast-math, no fused multiply-add contraction.
"""

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dspark_ref.c")
LIB = os.path.join(HERE, "_lib", "libdspark_ref.so")
FLAGS = ["-O3", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall"]


def build() -> str:
    cc = os.environ.get("CC") or shutil.which("gcc") or "cc"
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    tmp = LIB + ".tmp"
    res = subprocess.run([cc, *FLAGS, SRC, "-o", tmp, "-lm"], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C oracle build failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())

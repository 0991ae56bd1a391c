"""Build step of tests/c/abi_round.c: a plain C program that runs one round
through the library's C ABI with HIP runtime buffers (the entry script's
build() calls this after building the library).  The program links against the
in-tree libdspark.so (found through an rpath relative to the binary) and the
HIP runtime."""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN_DIR = os.path.join(HERE, "_bin")
BIN = os.path.join(BIN_DIR, "abi_round")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    os.makedirs(BIN_DIR, exist_ok=True)
    cc = shutil.which("gcc") or "cc"
    lib_dir = os.path.join(ROOT, "lossless_rejection_sampling_amd", "_lib")
    rel = os.path.relpath(lib_dir, BIN_DIR)
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "abi_round.c"), "-o", BIN + ".tmp",
           "-L", lib_dir, "-ldspark", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,$ORIGIN/{rel}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"building {BIN} failed:\n{res.stdout}\n{res.stderr}")
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build())

"""Compile tests/c_client/lcv_client (a plain C program using include/lcv_bsa.h) with gcc
against the in-tree liblcv_bsa.so and ROCm's HIP runtime."""
from __future__ import annotations

import shutil
import subprocess
from pathlib import Path

HERE = Path(__file__).resolve().parent
ROOT = HERE.parent.parent
PKG = ROOT / "block_sparse_attention_lcv_amd"
CLIENT = HERE / "lcv_client"
ROCM = Path("/opt/rocm")


def build() -> Path:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler (gcc) found")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROOT / 'include'}", f"-I{ROCM / 'include'}", str(HERE / "lcv_client.c"),
           f"-L{PKG}", "-llcv_bsa", f"-L{ROCM / 'lib'}", "-lamdhip64",
           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{ROCM / 'lib'}", "-o", str(CLIENT)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C client build failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    return CLIENT


if __name__ == "__main__":
    print(build())

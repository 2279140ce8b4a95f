"""Compile liblcv_bsa.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB_NAME = "liblcv_bsa.so"
LIB_PATH = PKG / LIB_NAME

SOURCES = ["lcv_bsa_host.cpp", "layout_kernels.hip", "rope3d_kernel.hip", "qk_prologue_kernel.hip",
           "bsa_fwd_kernel.hip", "bsa_bwd_kernel.hip", "attn_merge_kernel.hip",
           "qk_prologue_bwd_kernel.hip"]

# Packed-fp32 VALU forms are kept out of the generated code; the host pass ignores the flag.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblcv_bsa)")


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> Path:
    """Compile every source into LIB_PATH (always recompiles)."""
    tmp = LIB_PATH.with_suffix(".so.tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{ROOT / 'include'}", f"-I{CSRC}",
           *[str(CSRC / s) for s in SOURCES], "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l or "error" in l.lower())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))

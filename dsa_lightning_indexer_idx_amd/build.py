"""Build libdsaidx.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc.

    python -m dsa_lightning_indexer_idx_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libdsaidx.so"
OBJ = PKG / "_build"

SOURCES = ["api.cpp", "scan.hip", "prefill.hip", "topk.hip", "cand.hip", "attn.hip", "kcache.hip", "probe.hip", "noalloc.hip"]

# Device code never uses packed-fp32 instructions (the flag is a device-target
# feature; the host pass only warns that it does not know it). MFMA results stay in
# VGPRs: the epilogue reads every accumulator, and AGPR results would each cost a
# v_accvgpr_read.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdsaidx.so)")


def _compile(src: str) -> Path:
    OBJ.mkdir(exist_ok=True)
    out = OBJ / (src + ".o")
    cmd = [hipcc(), *FLAGS, "-c", str(CSRC / src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False) -> Path:
    """Compile every source for gfx950 and link libdsaidx.so; always rebuilds."""
    srcs = [s for s in SOURCES if (CSRC / s).exists()]
    with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB.with_suffix(f".so.tmp{os.getpid()}")
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

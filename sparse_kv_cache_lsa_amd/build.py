"""Build liblsa.so (gfx950) in-tree with hipcc.

    python -m sparse_kv_cache_lsa_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "liblsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["lsa_api.cpp", "lsa_score.hip", "lsa_select.hip", "lsa_select_masks.hip", "lsa_topk.hip",
           "lsa_gather.hip", "lsa_attention.hip", "lsa_lightning.hip", "lsa_fetch.hip", "lsa_project.hip", "lsa_labels.hip", "lsa_focal.hip"]

# Packed fp32 VALU ops are switched off for every HIP translation unit.  MFMA
# results are kept in ordinary VGPRs (not AGPRs), so fused epilogues read the
# accumulators without v_accvgpr_read copies.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-command-line-argument",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    out = os.path.join(OBJ, src + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", path, "-o", out]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + [f for f in FLAGS if f != "--offload-arch=gfx950"] + ["-c", path, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = int(os.environ.get("MAX_JOBS", "8"))
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

"""Build libvt.so in-tree: every HIP source compiled for gfx950 with hipcc.

Usage: ``python -m vision_transformer_encoder_tiled_amd.build`` (or
``__graft_entry__.build()``).  Objects go to ``_build/`` at the repository
root; the shared library lands next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libvt.so")
OBJ = os.path.join(ROOT, "_build")
SOURCES = ["meta.hip", "permute.hip", "layernorm.hip", "gemm.hip", "attention.hip", "attention_bwd.hip",
           "backward.hip", "clock.hip", "vt_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 instructions are disabled: the compiler would otherwise form
# v_pk_* fp32 ops from ordinary float code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


# Per-file flags.  The attention kernels (forward and backward) keep their
# MFMA accumulators in ordinary VGPRs (their working sets fit in 256, which
# allows two wavefronts per SIMD), avoiding AGPR<->VGPR copies around the
# softmax; the GEMM needs the AGPR file for its 256 accumulators.
EXTRA = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "attention_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, obj_dir: str, host_flags) -> str:
    obj = os.path.join(obj_dir, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *host_flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = OUT, obj_dir: str = OBJ, host_flags=()) -> str:
    """Compile and link the library.  ``host_flags`` go to every compile and
    the link (host-side options only, each behind -Xarch_host), e.g. the
    host-sanitizer build of the CPU tests; ``out`` / ``obj_dir`` place such a
    variant outside the package."""
    os.makedirs(obj_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, obj_dir, host_flags), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *host_flags, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

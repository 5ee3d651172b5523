"""Build libpaged_attn.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m paged_kv_cache_89_amd._build

compiles every source under csrc/ into _build/ (in parallel) and links
paged_kv_cache_89_amd/libpaged_attn.so.  A GPU is not needed to build.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpaged_attn.so")
ARCH = "gfx950"

MFMA_SOURCES = ["decode_gqa_d64_nt.hip", "decode_gqa_d64_t.hip", "decode_gqa_d128_nt.hip",
                "decode_gqa_d128_t.hip"]
SOURCES = ["api.hip", "validate.hip", "block_manager.cpp", "write_kv.hip", "merge.hip", "copy_blocks.hip",
           "decode_d64_nt.hip", "decode_d64_t.hip", "decode_d128_nt.hip", "decode_d128_t.hip",
           "decode_gqa.hip", "decode_cascade.hip", *MFMA_SOURCES]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}",
         # keep hipcc from emitting packed fp32 arithmetic (v_pk_*_f32)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


# Per-source extra flags.  The matrix-core kernels keep their MFMA accumulators in
# ordinary VGPRs (no AGPR round trips around the loop's rarely taken rescale branch).
EXTRA = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form=1"] for src in [*MFMA_SOURCES, "decode_cascade.hip"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else None))

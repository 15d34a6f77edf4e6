"""Build libgdn.so (the C ABI and its gfx950 HIP kernels) in-tree with hipcc.

Usage: python -m gated_delta_rule_56_amd.build  (or call build()).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libgdn.so")
ARCH = "gfx950"

SOURCES = ["gdn_abi.cpp", "gdn_decode.hip", "gdn_prefill_f32.hip",
           "gdn_prefill_chunk.hip", "gdn_prefill_scan.hip", "gdn_norm.hip",
           "gdn_prologue.hip", "gdn_varlen.hip", "gdn_kda.hip", "gdn_prefill_seg.hip", "gdn_static.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-mcode-object-version=5",
    # packed fp32 ops stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (no accvgpr copies around VALU work)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libgdn.so")
    return path


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *HIPCC_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")


def build(output: str = LIBRARY, jobs: int = 4) -> str:
    """Compile every source for gfx950 and link libgdn.so (always rebuilds)."""
    with tempfile.TemporaryDirectory(prefix="gdn_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(_compile, SOURCES, objs))
        tmp_out = output + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_out, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp_out, output)
    return output


if __name__ == "__main__":
    print(build(jobs=int(sys.argv[1]) if len(sys.argv) > 1 else 4))

"""Build liblora_nf4.so (gfx950) in-tree with hipcc.

    python -m qlora_linear_amd.build        # or qlora_linear_amd.build.build()

Compiles every csrc/*.hip to an object under qlora_linear_amd/_build/ and links
qlora_linear_amd/liblora_nf4.so. Always recompiles (the build check must build).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblora_nf4.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are disabled for all device code; denormals are kept
# (the NF4 dequantization must round exactly like IEEE float32).
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-file additions. The register-dequantizing tiles are scheduled for the most
# instruction-level parallelism (the AMDGPU backend's max-ilp strategy, an option
# of that backend only, so the host pass ignores it): measured on MI355X at q_proj,
# 8192 tokens, forward 283 -> 277 us, dX 0.6 % faster, the same bits.
FILE_FLAGS = {
    "lora_rw.hip": ["-mllvm", "--amdgpu-sched-strategy=max-ilp"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stdout}\n{p.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = min(len(srcs), max(1, (os.cpu_count() or 2) // 2), 8)
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)

"""Build libfp8dq.so (HIP for gfx950) in-tree.

Usage: python -m fp8_dynamic_quantized_amd.build  (or build() from Python).
Every HIP source under csrc/ is compiled with hipcc for gfx950 into
_build/, then linked into fp8_dynamic_quantized_amd/libfp8dq.so.
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
LIB = os.path.join(PKG, "libfp8dq.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    "-I", INCLUDE, "-I", CSRC,
    # correctly rounded fp32 division (the scale amax / 448 is bit-exact)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep fp32 denormals (subnormal scales and inputs are exact values)
    "-fno-gpu-flush-denormals-to-zero",
    # no packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _sources():
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    return [os.path.join(CSRC, f) for f in srcs]


# Per-source flags. gemm_block.hip: keep MFMA accumulators in ordinary VGPRs
# (the block kernel rescales its accumulator every 128 K columns).
PER_SOURCE = {
    "gemm_block.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    extra = PER_SOURCE.get(os.path.basename(src), [])
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every source and link `out` (default: the in-tree library)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = _sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
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

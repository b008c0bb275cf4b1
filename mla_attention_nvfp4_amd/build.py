"""Build libmla_nvfp4.so from csrc/*.hip with hipcc for gfx950.

Run ``python -m mla_attention_nvfp4_amd.build`` (or call ``build()``).  The
library is written next to this file; object files go to ``_build/``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla_nvfp4.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # one IEEE fp32 operation per quantization step: no contraction,
    # correctly rounded division
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-source extra flags.  decode kernels: MFMA accumulators in VGPRs, so the
# (rare) softmax rescale of the output accumulators needs no AGPR round trip
# and the loop-carried accumulators are not copied between register files.
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "decode_narrow.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "decode_qdq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         # MFMA rate loops: with AGPR accumulators the compiler copies the
         # loop-carried accumulators between register files every iteration,
         # which would time the copies instead of the products
         "roofline.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         # prefill: inputs are finite, so the max reductions of the softmax and
         # the P blocks need no NaN canonicalization (about 12% of the
         # attention loop's VALU instructions)
         "prefill.hip": ["-fno-honor-nans"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

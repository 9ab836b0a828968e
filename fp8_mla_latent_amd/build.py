"""Build libmla8.so (HIP, gfx950) in-tree with hipcc.

    python -m fp8_mla_latent_amd.build

Flags:
  * --offload-arch=gfx950 only: the kernels use CDNA4 instructions
    (v_mfma_f32_16x16x32_f16, v_mfma_scale_f32_16x16x128_f8f6f4,
    v_cvt_scalef32_pk_f16_fp8).
  * -fhip-fp32-correctly-rounded-divide-sqrt and no fast-math: the quantizer's
    amax/448 and 448/amax must be IEEE quotients for bit-exact scales and codes.
  * -Xclang -target-feature -Xclang -packed-fp32-ops: keep the compiler from
    forming packed-fp32 VALU instructions.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = [os.path.join(PKG, "csrc", f) for f in ("mla8_kernels.hip", "mla8_partial32.hip",
                                                   "mla8_index.hip", "mla8_kvfile.hip",
                                                   "mla8_api.hip")]
LIB = os.path.join(PKG, "libmla8.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", os.path.join(PKG, "csrc"),
]


def hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla8)")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libmla8.so")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

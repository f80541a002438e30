"""Build libmla.so (the HIP library behind include/mla.h) for gfx950 in-tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libmla.so")
SOURCES = ["mla_api.hip", "kernels_mfma.hip", "kernels_unabsorbed.hip", "kernels_decode.hip", "kernels_simt.hip",
           "profile.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in any kernel.
# -fno-honor-nans: max/min need not quiet signalling NaNs, so fmaxf is one
# v_max_f32 instead of two canonicalising ops plus the max (the softmax
# compares against +-infinity only; a NaN input gives a non-finite output).
# -amdgpu-mfma-vgpr-form: matrix instructions written with the builtins keep
# their accumulators in VGPRs; the flash kernels pin their large output
# accumulators to AGPRs explicitly (inline asm), so the two never compete.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=true", "-fno-honor-nans",
         "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    tmp = SO + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, *srcs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stderr[-8000:])
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libsage_attn.so for gfx950 with hipcc, in-tree.

    python -m bit_quantized_attention_sage_amd.build

Every translation unit is compiled with packed-FP32 instructions disabled;
the quantize and W8A8 units additionally with floating-point contraction off,
so each of their operations rounds exactly as written.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsage_attn.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]
UNITS = {
    "quant.hip": ["-ffp-contract=off"],
    "attn.hip": [],
    # int32 MFMA results are read by the VALU every K block: keep them in VGPRs
    "w8a8.hip": ["-ffp-contract=off", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "api.cpp": ["-x", "hip"],
}


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src, extra in UNITS.items():
        obj = os.path.join(BUILD, src.replace(".", "_") + ".o")
        cmd = [HIPCC] + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libqblk.so (the C-ABI library with the gfx950 kernels) in-tree.

    python bit_block_quant_amd/build.py [-v]     (by path: importing the package
                                                 loads the library it builds)

hipcc cross-compiles for gfx950 without a GPU present.  Flags:
  -ffp-contract=off            no implicit fused multiply-add: dequantized
                               weights must be the separately rounded products
  -fhip-fp32-correctly-rounded-divide-sqrt
                               IEEE fp32 division (quantizer codes)
  -fno-gpu-flush-denormals-to-zero
                               keep fp32 denormals (fp16 denormals are kept by
                               the default mode; super-scales can be subnormal)
  -packed-fp32-ops (disabled)  no packed-fp32 instructions in generated code
  -amdgpu-mfma-vgpr-form       MFMA results written to VGPRs, not AGPRs
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqblk.so")
SOURCES = ["qblk_abi.hip", "qblk_quant.hip", "qblk_gemv.hip", "qblk_gemm.hip", "qblk_w4a8.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs (the GEMM scales every partial product on the VALU)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.isabs(c) and os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [hipcc(), *FLAGS, *extra, *srcs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

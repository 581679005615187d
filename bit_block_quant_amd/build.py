"""Build libqblk.so (the C-ABI library with the gfx950 kernels) in-tree, and
libqblk_hbmref.so (bench.py's plain-read and empty-kernel references, kept
out of libqblk).

    python bit_block_quant_amd/build.py [-v]     (by path: importing the package
                                                 loads the library it builds)

hipcc cross-compiles for gfx950 without a GPU present.  Each source is
compiled to its own object (in parallel), then linked.  Flags:
  -ffp-contract=off            no implicit fused multiply-add: dequantized
                               weights must be the separately rounded products
  -fhip-fp32-correctly-rounded-divide-sqrt
                               IEEE fp32 division (quantizer codes)
  -fno-gpu-flush-denormals-to-zero
                               keep fp32 denormals (fp16 denormals are kept by
                               the default mode; super-scales can be subnormal)
  -packed-fp32-ops (disabled)  no packed-fp32 instructions in generated code
                               (the host pass prints that it does not know the
                               feature; that line is not a warning of the code)
  -amdgpu-mfma-vgpr-form       MFMA results written to VGPRs, not AGPRs
  -Wall -Werror                every diagnostic of the sources is an error
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqblk.so")
HBMREF_LIB = os.path.join(HERE, "libqblk_hbmref.so")
SOURCES = ["qblk_abi.hip", "qblk_quant.hip", "qblk_gemv.hip", "qblk_gemm.hip", "qblk_w4a8.hip"]
HBMREF_SOURCES = ["hbm_read.hip"]
ARCH = "gfx950"
OBJ_DIR = os.path.join(HERE, "_build")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs (the GEMM scales every partial product on the VALU)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # Kernel arguments preloaded into SGPRs at wave launch (gfx950): a kernel
    # starts without the memory round trip for its pointers, which the batch-1
    # products otherwise pay before x can even be requested (11008 x 4096
    # Type 0: 6.93 -> 6.37-6.50 us).  The code object keeps a prologue that
    # loads them the ordinary way where the hardware does not preload.
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-function", "-Werror",
]


def hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.isabs(c) and os.path.exists(c):
            return c
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass names the disabled packed-fp32 feature it does not know; nothing else is expected
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if out.strip():
        print(out, flush=True)
    if r.returncode != 0:
        raise subprocess.CalledProcessError(r.returncode, cmd)


def _link(sources, lib, extra, verbose, jobs):
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in sources]
    cmds = [[hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(sources, objs)]
    with ThreadPoolExecutor(max(1, min(jobs, len(cmds)))) as pool:
        list(pool.map(lambda c: _run(c, verbose), cmds))
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", lib + ".tmp"], verbose)
    os.replace(lib + ".tmp", lib)
    return lib


def build(verbose: bool = False, extra=()) -> str:
    extra = list(extra)
    jobs = int(os.environ.get("MAX_JOBS", "8"))
    _link(HBMREF_SOURCES, HBMREF_LIB, extra, verbose, jobs)
    return _link(SOURCES, LIB, extra, verbose, jobs)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libtpshard.so in-tree with hipcc for gfx950.

    python -m tensor_transformer_layer_mlp_amd.build [-v]

Each HIP source compiles to an object under _build/ (in parallel), then one shared library is
linked next to this file.  Packed fp32 instructions are disabled for the device code.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtpshard.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["abi.hip", "prof.hip", "dispatch.hip", "gemm_generic.hip", "gemm_bf16.hip", "reduce.hip",
           "attention_generic.hip", "attention_mfma.hip", "grouped.hip", "layernorm.hip", "moe.hip", "fp8.hip"]

CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]
# The attention kernels rescale and read their MFMA results with vector ops every block: MFMA results
# in ordinary VGPRs (not accumulation registers) save the copies between the two register files.
EXTRA = {"attention_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in srcs]
    cmds = [[HIPCC, *CFLAGS, *EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

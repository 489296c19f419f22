"""Build libtpshard.so in-tree with hipcc for gfx950.

    python -m tensor_transformer_layer_mlp_amd.build [-v] [--sanitize]

Each HIP source compiles to an object under _build/ (in parallel), then one shared library is
linked next to this file.  Packed fp32 instructions are disabled for the device code.

--sanitize builds libtpshard_san.so under _build_san/ instead: the host code instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer (device code unchanged, not sanitized), for the
CPU-side tests of argument validation.  Load it with TPSHARD_LIB pointing at it and the ASan
runtime preloaded (see sanitizer_env()).
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


# host-only sanitizers: each -fsanitize= applies to the host compilation alone
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined", "-g"]
SAN_LIB = os.path.join(PKG, "libtpshard_san.so")
SAN_BUILD_DIR = os.path.join(ROOT, "_build_san")


def build(verbose: bool = False, jobs: int = 8, sanitize: bool = False) -> str:
    bdir, lib = (SAN_BUILD_DIR, SAN_LIB) if sanitize else (BUILD_DIR, LIB)
    extra = SAN_FLAGS if sanitize else []
    os.makedirs(bdir, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objs = [os.path.join(bdir, s.replace(".hip", ".o")) for s in srcs]
    cmds = [[HIPCC, *CFLAGS, *EXTRA.get(s, []), *extra, "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = lib + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-shared-libsan"] if sanitize else []
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *link_extra, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


def sanitizer_env() -> dict:
    """Environment for a CPU-only process that loads the sanitized library: the ASan runtime
    preloaded (the Python interpreter itself is not instrumented), leak checking off (the
    interpreter's own allocations), and TPSHARD_LIB naming the sanitized build."""
    rt = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", TPSHARD_LIB=SAN_LIB)
    return env


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))

"""Compile the decode library (HIP for gfx950 + C++ host code) into
decode_megakernel_02_amd/libmk.so with hipcc.  Cross-compiles without a GPU."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmk.so")
ARCH = "gfx950"

# Packed-FP32 instructions are kept out of all device code.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass of hipcc does not know the packed-fp32 feature: harmless, filtered
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if out.strip() and (verbose or r.returncode):
        print(out, file=sys.stderr)
    if r.returncode:
        raise RuntimeError("build step failed: " + " ".join(cmd))


def build(verbose: bool = False) -> str:
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD, exist_ok=True)
    # (source, extra flags, object): the step kernels are built twice, for batch-1 handles and
    # for handles with several batch rows
    units = [("mk_kernels.hip", [], "mk_kernels.hip.o"),
             ("mk_kernels.hip", ["-DMK_BATCHED_TU=1"], "mk_kernels_batched.hip.o"),
             ("mk_prefill.hip", [], "mk_prefill.hip.o"), ("mk_api.cpp", ["-x", "hip"], "mk_api.cpp.o"),
             ("mk_plan.cpp", ["-x", "hip"], "mk_plan.cpp.o")]
    objs = [os.path.join(BUILD, obj) for _, _, obj in units]
    # the translation units are independent: compile them side by side
    with ThreadPoolExecutor(len(units)) as ex:
        for f in [ex.submit(_run, ["hipcc"] + HIP_FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
                  for (src, extra, _), obj in zip(units, objs)]:
            f.result()
    tmp = LIB + ".tmp"
    _run(["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

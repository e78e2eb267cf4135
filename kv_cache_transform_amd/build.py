"""Build libkvtc.so in-tree: hipcc for the gfx950 kernels and the host core,
g++ for the fp64 linear algebra, linked with zlib."""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvtc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division and square root (the quantizer divides)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-ffp-contract=on",
    # MFMA results in VGPRs (no AGPR round trips in the epilogues)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ...")


# gfx950 kernel translation units (compiled in parallel)
HIP_SOURCES = ["kvtc_encode.hip", "kvtc_decode.hip", "kvtc_lossless.hip"]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    steps = []
    for src in HIP_SOURCES:
        o = os.path.join(BUILD, src.replace(".hip", ".o"))
        steps.append((o, [HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", o]))
    o = os.path.join(BUILD, "kvtc_host.o")
    steps.append((o, [HIPCC, "-O3", "-std=c++17", "-fPIC", *inc, "-c",
                      os.path.join(CSRC, "kvtc_host.cpp"), "-o", o]))
    o = os.path.join(BUILD, "kvtc_linalg.o")
    steps.append((o, ["g++", "-O3", "-march=x86-64-v3", "-std=c++17", "-fPIC", *inc, "-c",
                      os.path.join(CSRC, "kvtc_linalg.cpp"), "-o", o]))
    with concurrent.futures.ThreadPoolExecutor(len(steps)) as ex:
        for f in [ex.submit(_run, cmd, verbose) for _, cmd in steps]:
            f.result()
    objs = [o for o, _ in steps]
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, "-lz", "-lpthread"],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libmxattn.so (HIP kernels + C ABI) for gfx950 with hipcc, in place.

    python -m mxfp4_quantized_attention_amd.build

Each source compiles to its own object (in parallel), then one shared library
is linked next to this file.  Packed-FP32 instruction forms are disabled for
all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxattn.so")
SOURCES = ["abi.hip", "quantize.hip", "attention.hip", "gemm.hip", "noalloc.hip"]
# The instruction-cost probe behind the attention kernel's vector-unit ceiling
# (bench.py --workload valu_probe): a library of its own, not part of the path.
PROBE_SOURCES = ["probe.hip"]
PROBE_LIB = os.path.join(HERE, "libmxprobe.so")
# The attention kernel never sees a NaN (inputs are finite by contract and the
# running max starts at -inf, never inf - inf); without NaNs the compiler drops
# the canonicalizing moves it otherwise puts in front of every fmaxf.
PER_FILE_FLAGS = {"attention.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fno-gpu-rdc",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *flags(), *PER_FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                         if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES) + len(PROBE_SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))
    link(objs[:len(SOURCES)], LIB)
    link(objs[len(SOURCES):], PROBE_LIB)
    build_abi_demo(objdir)
    return LIB


def link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-fno-gpu-rdc", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)


DEMO_SRC = os.path.join(ROOT, "tests", "abi_demo.c")
DEMO = os.path.join(HERE, "_build", "abi_demo")


def build_abi_demo(objdir: str) -> str:
    """The plain C consumer of the library (tests/abi_demo.c): gcc, C99, HIP
    runtime for memory and a stream, linked against libmxattn.so."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
           "-I", os.path.join(ROOT, "include"), DEMO_SRC, "-o", DEMO,
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-L", HERE, "-lmxattn", "-Wl,-rpath,$ORIGIN/.."]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("abi_demo build failed:\n" + r.stdout + r.stderr)
    return DEMO


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""The C ABI's host code under AddressSanitizer and UBSan.

abi.hip and noalloc.hip hold all of the library's host logic: argument and
size checks, workspace carving, the varlen and strided bookkeeping, and
mxq_dump's file writer.  They are compiled a second time with the host half
instrumented (-Xarch_host -fsanitize=address,undefined, every report fatal;
the device code is built as usual), linked with the other objects into a
scratch library, and a subprocess runs the host ABI tests against that build
(tests/conftest.py loads the library named by MXATTN_TEST_LIB).  Those tests
exercise every argument error path and a dump from host memory; an
out-of-bounds access, use after free or undefined operation on any of them
ends the subprocess with a sanitizer report, which fails this test.  CPU only:
nothing is launched.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from mxfp4_quantized_attention_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SOURCES = ["abi.hip", "noalloc.hip"]
SAN_HOST = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
            "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _rocm_llvm():
    return os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hip_build.hipcc()))), "llvm")


def _asan_runtime():
    hits = sorted(glob.glob(os.path.join(_rocm_llvm(), "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def _build_sanitized(out_dir):
    def compile_one(src):
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        extra = SAN_HOST if src in HOST_SOURCES else []
        cmd = [hip_build.hipcc(), *hip_build.flags(), *hip_build.PER_FILE_FLAGS.get(src, []), *extra,
               "-c", os.path.join(hip_build.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"hipcc failed for {src}:\n{r.stdout}{r.stderr}"
        return obj

    with ThreadPoolExecutor(max_workers=len(hip_build.SOURCES)) as ex:
        objs = list(ex.map(compile_one, hip_build.SOURCES))
    lib = os.path.join(out_dir, "libmxattn_san.so")
    rocm_lib = os.path.join(os.path.dirname(_rocm_llvm()), "lib")
    # the host objects are ordinary ELF objects with the device code embedded,
    # so the sanitizer-aware clang driver links them; the runtime is preloaded
    cmd = [os.path.join(_rocm_llvm(), "bin", "clang++"), "-shared", "-fsanitize=address,undefined",
           "-shared-libasan", *objs, "-L", rocm_lib, "-lamdhip64", "-Wl,-rpath," + rocm_lib, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "link failed:\n" + r.stdout + r.stderr
    return lib


def test_abi_host_paths_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists(hip_build.hipcc()):
        pytest.skip("ROCm clang sanitizer runtime or hipcc not installed")
    lib = _build_sanitized(str(tmp_path))
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join(p for p in (rt, env.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["MXATTN_TEST_LIB"] = lib
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           "tests/test_abi_host.py"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]

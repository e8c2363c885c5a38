"""Builds for the CPU sanitizer checks (test infrastructure; nothing here
runs on a GPU):

  * oracle.c with gcc's AddressSanitizer and UndefinedBehaviorSanitizer;
  * libgradcomp with both sanitizers on its host code only (every device
    code object is compiled exactly as in the product build);
  * the C driver of libgradcomp's host entry points (abi_host_checks.c),
    built with the same sanitizers and linked to that library.

Every build goes to a caller-given directory, never over the product's
libraries."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

from gradient_compression_dnn_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
ORACLE_FLAGS = ["-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
                "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                "-fno-omit-frame-pointer"]
# host-only sanitizer flags for hipcc: each one behind -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all",
            "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def gcc_runtime(name: str) -> str:
    """Path of a gcc runtime library (libasan.so, libubsan.so)."""
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True, check=True)
    return r.stdout.strip()


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd[:3])} ... failed:\n{r.stdout}\n{r.stderr}")


def build_oracle(out_dir: str) -> str:
    out = os.path.join(out_dir, "liboracle_san.so")
    _run(["gcc", *ORACLE_FLAGS, "-o", out, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    return out


def build_host_library(out_dir: str) -> str:
    """libgradcomp.so in out_dir, host code under ASan and UBSan."""
    srcs = sorted(glob.glob(os.path.join(hip_build.CSRC, "*.hip")))

    def one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        _run([hip_build.HIPCC, *hip_build.FLAGS, *HOST_SAN, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        objs = list(ex.map(one, srcs))
    lib = os.path.join(out_dir, "libgradcomp.so")
    _run([hip_build.HIPCC, "-shared", f"--offload-arch={hip_build.ARCH}", "-fPIC", "-o", lib, *objs])
    return lib


def build_driver(out_dir: str, libdir: str) -> str:
    exe = os.path.join(out_dir, "abi_host_checks")
    _run([CLANG, "-std=c99", "-g", "-Wall", "-Werror", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
          os.path.join(ROOT, "tests", "abi_host_checks.c"), "-o", exe,
          "-L", libdir, "-lgradcomp", f"-Wl,-rpath,{libdir}"])
    return exe

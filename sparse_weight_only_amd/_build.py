"""Build the in-tree C-ABI library ``_lib/libsgemv.so`` for gfx950.

Host sources (packer, layout) are compiled by g++ with -ffp-contract=off so
every FP64 operation of the packer is rounded on its own; the HIP source is
compiled by hipcc for gfx950 with packed-FP32 instructions disabled; hipcc
links the shared library against the HIP runtime.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libsgemv.so")
HOST_SRCS = ["host_pack.cpp", "host_layout.cpp"]
HIP_SRCS = ["sgemv_k_nk1.hip", "sgemv_k_nk2.hip", "sgemv_k_nk4.hip", "sgemv_k_f16.hip", "sgemv_k_rb.hip", "sgemv_launch.hip",
            "sgemv_probe.hip", "sgemv_k_list.hip"]


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the SparseGemv library needs ROCm's hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + out)
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, arch: str = "gfx950") -> str:
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(OUT_DIR, exist_ok=True)
    bdir = os.path.join(OUT_DIR, "obj")
    os.makedirs(bdir, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for s in HOST_SRCS:
        o = os.path.join(bdir, s + ".o")
        jobs.append((o, ["g++", "-std=c++17", "-O2", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
                         "-Wall", "-Wextra", "-c", os.path.join(CSRC, s), "-o", o]))
    for s in HIP_SRCS:
        o = os.path.join(bdir, s + ".o")
        jobs.append((o, [hipcc, f"--offload-arch={arch}", "-std=c++17", "-O3", "-fPIC",
                         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                         "-mllvm", "-amdgpu-kernarg-preload-count=16",
                         "-Wall", "-Wno-pass-failed", "-c", os.path.join(CSRC, s), "-o", o]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, cmd, verbose) for _, cmd in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "-o", tmp] + [o for o, _ in jobs], verbose)
    os.replace(tmp, LIB)
    build_c_driver(verbose)
    from . import _build_san
    _build_san.build_host_sanitized(verbose)
    return LIB


# The tests' plain-C driver of the library (tests/c_abi/sgemv_c_driver.c):
# built here, beside the library, so that no test compiles anything. Strict
# C99 against include/sgemv.h; the HIP runtime's C API for device memory.
REPO = os.path.dirname(HERE)
C_DRIVER_SRC = os.path.join(REPO, "tests", "c_abi", "sgemv_c_driver.c")
C_DRIVER = os.path.join(REPO, "tests", "c_abi", "_build", "sgemv_c_driver")


def build_c_driver(verbose: bool = False) -> str:
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(_hipcc())))
    os.makedirs(os.path.dirname(C_DRIVER), exist_ok=True)
    rel_lib = os.path.relpath(OUT_DIR, os.path.dirname(C_DRIVER))
    tmp = C_DRIVER + ".tmp"
    _run(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(REPO, "include"), "-isystem", os.path.join(rocm, "include"), C_DRIVER_SRC,
          "-L", OUT_DIR, "-lsgemv", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
          "-Wl,-rpath,$ORIGIN/" + rel_lib, "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", tmp], verbose)
    os.replace(tmp, C_DRIVER)
    return C_DRIVER


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

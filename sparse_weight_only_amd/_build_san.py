"""Host-only build of the packer and layout (no HIP code) with the address
and undefined-behaviour sanitizers, for the CPU tests.

The tests load it through the SGEMV_LIB variable in a child process whose
LD_PRELOAD starts with the address-sanitizer runtime; any report aborts that
process. The GPU code is never built this way.
"""
import os
import subprocess

from ._build import CSRC, HOST_SRCS, OUT_DIR, _run

SAN_LIB = os.path.join(OUT_DIR, "libsgemv_host_san.so")


def build_host_sanitized(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = SAN_LIB + ".tmp"
    _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-Wall", "-Wextra"] + [os.path.join(CSRC, s) for s in HOST_SRCS] + ["-o", tmp], verbose)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def asan_runtime() -> str:
    """Path of the compiler's address-sanitizer runtime (to preload)."""
    return subprocess.run(["g++", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True,
                          check=True).stdout.strip()

"""The host packer and layout built with the address and undefined-behaviour
sanitizers, running the CPU parity suite (pack and layout bit-exact against
the oracle, error paths, FP16 conversion) in a child process.

The child loads the host-only build (no HIP code) through SGEMV_LIB, with
the address-sanitizer runtime preloaded; any report (out-of-bounds access,
use after free, signed overflow, misaligned access, ...) aborts it. Tests of
the launcher's host arithmetic (plans, exported symbols) need the full
library and stay out; the largest shapes are left to the uninstrumented run.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

NEEDS_LAUNCHER = ["plan", "list_table", "exported", "layer_run", "balanced_split", "error_paths", "fp16_form"]
LARGEST = ["decoder_set_every", "dense_ablation_mlp", "adaptive_mlp_configs", "11008-4096-1"]


def test_cpu_parity_suite_under_sanitizers():
    from sparse_weight_only_amd import _build_san
    lib = _build_san.SAN_LIB
    srcs = [os.path.join(ROOT, "sparse_weight_only_amd", "csrc", f)
            for f in ("host_pack.cpp", "host_layout.cpp", "internal.hpp")]
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(s) for s in srcs):
        _build_san.build_host_sanitized()
    env = dict(os.environ)
    env.update({
        "SGEMV_LIB": lib,
        "LD_PRELOAD": _build_san.asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    deselect = " and ".join(f"not {k}" for k in NEEDS_LAUNCHER + LARGEST)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           "-k", deselect, "tests/test_pack_parity.py", "tests/test_host_fp16.py", "tests/test_oracle_pack.py"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=900)
    tail = r.stdout[-6000:]
    assert r.returncode == 0, tail
    assert "passed" in tail and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    print(tail.strip().splitlines()[-1])

"""The C ABI driven from plain C (tests/c_abi/sgemv_c_driver.c): no Python
binding and no torch between the caller and include/sgemv.h.

CPU: the driver's sgemv_describe / sgemv_pack / sgemv_layout output is
compared byte for byte with the oracle's canonical 2bit-CSR arrays and kernel
layout, and its host error paths are exercised (the driver exits non-zero if
any returns the wrong status). GPU: the driver allocates device memory with
the HIP runtime's C API, runs sgemv_run twice on a stream of its own (bit-equal
results required) and the output is checked against the FP64 oracle.
"""
import os
import subprocess

import numpy as np
import pytest

import synth
from oracle import gemv as ogemv, layout as olayout, pack as opack
from sparse_weight_only_amd import _build

TOL = 2e-3   # normalised error gate: max |y - y_ref| / sum |w' x|

# (name, N, K, nk, group sizes drawn from, B)
CASES = [
    ("cfg1_1024x1024_2of4_g128", 1024, 1024, 2, (128,), 1),
    ("ragged_37x768_1of4_mixed", 37, 768, 1, (32, 64, 128, 256), 3),
    ("ragged_21x512_dense_mixed", 21, 512, 4, (32, 128), 2),
    ("one_row_1x256_2of4_g32", 1, 256, 2, (32,), 16),
]


def driver() -> str:
    if not os.path.exists(_build.C_DRIVER):
        import torch
        if torch.cuda.is_available():
            pytest.fail(f"C driver not built ({_build.C_DRIVER}): run __graft_entry__.build() first")
        if not os.path.exists(_build.LIB):
            _build.build()
        else:
            _build.build_c_driver()
    return _build.C_DRIVER


def inputs(case, tmp):
    name, N, K, nk, gchoices, B = case
    i = CASES.index(case)
    if name.startswith("cfg1"):
        L = synth.cfg1()[0]
        W, X = L.W(), L.X(B)
    else:
        W = synth.weights(N, K, cfg=90 + i)
        X = synth.activations(B, K, cfg=90 + i)
    rng = synth.rng(90 + i, tag=7)
    gs = rng.choice(np.asarray(gchoices, np.int32), N).astype(np.int32)
    with open(os.path.join(tmp, "meta.txt"), "w") as f:
        f.write(f"{N} {K} {nk} {B}\n")
    W.view(np.uint16).tofile(os.path.join(tmp, "w.bin"))
    gs.tofile(os.path.join(tmp, "gs.bin"))
    X.view(np.uint16).tofile(os.path.join(tmp, "x.bin"))
    return W, X, gs


def call(mode, tmp):
    r = subprocess.run([driver(), mode, str(tmp)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout
    return r.stdout


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_c_driver_packs_like_the_oracle(case, tmp_path):
    name, N, K, nk, _, _ = case
    W, _, gs = inputs(case, str(tmp_path))
    call("pack", tmp_path)
    co = opack.pack_canonical(W, nk, gs)
    rd = lambda f, dt: np.fromfile(os.path.join(tmp_path, f), dtype=dt)
    desc = dict(l.split() for l in open(os.path.join(tmp_path, "desc.txt")))
    sizes = opack.sizes(N, K, nk, gs)
    assert int(desc["kept"]) == N * K * nk // 4
    assert int(desc["vals_bytes"]) == sizes["vals_bytes"] == co["vals"].nbytes
    assert int(desc["n_groups"]) == int(co["gptr"][-1])
    assert np.array_equal(rd("vals.bin", np.uint8), co["vals"].reshape(-1))
    assert np.array_equal(rd("offs.bin", np.uint8), co["offs"].reshape(-1))
    assert np.array_equal(rd("scale.bin", np.uint16), co["scale"].reshape(-1))
    assert np.array_equal(rd("zero.bin", np.uint16), co["zero"].reshape(-1))
    assert np.array_equal(rd("gptr.bin", np.int32), co["gptr"])
    assert np.array_equal(rd("rowptr.bin", np.int32), co["rowptr"])
    blob = rd("blob.bin", np.uint8)
    assert int(desc["blob_bytes"]) == blob.size
    assert np.array_equal(blob, olayout.build(co)["blob"])


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_c_driver_runs_on_the_gpu(case, tmp_path):
    name, N, K, nk, _, B = case
    print(f"case c-driver {name} B={B}", flush=True)
    W, X, gs = inputs(case, str(tmp_path))
    print(call("run", tmp_path).strip(), flush=True)
    y = np.fromfile(os.path.join(tmp_path, "y.bin"), dtype=np.uint16).view(np.float16).reshape(B, N)
    co = opack.pack_canonical(W, nk, gs)
    Wd = ogemv.dequant_dense(co)
    err = ogemv.normalized_error(y, ogemv.gemv(Wd, X), ogemv.abs_dot(Wd, X))
    assert err <= TOL, err

"""Helpers for the GPU parity tests: build layers through the C ABI, run, compare."""
import sys

import numpy as np

import synth
import sparse_weight_only_amd as sg
from oracle import gemv as ogemv, pack as opack

TOL = 2e-3          # normalised error gate: max |y - y_ref| / sum |w' x|


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def group_sizes(L, W):
    if not L.adaptive:
        return np.full(L.N, synth.G_COARSE, dtype=np.int32)
    return sg.select_groups(W, L.nk, L.Xcal(synth.CALIB_T), synth.FRAC_FINE, synth.G_FINE, synth.G_COARSE)


def make_layer(W, nk, gs):
    return sg.SparseGemvLayer.from_dense(W, nk, np.asarray(gs, np.int32))


def run_checked(layer, X16, guard=64):
    """Run on the GPU with sentinel guard bands around y; return y (FP16 numpy [B, N])."""
    import torch
    B = X16.shape[0]
    N = layer.desc.N
    x = torch.from_numpy(np.ascontiguousarray(X16)).cuda()
    sentinel = np.uint16(0x7E5A)
    ybuf = torch.full((B * N + 2 * guard,), int(np.int16(sentinel.view(np.int16))), dtype=torch.int16, device="cuda")
    y = ybuf[guard: guard + B * N]
    sg.run(layer.desc, layer.blob.data_ptr(), x.data_ptr(), y.data_ptr(), B,
           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    host = ybuf.cpu().numpy().view(np.uint16)
    assert np.all(host[:guard] == sentinel) and np.all(host[-guard:] == sentinel), "y guard band overwritten"
    return host[guard: guard + B * N].reshape(B, N).view(np.float16)


def oracle_y(canon_c, X16):
    """FP64 oracle on the C++ canonical arrays (checked bit-exact against the oracle's own pack)."""
    Wd = ogemv.dequant_dense(canon_c)
    return ogemv.gemv(Wd, X16), ogemv.abs_dot(Wd, X16), Wd


def canon_for_oracle(layer):
    c = dict(layer.canon)
    return c


def check_pack_matches_oracle(W, nk, gs, canon_c):
    co = opack.pack_canonical(W, nk, gs)
    for k in ("vals", "offs", "scale", "zero", "gptr"):
        assert np.array_equal(canon_c[k], co[k]), k
    return co

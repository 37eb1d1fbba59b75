"""Helpers for the GPU parity tests: build layers through the C ABI, run, compare.

Every reference output comes from the oracle's own pipeline, run on the dense
FP16 weights: its group choice, its 2bit-CSR pack, its dequantisation and its
FP64 product. The product packer's arrays are never the oracle's input; they
are only checked, byte for byte, against the oracle's (``Ref.check``).
"""
import sys

import numpy as np

import synth
import sparse_weight_only_amd as sg
from oracle import gemv as ogemv, groups as ogroups, layout as olayout, pack as opack, prune as oprune

TOL = 2e-3          # normalised error gate: max |y - y_ref| / sum |w' x|

CANON_KEYS = ("vals", "offs", "scale", "zero", "gptr", "rowptr")
CANON16_KEYS = ("vals16", "offs", "rowptr")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def group_sizes(L, W):
    """Group size per row of a workload layer: the oracle's choice, which the
    library's sgemv_select_groups must reproduce exactly."""
    if not L.adaptive:
        return ogroups.uniform_groups(L.N, synth.G_COARSE).astype(np.int32)
    _, mask = oprune.nm_prune(W, L.nk)
    Xcal = L.Xcal(synth.CALIB_T)
    gs_o = ogroups.select_groups(W, mask, Xcal, synth.FRAC_FINE, synth.G_FINE, synth.G_COARSE).astype(np.int32)
    gs_c = sg.select_groups(W, L.nk, Xcal, synth.FRAC_FINE, synth.G_FINE, synth.G_COARSE)
    assert np.array_equal(gs_c, gs_o), "sgemv_select_groups differs from the oracle"
    return gs_o


class Ref:
    """The oracle's pack of dense FP16 weights and its dense FP64 W'."""

    def __init__(self, W, nk, gs=None, fp16=False):
        self.fp16 = fp16
        self.co = opack.pack_fp16_canonical(W, nk) if fp16 else opack.pack_canonical(W, nk, gs)
        self.Wd = ogemv.dequant_dense(self.co)

    def check(self, layer):
        """The product layer's canonical arrays and its kernel-layout blob (the
        bytes the GPU reads) equal the oracle's, byte for byte."""
        for k in (CANON16_KEYS if self.fp16 else CANON_KEYS):
            assert np.array_equal(np.asarray(layer.canon[k]), np.asarray(self.co[k])), f"packed {k} differs"
        blob = (olayout.build16(self.co) if self.fp16 else olayout.build(self.co))["blob"]
        assert np.array_equal(layer.blob_host, blob), "kernel-layout blob differs"
        return self

    def y(self, X16):
        """(y_ref, D): FP64 W' x and sum |w' x| per output."""
        return ogemv.gemv(self.Wd, X16), ogemv.abs_dot(self.Wd, X16)


def make_layer(W, nk, gs):
    """Product layer (sgemv_pack + sgemv_layout, uploaded) and the oracle's
    reference for it, checked equal."""
    layer = sg.SparseGemvLayer.from_dense(W, nk, np.asarray(gs, np.int32))
    return layer, Ref(W, nk, gs).check(layer)


def make_layer_fp16(W, nk):
    layer = sg.SparseGemvLayer.from_dense_fp16(W, nk)
    return layer, Ref(W, nk, fp16=True).check(layer)


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


def assert_bit_exact(y, y_ref, what=""):
    """y_ref must be exactly representable in FP16 (the inputs make every
    partial sum exact); then y must carry exactly its bits."""
    want = y_ref.astype(np.float16)
    assert np.array_equal(want.astype(np.float64), y_ref), "reference not exact"
    assert np.array_equal(y.view(np.uint16), want.view(np.uint16)), what

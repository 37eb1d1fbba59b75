"""Host packer (C ABI) vs oracle: bit-exact canonical arrays, group choice and blob.

Runs on the CPU: the library is loaded but no GPU call is made.
"""
import re
import os

import numpy as np
import pytest

import synth
from oracle import groups as ogroups, layout as olayout, pack as opack, prune as oprune
import sparse_weight_only_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def oracle_groups(L, W):
    if not L.adaptive:
        return ogroups.uniform_groups(L.N, synth.G_COARSE)
    _, mask = oprune.nm_prune(W, L.nk)
    return ogroups.select_groups(W, mask, L.Xcal(synth.CALIB_T), synth.FRAC_FINE, synth.G_FINE, synth.G_COARSE)


def check_layer(L, rt=0, tpr=0, check_layout=True):
    W = L.W()
    gs_o = oracle_groups(L, W)
    if L.adaptive:
        gs_c = sg.select_groups(W, L.nk, L.Xcal(synth.CALIB_T), synth.FRAC_FINE, synth.G_FINE, synth.G_COARSE)
        assert np.array_equal(gs_c, gs_o), L.name
        assert int(np.sum(gs_c == synth.G_FINE)) == ogroups.fine_count(L.N, synth.FRAC_FINE)
    canon_o = opack.pack_canonical(W, L.nk, gs_o)
    canon_c = sg.pack(W, L.nk, gs_o)
    for k in ("vals", "offs", "scale", "zero", "gptr", "rowptr"):
        assert np.array_equal(canon_c[k], canon_o[k]), (L.name, k)
    d = sg.describe(L.N, L.K, L.nk, gs_o, rt, tpr)
    sz = opack.sizes(L.N, L.K, L.nk, gs_o)
    assert (d.kept, d.vals_bytes, d.offs_bytes, d.n_groups) == \
        (sz["kept"], sz["vals_bytes"], sz["offs_bytes"], sz["n_groups"])
    if check_layout:
        blob_c = sg.layout(d, canon_c)
        lay = olayout.build(canon_o, d.rt, d.tpr)
        off = lay["offsets"]
        assert (d.off_perm, d.off_vals, d.off_offs, d.off_sz, d.blob_bytes) == \
            (off["perm"], off["vals"], off["offs"], off["sz"], off["blob_bytes"])
        assert d.n_tiles == len(lay["tiles"])
        assert np.array_equal(blob_c, lay["blob"]), L.name
    return d


@pytest.mark.parametrize("L", synth.cfg1() + synth.cfg2(), ids=lambda L: L.name)
def test_uniform_configs(L):
    check_layer(L)


@pytest.mark.parametrize("L", synth.cfg3(), ids=lambda L: L.name)
def test_adaptive_mlp_configs(L):
    check_layer(L)


def test_decoder_set_sampled_layers():
    """32-layer set: every matrix shape at both N:M choices (layers 0 and 4), groups and blob."""
    layers = [L for L in synth.cfg4() if L.layer in (0, 4) and L.name.split("_", 2)[2] in
              ("q_proj", "gate_proj", "down_proj")]
    for L in layers:
        check_layer(L)


@pytest.mark.parametrize("rt,tpr", [(64, 4), (32, 8), (16, 16), (8, 32), (4, 64), (2, 32), (1, 64)])
def test_layout_parameters(rt, tpr):
    L = synth.Layer("lay", 768, 200, 2, True, 9, 0, 0, 9)
    check_layer(L, rt, tpr)
    L1 = synth.Layer("lay1", 1280, 77, 1, True, 9, 1, 0, 9)
    check_layer(L1, rt, tpr)


def test_quantizer_edge_groups():
    """Hand-shaped rows: all-zero groups, all-negative, tiny values, ties, -0."""
    rng = np.random.default_rng(0)
    N, K = 24, 512
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    W[0] = 0
    W[1] = -np.abs(W[1])
    W[2] = np.abs(W[2])
    W[3] = (W[3] * 1e-6).astype(np.float16)
    W[4] = np.float16(0.5)
    W[5, ::2] = -0.0
    W[6] = rng.choice(np.array([0.25, -0.25, 0.5], np.float16), K)
    W[7] = np.float16(65504.0) * rng.choice([-1, 1], K)
    W[8] = (rng.standard_normal(K) * 1e3).astype(np.float16)
    for nk in (1, 2):
        for g in (32, 64, 128, 256):
            gs = np.full(N, g, dtype=np.int32)
            co = opack.pack_canonical(W, nk, gs)
            cc = sg.pack(W, nk, gs)
            for k in ("vals", "offs", "scale", "zero", "gptr", "rowptr"):
                assert np.array_equal(cc[k], co[k]), (nk, g, k)


def test_random_scales_cover_fp16_rounding():
    """Many random groups of assorted magnitudes: every FP16 scale rounding path."""
    rng = np.random.default_rng(1)
    N, K = 64, 1024
    W = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-20, 10, (N, 1)))).astype(np.float16)
    gs = np.full(N, 32, dtype=np.int32)
    for nk in (1, 2):
        co = opack.pack_canonical(W, nk, gs)
        cc = sg.pack(W, nk, gs)
        assert np.array_equal(cc["scale"], co["scale"]) and np.array_equal(cc["zero"], co["zero"])
        assert np.array_equal(cc["vals"], co["vals"])


def test_every_header_symbol_is_exported():
    hdr = open(os.path.join(ROOT, "include", "sgemv.h")).read()
    names = re.findall(r"^\s*(?:int|const char\*)\s+(sgemv_\w+)\s*\(", hdr, re.M)
    assert len(names) >= 6
    L = sg.lib()
    for n in names:
        assert hasattr(L, n), n


def test_error_paths():
    g = np.full(8, 128, dtype=np.int32)
    with pytest.raises(sg.SgemvError) as e:
        sg.describe(8, 300, 2, g)
    assert e.value.code == sg.sgemv.SGEMV_EINVAL
    with pytest.raises(sg.SgemvError):
        sg.describe(8, 256, 3, g)
    with pytest.raises(sg.SgemvError):
        sg.describe(8, 256, 2, np.full(8, 48, np.int32))
    with pytest.raises(sg.SgemvError) as e:
        sg.describe(8, 256, 2, g, rt=4, tpr=3)
    assert e.value.code == sg.sgemv.SGEMV_ESIZE
    with pytest.raises(sg.SgemvError) as e:
        sg.describe(8, 11008, 2, np.full(8, 128, np.int32)[:8] * 0 + 64, rt=64, tpr=4)   # 43 chunks/thread
    assert e.value.code == sg.sgemv.SGEMV_ESIZE
    W = np.zeros((8, 256), dtype=np.float16)
    W[3, 7] = np.nan
    with pytest.raises(sg.SgemvError):
        sg.pack(W, 2, g)
    W[3, 7] = np.inf
    with pytest.raises(sg.SgemvError):
        sg.select_groups(W, 2, np.ones((4, 256), np.float16))
    d = sg.describe(8, 256, 2, g)
    # run: host-side checks fire before any HIP call (no GPU here)
    for args, code in [((0x1000, 0x1000, 0x1000, 0), sg.sgemv.SGEMV_EINVAL),     # B = 0
                       ((0x1000, 0x1000, 0x1000, 17), sg.sgemv.SGEMV_EINVAL),    # B = 17
                       ((0x1001, 0x1000, 0x1000, 1), sg.sgemv.SGEMV_EALIGN),     # blob misaligned
                       ((0x1000, 0x1008, 0x1000, 1), sg.sgemv.SGEMV_EALIGN),     # x misaligned
                       ((0x1000, 0x1000, 0x1001, 1), sg.sgemv.SGEMV_EALIGN),     # y misaligned
                       ((0, 0x1000, 0x1000, 1), sg.sgemv.SGEMV_EINVAL)]:         # NULL blob
        with pytest.raises(sg.SgemvError) as e:
            sg.run(d, *args)
        assert e.value.code == code
    bad = sg.Desc.from_buffer_copy(d)
    bad.off_sz += 256
    with pytest.raises(sg.SgemvError) as e:
        sg.run(bad, 0x1000, 0x1000, 0x1000, 1)
    assert e.value.code == sg.sgemv.SGEMV_ESIZE
    canon = sg.pack(np.zeros((8, 256), np.float16), 2, g)
    with pytest.raises(sg.SgemvError):
        sg.layout(bad, canon)


@pytest.mark.parametrize("seed", range(4))
def test_launch_plan_covers_each_tile_once(seed):
    """sgemv_plan (host arithmetic only): one workgroup per tile at batch 1, whole passes of
    256 lanes per tile for beam batches; the LDS holds every staged x column of a phase."""
    rng = np.random.default_rng(seed)
    for _ in range(25):
        nk = int(rng.choice([1, 2]))
        K = int(rng.choice([256, 512, 768, 1024, 1280, 2816, 4096, 11008]))
        N = int(rng.integers(1, 700))
        gs = rng.choice([g for g in (32, 64, 128) if K % g == 0], N).astype(np.int32)
        C = K * nk // 128
        tpr = int(rng.choice([4, 8, 16, 32, 64]))
        rt = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128, 256])) if seed else 0
        try:
            d = sg.describe(N, K, nk, gs, rt, tpr if rt else 0)
        except sg.SgemvError:
            continue
        cpc = 128 // nk
        for B in (1, 3, 16):
            pl = sg.plan(d, B)
            slots = d.rt * d.tpr
            if B == 1:
                assert pl.grid == d.n_tiles and pl.pass_log2 == 0 and not pl.batched
                assert pl.block * pl.rows_per_lane == slots and pl.block <= 256
                assert pl.lds_bytes >= C * (cpc // 8 + 1) * 16          # all of x, with pads
            else:
                assert pl.batched and pl.grid == d.n_tiles << pl.pass_log2
                assert pl.block << pl.pass_log2 == slots and pl.block <= 256
            assert pl.lds_bytes <= 160 * 1024
            assert pl.chunks_per_row_lane == -(-C // d.tpr)

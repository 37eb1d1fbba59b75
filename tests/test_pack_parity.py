"""Host packer (C ABI) vs oracle: bit-exact canonical arrays, group choice and blob.

Runs on the CPU: the library is loaded but no GPU call is made.
"""
import ctypes
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


def check_layer(L, check_layout=True):
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
    d = sg.describe(L.N, L.K, L.nk, gs_o)
    sz = opack.sizes(L.N, L.K, L.nk, gs_o)
    assert (d.kept, d.vals_bytes, d.offs_bytes, d.n_groups) == \
        (sz["kept"], sz["vals_bytes"], sz["offs_bytes"], sz["n_groups"])
    if check_layout:
        blob_c = sg.layout(d, canon_c)
        lay = olayout.build(canon_o)
        off = lay["offsets"]
        assert (d.off_codes, d.off_offs, d.off_perm, d.off_sz, d.blob_bytes) == \
            (off["codes"], off["offs"], off["perm"], off["sz"], off["blob_bytes"])
        assert d.n_blocks == -(-L.N // 16) and d.chunks == L.K // 256
        assert np.array_equal(blob_c, lay["blob"]), L.name
    return d


@pytest.mark.parametrize("L", synth.cfg1() + synth.cfg2(), ids=lambda L: L.name)
def test_uniform_configs(L):
    check_layer(L)


@pytest.mark.parametrize("L", synth.cfg3(), ids=lambda L: L.name)
def test_adaptive_mlp_configs(L):
    check_layer(L)


def _check_decoder_matrix(i):
    L = synth.cfg4()[i]
    check_layer(L)
    return L.name


def test_decoder_set_every_matrix():
    """All 224 matrices of the 32-layer set (which include the beam-batch
    layers: their weights are those of decoder layers 0 and 4): group choice,
    canonical arrays and blob bit-exact against the oracle. One matrix per
    task, spread over worker processes (about 5 s of oracle work each)."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    n = len(synth.cfg4())
    assert n == 224
    assert {(L.K, L.N, L.nk, L.w_cfg, L.layer, L.mat) for L in synth.cfg5()} <= \
        {(L.K, L.N, L.nk, L.w_cfg, L.layer, L.mat) for L in synth.cfg4()}
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ProcessPoolExecutor(workers, mp_context=multiprocessing.get_context("fork")) as ex:
        done = list(ex.map(_check_decoder_matrix, range(n)))
    assert done == [L.name for L in synth.cfg4()]


@pytest.mark.parametrize("N,K,nk", [(200, 768, 2), (77, 1280, 1), (1, 256, 2), (15, 512, 1), (33, 11008, 2),
                                    (45, 1280, 4), (17, 11008, 4)])
def test_ragged_blocks_and_mixed_classes(N, K, nk):
    """Partial last row block, row blocks that straddle two group sizes, every size."""
    rng = np.random.default_rng(N + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    gs = rng.choice([32, 64, 128, 256], N).astype(np.int32)
    canon_o = opack.pack_canonical(W, nk, gs)
    canon_c = sg.pack(W, nk, gs)
    d = sg.describe(N, K, nk, gs)
    assert list(d.class_rows) == [int(np.sum(gs == g)) for g in (32, 64, 128, 256)]
    assert np.array_equal(sg.layout(d, canon_c), olayout.build(canon_o)["blob"])


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
        sg.describe(8, 32768 + 256, 2, g)                      # K beyond 128 column chunks
    assert e.value.code == sg.sgemv.SGEMV_ESIZE
    with pytest.raises(sg.SgemvError) as e:
        sg.describe(1 << 20, 32768, 2, np.full(1 << 20, 128, np.int32))   # blob of 2^31 bytes or more
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


def wave_chunks(pl, C):
    """Chunk range [c0, c0 + n) of every wave of a plan: chunks_per_wave for
    the first full_waves waves, one less after, contiguous, clipped to C."""
    out = []
    for w in range(pl.waves):
        c0 = w * pl.chunks_per_wave - max(0, w - pl.full_waves)
        n = pl.chunks_per_wave - (1 if w >= pl.full_waves else 0)
        out.append((c0, max(0, min(n, C - c0))))
    return out


def covers_exactly(pl, C):
    """The waves' ranges tile the C chunks in order, none left over."""
    assert 1 <= pl.full_waves <= pl.waves
    nxt = 0
    for c0, n in wave_chunks(pl, C):
        assert c0 == nxt or n == 0
        nxt = c0 + n if n else nxt
    assert nxt == C
    # the last wave has work, unless a wider layer set the geometry
    return wave_chunks(pl, C)[-1][1] > 0


def test_balanced_split_of_the_11008_column_layer():
    """K = 11008 (43 chunks) at one vector: 12 waves, 7 of 4 chunks and 5
    of 3, so that no SIMD of the workgroup (wave w on SIMD w % 4) holds more
    than 11 chunks; 11 waves of 4 would put 12 on one."""
    d = sg.describe(4096, 11008, 1, np.full(4096, 128, np.int32))
    pl = sg.plan(d, 1)
    assert (pl.waves, pl.chunks_per_wave, pl.full_waves) == (12, 4, 7)
    per = [0, 0, 0, 0]
    for w, (c0, n) in enumerate(wave_chunks(pl, 43)):
        per[w % 4] += n
    assert max(per) == 11 and sum(per) == 43
    # 4096 columns (16 chunks): 8 waves of 2, already even
    d = sg.describe(11008, 4096, 2, np.full(11008, 128, np.int32))
    pl = sg.plan(d, 1)
    assert (pl.waves, pl.chunks_per_wave, pl.full_waves) == (8, 2, 8)


@pytest.mark.parametrize("seed", range(4))
def test_launch_plan_covers_every_chunk_once(seed):
    """sgemv_plan (host arithmetic only): one workgroup per row_blocks row
    blocks (1, or 4 for 8+ vectors on INT4 sparse layers with K <= 4096 and
    640+ row blocks); its waves split the column chunks in contiguous ranges; x
    phases fit the 8 loads per lane, the weights of row_blocks x
    chunks_per_wave pieces fit the register budget, and the LDS holds every
    wave's slice plus the partial sums."""
    rng = np.random.default_rng(seed)
    seen = set()
    for it in range(48):
        nk = int(rng.choice([1, 2, 4]))
        K = 256 * int(rng.choice([1, 2, 3, 4, 5, 11, 16, 43, 64, 65, 128]))
        N = int(rng.integers(1, 12000)) if it % 4 else int(rng.integers(8000, 40000))
        gs = rng.choice([32, 64, 128, 256], N).astype(np.int32)
        d = sg.describe(N, K, nk, gs)
        C = K // 256
        for B in (1, 2, 3, 4, 7, 8, 9, 16):
            pl = sg.plan(d, B)
            rb = pl.row_blocks
            seen.add(rb)
            assert rb == (4 if nk != 4 and B >= 8 and C <= 16 and d.n_blocks >= 640 else 1)
            assert d.n_blocks == -(-N // 16) and pl.grid == -(-d.n_blocks // rb)
            assert pl.block == 64 * pl.waves and 1 <= pl.waves <= 16
            assert 1 <= pl.chunks_per_wave <= 8
            imax = 1 << (pl.chunks_per_wave - 1).bit_length()
            assert rb * imax <= 8
            assert covers_exactly(pl, C)
            assert 1 <= pl.phase_chunks <= pl.chunks_per_wave
            assert pl.phase_chunks & (pl.phase_chunks - 1) == 0          # a power of two
            assert pl.x_loads == -(-(B * pl.phase_chunks * 32) // 64) and pl.x_loads <= 8
            xs = pl.waves * B * (pl.phase_chunks * 512 + 16)
            if rb == 1:
                assert pl.lds_bytes == xs + B * 16 * 16 * 4
            else:
                assert pl.lds_bytes == xs + pl.waves * rb * B * 16 * 4 + rb * 16 * 4
            assert pl.lds_bytes <= 160 * 1024
    assert seen == {1, 4}


def test_plan_rejects_bad_batch_and_descriptor():
    g = np.full(40, 64, np.int32)
    d = sg.describe(40, 1024, 1, g)
    for B in (0, 17, -1):
        with pytest.raises(sg.SgemvError) as e:
            sg.plan(d, B)
        assert e.value.code == sg.sgemv.SGEMV_EINVAL
    for field, delta in [("n_blocks", 1), ("chunks", -1), ("n_groups", 1), ("off_perm", 256), ("value_format", 1),
                         ("blob_bytes", 256)]:
        bad = sg.Desc.from_buffer_copy(d)
        setattr(bad, field, getattr(bad, field) + delta)
        with pytest.raises(sg.SgemvError) as e:
            sg.plan(bad, 1)
        assert e.value.code == sg.sgemv.SGEMV_ESIZE, field
    bad = sg.Desc.from_buffer_copy(d)
    bad.class_rows[0] += 1
    bad.class_rows[1] -= 1
    with pytest.raises(sg.SgemvError):
        sg.plan(bad, 1)


def test_layout_rejects_dequantised_weights_beyond_fp16():
    """The kernel holds (code - zero) * scale in FP16: a group spanning [0, 65504]
    gets scale fp16(65504/15) = 4368 and code 15 -> 65520, which rounds to +inf."""
    N, K = 2, 256
    W = np.zeros((N, K), np.float16)
    W[1, 0] = 65504.0                     # row 1, group 0: lo = 0, hi = 65504
    gs = np.full(N, 32, np.int32)
    canon_o = opack.pack_canonical(W, 2, gs)
    from oracle import gemv as ogemv
    Wd = ogemv.dequant_dense(canon_o)
    assert Wd[1, 0] == 65520.0 and np.isinf(np.float16(Wd[1, 0]))
    canon_c = sg.pack(W, 2, gs)
    d = sg.describe(N, K, 2, gs)
    with pytest.raises(sg.SgemvError) as e:
        sg.layout(d, canon_c)
    assert e.value.code == sg.sgemv.SGEMV_EINVAL
    W[1, 0] = 65000.0                     # scale 4332, 15 * 4332 = 64980: finite
    canon_c = sg.pack(W, 2, gs)
    assert sg.layout(d, canon_c).nbytes == d.blob_bytes


def test_group_plan_and_host_errors():
    """sgemv_plan_group / sgemv_run_group host checks (no HIP call before them)."""
    rng = np.random.default_rng(11)
    E = sg.sgemv
    shapes = [(4096, 4096), (4096, 4096), (11008, 4096), (4096, 11008), (17, 256)]
    descs = {}
    for nk in (1, 2):
        descs[nk] = [sg.describe(N, K, nk, rng.choice([32, 128], N).astype(np.int32)) for N, K in shapes]
    fake = lambda ds: [(d, 0x1000 * (i + 1), 0x100000, 0x200000 + 0x40000 * i) for i, d in enumerate(ds)]
    for nk in (1, 2):
        for B in (1, 4, 16):
            for k in range(1, len(shapes) + 1):
                ds = descs[nk][:k]
                pl = sg.plan_group(fake(ds), B)
                cmax = max(d.chunks for d in ds)
                assert pl.grid == sum(d.n_blocks for d in ds)
                assert pl.block == 64 * pl.waves and 1 <= pl.waves <= 16
                assert covers_exactly(pl, cmax)
                for d in ds:                      # narrower layers: a prefix, the rest idle
                    covers_exactly(pl, d.chunks)
                assert pl.lds_bytes == pl.waves * B * (pl.phase_chunks * 512 + 16) + B * 16 * 16 * 4
            # a group of one is planned like the single call
            # (the single call may merge row blocks; the group launch does not)
            for d in descs[nk]:
                a, b = sg.plan_group(fake([d]), B), sg.plan(d, B)
                assert a.row_blocks == 1
                if b.row_blocks == 1:
                    assert a.as_dict() == b.as_dict()
                else:
                    assert a.grid == d.n_blocks and b.grid == -(-d.n_blocks // b.row_blocks)
    # up to 32 layers; 0, 33 and mixed N:M choices are rejected
    small = sg.describe(16, 256, 2, np.full(16, 128, np.int32))
    assert sg.plan_group(fake([small] * 32), 1).grid == 32
    for tasks, B, code in [([], 1, E.SGEMV_EINVAL), (fake([small] * 33), 1, E.SGEMV_EINVAL),
                           (fake([descs[1][0], descs[2][0]]), 1, E.SGEMV_EINVAL),
                           (fake([small]), 0, E.SGEMV_EINVAL), (fake([small]), 17, E.SGEMV_EINVAL)]:
        with pytest.raises(sg.SgemvError) as e:
            sg.plan_group(tasks, B)
        assert e.value.code == code
        with pytest.raises(sg.SgemvError) as e:
            sg.run_group(tasks, B)
        assert e.value.code == code
    bad = sg.Desc.from_buffer_copy(small)
    bad.n_blocks += 1
    with pytest.raises(sg.SgemvError) as e:
        sg.run_group(fake([small, bad]), 1)
    assert e.value.code == E.SGEMV_ESIZE
    for task, code in [((small, 0x1001, 0x1000, 0x1000), E.SGEMV_EALIGN), ((small, 0x1000, 0x1008, 0x1000), E.SGEMV_EALIGN),
                       ((small, 0x1000, 0x1000, 0x1001), E.SGEMV_EALIGN), ((small, 0, 0x1000, 0x1000), E.SGEMV_EINVAL),
                       ((small, 0x1000, 0x1000, 0), E.SGEMV_EINVAL)]:
        with pytest.raises(sg.SgemvError) as e:
            sg.run_group(fake([small]) + [task], 1)
        assert e.value.code == code


@pytest.mark.parametrize("nk", [1, 2])
def test_prune_scored_matches_oracle(nk):
    """sgemv_prune (C++) against oracle.prune.nm_prune_scored, bit for bit, on
    random, tie-heavy and outlier-channel inputs, with and without a
    calibration batch."""
    from oracle import prune as oprune
    rng = np.random.default_rng(31 + nk)
    pool = np.array([0.0, -0.0, 0.5, -0.5, 1.0, 0.25, -2.0], dtype=np.float16)
    cases = [((rng.standard_normal((40, 512)) * 0.02).astype(np.float16), rng.standard_normal((8, 512)).astype(np.float16)),
             (pool[rng.integers(0, len(pool), (33, 256))], pool[rng.integers(0, len(pool), (3, 256))]),
             (synth.cfg2()[0].W()[:64], synth.cfg2()[0].X(4)),                # 41 channels x20
             ((rng.standard_normal((9, 256)) * 0.02).astype(np.float16), np.zeros((2, 256), np.float16))]
    for W, X in cases:
        for xc in (X, None):
            got = sg.prune(W, nk, xc)
            want = oprune.pruned_dense(W, oprune.nm_prune_scored(W, nk, xc)[1])
            assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
    with pytest.raises(sg.SgemvError):
        sg.prune(np.full((4, 256), np.nan, np.float16), nk)
    with pytest.raises(sg.SgemvError):
        sg.prune(np.zeros((4, 256), np.float16), nk, np.full((1, 256), np.inf, np.float16))


def test_pack_of_pruned_matrix_keeps_the_pruned_weights():
    """sgemv_pack on sgemv_prune's output dequantises to the same matrix as
    quantising the scored selection directly (oracle)."""
    from oracle import prune as oprune, quant as oquant, gemv as ogemv
    L = synth.cfg2()[0]
    W = L.W()[:96]
    X = L.Xcal(synth.CALIB_T)
    for nk in (1, 2):
        Wp = sg.prune(W, nk, X)
        gs = sg.select_groups(Wp, nk, X)
        canon = sg.pack(Wp, nk, gs)
        Wd = ogemv.dequant_dense(canon)
        # oracle: scored selection, then the same quantiser on the kept values
        offs, mask = oprune.nm_prune_scored(W, nk, X)
        co = opack.pack_canonical(oprune.pruned_dense(W, mask), nk, gs)
        assert np.array_equal(ogemv.dequant_dense(co), Wd)
        assert np.all(Wd[~mask] == 0)


def test_activation_aware_pruning_lowers_output_error_with_outlier_channels():
    """On the 4096 x 4096 workload (41 input channels x20) the |w| * ||x||
    selection keeps the outlier channels' weights and so approximates the
    dense product better than |w| alone (measured on the oracle)."""
    from oracle import prune as oprune
    L = synth.cfg2()[0]
    W = L.W()[:256]
    Xall = L.X(72)                       # calibration rows and test rows share the outlier channels
    Xcal, X = Xall[:64], Xall[64:]
    dense = X.astype(np.float64) @ W.astype(np.float64).T
    for nk in (1, 2):
        errs = {}
        for name, xc in (("magnitude", None), ("activation_aware", Xcal)):
            Wp = oprune.pruned_dense(W, oprune.nm_prune_scored(W, nk, xc)[1]).astype(np.float64)
            errs[name] = np.linalg.norm(X.astype(np.float64) @ Wp.T - dense) / np.linalg.norm(dense)
        assert errs["activation_aware"] < errs["magnitude"], errs



@pytest.mark.parametrize("L", [L for L in synth.cfg3() if L.nk == 2], ids=lambda L: L.name + "_dense")
def test_dense_ablation_mlp_shapes(L):
    """The dense INT4 ablation (nk = 4: every element kept, no offsets) of the
    MLP shapes: groups, canonical arrays and blob bit-exact against the oracle."""
    import dataclasses
    check_layer(dataclasses.replace(L, nk=4, name=L.name.replace("2of4", "dense")))


@pytest.mark.parametrize("N,K,nk", [(4096, 4096, 2), (11008, 4096, 1), (77, 1280, 1), (33, 11008, 2), (1, 256, 2)])
def test_fp16_form_matches_oracle(N, K, nk):
    """FP16-valued form: canonical arrays, descriptor and blob bit-exact against the oracle."""
    rng = np.random.default_rng(N + K + nk)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    c = sg.pack_fp16(W, nk)
    co = opack.pack_fp16_canonical(W, nk)
    for k in ("vals16", "offs", "rowptr"):
        assert np.array_equal(c[k], co[k]), k
    d = sg.describe_fp16(N, K, nk)
    lay = olayout.build16(co)
    off = lay["offsets"]
    assert (d.value_format, d.n_groups, list(d.class_rows), d.g_min, d.g_max) == (1, 0, [0, 0, 0, 0], 0, 0)
    assert (d.kept, d.vals_bytes, d.offs_bytes) == (N * K * nk // 4, N * K * nk // 2, N * K * nk // 16)
    assert (d.off_codes, d.off_offs, d.off_perm, d.blob_bytes) == (off["values"], off["offs"], off["perm"], off["blob_bytes"])
    assert np.array_equal(sg.layout_fp16(d, c), lay["blob"])
    pl = sg.plan(d, 1)
    assert pl.grid == -(-N // 16)


def test_fp16_form_errors():
    E = sg.sgemv
    W = np.zeros((8, 256), np.float16)
    with pytest.raises(sg.SgemvError) as e:
        sg.describe_fp16(8, 256, 4)
    assert e.value.code == E.SGEMV_EINVAL
    with pytest.raises(sg.SgemvError):
        sg.pack_fp16(W, 4)
    W[2, 3] = np.inf
    with pytest.raises(sg.SgemvError):
        sg.pack_fp16(W, 2)
    W[2, 3] = 0
    d16 = sg.describe_fp16(8, 256, 2)
    d4 = sg.describe(8, 256, 2, np.full(8, 128, np.int32))
    c16 = sg.pack_fp16(W, 2)
    with pytest.raises(sg.SgemvError) as e:                    # an INT4 descriptor
        sg.layout_fp16(d4, c16)
    assert e.value.code == E.SGEMV_EINVAL
    with pytest.raises(sg.SgemvError):                         # an FP16 descriptor in the INT4 layout
        sg.layout(d16, sg.pack(W, 2, np.full(8, 128, np.int32)))
    bad = sg.Desc.from_buffer_copy(d16)
    bad.n_groups = 1
    with pytest.raises(sg.SgemvError) as e:
        sg.plan(bad, 1)
    assert e.value.code == E.SGEMV_ESIZE
    # one launch cannot mix the two value formats
    fake = [(d16, 0x1000, 0x1000, 0x1000), (d4, 0x2000, 0x1000, 0x2000)]
    with pytest.raises(sg.SgemvError) as e:
        sg.plan_group(fake, 1)
    assert e.value.code == E.SGEMV_EINVAL


def test_layer_run_rejects_bad_buffers_before_any_launch():
    """SparseGemvLayer.run checks x and y on the host: a y smaller than B x N,
    of another dtype or not contiguous, an x of the wrong width or dtype, or
    tensors on another device than the layer raise before sg.run is called
    (the layer is built on the CPU here, so a launch would be an error too)."""
    import torch
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((40, 512)) * 0.02).astype(np.float16)
    gs = np.full(40, 128, np.int32)
    canon = sg.pack(W, 2, gs)
    d = sg.describe(40, 512, 2, gs)
    # a host-resident layer (the constructor's device-alignment check is for
    # device blobs, so the attributes are set directly)
    layer = object.__new__(sg.SparseGemvLayer)
    layer.desc, layer.canon, layer.blob_host = d, canon, sg.layout(d, canon)
    layer.blob = torch.from_numpy(layer.blob_host)
    x = torch.zeros((3, 512), dtype=torch.float16)
    bad = [
        dict(x=torch.zeros((3, 256), dtype=torch.float16)),                  # wrong K
        dict(x=torch.zeros((3, 512), dtype=torch.float32)),                  # wrong dtype
        dict(x=torch.zeros((512, 3), dtype=torch.float16).t()),              # not contiguous
        dict(x=x, y=torch.empty((2, 40), dtype=torch.float16)),              # y too small
        dict(x=x, y=torch.empty((3, 40), dtype=torch.float32)),              # y of another dtype
        dict(x=x, y=torch.empty((40, 3), dtype=torch.float16).t()),          # y not contiguous
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            layer.run(kw["x"], kw.get("y"))
    if torch.cuda.is_available():
        with pytest.raises(ValueError):
            layer.run(x.cuda())                                               # x on another device


def test_select_groups_rejects_calibration_of_wrong_width():
    """xcal must be [T, K]: a flat or narrower batch is refused before the
    library reads T x K halves from it."""
    W = np.zeros((8, 1024), np.float16)
    with pytest.raises(ValueError):
        sg.select_groups(W, 2, np.ones(4096, np.float16))
    with pytest.raises(ValueError):
        sg.select_groups(W, 2, np.ones((4, 512), np.float16))
    assert sg.select_groups(W, 2, np.ones((4, 1024), np.float16)).shape == (8,)


def test_list_plan_and_host_errors():
    """sgemv_plan_list / sgemv_run_list host checks and launch shape (no HIP
    call before them)."""
    E = sg.sgemv
    rng = np.random.default_rng(12)
    d_up = sg.describe(11008, 4096, 1, rng.choice([32, 128], 11008).astype(np.int32))
    d_down = sg.describe(4096, 11008, 2, rng.choice([32, 128], 4096).astype(np.int32))
    d_small = sg.describe(40, 1024, 2, np.full(40, 64, np.int32))
    # 8 waves a workgroup, each with a run of at least one block where the
    # task has that many: 688 and 256 blocks give at most 86 and 32 workgroups
    pl = sg.plan_list([(d_up, 0, 0, 0), (d_down, 0, 0, 0)], 1)
    assert (pl.waves, pl.block, pl.grid) == (8, 512, 86 + 32)
    assert pl.lds_bytes == 43 * 512 + pl.row_blocks * 96      # x of K = 11008, rows and results of a run
    pl = sg.plan_list([(d_up, 0, 0, 0)], 1)
    assert (pl.waves, pl.grid, pl.row_blocks) == (8, 86, 8)
    pl = sg.plan_list([(d_small, 0, 0, 0)], 1)
    assert pl.grid == 1 and pl.row_blocks == 3
    # many tasks: at most 1536 workgroups (6 a compute unit), each with at
    # least 8 blocks: 40 tasks of 256 blocks fill 40 x 32
    many = [(sg.describe(4096, 4096, 1, np.full(4096, 128, np.int32)), 0, 0, 0) for i in range(40)]
    pl = sg.plan_list(many, 1)
    assert pl.grid == 1280 and pl.row_blocks == 8
    big = [(sg.describe(4096 * 4, 4096, 1, np.full(4096 * 4, 128, np.int32)), 0, 0, 0) for i in range(40)]
    pl = sg.plan_list(big, 1)
    assert pl.grid == 1536 and pl.row_blocks <= 256
    for tasks, B, code in [([], 1, E.SGEMV_EINVAL), ([(d_up, 0, 0, 0)], 2, E.SGEMV_EINVAL),
                           ([(d_small, 0, 0, 0)] * 49, 1, E.SGEMV_EINVAL)]:
        with pytest.raises(sg.SgemvError) as e:
            sg.plan_list(tasks, B)
        assert e.value.code == code
    d16 = sg.describe_fp16(64, 1024, 2)
    d4 = sg.describe(64, 1024, 4, np.full(64, 128, np.int32))
    for d in (d16, d4):
        with pytest.raises(sg.SgemvError) as e:
            sg.plan_list([(d, 0, 0, 0)], 1)
        assert e.value.code == E.SGEMV_EINVAL
    bad = sg.describe(40, 1024, 2, np.full(40, 64, np.int32))
    bad.n_blocks += 1
    with pytest.raises(sg.SgemvError) as e:
        sg.plan_list([(bad, 0, 0, 0)], 1)
    assert e.value.code == E.SGEMV_ESIZE
    # run: NULL and misaligned pointers are refused on the host
    for ptrs, code in [((0, 0x1000, 0x1000), E.SGEMV_EINVAL), ((0x1001, 0x1000, 0x1000), E.SGEMV_EALIGN),
                       ((0x1000, 0x1008, 0x1000), E.SGEMV_EALIGN)]:
        with pytest.raises(sg.SgemvError) as e:
            sg.run_list([(d_small,) + ptrs], 1, 0)
        assert e.value.code == code


ROW = np.dtype([("blob", "<u8"), ("x", "<u8"), ("y", "<u8"), ("blob_bytes", "<u4"), ("off_offs", "<u4"),
                ("off_perm", "<u4"), ("off_sz", "<u4"), ("N", "<i4"), ("cls1", "<i4"), ("cls2", "<i4"),
                ("cls3", "<i4"), ("c_nk", "<u4"), ("n_wg", "<i4"), ("q", "<i4"), ("r", "<i4"), ("j0", "<i4"),
                ("pad", "<i4")])


def test_list_table_covers_every_block_once():
    """sgemv_list_table: the rows of the table cover every row block of every
    task exactly once, a task's rows are consecutive, and up to 48 tasks get
    the shares of sgemv_plan_list. Beyond 48 tasks the workgroups grow with
    the count (a share like that in a list of 48)."""
    assert ROW.itemsize == 80
    rng = np.random.default_rng(14)
    shapes = [(4096, 4096), (11008, 4096), (4096, 11008), (40, 1024), (3000, 2048)]
    descs = [sg.describe(N, K, nk, rng.choice([32, 64, 128, 256], N).astype(np.int32))
             for N, K in shapes for nk in (1, 2)]
    for count in (1, 7, 48, 49, 224, 300):
        tasks = [(descs[int(i)], 0x100000 * (k + 1), 0x1000 * (k + 1), 0x2000 * (k + 1))
                 for k, i in enumerate(rng.integers(0, len(descs), count))]
        table, L = sg.list_table(tasks, 1)
        assert (L.tasks, L.block) == (count, 512) and table.size == L.table_bytes == 80 * L.rows
        rows = table.view(ROW)
        seen = {}
        for k, row in enumerate(rows):
            key = int(row["y"])
            assert row["j0"] % L.row_width == 0 and row["j0"] < row["n_wg"]
            if key in seen:
                assert seen[key][-1] == k - 1, "a task's rows are consecutive"
            seen.setdefault(key, []).append(k)
        assert len(seen) == count
        total = 0
        for (d, blob, x, y) in tasks:
            ks = seen[y]
            r0 = rows[ks[0]]
            assert (int(r0["blob"]), int(r0["x"]), r0["N"]) == (blob, x, d.N)
            n, q, r = int(r0["n_wg"]), int(r0["q"]), int(r0["r"])
            assert len(ks) == -(-n // L.row_width) and n * q + r == d.n_blocks and q + (r > 0) <= 256
            total += n
        assert total == L.workgroups
        if count <= sg.LIST_MAX:
            assert L.workgroups == sg.plan_list(tasks, 1).grid
        else:
            assert L.workgroups > sg.plan_list(tasks[:48], 1).grid


def test_list_table_host_errors():
    """sgemv_list_table / sgemv_run_list_table host checks (no HIP call before them)."""
    E = sg.sgemv
    d = sg.describe(40, 1024, 2, np.full(40, 64, np.int32))
    for tasks, B, code in [([], 1, E.SGEMV_EINVAL), ([(d, 0x1000, 0x1000, 0x1000)], 2, E.SGEMV_EINVAL),
                           ([(d, 0x1000, 0x1000, 0x1000)] * (sg.LIST_TABLE_MAX + 1), 1, E.SGEMV_EINVAL),
                           ([(d, 0, 0x1000, 0x1000)], 1, E.SGEMV_EINVAL),
                           ([(d, 0x1001, 0x1000, 0x1000)], 1, E.SGEMV_EALIGN),
                           ([(sg.describe_fp16(64, 1024, 2), 0x1000, 0x1000, 0x1000)], 1, E.SGEMV_EINVAL)]:
        with pytest.raises(sg.SgemvError) as e:
            sg.list_table(tasks, B)
        assert e.value.code == code
    # a table buffer smaller than the table
    launch = sg.ListLaunch()
    arr = sg.sgemv._tasks([(d, 0x1000, 0x1000, 0x1000)])
    buf = np.zeros(79, np.uint8)
    assert sg.lib().sgemv_list_table(arr, 1, 1, sg.sgemv._ptr(buf), buf.size, ctypes.byref(launch)) == E.SGEMV_ESIZE
    assert sg.lib().sgemv_list_table(arr, 1, 1, None, 0, None) == E.SGEMV_EINVAL
    # launches that no table describes, and a misaligned table
    _, good = sg.list_table([(d, 0x1000, 0x1000, 0x1000)], 1)
    for field, value in [("rows", 0), ("rows", 65536), ("row_width", 0), ("row_width", 33), ("block", 256),
                         ("lds_bytes", 160 * 1024 + 1), ("table_bytes", 81)]:
        bad = sg.ListLaunch.from_buffer_copy(good)
        setattr(bad, field, value)
        with pytest.raises(sg.SgemvError) as e:
            sg.run_list_table(0x1000, bad, 0)
        assert e.value.code == E.SGEMV_EINVAL, field
    for ptr, code in [(0, E.SGEMV_EINVAL), (0x1008, E.SGEMV_EALIGN)]:
        with pytest.raises(sg.SgemvError) as e:
            sg.run_list_table(ptr, good, 0)
        assert e.value.code == code

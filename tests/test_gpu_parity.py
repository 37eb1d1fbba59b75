"""GPU parity: the HIP SparseGemv kernels through the C ABI against the FP64 oracle.

Bars: bit-exact where the arithmetic is exact (grid weights with x in
{-1,0,1}; one-hot x), normalised error <= 2e-3 elsewhere, guard bands intact,
identical bits on repeated runs.
"""
import numpy as np
import pytest

import synth
import sparse_weight_only_amd as sg
from oracle import gemv as ogemv
from gpu_util import TOL, say, group_sizes, make_layer, make_layer_fp16, run_checked, assert_bit_exact, Ref

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.lib()


def grid_weights(N, K, nk, g, rng, s=2.0 ** -6):
    """Values k*s, k in [-8, 7], with every quantisation group keeping -8s and 7s."""
    W = rng.integers(-8, 8, (N, K)).astype(np.float64)
    for c0 in range(0, K, g):
        W[:, c0: c0 + 4] = [-8, 7, 0, 0] if nk in (2, 4) else [-8, 0, 0, 0]
        if nk == 1:
            W[:, c0 + 4: c0 + 8] = [7, 0, 0, 0]
    return (W * s).astype(np.float16)


@pytest.mark.parametrize("nk", [2, 1, 4])
@pytest.mark.parametrize("N,K,gs_kind", [
    (1024, 1024, "u128"), (300, 4096, "mixed"), (77, 11008, "mixed"), (513, 2048, "all"),
    (40, 768, "mixed"), (1, 256, "u128"), (130, 1280, "all"), (96, 512, "u32"), (17, 32768, "all"),
])
def test_exact_arithmetic_bit_exact(nk, N, K, gs_kind):
    rng = np.random.default_rng(N + K + nk)
    gchoices = {"u128": [128], "u32": [32], "mixed": [32, 128], "all": [32, 64, 128, 256]}[gs_kind]
    gs = rng.choice(gchoices, N).astype(np.int32)
    W = np.zeros((N, K), np.float16)
    for g in np.unique(gs):
        rows = gs == g
        W[rows] = grid_weights(int(rows.sum()), K, nk, int(g), rng)
    say(f"case exact nk={nk} N={N} K={K} groups={gs_kind}")
    layer, ref = make_layer(W, nk, gs)
    assert np.all(np.abs(ref.co["scale"].view(np.float16).astype(np.float64) - 2.0 ** -6) == 0)
    for B in (1, 3, 16):
        X = np.zeros((B, K), np.float16)
        for b in range(B):
            idx = rng.choice(K, size=min(64, K), replace=False)
            X[b, idx] = rng.choice([-1.0, 1.0], len(idx))
        y = run_checked(layer, X)
        assert_bit_exact(y, ref.y(X)[0], f"B={B}")


@pytest.mark.parametrize("L", synth.cfg1() + synth.cfg2() + synth.cfg3(), ids=lambda L: L.name)
def test_one_hot_columns_bit_exact(L):
    W = L.W()
    gs = group_sizes(L, W)
    say(f"case one-hot {L.name}")
    layer, ref = make_layer(W, L.nk, gs)
    Wd = ref.Wd
    rng = np.random.default_rng(5)
    cols = np.concatenate([[0, L.K - 1], rng.choice(L.K, 14, replace=False)])
    X = np.zeros((16, L.K), np.float16)
    X[np.arange(16), cols] = 1.0
    y = run_checked(layer, X)
    want = Wd[:, cols].T.astype(np.float16)
    assert np.array_equal(y.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("L", synth.cfg1() + synth.cfg2() + synth.cfg3(), ids=lambda L: L.name)
def test_configs_within_tolerance(L):
    W = L.W()
    gs = group_sizes(L, W)
    say(f"case config {L.name}")
    layer, ref = make_layer(W, L.nk, gs)
    X = L.X(1)
    y = run_checked(layer, X)
    y_ref, D = ref.y(X)
    err = ogemv.normalized_error(y, y_ref, D)
    say(f"  {L.name}: normalised error {err:.3e}")
    assert err <= TOL
    y2 = run_checked(layer, X)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), "not deterministic"


@pytest.mark.parametrize("L", synth.cfg5(), ids=lambda L: L.name)
def test_beam_batches_within_tolerance(L):
    W = L.W()
    gs = group_sizes(L, W)
    say(f"case beam {L.name}")
    layer, ref = make_layer(W, L.nk, gs)
    for B in synth.CFG5_BATCHES:
        X = L.X(B)
        y = run_checked(layer, X)
        y_ref, D = ref.y(X)
        err = ogemv.normalized_error(y, y_ref, D)
        say(f"  B={B}: normalised error {err:.3e}")
        assert err <= TOL
        # each batch row equals the batch-1 result of that row (same kernel arithmetic per row)
        y1 = run_checked(layer, X[B - 1: B])
        assert ogemv.normalized_error(y1, y_ref[B - 1: B], D[B - 1: B]) <= TOL


@pytest.mark.parametrize("layer_idx", [0, 4, 31])
def test_decoder_layer_back_to_back(layer_idx):
    """Decoder layers 0 (2:4), 4 (1:4) and 31 (2:4) of the 32-layer set: the 7
    projections launched back to back on one stream, each with its own x."""
    import torch
    Ls = [L for L in synth.cfg4() if L.layer == layer_idx]
    layers, xs, ys = [], [], []
    for L in Ls:
        W = L.W()
        layers.append((L,) + make_layer(W, L.nk, group_sizes(L, W)))
    say(f"case decoder layer {layer_idx}, {len(layers)} GEMVs back to back")
    for L, layer, _ in layers:
        x = torch.from_numpy(L.X(1)).cuda()
        y = torch.empty((1, L.N), dtype=torch.float16, device="cuda")
        sg.run(layer.desc, layer.blob.data_ptr(), x.data_ptr(), y.data_ptr(), 1,
               torch.cuda.current_stream().cuda_stream)
        xs.append(x)
        ys.append(y)
    torch.cuda.synchronize()
    for (L, layer, ref), y in zip(layers, ys):
        err = ogemv.normalized_error(y.cpu().numpy(), *ref.y(L.X(1)))
        assert err <= TOL, (L.name, err)


@pytest.mark.parametrize("B", [1, 2, 5, 16])
def test_odd_shapes_and_batches(B):
    rng = np.random.default_rng(B)
    for (N, K, nk) in [(1, 256, 2), (3, 256, 1), (257, 1536, 2), (129, 2816, 1)]:
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
        gs = rng.choice([32, 64, 128], N).astype(np.int32)
        say(f"case odd N={N} K={K} nk={nk} B={B}")
        layer, ref = make_layer(W, nk, gs)
        X = rng.standard_normal((B, K)).astype(np.float16)
        X[:, :8] = 0
        y = run_checked(layer, X)
        y_ref, D = ref.y(X)
        assert ogemv.normalized_error(y, y_ref, D) <= TOL


@pytest.mark.parametrize("nk", [2, 1])
def test_every_batch_size(nk):
    """Every batch size from 1 to 16 through the kernels the plan picks for it
    (one vector, several vectors, 4 row blocks a workgroup from 8 vectors on
    the 10250 x 2048 layer; phased x staging on the 11008-column one): within
    the tolerance."""
    rng = np.random.default_rng(700 + nk)
    for (N, K) in [(10250, 2048), (300, 11008)]:
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
        gs = rng.choice([32, 128], N).astype(np.int32)
        layer, ref = make_layer(W, nk, gs)
        X = rng.standard_normal((16, K)).astype(np.float16)
        y_ref, D = ref.y(X)
        for B in range(1, 17):
            pl = sg.plan(layer.desc, B)
            say(f"case batch N={N} K={K} nk={nk} B={B} row_blocks={pl.row_blocks} waves={pl.waves} "
                f"phase={pl.phase_chunks}")
            y = run_checked(layer, X[:B])
            err = ogemv.normalized_error(y, y_ref[:B], D[:B])
            assert err <= TOL, (N, K, B, err)


def test_zero_input_gives_zero_output():
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((64, 512)) * 0.02).astype(np.float16)
    layer, _ = make_layer(W, 2, np.full(64, 128, np.int32))
    y = run_checked(layer, np.zeros((2, 512), np.float16))
    assert np.all(y.view(np.uint16) == 0)


@pytest.mark.parametrize("nk", [2, 1, 4])
@pytest.mark.parametrize("N,K", [(16, 256), (600, 8192), (40, 11008), (17, 32768)])
def test_every_launch_geometry(nk, N, K):
    """Shapes and batches that together launch every reachable kernel instance
    (chunks per wave 1..8, x loads per lane 1..8, phased staging of x)."""
    rng = np.random.default_rng(N + nk)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    gs = rng.choice([32, 64, 128, 256], N).astype(np.int32)
    layer, ref = make_layer(W, nk, gs)
    for B in (1, 2, 3, 4, 8, 16):
        pl = sg.plan(layer.desc, B)
        say(f"case geometry N={N} K={K} nk={nk} B={B} waves={pl.waves} cpw={pl.chunks_per_wave} "
            f"phase={pl.phase_chunks} xloads={pl.x_loads}")
        X = rng.standard_normal((B, K)).astype(np.float16)
        y = run_checked(layer, X)
        y_ref, D = ref.y(X)
        err = ogemv.normalized_error(y, y_ref, D)
        assert err <= TOL, (B, err)


@pytest.mark.parametrize("nk", [2, 1])
@pytest.mark.parametrize("N,K", [(16390, 4096), (10250, 2048), (10255, 768)])
def test_several_row_blocks_per_workgroup(nk, N, K):
    """Batches of 8+ vectors on layers with many row blocks take the kernel
    that computes 4 row blocks per workgroup (x loaded once for all of them).
    These shapes give a last workgroup with fewer blocks than it computes, a
    last block of fewer than 16 rows, a last wave with one chunk and blocks of
    different group sizes in one workgroup: bit for bit where the arithmetic
    is exact, within tolerance on Gaussian inputs, and the same bits on a
    second run. At 4 vectors the same layer takes one block per workgroup."""
    rng = np.random.default_rng(N + K + nk)
    T = -(-N // 16)
    gs = rng.choice([32, 64, 128, 256], N).astype(np.int32)
    W = np.zeros((N, K), np.float16)
    for g in np.unique(gs):
        rows = gs == g
        W[rows] = grid_weights(int(rows.sum()), K, nk, int(g), rng)
    layer, ref = make_layer(W, nk, gs)
    for B in (4, 8, 9, 16):
        pl = sg.plan(layer.desc, B)
        want_rb = 4 if B >= 8 else 1
        say(f"case row blocks N={N} K={K} nk={nk} B={B} row_blocks={pl.row_blocks} waves={pl.waves} "
            f"cpw={pl.chunks_per_wave} xloads={pl.x_loads}")
        assert pl.row_blocks == want_rb and pl.grid == -(-T // want_rb)
        X = np.zeros((B, K), np.float16)
        for b in range(B):
            idx = rng.choice(K, size=64, replace=False)
            X[b, idx] = rng.choice([-1.0, 1.0], 64)
        y = run_checked(layer, X)
        assert_bit_exact(y, ref.y(X)[0], f"B={B}")
    # Gaussian weights and inputs: tolerance, then determinism
    Wg = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    layer, ref = make_layer(Wg, nk, gs)
    X = rng.standard_normal((16, K)).astype(np.float16)
    y = run_checked(layer, X)
    err = ogemv.normalized_error(y, *ref.y(X))
    say(f"  gaussian B=16: normalised error {err:.3e}")
    assert err <= TOL
    y2 = run_checked(layer, X)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), "not deterministic"


def _run_group_checked(layers, Xs, B, guard=64):
    """One sgemv_run_group launch over layers (each with its own x and guarded y)."""
    import torch
    sentinel = np.uint16(0x7E5A)
    bufs, tasks, xs = [], [], []
    for layer, X in zip(layers, Xs):
        N = layer.desc.N
        x = torch.from_numpy(np.ascontiguousarray(X)).cuda()
        ybuf = torch.full((B * N + 2 * guard,), int(np.int16(sentinel.view(np.int16))), dtype=torch.int16, device="cuda")
        xs.append(x)
        bufs.append(ybuf)
        tasks.append((layer.desc, layer.blob.data_ptr(), x.data_ptr(), ybuf[guard:].data_ptr()))
    sg.run_group(tasks, B, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    out = []
    for layer, ybuf in zip(layers, bufs):
        host = ybuf.cpu().numpy().view(np.uint16)
        assert np.all(host[:guard] == sentinel) and np.all(host[-guard:] == sentinel), "y guard band overwritten"
        out.append(host[guard: guard + B * layer.desc.N].reshape(B, layer.desc.N).view(np.float16))
    return out


@pytest.mark.parametrize("nk", [2, 1, 4])
def test_group_launch_exact_arithmetic(nk):
    """Several layers of different N and K in one launch: bit-exact on grid weights."""
    rng = np.random.default_rng(40 + nk)
    shapes = [(600, 4096), (33, 4096), (1000, 2048), (77, 11008), (16, 256), (300, 4096)]
    layers = []
    for N, K in shapes:
        gs = rng.choice([32, 64, 128, 256], N).astype(np.int32)
        W = np.zeros((N, K), np.float16)
        for g in np.unique(gs):
            W[gs == g] = grid_weights(int((gs == g).sum()), K, nk, int(g), rng)
        layers.append(make_layer(W, nk, gs))
    for B in (1, 3, 16):
        say(f"case group exact nk={nk} B={B} layers={shapes}")
        Xs = []
        for N, K in shapes:
            X = np.zeros((B, K), np.float16)
            for b in range(B):
                idx = rng.choice(K, size=min(64, K), replace=False)
                X[b, idx] = rng.choice([-1.0, 1.0], len(idx))
            Xs.append(X)
        ys = _run_group_checked([lay for lay, _ in layers], Xs, B)
        for (layer, ref), X, y in zip(layers, Xs, ys):
            assert_bit_exact(y, ref.y(X)[0], (layer.desc.N, layer.desc.K, B))


def test_group_launch_many_small_layers():
    """32 layers (the maximum) in one launch: every row block lands in its own layer."""
    rng = np.random.default_rng(77)
    layers, Xs = [], []
    for i in range(32):
        N, K = int(rng.integers(1, 70)), 256 * int(rng.integers(1, 6))
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
        gs = rng.choice([32, 128], N).astype(np.int32)
        layers.append(make_layer(W, 2, gs))
        Xs.append(rng.standard_normal((2, K)).astype(np.float16))
    say("case group of 32 small layers")
    ys = _run_group_checked([lay for lay, _ in layers], Xs, 2)
    for (layer, ref), X, y in zip(layers, Xs, ys):
        assert ogemv.normalized_error(y, *ref.y(X)) <= TOL


def test_group_launch_decoder_layer():
    """The GEMVs of decoder layer 0 grouped as a decode step issues them (q, k, v; o; gate, up; down)."""
    Ls = [L for L in synth.cfg4() if L.layer == 0]
    made = {}
    for L in Ls:
        W = L.W()
        made[L.name] = (L,) + make_layer(W, L.nk, group_sizes(L, W))
    groups = [["q_proj", "k_proj", "v_proj"], ["o_proj"], ["gate_proj", "up_proj"], ["down_proj"]]
    for grp in groups:
        members = [made[f"cfg4_l00_{m}"] for m in grp]
        say(f"case group decoder layer 0: {grp}")
        ys = _run_group_checked([lay for _, lay, _ in members], [L.X(1) for L, _, _ in members], 1)
        for (L, layer, ref), y in zip(members, ys):
            err = ogemv.normalized_error(y, *ref.y(L.X(1)))
            assert err <= TOL, (L.name, err)
            if len(grp) == 1:
                # a group of one is the single call: same kernel, same geometry, same bits
                assert np.array_equal(y.view(np.uint16), run_checked(layer, L.X(1)).view(np.uint16))


@pytest.mark.parametrize("nk", [2, 1])
def test_activation_aware_pruned_layer(nk):
    """Weights pruned by |w| * ||x_k|| (sgemv_prune) through pack, layout and the
    kernel, against the oracle's scored selection quantised and multiplied in FP64."""
    from oracle import prune as oprune, groups as ogroups
    L = synth.cfg2()[0]
    W = L.W()
    Xall = L.X(72)
    Xcal, X = Xall[:64], Xall[64:]
    Wp = sg.prune(W, nk, Xcal)
    Wp_o = oprune.pruned_dense(W, oprune.nm_prune_scored(W, nk, Xcal)[1])
    assert np.array_equal(Wp.view(np.uint16), Wp_o.view(np.uint16)), "sgemv_prune differs from the oracle"
    _, mask = oprune.nm_prune(Wp_o, nk)
    gs = ogroups.select_groups(Wp_o, mask, Xcal)
    assert np.array_equal(sg.select_groups(Wp, nk, Xcal), gs)
    say(f"case activation-aware pruning nk={nk}")
    layer, ref = make_layer(Wp, nk, gs)
    y = run_checked(layer, X)
    err = ogemv.normalized_error(y, *ref.y(X))
    say(f"  normalised error {err:.3e}")
    assert err <= TOL



@pytest.mark.parametrize("L", [L for L in synth.cfg3() if L.nk == 2], ids=lambda L: L.name + "_dense")
def test_dense_ablation_within_tolerance(L):
    """Dense INT4 ablation (every element kept, same quantiser) of the MLP shapes."""
    import dataclasses
    Ld = dataclasses.replace(L, nk=4)
    W = Ld.W()
    gs = group_sizes(Ld, W)
    say(f"case dense ablation {L.name}")
    layer, ref = make_layer(W, 4, gs)
    for B in (1, 4):
        X = Ld.X(B)
        y = run_checked(layer, X)
        y_ref, D = ref.y(X)
        err = ogemv.normalized_error(y, y_ref, D)
        say(f"  B={B}: normalised error {err:.3e}")
        assert err <= TOL


@pytest.mark.parametrize("nk", [2, 1])
@pytest.mark.parametrize("N,K", [(300, 4096), (77, 11008), (16, 256), (1000, 2048), (17, 32768)])
def test_fp16_form_exact_arithmetic(nk, N, K):
    """FP16-valued form on grid weights (multiples of 2^-6, |w| <= 1/8) and 64
    entries of x in {-1, 1}: every partial sum and y (|y| <= 8) are exact, so y
    must equal the oracle's bits."""
    rng = np.random.default_rng(N + K + 7 * nk)
    W = (rng.integers(-8, 9, (N, K)) * 2.0 ** -6).astype(np.float16)
    layer, ref = make_layer_fp16(W, nk)
    say(f"case fp16 form exact nk={nk} N={N} K={K}")
    for B in (1, 3, 16):
        X = np.zeros((B, K), np.float16)
        for b in range(B):
            idx = rng.choice(K, size=min(64, K), replace=False)
            X[b, idx] = rng.choice([-1.0, 1.0], len(idx))
        y = run_checked(layer, X)
        assert_bit_exact(y, ref.y(X)[0], B)


@pytest.mark.parametrize("L", synth.cfg3(), ids=lambda L: L.name + "_fp16")
def test_fp16_form_mlp_within_tolerance(L):
    W = L.W()
    say(f"case fp16 form {L.name}")
    layer, ref = make_layer_fp16(W, L.nk)
    for B in (1, 4):
        X = L.X(B)
        y = run_checked(layer, X)
        y_ref, D = ref.y(X)
        err = ogemv.normalized_error(y, y_ref, D)
        say(f"  B={B}: normalised error {err:.3e}")
        assert err <= TOL


def test_fp16_form_group_launch():
    rng = np.random.default_rng(5)
    layers, Xs = [], []
    for N, K in [(600, 4096), (33, 4096), (256, 1024)]:
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
        layers.append(make_layer_fp16(W, 2))
        Xs.append(rng.standard_normal((2, K)).astype(np.float16))
    say("case fp16 form group launch")
    ys = _run_group_checked([lay for lay, _ in layers], Xs, 2)
    for (layer, ref), X, y in zip(layers, Xs, ys):
        assert ogemv.normalized_error(y, *ref.y(X)) <= TOL


@pytest.mark.parametrize("nk", [2, 1])
def test_large_layer_sampled_rows(nk):
    """A large layer (262144 x 4096: blobs of 0.25-0.45 GB, offsets far into
    the 32-bit range) in the launch geometry the workloads use; the oracle
    checks 64 sampled rows (uniform groups keep rows independent, so the
    oracle packs only those rows)."""
    from oracle import pack as opack
    N, K = 262144, 4096
    rng = np.random.default_rng(99 + nk)
    # 8192 random rows, tiled: the address arithmetic sees every row block
    W = np.tile((rng.standard_normal((8192, K), dtype=np.float32) * 0.02).astype(np.float16), (N // 8192, 1))
    gs = np.full(N, 128, np.int32)
    say(f"case large layer nk={nk} N={N} K={K}")
    layer = sg.SparseGemvLayer.from_dense(W, nk, gs)
    say(f"  blob {layer.desc.blob_bytes / 2**20:.0f} MiB, grid {sg.plan(layer.desc, 1).grid}")
    X = rng.standard_normal((2, K)).astype(np.float16)
    y = run_checked(layer, X)
    rows = np.concatenate([[0, 1, N - 1, N - 16, N // 2], rng.choice(N, 59, replace=False)])
    co = opack.pack_canonical(W[rows], nk, gs[rows])
    # the product's arrays for those rows equal the oracle's (uniform groups:
    # row n's scale/zero words are n * K/128 ... (n + 1) * K/128 - 1)
    for k in ("vals", "offs"):
        assert np.array_equal(layer.canon[k][rows], co[k]), k
    words = (rows[:, None] * (K // 128) + np.arange(K // 128)[None, :]).reshape(-1)
    for k in ("scale", "zero"):
        assert np.array_equal(layer.canon[k][words], co[k]), k
    Wd = ogemv.dequant_dense(co)
    y_ref, D = ogemv.gemv(Wd, X), ogemv.abs_dot(Wd, X)
    err = ogemv.normalized_error(y[:, rows], y_ref, D)
    say(f"  sampled normalised error {err:.3e}")
    assert err <= TOL
    del layer
    torch.cuda.empty_cache()


def degenerate_layer(N, K, rng):
    """Gaussian rows (std 0.02) with hand-shaped degenerate rows on every
    fifth row, cycling through: all +0; all -0; -0 among positive values;
    every group one-signed positive; every group one-signed negative; values
    x 1e-4 (FP16-subnormal values and scales); values x 3e-5 (scales that
    round below 2^-24 and are raised to it); group 0 (columns 0 .. g - 1)
    one-signed up to +65000; group 0 one-signed down to -65000. Group sizes
    cycle through 32, 64, 128, 256 (rows of every kind at every size)."""
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    gs = np.array([32, 64, 128, 256], np.int32)[rng.integers(0, 4, N)]
    special = np.arange(0, N, 5)
    for i, n in enumerate(special):
        kind = i % 9
        g = int(gs[n])
        row = rng.standard_normal(K) * 0.02
        if kind == 0:
            W[n] = np.float16(0.0)
        elif kind == 1:
            W[n] = np.float16(-0.0)
        elif kind == 2:
            r = np.abs(row).astype(np.float16)
            r[rng.random(K) < 0.5] = np.float16(-0.0)
            W[n] = r
        elif kind == 3:
            W[n] = np.abs(row).astype(np.float16)
        elif kind == 4:
            W[n] = (-np.abs(row)).astype(np.float16)
        elif kind == 5:
            W[n] = (row * 1e-4).astype(np.float16)
        elif kind == 6:
            W[n] = (row * 3e-5).astype(np.float16)
        elif kind in (7, 8):
            r = row.copy()
            r[:g] = np.abs(r[:g]) / np.max(np.abs(r[:g])) * 65000.0
            if kind == 8:
                r[:g] = -r[:g]
            W[n] = r.astype(np.float16)
    return W, gs


@pytest.mark.parametrize("nk", [2, 1, 4])
def test_degenerate_groups_every_kernel(nk):
    """Degenerate quantisation groups (all zero, -0, one-signed, FP16-subnormal
    scales, values near 65000) through the one-vector, general, several-row-
    block, dense and several-layer kernels. One-hot x: y equals the FP16
    rounding of the oracle's column bit for bit (the kernel rounds each
    dequantised weight once, as the cast of the exact value does). Gaussian
    x, scaled by 2^-8 on the columns of the large groups so that y stays in
    FP16 range: within the tolerance."""
    rng = np.random.default_rng(500 + nk)
    N, K = (10250, 2048) if nk != 4 else (1000, 2048)
    W, gs = degenerate_layer(N, K, rng)
    layer, ref = make_layer(W, nk, gs)
    s = ref.co["scale"].view(np.float16).astype(np.float64)
    assert np.any((s > 0) & (s < 2.0 ** -14)), "no FP16-subnormal scale in the layer"
    assert np.max(np.abs(ref.Wd)) > 60000
    cols = np.concatenate([[0, 1, 2, 3, 31, 32, 255, 256, K - 1], rng.choice(K, 7, replace=False)])
    for B in (1, 3, 16):
        pl = sg.plan(layer.desc, B)
        say(f"case degenerate nk={nk} B={B} one-hot row_blocks={pl.row_blocks} waves={pl.waves}")
        for c0 in range(0, len(cols), B):
            cc = cols[c0: c0 + B]
            X = np.zeros((len(cc), K), np.float16)
            X[np.arange(len(cc)), cc] = 1.0
            y = run_checked(layer, X)
            want = ref.Wd[:, cc].T.astype(np.float16)
            assert np.array_equal(y.view(np.uint16), want.view(np.uint16)), (B, cc)
    for B in (1, 3, 8, 16):
        say(f"case degenerate nk={nk} B={B} gaussian")
        X = rng.standard_normal((B, K))
        X[:, :256] *= 2.0 ** -8
        X = X.astype(np.float16)
        y = run_checked(layer, X)
        err = ogemv.normalized_error(y, *ref.y(X))
        say(f"  normalised error {err:.3e}")
        assert err <= TOL, (B, err)
    # several layers in one launch: the degenerate layer beside a small one
    Ws = (rng.standard_normal((40, 512)) * 0.02).astype(np.float16)
    small, ref_s = make_layer(Ws, nk, np.full(40, 64, np.int32))
    for B in (1, 3):
        say(f"case degenerate nk={nk} B={B} group launch")
        X = rng.standard_normal((B, K))
        X[:, :256] *= 2.0 ** -8
        X = X.astype(np.float16)
        Xs = rng.standard_normal((B, 512)).astype(np.float16)
        y, ys = _run_group_checked([layer, small], [X, Xs], B)
        assert ogemv.normalized_error(y, *ref.y(X)) <= TOL
        assert ogemv.normalized_error(ys, *ref_s.y(Xs)) <= TOL


def test_stale_hip_error_is_not_reported_by_a_good_launch():
    """A HIP error left on this thread by an earlier, unrelated runtime call
    does not come back as SGEMV_EHIP from launches that succeed (each entry
    point is called right after the error is planted, with no other runtime
    call in between)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")      # the runtime this process already uses
    rng = np.random.default_rng(31)
    W = (rng.standard_normal((100, 1024)) * 0.02).astype(np.float16)
    layer, ref = make_layer(W, 2, np.full(100, 128, np.int32))
    X = rng.standard_normal((2, 1024)).astype(np.float16)
    x = torch.from_numpy(X).cuda()
    ys = [torch.zeros((2, 100), dtype=torch.float16, device="cuda") for _ in range(3)]
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    dst = torch.zeros(64, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    say("case stale HIP error before sgemv_run / sgemv_run_group / probes")

    def plant():
        assert hip.hipSetDevice(ctypes.c_int(1 << 20)) != 0     # leaves hipErrorInvalidDevice behind

    plant()
    sg.run(layer.desc, layer.blob.data_ptr(), x.data_ptr(), ys[0].data_ptr(), 1, s)   # raises on a non-zero status
    plant()
    sg.run(layer.desc, layer.blob.data_ptr(), x.data_ptr(), ys[1].data_ptr(), 2, s)
    plant()
    sg.run_group([(layer.desc, layer.blob.data_ptr(), x.data_ptr(), ys[2].data_ptr())], 2, s)
    plant()
    sg.probe_read(buf.data_ptr(), buf.numel(), dst.data_ptr(), 16, stream=s)
    plant()
    sg.probe_empty(1, 64, s)
    assert hip.hipGetLastError() == 0          # each entry point cleared what it found
    torch.cuda.synchronize()
    y_ref, D = ref.y(X)
    assert ogemv.normalized_error(ys[0].cpu().numpy()[:1], y_ref[:1], D[:1]) <= TOL
    assert ogemv.normalized_error(ys[1].cpu().numpy(), y_ref, D) <= TOL
    assert ogemv.normalized_error(ys[2].cpu().numpy(), y_ref, D) <= TOL


def test_measurement_probes():
    """The plain-read probe folds each lane's 16 bytes into one word (XOR of
    its four words) and stores the words of the first store_bytes / 4 lanes;
    the empty probe launches and returns."""
    rng = np.random.default_rng(32)
    nbytes = 3 * 4096 + 48                       # a last, partial workgroup
    host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    dst = torch.full((300,), -1, dtype=torch.int32, device="cuda")
    say("case probes: read 12336 bytes, store 1024 bytes")
    s = torch.cuda.current_stream().cuda_stream
    magic = 0x9E3779B9                           # no lane's word equals it (checked below)
    sg.probe_read(src.data_ptr(), nbytes, dst.data_ptr(), 1024, magic=magic, stream=s)
    sg.probe_empty(4, 256, s)
    torch.cuda.synchronize()
    fold = np.bitwise_xor.reduce(host.reshape(-1, 4), axis=1)
    assert not np.any(fold == magic)
    got = dst.cpu().numpy().view(np.uint32)
    assert np.array_equal(got[:256], fold[:256])
    assert np.all(got[256:] == 0xFFFFFFFF)     # only the 256 store lanes wrote
    with pytest.raises(sg.SgemvError):
        sg.probe_read(src.data_ptr(), nbytes + 8, dst.data_ptr(), 0, stream=s)
    with pytest.raises(sg.SgemvError):
        sg.probe_empty(1, 100, s)


def _run_list_checked(layers, Xs, guard=64, table=False):
    """One sgemv_run_list launch over one-vector layers (guarded outputs); with
    ``table``, one sgemv_run_list_table launch from a device task table."""
    sentinel = np.uint16(0x7E5A)
    bufs, tasks, xs = [], [], []
    for layer, X in zip(layers, Xs):
        N = layer.desc.N
        x = torch.from_numpy(np.ascontiguousarray(X)).cuda()
        ybuf = torch.full((N + 2 * guard,), int(np.int16(sentinel.view(np.int16))), dtype=torch.int16, device="cuda")
        xs.append(x)
        bufs.append(ybuf)
        tasks.append((layer.desc, layer.blob.data_ptr(), x.data_ptr(), ybuf[guard:].data_ptr()))
    if table:
        host, launch = sg.list_table(tasks, 1)
        say(f"  table launch: {launch.tasks} tasks, {launch.rows} rows of {launch.row_width}, "
            f"{launch.workgroups} workgroups")
        tdev = torch.from_numpy(host).cuda()
        sg.run_list_table(tdev.data_ptr(), launch, torch.cuda.current_stream().cuda_stream)
    else:
        sg.run_list(tasks, 1, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    out = []
    for layer, ybuf in zip(layers, bufs):
        host = ybuf.cpu().numpy().view(np.uint16)
        assert np.all(host[:guard] == sentinel) and np.all(host[-guard:] == sentinel), "y guard band overwritten"
        out.append(host[guard: guard + layer.desc.N].reshape(1, layer.desc.N).view(np.float16))
    return out


def test_list_launch_exact_arithmetic():
    """Layers of different N, K and N:M in one task-list launch: bit-exact on
    grid weights with x in {-1, 0, 1}; row-block runs of one to many blocks
    per workgroup, layers of 1 to 128 column chunks (K = 32768, the largest:
    64 KiB of x in LDS), ragged last blocks. The same launch with the tasks
    in reverse order gives the same bits per layer."""
    rng = np.random.default_rng(61)
    specs = [(600, 4096, 2), (33, 4096, 1), (1000, 2048, 1), (77, 11008, 2), (16, 256, 2), (300, 4096, 1),
             (4100, 1024, 2), (5, 768, 1), (2000, 11008, 1), (40, 32768, 2), (17, 32768, 1)]
    layers, Xs = [], []
    for N, K, nk in specs:
        gs = rng.choice([32, 64, 128, 256], N).astype(np.int32)
        W = np.zeros((N, K), np.float16)
        for g in np.unique(gs):
            W[gs == g] = grid_weights(int((gs == g).sum()), K, nk, int(g), rng)
        layers.append(make_layer(W, nk, gs))
        X = np.zeros((1, K), np.float16)
        idx = rng.choice(K, size=min(64, K), replace=False)
        X[0, idx] = rng.choice([-1.0, 1.0], len(idx))
        Xs.append(X)
    pl = sg.plan_list([(lay.desc, 0, 0, 0) for lay, _ in layers], 1)
    say(f"case list exact, {len(specs)} layers: grid={pl.grid} waves={pl.waves} cpw={pl.chunks_per_wave}")
    ys = _run_list_checked([lay for lay, _ in layers], Xs)
    for (layer, ref), X, y in zip(layers, Xs, ys):
        assert_bit_exact(y, ref.y(X)[0], (layer.desc.N, layer.desc.K, layer.desc.nk))
    ys2 = _run_list_checked([lay for lay, _ in layers], Xs)
    for y, y2 in zip(ys, ys2):
        assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))
    ys3 = _run_list_checked([lay for lay, _ in layers][::-1], Xs[::-1])[::-1]
    for y, y3 in zip(ys, ys3):
        assert np.array_equal(y.view(np.uint16), y3.view(np.uint16))


def test_list_table_exact_arithmetic():
    """The layers of the exact-arithmetic list case through a task table in
    device memory: bit-exact against the oracle, and the same bits as the
    kernel-argument launch of the same tasks."""
    rng = np.random.default_rng(63)
    specs = [(600, 4096, 2), (33, 4096, 1), (1000, 2048, 1), (77, 11008, 2), (16, 256, 2), (300, 4096, 1),
             (4100, 1024, 2), (5, 768, 1), (2000, 11008, 1), (40, 32768, 2), (17, 32768, 1)]
    layers, Xs = [], []
    for N, K, nk in specs:
        gs = rng.choice([32, 64, 128, 256], N).astype(np.int32)
        W = np.zeros((N, K), np.float16)
        for g in np.unique(gs):
            W[gs == g] = grid_weights(int((gs == g).sum()), K, nk, int(g), rng)
        layers.append(make_layer(W, nk, gs))
        X = np.zeros((1, K), np.float16)
        idx = rng.choice(K, size=min(64, K), replace=False)
        X[0, idx] = rng.choice([-1.0, 1.0], len(idx))
        Xs.append(X)
    say(f"case list table exact, {len(specs)} layers")
    ys = _run_list_checked([lay for lay, _ in layers], Xs, table=True)
    for (layer, ref), X, y in zip(layers, Xs, ys):
        assert_bit_exact(y, ref.y(X)[0], (layer.desc.N, layer.desc.K, layer.desc.nk))
    ys2 = _run_list_checked([lay for lay, _ in layers], Xs)
    for y, y2 in zip(ys, ys2):
        assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))


def test_list_table_decoder_step():
    """All 224 GEMVs of the 32-layer decoder set as one table launch (the
    launch bench.py times; each GEMV with its own x and y, the weights of one
    (shape, N:M) pair shared): within the tolerance of the oracle for every
    GEMV, the same bits as five kernel-argument launches of 48 and on a
    second table launch."""
    made, layers, Xs = {}, [], []
    for L in synth.cfg4():
        key = (L.K, L.N, L.nk)
        if key not in made:
            W = L.W()
            made[key] = make_layer(W, L.nk, group_sizes(L, W))
        layers.append(made[key])
        Xs.append(L.X(1))
    say(f"case list table: decoder step, {len(layers)} GEMVs, {len(made)} weight sets")
    ys = _run_list_checked([lay for lay, _ in layers], Xs, table=True)
    for (layer, ref), X, y in zip(layers, Xs, ys):
        assert ogemv.normalized_error(y, *ref.y(X)) <= TOL, (layer.desc.N, layer.desc.K, layer.desc.nk)
    ys2 = []
    for i in range(0, len(layers), sg.LIST_MAX):
        ys2 += _run_list_checked([lay for lay, _ in layers[i: i + sg.LIST_MAX]], Xs[i: i + sg.LIST_MAX])
    ys3 = _run_list_checked([lay for lay, _ in layers], Xs, table=True)
    for y, y2, y3 in zip(ys, ys2, ys3):
        assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))
        assert np.array_equal(y.view(np.uint16), y3.view(np.uint16))


def test_list_table_many_small_tasks():
    """600 small layers (1 to 200 rows, 256 to 2048 columns, 2:4 and 1:4
    mixed) and the degenerate-groups layer as one table launch: many tasks
    of one or two workgroups, rows of the table shared by none; within the
    tolerance of the oracle, the same bits as kernel-argument launches of 48."""
    rng = np.random.default_rng(64)
    layers, Xs = [], []
    for i in range(600):
        N, K = int(rng.integers(1, 201)), 256 * int(rng.integers(1, 9))
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
        layers.append(make_layer(W, int(rng.choice([1, 2])), rng.choice([32, 64, 128, 256], N).astype(np.int32)))
        Xs.append(rng.standard_normal((1, K)).astype(np.float16))
    Wd, gs = degenerate_layer(3000, 2048, rng)
    layers.append(make_layer(Wd, 2, gs))
    X = rng.standard_normal((1, 2048))
    X[:, :256] *= 2.0 ** -8
    Xs.append(X.astype(np.float16))
    say(f"case list table: {len(layers)} small layers")
    ys = _run_list_checked([lay for lay, _ in layers], Xs, table=True)
    for (layer, ref), X, y in zip(layers, Xs, ys):
        assert ogemv.normalized_error(y, *ref.y(X)) <= TOL, (layer.desc.N, layer.desc.K)
    for i in range(0, len(layers), sg.LIST_MAX):
        part = _run_list_checked([lay for lay, _ in layers[i: i + sg.LIST_MAX]], Xs[i: i + sg.LIST_MAX])
        for y, y2 in zip(ys[i: i + sg.LIST_MAX], part):
            assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))


def test_list_table_most_tasks():
    """SGEMV_LIST_TABLE_MAX (4096) layers of 1 to 48 rows and 256 or 512
    columns, 2:4 and 1:4 mixed, as one table launch: within the tolerance of
    the oracle, and the same bits for the first 48 as a kernel-argument
    launch of them."""
    rng = np.random.default_rng(65)
    layers, Xs = [], []
    for i in range(sg.LIST_TABLE_MAX):
        N, K = int(rng.integers(1, 49)), 256 * int(rng.integers(1, 3))
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
        layers.append(make_layer(W, int(rng.choice([1, 2])), rng.choice([32, 64, 128, 256], N).astype(np.int32)))
        Xs.append(rng.standard_normal((1, K)).astype(np.float16))
    say(f"case list table: {len(layers)} layers, the most a table takes")
    ys = _run_list_checked([lay for lay, _ in layers], Xs, table=True)
    for (layer, ref), X, y in zip(layers, Xs, ys):
        assert ogemv.normalized_error(y, *ref.y(X)) <= TOL, (layer.desc.N, layer.desc.K)
    part = _run_list_checked([lay for lay, _ in layers[:sg.LIST_MAX]], Xs[:sg.LIST_MAX])
    for y, y2 in zip(ys, part):
        assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))


def test_list_launch_mlp_layers_and_single_tasks():
    """The four MLP layers (up/down at 1:4 and 2:4, adaptive groups) as one
    list launch, and each alone (every workgroup then walks many blocks):
    within the tolerance, the same bits on a second run."""
    made = []
    for L in synth.cfg3():
        W = L.W()
        made.append((L,) + make_layer(W, L.nk, group_sizes(L, W)))
    say("case list: the four MLP layers in one launch")
    ys = _run_list_checked([lay for _, lay, _ in made], [L.X(1) for L, _, _ in made])
    for (L, layer, ref), y in zip(made, ys):
        err = ogemv.normalized_error(y, *ref.y(L.X(1)))
        say(f"  {L.name}: normalised error {err:.3e}")
        assert err <= TOL, (L.name, err)
    for L, layer, ref in made:
        say(f"case list: {L.name} alone, grid {sg.plan_list([(layer.desc, 0, 0, 0)], 1).grid}")
        (y,) = _run_list_checked([layer], [L.X(1)])
        assert ogemv.normalized_error(y, *ref.y(L.X(1))) <= TOL
        (y2,) = _run_list_checked([layer], [L.X(1)])
        assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))


def test_list_launch_decoder_layers():
    """Decoder layers 3 (2:4) and 4 (1:4) of the 32-layer set: 14 GEMVs with
    their own x in one launch, against the oracle."""
    made = []
    for L in synth.cfg4():
        if L.layer in (3, 4):
            W = L.W()
            made.append((L,) + make_layer(W, L.nk, group_sizes(L, W)))
    say(f"case list: decoder layers 3 and 4, {len(made)} GEMVs")
    ys = _run_list_checked([lay for _, lay, _ in made], [L.X(1) for L, _, _ in made])
    for (L, layer, ref), y in zip(made, ys):
        err = ogemv.normalized_error(y, *ref.y(L.X(1)))
        assert err <= TOL, (L.name, err)


def test_list_launch_most_tasks():
    """SGEMV_LIST_MAX (48) small layers in one launch, and the degenerate
    groups layer among them."""
    rng = np.random.default_rng(62)
    layers, Xs = [], []
    for i in range(sg.LIST_MAX - 1):
        N, K = int(rng.integers(1, 90)), 256 * int(rng.integers(1, 12))
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
        layers.append(make_layer(W, int(rng.choice([1, 2])), rng.choice([32, 64, 128, 256], N).astype(np.int32)))
        Xs.append(rng.standard_normal((1, K)).astype(np.float16))
    Wd, gs = degenerate_layer(3000, 2048, rng)
    layers.append(make_layer(Wd, 1, gs))
    X = rng.standard_normal((1, 2048))
    X[:, :256] *= 2.0 ** -8
    Xs.append(X.astype(np.float16))
    say(f"case list: {len(layers)} layers")
    ys = _run_list_checked([lay for lay, _ in layers], Xs)
    for (layer, ref), X, y in zip(layers, Xs, ys):
        assert ogemv.normalized_error(y, *ref.y(X)) <= TOL, (layer.desc.N, layer.desc.K)


def _guarded(host_bytes, guard, fill):
    """Device copy of host bytes between two sentinel bands (the copy stays 256-byte aligned)."""
    buf = torch.full((host_bytes.size + 2 * guard,), fill, dtype=torch.uint8, device="cuda")
    buf[guard: guard + host_bytes.size] = torch.from_numpy(np.ascontiguousarray(host_bytes)).cuda()
    return buf


def _bands_intact(buf, n, guard, fill):
    h = buf.cpu().numpy()
    return np.all(h[:guard] == fill) and np.all(h[guard + n:] == fill)


@pytest.mark.parametrize("case", ["b1_2of4", "b1_1of4", "general_B3", "rows_B16", "dense_B1", "fp16_B2", "group_B1",
                                  "list_B1"])
def test_inputs_untouched_and_guard_bands(case):
    """The kernels only read the blob and x: sentinel bands around both (and
    the bytes themselves) are unchanged after a launch, and y is right."""
    rng = np.random.default_rng(sum(map(ord, case)))
    N, K, nk, B = {"b1_2of4": (300, 4096, 2, 1), "b1_1of4": (300, 11008, 1, 1), "general_B3": (200, 2048, 2, 3),
                   "rows_B16": (10250, 2048, 1, 16), "dense_B1": (64, 1024, 4, 1), "fp16_B2": (100, 1024, 2, 2),
                   "group_B1": (500, 4096, 1, 1), "list_B1": (700, 4096, 2, 1)}[case]
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    if case == "fp16_B2":
        layer, ref = make_layer_fp16(W, nk)
    else:
        layer, ref = make_layer(W, nk, rng.choice([32, 128], N).astype(np.int32))
    X = rng.standard_normal((B, K)).astype(np.float16)
    G, FILL = 256, 0xA5
    blob = _guarded(layer.blob_host, G, FILL)
    xb = _guarded(X.view(np.uint8).reshape(-1), G, FILL)
    y = torch.zeros((B, N), dtype=torch.float16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    say(f"case guard bands {case}")
    task = (layer.desc, blob[G:].data_ptr(), xb[G:].data_ptr(), y.data_ptr())
    if case.startswith("group"):
        sg.run_group([task], B, s)
    elif case.startswith("list"):
        sg.run_list([task], B, s)
    else:
        sg.run(layer.desc, blob[G:].data_ptr(), xb[G:].data_ptr(), y.data_ptr(), B, s)
    torch.cuda.synchronize()
    assert _bands_intact(blob, layer.blob_host.size, G, FILL) and _bands_intact(xb, X.nbytes, G, FILL)
    assert np.array_equal(blob[G: G + layer.blob_host.size].cpu().numpy(), layer.blob_host)
    assert np.array_equal(xb[G: G + X.nbytes].cpu().numpy().view(np.float16).reshape(B, K), X)
    assert ogemv.normalized_error(y.cpu().numpy(), *ref.y(X)) <= TOL

"""Pins oracle.pack: hand-packed rows, round trips, closed-form sizes, the 30 % claim."""
import numpy as np
import pytest

from oracle import pack, prune, quant, groups, gemv
from conftest import read_golden


def test_pack_bytes_hand_example():
    q = np.array([[1, 2, 3, 4, 5, 6, 7, 8]], dtype=np.uint8)
    o = np.array([[0, 3, 1, 2, 3, 3, 0, 1]], dtype=np.uint8)
    vals, offs = pack.pack_bytes(q, o)
    assert vals.tolist() == [[0x21, 0x43, 0x65, 0x87]]          # low nibble = even element
    # byte 0: 0 | 3<<2 | 1<<4 | 2<<6 = 0x9C ; byte 1: 3 | 3<<2 | 0<<4 | 1<<6 = 0x4F
    assert offs.tolist() == [[0x9C, 0x4F]]
    q2, o2 = pack.unpack_bytes(vals, offs)
    assert np.array_equal(q2, q) and np.array_equal(o2, o)


def test_hand_packed_rows_golden():
    for rec in read_golden("pack_hand.txt"):
        grp = np.array([float(t) for t in rec["group"].split()], dtype=np.float16)
        W = np.tile(grp, 64)[None, :]
        nk = int(rec["nk"])
        c = pack.pack_canonical(W, nk, [128])
        assert np.all(c["vals"] == int(rec["vals_byte"], 16)) and c["vals"].shape == (1, 32 * nk)
        assert np.all(c["offs"] == int(rec["offs_byte"], 16)) and c["offs"].shape == (1, 16 * nk)
        assert c["scale"].tolist() == [int(rec["scale"], 16)] * 2
        assert c["zero"].tolist() == [int(rec["zero"], 16)] * 2
        assert c["gptr"].tolist() == [0, 2]
        assert c["rowptr"].tolist() == [0, 64 * nk]


@pytest.mark.parametrize("nk", [1, 2, 4])
def test_round_trip_and_sizes(nk):
    rng = np.random.default_rng(nk)
    N, K = 37, 512
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    gs = np.where(rng.random(N) < 0.3, 32, 128).astype(np.int32)
    c = pack.pack_canonical(W, nk, gs)
    sz = pack.sizes(N, K, nk, gs)
    assert c["vals"].size == sz["vals_bytes"] == N * K * nk // 8
    assert c["offs"].size == sz["offs_bytes"] == (0 if nk == 4 else N * K * nk // 16)
    assert c["scale"].size == c["zero"].size == sz["n_groups"] == int(np.sum(K // gs))
    assert c["gptr"][-1] == sz["n_groups"]
    q, o = pack.unpack_bytes(c["vals"], c["offs"])
    offs3, mask = prune.nm_prune(W, nk)
    if nk == 4:
        assert mask.all() and np.array_equal(offs3.reshape(N, -1), np.tile(np.arange(4), (N, K // 4)))
    else:
        assert np.array_equal(o, offs3.reshape(N, -1))
    # re-quantising each group of the kept values gives the stored codes/scales
    kept = prune.kept_values(W, offs3)
    for n in range(N):
        g = int(gs[n])
        m = g * nk // 4
        s16, z16, qq = quant.quantize_groups(kept[n].reshape(K // g, m))
        lo, hi = c["gptr"][n], c["gptr"][n + 1]
        assert np.array_equal(s16.view(np.uint16), c["scale"][lo:hi])
        assert np.array_equal(z16.view(np.uint16), c["zero"][lo:hi])
        assert np.array_equal(qq.reshape(-1), q[n])


def test_thirty_percent_of_csr():
    """Index + value bits of 2bit-CSR vs INT4 + int16 column index CSR = 6/20 = 30 %."""
    for nk in (1, 2):
        sz = pack.sizes(64, 1024, nk, [128] * 64)
        bits_2bit_csr = 8 * (sz["vals_bytes"] + sz["offs_bytes"])
        bits_csr = sz["kept"] * (4 + 16)
        assert bits_2bit_csr * 10 == bits_csr * 3


def test_rejects_bad_groups():
    W = np.zeros((2, 256), dtype=np.float16)
    for gs in ([48, 128], [128], [512, 128]):
        with pytest.raises(ValueError):
            pack.pack_canonical(W, 2, gs)


def test_fp16_valued_form_hand_example_and_round_trip():
    """FP16-valued 2bit-CSR: kept values as FP16 bits, same offsets as the INT4 form."""
    W = np.zeros((1, 256), dtype=np.float16)
    W[0, :8] = [0.5, -2.0, 0.25, 1.0, 0.0, -0.0, 3.0, -3.0]
    c = pack.pack_fp16_canonical(W, 2)
    # group 0 keeps -2 (col 1) and 1 (col 3); group 1 keeps 3 and -3 (cols 6, 7):
    # values -2, 1, 3, -3 (bits 0xC000, 0x3C00, 0x4200, 0xC200), offsets 1, 3, 2, 3
    assert c["vals16"][0, :4].tolist() == [0xC000, 0x3C00, 0x4200, 0xC200]
    assert c["offs"][0, 0] == (1 | 3 << 2 | 2 << 4 | 3 << 6)
    c1 = pack.pack_fp16_canonical(W, 1)
    assert c1["vals16"][0, :2].tolist() == [0xC000, 0x4200]          # -2 at col 1, 3 at col 6 (tie -> lower)
    rng = np.random.default_rng(4)
    Wr = (rng.standard_normal((9, 512)) * 0.02).astype(np.float16)
    for nk in (1, 2):
        c = pack.pack_fp16_canonical(Wr, nk)
        assert c["vals16"].size * 2 == 9 * 512 * nk // 4 * 2 and c["offs"].size == 9 * 512 * nk // 16
        _, mask = prune.nm_prune(Wr, nk)
        assert np.array_equal(gemv.dequant_dense(c), np.where(mask, Wr.astype(np.float64), 0.0))

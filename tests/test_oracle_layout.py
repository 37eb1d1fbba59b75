"""Pins oracle.layout: hand-placed bytes and decode(build(.)) == identity."""
import numpy as np
import pytest

from oracle import layout, pack


def synthetic_canon(N, K, nk, gs, seed=0):
    """Canonical arrays filled with arbitrary codes/offsets (no quantisation needed)."""
    rng = np.random.default_rng(seed)
    kpr = K * nk // 4
    q = rng.integers(0, 16, (N, kpr)).astype(np.uint8)
    o = rng.integers(0, 4, (N, kpr)).astype(np.uint8)
    vals, offs = pack.pack_bytes(q, o)
    gs = np.asarray(gs, dtype=np.int32)
    gptr = np.zeros(N + 1, dtype=np.int64)
    gptr[1:] = np.cumsum(K // gs)
    ng = int(gptr[-1])
    return {"N": N, "K": K, "nk": nk, "group_size": gs, "vals": vals, "offs": offs,
            "scale": rng.integers(0, 65536, ng).astype(np.uint16),
            "zero": rng.integers(0, 65536, ng).astype(np.uint16),
            "gptr": gptr.astype(np.int32)}, q, o


def test_hand_placed_bytes():
    N, K, nk = 2, 256, 2                      # C = 4 chunks per row
    kpr = K * nk // 4
    q = np.array([[(j + n) % 16 for j in range(kpr)] for n in range(N)], dtype=np.uint8)
    o = np.array([[j % 4 for j in range(kpr)] for n in range(N)], dtype=np.uint8)
    vals, offs = pack.pack_bytes(q, o)
    canon = {"N": N, "K": K, "nk": nk, "group_size": np.array([128, 128], np.int32),
             "vals": vals, "offs": offs,
             "scale": np.array([0x1111, 0x2222, 0x3333, 0x4444], np.uint16),
             "zero": np.array([0xAAAA, 0xBBBB, 0xCCCC, 0xDDDD], np.uint16),
             "gptr": np.array([0, 2, 4], np.int32)}
    L = layout.build(canon, RT=2, TPR=4)
    # one tile, one iteration: chunk c of row r sits at slot r*4 + c
    # slot 0, dword 0 = elements 0..7 of row 0 (codes 0..7); nibble k holds
    # element [0,2,4,6,1,3,5,7][k] -> 0x75316420
    assert L["vals"][0][:4].tolist() == [0x20, 0x64, 0x31, 0x75]
    # slot 5 = row 1, chunk 1: elements 32..39 of row 1 have codes (j+1)%16 = 1..8
    # nibbles [1,3,5,7,2,4,6,8] -> 0x86427531
    assert L["vals"][5][:4].tolist() == [0x31, 0x75, 0x42, 0x86]
    # offsets j%4: element 4q+b at bits 8b+2q -> byte b = b*0x55
    assert L["offs"][0].tolist() == [0x00, 0x55, 0xAA, 0xFF] * 2
    # group 128 covers two 64-column chunks at 2:4: slots (0,1) share entry 0
    assert L["sz"].tolist() == [0xAAAA1111, 0xBBBB2222, 0xCCCC3333, 0xDDDD4444]
    assert L["tiles"].tolist() == [[0, 2, 128, 0]]
    assert L["perm"].tolist() == [0, 1]
    off = L["offsets"]
    assert off["perm"] == 256 and off["vals"] == 512 and off["offs"] == 512 + 256
    assert off["sz"] == 512 + 256 + 256 and off["blob_bytes"] == 1280


def test_hand_ragged_slot():
    # K=768 at 2:4 -> C = 12; TPR = 8 -> iterations of 8 and 4 chunks
    N, K, nk = 2, 768, 2
    canon, q, o = synthetic_canon(N, K, nk, [128, 128], seed=4)
    L = layout.build(canon, RT=2, TPR=8)
    # row 1, chunk 9 -> i = 1, kl = 1, cnt = 4 -> slot 1*2*8 + 1*4 + 1 = 21
    e = 32 * 9 + np.array([0, 2, 4, 6, 1, 3, 5, 7])
    want = sum(int(q[1, e[k]]) << (4 * k) for k in range(8))
    got = int.from_bytes(L["vals"][21][:4].tobytes(), "little")
    assert got == want


def test_row_order_and_tiles():
    gs = np.array([128, 32, 128, 32, 64, 128, 32], dtype=np.int32)
    assert layout.row_order(gs).tolist() == [1, 3, 6, 4, 0, 2, 5]
    assert layout.tile_list(gs, 2) == [(0, 2, 32), (2, 1, 32), (3, 1, 64), (4, 2, 128), (6, 1, 128)]


@pytest.mark.parametrize("N,K,nk,RT,TPR", [
    (7, 256, 2, 4, 4), (9, 768, 2, 2, 8), (11, 768, 1, 4, 4), (5, 1024, 1, 16, 16),
    (13, 2816, 2, 4, 16), (6, 2816, 1, 8, 32), (3, 512, 2, 1, 64),
])
def test_decode_inverts_build(N, K, nk, RT, TPR):
    rng = np.random.default_rng(N * K + nk)
    choices = [g for g in (32, 64, 128, 256) if K % g == 0 and
               (g <= 128 // nk or (TPR % (g // (128 // nk)) == 0 and (K * nk // 128) % (g // (128 // nk)) == 0))]
    gs = rng.choice(choices, N).astype(np.int32)
    canon, q, o = synthetic_canon(N, K, nk, gs, seed=N)
    L = layout.build(canon, RT, TPR)
    q2, o2, szr, perm = layout.decode(L["blob"], N, K, nk, RT, TPR)
    assert np.array_equal(q2, q) and np.array_equal(o2, o)
    sz = canon["scale"].astype(np.uint32) | (canon["zero"].astype(np.uint32) << 16)
    for n in range(N):
        assert np.array_equal(szr[n], sz[canon["gptr"][n]: canon["gptr"][n + 1]])
    assert sorted(perm.tolist()) == list(range(N))

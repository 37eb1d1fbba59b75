"""Pins oracle.layout: hand-placed bytes, row order, record order and
decode(build(.)) == identity over ragged and mixed-class shapes."""
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
    if nk == 4:
        offs = np.zeros((N, 0), np.uint8)
    gs = np.asarray(gs, dtype=np.int32)
    gptr = np.zeros(N + 1, dtype=np.int64)
    gptr[1:] = np.cumsum(K // gs)
    ng = int(gptr[-1])
    return {"N": N, "K": K, "nk": nk, "group_size": gs, "vals": vals, "offs": offs,
            "scale": rng.integers(0, 65536, ng).astype(np.uint16),
            "zero": rng.integers(0, 65536, ng).astype(np.uint16),
            "gptr": gptr.astype(np.int32)}, q, o


def u32_at(blob, at):
    return int.from_bytes(blob[at: at + 4].tobytes(), "little")


def test_hand_placed_bytes_2of4():
    N, K, nk = 2, 256, 2                      # one row block, one column chunk
    kpr = K * nk // 4
    q = np.array([[(j + n) % 16 for j in range(kpr)] for n in range(N)], dtype=np.uint8)
    o = np.array([[j % 4 for j in range(kpr)] for n in range(N)], dtype=np.uint8)
    vals, offs = pack.pack_bytes(q, o)
    canon = {"N": N, "K": K, "nk": nk, "group_size": np.array([128, 128], np.int32),
             "vals": vals, "offs": offs,
             "scale": np.array([0x1111, 0x2222, 0x3333, 0x4444], np.uint16),
             "zero": np.array([0xAAAA, 0xBBBB, 0xCCCC, 0xDDDD], np.uint16),
             "gptr": np.array([0, 2, 4], np.int32)}
    L = layout.build(canon)
    off = L["offsets"]
    # records of 64 lanes x 16 bytes: 1024 bytes of codes, then 512 of offsets,
    # 64 of perm (16 rows) and 4 words + 8 spare bytes of scale|zero
    assert (off["codes"], off["offs"], off["perm"], off["sz"], off["blob_bytes"]) == (0, 1024, 1536, 1792, 2048)
    blob = L["blob"]
    # lane 0 = row 0, columns 0..63 = kept elements 0..31; dword 0 = elements
    # 0..7 (codes 0..7) with element k at nibble [0,4,1,5,2,6,3,7][k]:
    # nibbles 0..7 hold 0,2,4,6,1,3,5,7 -> 0x75316420
    assert u32_at(blob, 0) == 0x75316420
    # lane 17 = row 1, columns 64..127 = elements 32..63; dword 0 = elements
    # 32..39 with codes (j+1)%16 = 1..8 -> nibbles 1,3,5,7,2,4,6,8 -> 0x86427531
    assert u32_at(blob, 17 * 16) == 0x86427531
    # lane 48 = row 0, columns 192..255 = elements 96..127; dword 3 = elements
    # 120..127, codes 8..15 -> nibbles 8,10,12,14,9,11,13,15 -> 0xFDB9ECA8
    assert u32_at(blob, 48 * 16 + 12) == 0xFDB9ECA8
    # offsets at 2:4 are the canonical bytes: offsets 0,1,2,3 at bits 0,2,4,6 -> 0xE4
    assert blob[1024: 1024 + 8].tolist() == [0xE4] * 8
    assert np.frombuffer(blob[1536: 1600].tobytes(), "<i4").tolist() == [0, 1] + [-1] * 14
    # one record: row 0 with its 2 words of chunk 0, then row 1 with its 2
    assert [u32_at(blob, 1792 + 4 * i) for i in range(4)] == [0xAAAA1111, 0xBBBB2222, 0xCCCC3333, 0xDDDD4444]
    assert blob[1808: 2048].tolist() == [0] * 240


def test_hand_placed_bytes_1of4():
    N, K, nk = 1, 256, 1                      # 64 kept elements, 16 per piece
    kpr = K * nk // 4
    q = np.array([[j % 16 for j in range(kpr)]], dtype=np.uint8)
    o = np.array([[(j // 4) % 4 for j in range(kpr)]], dtype=np.uint8)
    vals, offs = pack.pack_bytes(q, o)
    canon = {"N": N, "K": K, "nk": nk, "group_size": np.array([256], np.int32), "vals": vals, "offs": offs,
             "scale": np.array([0x3C00], np.uint16), "zero": np.array([0x4800], np.uint16),
             "gptr": np.array([0, 1], np.int32)}
    L = layout.build(canon)
    off = L["offsets"]
    # 64 lanes x 12 bytes (2 code dwords, then the offset dword) = 768 bytes of
    # codes; the offset section is empty; 64 bytes of perm; the scale|zero word
    assert (off["codes"], off["offs"], off["perm"], off["sz"], off["blob_bytes"]) == (0, 768, 768, 1024, 1280)
    blob = L["blob"]
    # lane 16 = columns 64..127 = elements 16..31; dword 0 = elements 16..23 with
    # codes 0..7, element k at nibble [0,1,4,5,2,3,6,7][k]: nibbles 0..7 hold
    # 0,1,4,5,2,3,6,7 -> 0x76325410
    assert u32_at(blob, 16 * 12) == 0x76325410
    # lane 0 offsets, its third dword: element m = 4t + e has offset t and sits
    # at bit 16*(t%2) + ([0,4,10,14] if t < 2 else [2,6,8,12])[e]:
    # t=1 -> 1 at bits 16,20,26,30 = 0x44110000; t=2 -> 2 at bits 2,6,8,12 =
    # 0x00002288; t=3 -> 3 at bits 18,22,24,28 = 0x33CC0000
    assert u32_at(blob, 8) == 0x77DD2288
    # lane 1 (the padding row 1, no data) is all zero, then lane 16's codes
    assert blob[12: 24].tolist() == [0] * 12
    assert u32_at(blob, 1024) == 0x48003C00
    assert np.frombuffer(blob[768: 832].tobytes(), "<i4").tolist() == [0] + [-1] * 15


def test_row_order_and_mixed_class_record():
    gs = np.array([128, 32, 128, 32, 64, 128, 32], dtype=np.int32)
    assert layout.row_order(gs).tolist() == [1, 3, 6, 4, 0, 2, 5]
    N, K = 7, 256
    gptr = np.concatenate([[0], np.cumsum(K // gs)]).astype(np.int32)
    ng = int(gptr[-1])
    assert ng == 3 * 8 + 4 + 3 * 2
    kpr = K * 2 // 4
    vals, offs = pack.pack_bytes(np.zeros((N, kpr), np.uint8), np.zeros((N, kpr), np.uint8))
    canon = {"N": N, "K": K, "nk": 2, "group_size": gs, "vals": vals, "offs": offs,
             "scale": np.arange(ng, dtype=np.uint16), "zero": np.zeros(ng, np.uint16), "gptr": gptr}
    L = layout.build(canon)
    # one record: rows in sorted order 1, 3, 6 (8 words each), 4 (4), 0, 2, 5 (2 each)
    want = (list(range(gptr[1], gptr[2])) + list(range(gptr[3], gptr[4])) + list(range(gptr[6], gptr[7]))
            + list(range(gptr[4], gptr[5])) + list(range(gptr[0], gptr[1])) + list(range(gptr[2], gptr[3]))
            + list(range(gptr[5], gptr[6])))
    assert L["sz"].tolist() == want


def test_records_follow_chunks_within_a_block():
    # K = 512: two chunks; a g32 row has 8 words per chunk, in chunk order
    gs = np.array([32, 128], dtype=np.int32)
    canon, _, _ = synthetic_canon(2, 512, 2, gs, seed=3)
    L = layout.build(canon)
    sz = canon["scale"].astype(np.uint32) | (canon["zero"].astype(np.uint32) << 16)
    row0, row1 = sz[0:16], sz[16:20]
    want = np.concatenate([row0[0:8], row1[0:2], row0[8:16], row1[2:4]])
    assert np.array_equal(L["sz"], want)


@pytest.mark.parametrize("N,K,nk", [
    (7, 256, 2), (16, 512, 2), (17, 768, 2), (33, 512, 1), (5, 1024, 1), (40, 256, 1),
    (3, 2816, 2), (19, 2816, 1), (7, 256, 4), (21, 1280, 4),
])
def test_decode_inverts_build(N, K, nk):
    rng = np.random.default_rng(N * K + nk)
    gs = rng.choice([32, 64, 128, 256], N).astype(np.int32)
    canon, q, o = synthetic_canon(N, K, nk, gs, seed=N)
    L = layout.build(canon)
    q2, o2, szr, perm = layout.decode(L["blob"], N, K, nk, gs)
    assert np.array_equal(q2, q) and (nk == 4 or np.array_equal(o2, o))
    sz = canon["scale"].astype(np.uint32) | (canon["zero"].astype(np.uint32) << 16)
    for n in range(N):
        assert np.array_equal(szr[n], sz[canon["gptr"][n]: canon["gptr"][n + 1]])
    assert sorted(perm.tolist()) == list(range(N))
    # no byte is duplicated: the sections hold exactly the canonical bits plus zero padding
    off = L["offsets"]
    T = -(-N // 16)
    assert off["offs"] >= T * (K // 256) * 64 * 8 * nk


def test_off14_positions_are_a_permutation():
    pos = [layout.off14_bit(m) for m in range(16)]
    assert sorted(pos) == list(range(0, 32, 2))


def test_hand_placed_bytes_dense():
    """Dense ablation (nk = 4): 64 elements per piece, no offset section."""
    N, K, nk = 1, 256, 4
    q = np.array([[j % 16 for j in range(K)]], dtype=np.uint8)
    vals, _ = pack.pack_bytes(q, np.zeros((N, K), np.uint8))
    canon = {"N": N, "K": K, "nk": nk, "group_size": np.array([256], np.int32), "vals": vals,
             "offs": np.zeros((N, 0), np.uint8), "scale": np.array([0x3C00], np.uint16),
             "zero": np.array([0x4800], np.uint16), "gptr": np.array([0, 1], np.int32)}
    L = layout.build(canon)
    off = L["offsets"]
    # 64 lanes x 32 bytes of codes; the offset section is empty
    assert (off["codes"], off["offs"], off["perm"], off["sz"], off["blob_bytes"]) == (0, 2048, 2048, 2304, 2560)
    blob = L["blob"]
    # lane 0, dword 0: positions 0 and 1 of the groups at columns 0-3, 4-7,
    # 8-11, 12-15, i.e. elements 0,1,4,5,8,9,12,13 (codes equal), element k at
    # nibble [0,4,1,5,2,6,3,7][k]: nibbles 0..7 hold 0,4,8,12,1,5,9,13
    assert u32_at(blob, 0) == 0xD951C840
    # dword 1: positions 2 and 3: elements 2,3,6,7,10,11,14,15 -> nibbles
    # 2,6,10,14,3,7,11,15
    assert u32_at(blob, 4) == 0xFB73EA62
    # lane 16 (columns 64..127): dword 7 = columns 112..127, positions 2, 3:
    # elements 114,115,118,119,122,123,126,127 -> codes 2,3,6,7,10,11,14,15;
    # dwords 4-7 of every lane follow dwords 0-3 of every lane (1 KiB slices)
    assert u32_at(blob, 1024 + 16 * 16 + 12) == 0xFB73EA62
    assert u32_at(blob, 2304) == 0x48003C00


@pytest.mark.parametrize("N,K,nk", [(7, 256, 2), (19, 768, 2), (33, 512, 1), (5, 2816, 1)])
def test_fp16_form_decode_inverts_build(N, K, nk):
    rng = np.random.default_rng(N + nk)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    c = pack.pack_fp16_canonical(W, nk)
    L = layout.build16(c)
    q16, o = layout.decode16(L["blob"], N, K, nk)
    _, o_ref = pack.unpack_bytes(np.zeros((N, 1), np.uint8), c["offs"])
    assert np.array_equal(q16, c["vals16"]) and np.array_equal(o, o_ref)
    off = L["offsets"]
    assert off["blob_bytes"] == layout._align(off["perm"] + 64 * (-(-N // 16)))


def test_fp16_form_hand_placed_values():
    # one row, 2:4: lane 16 (columns 64..127) holds kept elements 32..63 in
    # order: 64 bytes; its first value is element 32
    N, K, nk = 1, 256, 2
    W = np.zeros((N, K), np.float16)
    W[0, 0::4] = np.arange(64, dtype=np.float16)          # column 4j holds j, kept with column 4j+1 (0)
    c = pack.pack_fp16_canonical(W, nk)
    L = layout.build16(c)
    blob = L["blob"]
    # element 32 = column 64 (value 16), element 33 = column 65 (value 0);
    # slice 0 (values 0-7) of lane 16 sits at 16 * 16
    v = np.frombuffer(blob[16 * 16: 16 * 16 + 8].tobytes(), "<u2").view(np.float16)
    assert v.tolist() == [16.0, 0.0, 17.0, 0.0]
    # slice 1 of lane 16 (elements 40..47 = columns 80, 81, ...) follows all 64 lanes' slice 0
    v = np.frombuffer(blob[1024 + 16 * 16: 1024 + 16 * 16 + 4].tobytes(), "<u2").view(np.float16)
    assert v.tolist() == [20.0, 0.0]
    # 64 lanes x 64 bytes of values, then 64 lanes x 8 bytes of offsets
    assert L["offsets"]["offs"] == 4096 and L["offsets"]["perm"] == 4096 + 512

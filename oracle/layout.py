"""Kernel layout: a documented permutation of the canonical 2bit-CSR arrays.

The GPU kernel reads the same bits as the canonical arrays (no padding, no
duplication), reordered so that every load is a coalesced 16-byte (values),
8-byte (offsets) or 4-byte (scale+zero) access. This module builds that
blob from the canonical arrays, element by element, from the rules below.

Terms
* chunk: 32 consecutive kept elements of a row (16 bytes of codes, 8 bytes of
  offsets); it spans cpc = 128/nk dense columns (64 at 2:4, 128 at 1:4).
  A row has C = K*nk/128 chunks.
* row order: rows sorted by group size (smaller first), ascending row index
  within a size (``perm[i]`` = original row of sorted position i).
* tile: up to RT consecutive sorted rows of one group size. Within a tile,
  TPR threads work on each row; chunk c of a row goes to k-lane c % TPR at
  iteration c // TPR. There are I = ceil(C/TPR) iterations; all but the last
  hold TPR chunks per row, the last holds rem = C - (I-1)*TPR.
* slot: position of a chunk in the tile's streams,
      slot = row0*C + i*nr*TPR + r*cnt_i + kl
  with row0 the tile's first sorted row, nr its row count, r the row within
  the tile, kl the k-lane and cnt_i the chunks per row of iteration i.

Bits inside a chunk (element e = 0..31 of the chunk)
* codes: 4 little-endian dwords; dword d holds elements 8d..8d+7, nibble k
  (bits 4k..4k+3) holds element 8d + 2k for k < 4 and 8d + 2(k-4) + 1 for
  k >= 4, so that masking 0x000F000F / 0x00F000F0 yields consecutive pairs;
* offsets: 2 little-endian dwords; dword D holds elements 16D..16D+15,
  element 16D + 4q + b at bits 8b + 2q, so that (dword >> 2q) & 0x03030303
  gives the offsets of 4 consecutive elements in 4 bytes.

Scale/zero stream: one 32-bit entry per group, FP16 scale in the low half,
FP16 zero in the high half. A chunk at slot s of a tile with group size g
uses entries sz_base + (s*cpc)//g + j, j < max(1, cpc//g); chunks that share
a group share its entry (consecutive slots, so the entry is stored once).

Blob sections (each starting on a 256-byte boundary, in this order):
tiles int32[n_tiles][4] = (row0, nr, g, sz_base); perm int32[N];
codes (N*C*16 B); offsets (N*C*8 B); scale/zero (n_groups*4 B).
"""
import numpy as np

from .pack import unpack_bytes

ALIGN = 256


def _align(x: int) -> int:
    return (x + ALIGN - 1) // ALIGN * ALIGN


def cols_per_chunk(nk: int) -> int:
    return 128 // nk


def row_order(group_size) -> np.ndarray:
    return np.argsort(np.asarray(group_size, dtype=np.int64), kind="stable").astype(np.int32)


def tile_list(group_size, RT: int):
    """[(row0, nr, g)] in sorted-row order, class by class."""
    gs_sorted = np.asarray(group_size, dtype=np.int64)[row_order(group_size)]
    tiles, i, N = [], 0, len(gs_sorted)
    while i < N:
        g = int(gs_sorted[i])
        j = i
        while j < N and gs_sorted[j] == g:
            j += 1
        for r0 in range(i, j, RT):
            tiles.append((r0, min(RT, j - r0), g))
        i = j
    return tiles


def section_offsets(N: int, K: int, nk: int, n_tiles: int, n_groups: int) -> dict:
    C = K * nk // 128
    off = {"tiles": 0}
    off["perm"] = _align(16 * n_tiles)
    off["vals"] = _align(off["perm"] + 4 * N)
    off["offs"] = _align(off["vals"] + 16 * N * C)
    off["sz"] = _align(off["offs"] + 8 * N * C)
    off["blob_bytes"] = _align(off["sz"] + 4 * n_groups)
    return off


def _encode_codes(q32: np.ndarray) -> np.ndarray:
    """[S, 32] codes -> [S, 16] bytes."""
    S = q32.shape[0]
    q = q32.astype(np.uint32).reshape(S, 4, 8)
    src = [0, 2, 4, 6, 1, 3, 5, 7]            # element held by nibble k
    dw = np.zeros((S, 4), dtype=np.uint32)
    for k in range(8):
        dw |= q[:, :, src[k]] << np.uint32(4 * k)
    return dw.astype("<u4").view(np.uint8).reshape(S, 16)


def _encode_offs(o32: np.ndarray) -> np.ndarray:
    """[S, 32] offsets -> [S, 8] bytes."""
    S = o32.shape[0]
    o = o32.astype(np.uint32).reshape(S, 2, 4, 4)   # [S, D, q, b]
    dw = np.zeros((S, 2), dtype=np.uint32)
    for q in range(4):
        for b in range(4):
            dw |= o[:, :, q, b] << np.uint32(8 * b + 2 * q)
    return dw.astype("<u4").view(np.uint8).reshape(S, 8)


def build(canon: dict, RT: int, TPR: int) -> dict:
    """Canonical arrays -> kernel blob (bytes) plus its parts for inspection."""
    N, K, nk = canon["N"], canon["K"], canon["nk"]
    gs = np.asarray(canon["group_size"], dtype=np.int64)
    cpc = cols_per_chunk(nk)
    C = K * nk // 128
    q, o = unpack_bytes(canon["vals"], canon["offs"])
    scale = np.asarray(canon["scale"], dtype=np.uint32)
    zero = np.asarray(canon["zero"], dtype=np.uint32)
    sz_all = scale | (zero << np.uint32(16))
    gptr = np.asarray(canon["gptr"], dtype=np.int64)
    perm = row_order(gs)
    tiles = tile_list(gs, RT)
    vals_blob = np.zeros((N * C, 16), dtype=np.uint8)
    offs_blob = np.zeros((N * C, 8), dtype=np.uint8)
    n_groups = int(gptr[N])
    sz_blob = np.zeros(n_groups, dtype=np.uint32)
    sz_filled = np.zeros(n_groups, dtype=bool)
    tile_tab = np.zeros((len(tiles), 4), dtype=np.int32)
    sz_base = 0
    I = -(-C // TPR)
    for t, (row0, nr, g) in enumerate(tiles):
        tile_tab[t] = (row0, nr, g, sz_base)
        rows = perm[row0: row0 + nr].astype(np.int64)
        for i in range(I):
            cnt = min(TPR, C - i * TPR)
            r = np.arange(nr)[:, None]
            kl = np.arange(cnt)[None, :]
            c = (i * TPR + kl) + 0 * r                      # [nr, cnt] chunk index
            s_rel = i * nr * TPR + r * cnt + kl             # tile-relative slot
            slot = (row0 * C + s_rel).reshape(-1)
            n_of = (rows[:, None] + 0 * kl).reshape(-1)
            c_f = c.reshape(-1)
            e = 32 * c_f[:, None] + np.arange(32)[None, :]
            vals_blob[slot] = _encode_codes(q[n_of[:, None], e])
            offs_blob[slot] = _encode_offs(o[n_of[:, None], e])
            # scale/zero entries of the groups this chunk touches
            per = max(1, cpc // g)
            for j in range(per):
                grp = gptr[n_of] + (c_f * cpc) // g + j
                dst = sz_base + (s_rel.reshape(-1) * cpc) // g + j
                if np.any(sz_filled[dst] & (sz_blob[dst] != sz_all[grp])):
                    raise AssertionError("shared scale/zero entry disagrees")
                sz_blob[dst] = sz_all[grp]
                sz_filled[dst] = True
        sz_base += nr * C * cpc // g
    assert sz_base == n_groups and np.all(sz_filled)
    off = section_offsets(N, K, nk, len(tiles), n_groups)
    blob = np.zeros(off["blob_bytes"], dtype=np.uint8)
    blob[off["tiles"]: off["tiles"] + 16 * len(tiles)] = tile_tab.astype("<i4").view(np.uint8).reshape(-1)
    blob[off["perm"]: off["perm"] + 4 * N] = perm.astype("<i4").view(np.uint8)
    blob[off["vals"]: off["vals"] + 16 * N * C] = vals_blob.reshape(-1)
    blob[off["offs"]: off["offs"] + 8 * N * C] = offs_blob.reshape(-1)
    blob[off["sz"]: off["sz"] + 4 * n_groups] = sz_blob.astype("<u4").view(np.uint8)
    return {"blob": blob, "offsets": off, "tiles": tile_tab, "perm": perm,
            "vals": vals_blob, "offs": offs_blob, "sz": sz_blob}


def decode(blob: np.ndarray, N: int, K: int, nk: int, RT: int, TPR: int):
    """Inverse of build: blob -> per-element codes [N, kpr], offsets [N, kpr],
    and per-row (scale, zero) lists, read through the same rules."""
    C = K * nk // 128
    cpc = cols_per_chunk(nk)
    kpr = K * nk // 4
    # the tile table's size is implied by the group sizes, which the tile
    # table itself records; read tiles until the rows are covered
    tiles, rows_seen, t = [], 0, 0
    while rows_seen < N:
        row0, nr, g, szb = np.frombuffer(blob[16 * t: 16 * t + 16].tobytes(), dtype="<i4")
        tiles.append((int(row0), int(nr), int(g), int(szb)))
        rows_seen += int(nr)
        t += 1
    n_groups = sum(nr * K // g for (_, nr, g, _) in tiles)
    off = section_offsets(N, K, nk, len(tiles), n_groups)
    perm = np.frombuffer(blob[off["perm"]: off["perm"] + 4 * N].tobytes(), dtype="<i4")
    vb = blob[off["vals"]: off["vals"] + 16 * N * C].reshape(N * C, 4, 4)
    ob = blob[off["offs"]: off["offs"] + 8 * N * C].reshape(N * C, 2, 4)
    vd = vb.astype(np.uint32)
    vd = vd[..., 0] | (vd[..., 1] << 8) | (vd[..., 2] << 16) | (vd[..., 3] << 24)   # [S, 4]
    od = ob.astype(np.uint32)
    od = od[..., 0] | (od[..., 1] << 8) | (od[..., 2] << 16) | (od[..., 3] << 24)   # [S, 2]
    szb = np.frombuffer(blob[off["sz"]: off["sz"] + 4 * n_groups].tobytes(), dtype="<u4")
    q = np.zeros((N, kpr), dtype=np.uint8)
    o = np.zeros((N, kpr), dtype=np.uint8)
    sz_rows = {}
    I = -(-C // TPR)
    for (row0, nr, g, sz_base) in tiles:
        for r in range(nr):
            n = int(perm[row0 + r])
            ng = K // g
            sz_rows[n] = np.zeros(ng, dtype=np.uint32)
            for c in range(C):
                i, kl = divmod(c, TPR)
                cnt = min(TPR, C - i * TPR)
                s_rel = i * nr * TPR + r * cnt + kl
                slot = row0 * C + s_rel
                for e in range(32):
                    d, m = divmod(e, 8)
                    k = m // 2 if m % 2 == 0 else 4 + m // 2
                    q[n, 32 * c + e] = (vd[slot, d] >> (4 * k)) & 0xF
                    D, rest = divmod(e, 16)
                    qq, b = divmod(rest, 4)
                    o[n, 32 * c + e] = (od[slot, D] >> (8 * b + 2 * qq)) & 3
                for j in range(max(1, cpc // g)):
                    sz_rows[n][(c * cpc) // g + j] = szb[sz_base + (s_rel * cpc) // g + j]
    return q, o, sz_rows, perm

"""Kernel layout: a documented permutation of the canonical 2bit-CSR arrays.

Test infrastructure (see the package docstring). The GPU kernel reads the
same bits as the canonical arrays, reordered for the 2-of-4 sparse
matrix-core instruction (16 rows x 64 dense columns per instruction); this
module builds that blob from the canonical arrays, element by element, from
the rules below, and reads it back.

Terms
* sorted rows: rows ordered by group size (smaller first), ascending row
  index within a size; ``perm[i]`` = original row of sorted position i.
* row block b: sorted rows 16b .. 16b+15; T = ceil(N / 16) blocks; rows past
  N in the last block are padding.
* column chunk c: dense columns 256c .. 256c+255; C = K / 256 chunks.
* piece (i, c, q), q = 0..3: sorted row i, dense columns 256c + 64q .. +63;
  it holds the row's kept elements e0 .. e0 + 16*nk - 1, e0 = 16*nk*(4c + q)
  (an N:M row keeps exactly nk per 4 columns, so pieces are aligned).
* record (b, c): 64 lanes; lane r + 16q holds piece (16b + r, c, q).

Bits of a piece
* codes (8*nk bytes): little-endian dwords of 8 consecutive elements; element
  k (0..7) of a dword sits at nibble NIB[k], NIB = [0,4,1,5,2,6,3,7] at 2:4
  and [0,1,4,5,2,3,6,7] at 1:4 (so that the masks 0x000F000F / 0x00F000F0
  pick the pairs the kernel feeds into one matrix-core register);
* offsets (4*nk bytes): at 2:4 the canonical 2-bit fields, element m at bits
  2m of a little-endian 64-bit word (bytes unchanged); at 1:4 one dword with
  element m at bit 16*((m//4) % 2) + (REAL if m//4 < 2 else DUMMY)[m % 4],
  REAL = [0,4,10,14], DUMMY = [2,6,8,12].
* at 1:4 a lane's piece is 12 bytes in the code section: its 2 code dwords,
  then its offset dword (one load reads both); the offset section is empty.

Dense ablation (nk = 4, every element kept, no offsets): a piece holds the
64 elements of its columns in 8 dwords; dword 2t + h (t = 0..3, h = 0, 1)
holds, for the 4 groups of columns 16t .. 16t + 15 of the piece, the
elements at in-group positions 2h and 2h + 1: dword element k = 2g + p'
(group g, position 2h + p') at nibble NIB[2][k], so that each dword is a
2-of-4 operand whose index field is the constant (0, 1) or (2, 3) per
group. A record stores the pieces' dwords 0-3 for all 64 lanes, then dwords
4-7 (16-byte slices, so that one load instruction reads 1 KiB
contiguously). The offset section is empty.

Scale/zero: one 32-bit word per group, FP16 scale in the low half, FP16 zero
in the high half; records (b, c) in (b, c) order, each listing the rows of
block b in order, each row with its 256/g words of chunk c (its groups
c*256/g .. (c+1)*256/g - 1). Padding rows have no words.

Blob sections (each starting on a 256-byte boundary, in this order): codes
[T][C][64][8*nk] (1:4: [T][C][64][12], codes and offsets); offsets
[T][C][64][8] (2:4 only); perm int32[16*T] (-1 for padding rows);
scale/zero words, followed by 8 zero bytes.
"""
import numpy as np

from .pack import unpack_bytes

ALIGN = 256
NIB = {2: [0, 4, 1, 5, 2, 6, 3, 7], 1: [0, 1, 4, 5, 2, 3, 6, 7]}
REAL = [0, 4, 10, 14]
DUMMY = [2, 6, 8, 12]


def _align(x: int) -> int:
    return (x + ALIGN - 1) // ALIGN * ALIGN


def row_order(group_size) -> np.ndarray:
    return np.argsort(np.asarray(group_size, dtype=np.int64), kind="stable").astype(np.int32)


def off14_bit(m: int) -> int:
    """Bit position of element m (0..15) of a 1:4 piece in its offset dword."""
    t, e = divmod(m, 4)
    return 16 * (t % 2) + (REAL if t < 2 else DUMMY)[e]


def piece_code_bytes(nk: int) -> int:
    """Bytes of a piece in the code section (1:4: codes and the offset dword)."""
    return 12 if nk == 1 else 8 * nk


def piece_offs_bytes(nk: int) -> int:
    """Bytes of a piece in the offset section (2:4 only)."""
    return 8 if nk == 2 else 0


def dense_dword_element(d: int, k: int) -> int:
    """Element (0..63) of a dense piece held by element k of code dword d."""
    t, h = divmod(d, 2)
    g, pp = divmod(k, 2)
    return 16 * t + 4 * g + 2 * h + pp


def section_offsets(N: int, K: int, nk: int, n_groups: int) -> dict:
    T, C = -(-N // 16), K // 256
    records = T * C * 64
    off = {"codes": 0}
    off["offs"] = _align(records * piece_code_bytes(nk))
    off["perm"] = _align(off["offs"] + records * piece_offs_bytes(nk))
    off["sz"] = _align(off["perm"] + 4 * 16 * T)
    off["blob_bytes"] = _align(off["sz"] + 4 * n_groups + 8)
    return off


def build(canon: dict) -> dict:
    """Canonical arrays -> kernel blob (bytes) plus its parts for inspection."""
    N, K, nk = canon["N"], canon["K"], canon["nk"]
    gs = np.asarray(canon["group_size"], dtype=np.int64)
    T, C, kpp = -(-N // 16), K // 256, 16 * nk
    q, o = unpack_bytes(canon["vals"], canon["offs"])           # [N, K*nk/4] each
    if nk == 4:
        o = np.zeros_like(q)                                     # no offsets stored
    sz_all = (np.asarray(canon["scale"], dtype=np.uint32)
              | (np.asarray(canon["zero"], dtype=np.uint32) << np.uint32(16)))
    gptr = np.asarray(canon["gptr"], dtype=np.int64)
    perm = row_order(gs)
    # per sorted row: pieces [C, 4, kpp] of codes and offsets
    qs = q[perm].astype(np.uint32).reshape(N, C, 4, kpp)
    os_ = o[perm].astype(np.uint32).reshape(N, C, 4, kpp)
    # codes: dwords of 8 elements, element k at nibble NIB[k]
    cw = np.zeros((N, C, 4, kpp // 8), dtype=np.uint32)
    if nk == 4:
        for d in range(8):
            for k in range(8):
                cw[..., d] |= qs[..., dense_dword_element(d, k)] << np.uint32(4 * NIB[2][k])
    else:
        qd = qs.reshape(N, C, 4, kpp // 8, 8)
        for k in range(8):
            cw |= qd[..., k] << np.uint32(4 * NIB[nk][k])
    # offsets
    if nk == 4:
        ow = np.zeros((N, C, 4, 0), dtype=np.uint32)
    elif nk == 2:
        od = os_.reshape(N, C, 4, 2, 16)
        ow = np.zeros((N, C, 4, 2), dtype=np.uint32)
        for m in range(16):
            ow |= od[..., m] << np.uint32(2 * m)
    else:
        ow = np.zeros((N, C, 4, 1), dtype=np.uint32)
        for m in range(16):
            ow[..., 0] |= os_[..., m] << np.uint32(off14_bit(m))
    # records (b, c): lane r + 16q <- piece (16b + r, c, q); padding rows stay zero
    cwp = np.zeros((T * 16,) + cw.shape[1:], dtype=np.uint32)
    owp = np.zeros((T * 16,) + ow.shape[1:], dtype=np.uint32)
    cwp[:N], owp[:N] = cw, ow
    codes = cwp.reshape(T, 16, C, 4, -1).transpose(0, 2, 3, 1, 4)     # [T, C, q, r, dw]
    if nk == 4:
        # 16-byte slices: slice h of every lane, then slice h + 1
        codes = codes.reshape(T, C, 64, 2, 4).transpose(0, 1, 3, 2, 4)   # [T, C, h, lane, 4 dwords]
    offs = owp.reshape(T, 16, C, 4, -1).transpose(0, 2, 3, 1, 4)
    if nk == 1:
        # a lane's 2 code dwords, then its offset dword
        codes = np.concatenate([codes, offs], axis=-1)                    # [T, C, q, r, 3]
        offs = offs[..., :0]
    # scale/zero records
    sz_words = []
    for b in range(T):
        rows = perm[16 * b: 16 * b + 16]
        per_row = []
        for n in rows:
            g = int(gs[n])
            per_row.append(sz_all[gptr[n]: gptr[n + 1]].reshape(C, 256 // g))
        sz_words.append(np.concatenate(per_row, axis=1).reshape(-1))      # chunk-major
    sz = np.concatenate(sz_words).astype(np.uint32)
    n_groups = int(gptr[N])
    assert sz.size == n_groups
    perm_pad = np.full(16 * T, -1, dtype=np.int32)
    perm_pad[:N] = perm
    off = section_offsets(N, K, nk, n_groups)
    blob = np.zeros(off["blob_bytes"], dtype=np.uint8)

    def put(at, arr):
        raw = np.ascontiguousarray(arr).astype("<u4").view(np.uint8).reshape(-1)
        blob[at: at + raw.size] = raw

    put(off["codes"], codes)
    put(off["offs"], offs)
    put(off["perm"], perm_pad.view(np.uint32))
    put(off["sz"], sz)
    return {"blob": blob, "offsets": off, "perm": perm_pad, "codes": codes, "offs": offs, "sz": sz}


def decode(blob: np.ndarray, N: int, K: int, nk: int, group_size):
    """Inverse of build: blob -> per-element codes [N, K*nk/4] and offsets
    [N, K*nk/4] in original row order, per-row scale|zero word lists and the
    sorted-row permutation, read back through the same rules."""
    gs = np.asarray(group_size, dtype=np.int64)
    T, C, kpp = -(-N // 16), K // 256, 16 * nk
    n_groups = int(np.sum(K // gs))
    off = section_offsets(N, K, nk, n_groups)
    u32 = lambda at, n: np.frombuffer(blob[at: at + 4 * n].tobytes(), dtype="<u4")
    perm = np.frombuffer(blob[off["perm"]: off["perm"] + 64 * T].tobytes(), dtype="<i4")
    pcw = piece_code_bytes(nk) // 4
    cw = u32(off["codes"], T * C * 64 * pcw).reshape(T, C, 64, pcw)
    if nk == 4:
        cw = cw.reshape(T, C, 2, 64, 4).transpose(0, 1, 3, 2, 4).reshape(T, C, 64, 8)
    if nk == 1:
        cw, ow = cw[..., :2], cw[..., 2:]
    else:
        now = piece_offs_bytes(nk) // 4
        ow = u32(off["offs"], T * C * 64 * now).reshape(T, C, 64, now)
    szw = u32(off["sz"], n_groups)
    kpr = K * nk // 4
    q = np.zeros((N, kpr), dtype=np.uint8)
    o = np.zeros((N, kpr), dtype=np.uint8)
    sz_rows = {}
    at = 0
    for b in range(T):
        for c in range(C):
            for r in range(16):
                i = 16 * b + r
                if i >= N:
                    break
                n = int(perm[i])
                for qq in range(4):
                    lane = r + 16 * qq
                    e0 = kpp * (4 * c + qq)
                    if nk == 4:
                        for d in range(8):
                            for k in range(8):
                                q[n, e0 + dense_dword_element(d, k)] = (cw[b, c, lane, d] >> (4 * NIB[2][k])) & 0xF
                        continue
                    for m in range(kpp):
                        dw, k = divmod(m, 8)
                        q[n, e0 + m] = (cw[b, c, lane, dw] >> (4 * NIB[nk][k])) & 0xF
                        if nk == 2:
                            word, bit = divmod(m, 16)
                            o[n, e0 + m] = (ow[b, c, lane, word] >> (2 * bit)) & 3
                        else:
                            o[n, e0 + m] = (ow[b, c, lane, 0] >> off14_bit(m)) & 3
                per = 256 // int(gs[n])
                sz_rows.setdefault(n, np.zeros(K // int(gs[n]), dtype=np.uint32))
                sz_rows[n][c * per: (c + 1) * per] = szw[at: at + per]
                at += per
    assert at == n_groups
    return q, o, sz_rows, perm[:N]


# ---- FP16-valued form (no groups): values in place of codes, no scale/zero

def section_offsets16(N: int, K: int, nk: int) -> dict:
    """Sections of the FP16-valued blob: values, offsets as in the INT4 form,
    perm; no scale/zero words. A lane's piece holds its 16*nk kept values
    (FP16, element order) in 2*nk 16-byte slices; record (b, c) stores slice
    0 of all 64 lanes, then slice 1, and so on."""
    T, C = -(-N // 16), K // 256
    records = T * C * 64
    off = {"values": 0}
    off["offs"] = _align(records * 32 * nk)
    off["perm"] = _align(off["offs"] + records * 4 * nk)   # offsets stay a section of their own here
    off["blob_bytes"] = _align(off["perm"] + 4 * 16 * T)
    return off


def _piece_offsets(o_sorted: np.ndarray, N: int, C: int, nk: int) -> np.ndarray:
    """Offset words [N, C, 4, nk] of every piece (same rules as the INT4 form)."""
    kpp = 16 * nk
    os_ = o_sorted.astype(np.uint32).reshape(N, C, 4, kpp)
    if nk == 2:
        od = os_.reshape(N, C, 4, 2, 16)
        ow = np.zeros((N, C, 4, 2), dtype=np.uint32)
        for m in range(16):
            ow |= od[..., m] << np.uint32(2 * m)
    else:
        ow = np.zeros((N, C, 4, 1), dtype=np.uint32)
        for m in range(16):
            ow[..., 0] |= os_[..., m] << np.uint32(off14_bit(m))
    return ow


def build16(canon16: dict) -> dict:
    """FP16-valued canonical arrays -> kernel blob (rows in index order: with
    no group sizes there is nothing to sort by, perm is the identity)."""
    N, K, nk = canon16["N"], canon16["K"], canon16["nk"]
    T, C, kpp = -(-N // 16), K // 256, 16 * nk
    v16 = np.asarray(canon16["vals16"], dtype=np.uint16)
    _, o = unpack_bytes(np.zeros((N, 1), np.uint8), canon16["offs"])
    vals = np.zeros((T * 16, C, 4, kpp), dtype=np.uint16)
    vals[:N] = v16.reshape(N, C, 4, kpp)
    ow = np.zeros((T * 16, C, 4, nk), dtype=np.uint32)
    ow[:N] = _piece_offsets(o, N, C, nk)
    values = vals.reshape(T, 16, C, 4, kpp).transpose(0, 2, 3, 1, 4)      # [T, C, q, r, kpp]
    # 16-byte slices (8 values): slice k of all 64 lanes, then slice k + 1
    values = values.reshape(T, C, 64, 2 * nk, 8).transpose(0, 1, 3, 2, 4)  # [T, C, k, lane, 8]
    offs = ow.reshape(T, 16, C, 4, nk).transpose(0, 2, 3, 1, 4)
    perm = np.full(16 * T, -1, dtype=np.int32)
    perm[:N] = np.arange(N, dtype=np.int32)
    off = section_offsets16(N, K, nk)
    blob = np.zeros(off["blob_bytes"], dtype=np.uint8)
    raw = np.ascontiguousarray(values).astype("<u2").view(np.uint8).reshape(-1)
    blob[off["values"]: off["values"] + raw.size] = raw
    raw = np.ascontiguousarray(offs).astype("<u4").view(np.uint8).reshape(-1)
    blob[off["offs"]: off["offs"] + raw.size] = raw
    raw = perm.astype("<i4").view(np.uint8)
    blob[off["perm"]: off["perm"] + raw.size] = raw
    return {"blob": blob, "offsets": off, "perm": perm}


def decode16(blob: np.ndarray, N: int, K: int, nk: int):
    """Inverse of build16: FP16 bits [N, K*nk/4] and offsets [N, K*nk/4]."""
    T, C, kpp = -(-N // 16), K // 256, 16 * nk
    off = section_offsets16(N, K, nk)
    v = np.frombuffer(blob[off["values"]: off["values"] + T * C * 64 * kpp * 2].tobytes(), dtype="<u2")
    v = v.reshape(T, C, 2 * nk, 64, 8).transpose(0, 1, 3, 2, 4).reshape(T, C, 4, 16, kpp)
    ow = np.frombuffer(blob[off["offs"]: off["offs"] + T * C * 64 * 4 * nk].tobytes(), dtype="<u4")
    ow = ow.reshape(T, C, 4, 16, nk)
    kpr = K * nk // 4
    q16 = np.zeros((N, kpr), dtype=np.uint16)
    o = np.zeros((N, kpr), dtype=np.uint8)
    for n in range(N):
        b, r = divmod(n, 16)
        for c in range(C):
            for qq in range(4):
                e0 = kpp * (4 * c + qq)
                q16[n, e0: e0 + kpp] = v[b, c, qq, r]
                for m in range(kpp):
                    if nk == 2:
                        word, bit = divmod(m, 16)
                        o[n, e0 + m] = (ow[b, c, qq, r, word] >> (2 * bit)) & 3
                    else:
                        o[n, e0 + m] = (ow[b, c, qq, r, 0] >> off14_bit(m)) & 3
    return q16, o

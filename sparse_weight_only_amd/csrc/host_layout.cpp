// Layer descriptor and kernel layout of the 2bit-CSR arrays.
//
// The kernel layout is a permutation of the canonical bits, with zero
// padding only for the rows of a last, partial row block, arranged for the
// matrix-core kernel (v_smfmac_f32_16x16x64_f16: 16 rows x 64 dense columns
// per instruction, A operand 2-of-4 sparse with 2-bit indices):
//  - sorted rows: rows ordered by group size (ascending, stable);
//  - row block b: sorted rows 16b .. 16b+15 (T = ceil(N/16) blocks);
//  - piece (i, c, q): sorted row i, dense columns 256c + 64q .. 256c + 64q + 63,
//    i.e. its 16*nk consecutive kept elements starting at 16*nk*(4c + q);
//  - record (b, c) of the code and offset sections: 64 lanes, lane r + 16q
//    holding piece (16b + r, c, q);
//  - codes of a piece: little-endian dwords of 8 consecutive elements; element
//    k of a dword sits at nibble [0,4,1,5,2,6,3,7][k] (2:4) or
//    [0,1,4,5,2,3,6,7][k] (1:4);
//  - offsets of a piece: 2:4 = the canonical 2-bit fields (element m at bits
//    2m of a little-endian 64-bit word); 1:4 = one dword, element m at bit
//    16*((m/4)%2) + (m/4 < 2 ? [0,4,10,14] : [2,6,8,12])[m%4];
//  - at 1:4 a lane's piece is 12 bytes of the code section, its 2 code
//    dwords and then its offset dword (one 12-byte load reads both), and the
//    offset section is empty;
//  - dense ablation (nk = 4, no offsets): code dword 2t + h holds positions
//    2h and 2h + 1 of the 4 groups of piece columns 16t .. 16t + 15, element
//    k = 2g + p at nibble [0,4,1,5,2,6,3,7][k]; a record stores dwords 0-3 of
//    all 64 lanes, then dwords 4-7 (so one load reads 1 KiB contiguously);
//  - perm: original row of each sorted row, -1 for padding rows;
//  - scale|zero<<16 words: records (b, c) in order, each the rows of block b
//    in order, each with its 256/g words of chunk c (groups c*256/g ..).
// Reference: the first contribution item of the page "Efficient large-model
// ad applications through model compression and parallel verification"
// (English gloss of its Chinese title; a translation of arXiv 2605.11582), which introduces the index-compressed 2bit-CSR format
// but leaves its bit layout open.
#include <algorithm>
#include <cmath>
#include <numeric>
#include <vector>

#include "internal.hpp"

using namespace sgemv;

namespace {

std::vector<int32_t> sorted_rows(const int32_t* gs, int32_t N) {
  std::vector<int32_t> perm(N);
  std::iota(perm.begin(), perm.end(), 0);
  std::stable_sort(perm.begin(), perm.end(), [&](int32_t a, int32_t b) { return gs[a] < gs[b]; });
  return perm;
}

constexpr int kNib24[8] = {0, 4, 1, 5, 2, 6, 3, 7};
constexpr int kNib14[8] = {0, 1, 4, 5, 2, 3, 6, 7};
constexpr int kOff14Real[4] = {0, 4, 10, 14};
constexpr int kOff14Dummy[4] = {2, 6, 8, 12};

}  // namespace

extern "C" int sgemv_describe(int32_t N, int32_t K, int32_t nk, const int32_t* group_size,
                              sgemv_desc* out) {
  if (!group_size || !out) return SGEMV_EINVAL;
  if (N < 1 || K < kChunkCols || K % kChunkCols != 0 || !valid_nk(nk)) return SGEMV_EINVAL;
  if (K / kChunkCols > kMaxChunks) return SGEMV_ESIZE;
  int g_min = 1 << 30, g_max = 0;
  int64_t n_groups = 0;
  sgemv_desc d;
  memset(&d, 0, sizeof d);
  for (int32_t n = 0; n < N; ++n) {
    const int g = group_size[n];
    if (!valid_group(g, K)) return SGEMV_EINVAL;
    g_min = std::min(g_min, g);
    g_max = std::max(g_max, g);
    n_groups += K / g;
    d.class_rows[ilog2(g / 32)] += 1;
  }
  const int32_t T = (N + kBlockRows - 1) / kBlockRows, C = K / kChunkCols;
  d.N = N; d.K = K; d.nk = nk;
  d.n_blocks = T;
  d.chunks = C;
  d.g_min = g_min; d.g_max = g_max;
  d.kept = (int64_t)N * K * nk / 4;
  d.vals_bytes = d.kept / 2;
  d.offs_bytes = nk == 4 ? 0 : d.kept / 4;
  d.n_groups = n_groups;
  const int64_t records = (int64_t)T * C * 64;
  d.off_codes = 0;
  d.off_offs = align_up(records * piece_code_bytes(nk));
  d.off_perm = align_up(d.off_offs + records * piece_offs_bytes(nk));
  d.off_sz = align_up(d.off_perm + 4 * (int64_t)T * kBlockRows);
  // 8 spare bytes after the words: a lane reads two words where it needs one
  d.blob_bytes = align_up(d.off_sz + 4 * n_groups + 8);
  if (d.blob_bytes >= ((int64_t)1 << 31)) return SGEMV_ESIZE;
  *out = d;
  return SGEMV_OK;
}

extern "C" int sgemv_describe_fp16(int32_t N, int32_t K, int32_t nk, sgemv_desc* out) {
  if (!out) return SGEMV_EINVAL;
  if (N < 1 || K < kChunkCols || K % kChunkCols != 0 || (nk != 1 && nk != 2)) return SGEMV_EINVAL;
  if (K / kChunkCols > kMaxChunks) return SGEMV_ESIZE;
  sgemv_desc d;
  memset(&d, 0, sizeof d);
  const int32_t T = (N + kBlockRows - 1) / kBlockRows, C = K / kChunkCols;
  d.N = N; d.K = K; d.nk = nk;
  d.n_blocks = T;
  d.chunks = C;
  d.value_format = 1;
  d.kept = (int64_t)N * K * nk / 4;
  d.vals_bytes = d.kept * 2;
  d.offs_bytes = d.kept / 4;
  const int64_t records = (int64_t)T * C * 64;
  d.off_codes = 0;
  d.off_offs = align_up(records * piece_value16_bytes(nk));
  d.off_perm = align_up(d.off_offs + records * piece_offs16_bytes(nk));
  d.off_sz = align_up(d.off_perm + 4 * (int64_t)T * kBlockRows);   // no words: the blob ends here
  d.blob_bytes = d.off_sz;
  if (d.blob_bytes >= ((int64_t)1 << 31)) return SGEMV_ESIZE;
  *out = d;
  return SGEMV_OK;
}

extern "C" int sgemv_layout_fp16(const sgemv_desc* d, const uint16_t* vals16, const uint8_t* offs, void* blob_v) {
  if (!d || !vals16 || !offs || !blob_v || d->value_format != 1) return SGEMV_EINVAL;
  sgemv_desc chk;
  const int rc = sgemv_describe_fp16(d->N, d->K, d->nk, &chk);
  if (rc) return rc;
  if (memcmp(&chk, d, sizeof chk) != 0) return SGEMV_ESIZE;
  const int32_t N = d->N, K = d->K, nk = d->nk, T = d->n_blocks, C = d->chunks, kpr = K * nk / 4;
  const int kpp = 16 * nk, pvb = piece_value16_bytes(nk), pob = piece_offs16_bytes(nk);
  uint8_t* blob = (uint8_t*)blob_v;
  memset(blob, 0, (size_t)d->blob_bytes);
  int32_t* pm = (int32_t*)(blob + d->off_perm);
  for (int32_t i = 0; i < T * kBlockRows; ++i) pm[i] = i < N ? i : -1;
  for (int32_t n = 0; n < N; ++n) {
    const int32_t b = n / kBlockRows, r = n % kBlockRows;
    const uint16_t* vrow = vals16 + (int64_t)n * kpr;
    const uint8_t* orow = offs + (int64_t)n * (kpr / 4);
    for (int32_t c = 0; c < C; ++c)
      for (int q = 0; q < 4; ++q) {
        const int64_t rec = ((int64_t)b * C + c) * 64 + r + 16 * q;
        const int64_t e0 = (int64_t)kpp * (4 * c + q);
        // values in element order, in 16-byte slices: slice k of all 64 lanes, then slice k + 1
        const int64_t rec0 = ((int64_t)b * C + c) * 64;
        for (int k = 0; k < pvb / 16; ++k)
          memcpy(blob + d->off_codes + rec0 * pvb + (k * 64 + r + 16 * q) * 16, vrow + e0 + 8 * k, 16);
        if (nk == 2) {
          memcpy(blob + d->off_offs + rec * pob, orow + e0 / 4, pob);
        } else {
          uint32_t word = 0;
          for (int m = 0; m < 16; ++m) {
            const int64_t j = e0 + m;
            const uint32_t o = (orow[j >> 2] >> (2 * (j & 3))) & 3u;
            const int t = m / 4, e = m % 4;
            word |= o << (16 * (t % 2) + (t < 2 ? kOff14Real[e] : kOff14Dummy[e]));
          }
          memcpy(blob + d->off_offs + rec * pob, &word, 4);
        }
      }
  }
  return SGEMV_OK;
}

extern "C" int sgemv_layout(const sgemv_desc* d, const uint8_t* vals, const uint8_t* offs,
                            const uint16_t* scale, const uint16_t* zero, const int32_t* gptr,
                            void* blob_v) {
  if (!d || !vals || (!offs && d->nk != 4) || !scale || !zero || !gptr || !blob_v) return SGEMV_EINVAL;
  const int32_t N = d->N, K = d->K, nk = d->nk;
  if (N < 1 || K < kChunkCols || K % kChunkCols || !valid_nk(nk)) return SGEMV_EINVAL;
  // group sizes from the ragged row pointer of the scale/zero arrays
  std::vector<int32_t> gs(N);
  if (gptr[0] != 0) return SGEMV_EINVAL;
  for (int32_t n = 0; n < N; ++n) {
    const int32_t ng = gptr[n + 1] - gptr[n];
    if (ng <= 0 || K % ng) return SGEMV_EINVAL;
    gs[n] = K / ng;
    if (!valid_group(gs[n], K)) return SGEMV_EINVAL;
  }
  sgemv_desc chk;
  const int rc = sgemv_describe(N, K, nk, gs.data(), &chk);
  if (rc) return rc;
  if (memcmp(&chk, d, sizeof chk) != 0) return SGEMV_ESIZE;
  const int32_t T = d->n_blocks, C = d->chunks, kpr = K * nk / 4;
  const int pcb = piece_code_bytes(nk), pob = piece_offs_bytes(nk), kpp = 16 * nk;
  const std::vector<int32_t> perm = sorted_rows(gs.data(), N);
  // The kernel holds each weight as the FP16 value (code - zero) * scale:
  // reject layers where that rounds outside the FP16 range.
  for (int32_t n = 0; n < N; ++n) {
    const uint8_t* vrow = vals + (int64_t)n * (kpr / 2);
    const int32_t kpg = gs[n] * nk / 4;                // kept elements per group
    for (int32_t g = 0; g < kpr / kpg; ++g) {
      int lo = 15, hi = 0;
      for (int32_t j = g * kpg; j < (g + 1) * kpg; ++j) {
        const int code = (vrow[j >> 1] >> (4 * (j & 1))) & 0xF;
        lo = std::min(lo, code);
        hi = std::max(hi, code);
      }
      const int64_t grp = gptr[n] + g;
      const double s = f16_to_f64(scale[grp]), z = f16_to_f64(zero[grp]);
      if (!f16_finite(f64_to_f16((lo - z) * s)) || !f16_finite(f64_to_f16((hi - z) * s))) return SGEMV_EINVAL;
    }
  }
  uint8_t* blob = (uint8_t*)blob_v;
  memset(blob, 0, (size_t)d->blob_bytes);
  uint8_t* cb = blob + d->off_codes;
  uint8_t* ob = blob + d->off_offs;
  int32_t* pm = (int32_t*)(blob + d->off_perm);
  uint32_t* szb = (uint32_t*)(blob + d->off_sz);
  for (int32_t i = 0; i < T * kBlockRows; ++i) pm[i] = i < N ? perm[i] : -1;
  int64_t szw = 0;
  for (int32_t b = 0; b < T; ++b) {
    for (int32_t c = 0; c < C; ++c) {
      for (int32_t r = 0; r < kBlockRows; ++r) {
        const int32_t i = b * kBlockRows + r;
        if (i >= N) break;
        const int32_t n = perm[i];
        const uint8_t* vrow = vals + (int64_t)n * (kpr / 2);
        const uint8_t* orow = nk == 4 ? nullptr : offs + (int64_t)n * (kpr / 4);
        for (int q = 0; q < 4; ++q) {
          const int64_t rec = ((int64_t)b * C + c) * 64 + r + 16 * q;
          const int64_t e0 = (int64_t)kpp * (4 * c + q);        // first kept element of the piece
          if (nk == 4) {
            // dense: dword 2t + h holds in-group positions 2h, 2h + 1 of the 4
            // groups of columns 16t .. 16t + 15 (a 2-of-4 operand each)
            for (int dw = 0; dw < 8; ++dw) {
              uint32_t word = 0;
              for (int k = 0; k < 8; ++k) {
                const int64_t j = e0 + 16 * (dw / 2) + 4 * (k / 2) + 2 * (dw % 2) + (k % 2);
                const uint32_t code = (vrow[j >> 1] >> (4 * (j & 1))) & 0xFu;
                word |= code << (4 * kNib24[k]);
              }
              // 16-byte slices: dwords 0-3 of all 64 lanes, then dwords 4-7
              const int64_t rec0 = ((int64_t)b * C + c) * 64;
              memcpy(cb + rec0 * pcb + ((dw / 4) * 64 + r + 16 * q) * 16 + 4 * (dw % 4), &word, 4);
            }
            continue;
          }
          // codes: dwords of 8 elements with the nibble order of the N:M choice
          for (int dw = 0; dw < 2 * nk; ++dw) {
            uint32_t word = 0;
            for (int k = 0; k < 8; ++k) {
              const int64_t j = e0 + 8 * dw + k;
              const uint32_t code = (vrow[j >> 1] >> (4 * (j & 1))) & 0xFu;
              word |= code << (4 * (nk == 2 ? kNib24[k] : kNib14[k]));
            }
            memcpy(cb + rec * pcb + 4 * dw, &word, 4);
          }
          // offsets
          if (nk == 2) {
            memcpy(ob + rec * pob, orow + e0 / 4, pob);        // canonical bytes, unchanged
          } else {
            uint32_t word = 0;
            for (int m = 0; m < 16; ++m) {
              const int64_t j = e0 + m;
              const uint32_t o = (orow[j >> 2] >> (2 * (j & 3))) & 3u;
              const int t = m / 4, e = m % 4;
              word |= o << (16 * (t % 2) + (t < 2 ? kOff14Real[e] : kOff14Dummy[e]));
            }
            memcpy(cb + rec * pcb + 8, &word, 4);      // after the piece's 2 code dwords
          }
        }
        // scale|zero words of chunk c of this row
        const int per = kChunkCols / gs[n];
        for (int j = 0; j < per; ++j) {
          const int64_t src = gptr[n] + (int64_t)c * per + j;
          szb[szw++] = (uint32_t)scale[src] | ((uint32_t)zero[src] << 16);
        }
      }
    }
  }
  if (szw != d->n_groups) return SGEMV_ESIZE;
  return SGEMV_OK;
}

// Layer descriptor and kernel layout of the 2bit-CSR arrays.
//
// The kernel layout is a permutation of the canonical bits (no padding and
// no duplication) so that the SparseGemv kernel reads codes with 16-byte,
// offsets with 8-byte and scale|zero words with 4..16-byte coalesced loads:
//  - rows sorted by group size (ascending), ascending row index within a size;
//  - tiles of up to rt sorted rows of one group size, one workgroup each;
//  - a chunk = 32 consecutive kept elements of a row (cpc = 128/nk columns);
//    chunk c of a row goes to k-lane c % tpr at iteration c / tpr, and its
//    slot is row0*C + i*nr*tpr + r*cnt_i + kl (cnt_i chunks per row in
//    iteration i: tpr, or the remainder in the last one);
//  - inside a chunk, codes dword d holds elements 8d..8d+7 with nibble k
//    holding element 8d + 2k (k < 4) or 8d + 2(k-4) + 1 (k >= 4); offsets
//    dword D holds elements 16D..16D+15, element 16D + 4q + b at bits 8b + 2q;
//  - scale|zero<<16 words: chunk at tile slot s uses sz_base + (s*cpc)/g + j,
//    j < max(1, cpc/g), so chunks sharing a group share one stored word.
// Reference: the first contribution item of the page "Efficient LLM ad
// generation via model compression and parallel verification" (translation
// of arXiv 2605.11582), which introduces the index-compressed 2bit-CSR format
// but leaves its bit layout open.
#include <algorithm>
#include <numeric>
#include <vector>

#include "internal.hpp"

using namespace sgemv;

namespace {

struct Tile { int32_t row0, nr, g; };

// Sorted row order (by group size, stable) and the tile list.
void order_and_tiles(const int32_t* gs, int32_t N, int32_t rt, std::vector<int32_t>& perm,
                     std::vector<Tile>& tiles) {
  perm.resize(N);
  std::iota(perm.begin(), perm.end(), 0);
  std::stable_sort(perm.begin(), perm.end(), [&](int32_t a, int32_t b) { return gs[a] < gs[b]; });
  tiles.clear();
  int32_t i = 0;
  while (i < N) {
    int32_t g = gs[perm[i]], j = i;
    while (j < N && gs[perm[j]] == g) ++j;
    for (int32_t r0 = i; r0 < j; r0 += rt) tiles.push_back({r0, std::min(rt, j - r0), g});
    i = j;
  }
}

}  // namespace

extern "C" int sgemv_describe(int32_t N, int32_t K, int32_t nk, const int32_t* group_size,
                              int32_t rt, int32_t tpr, sgemv_desc* out) {
  if (!group_size || !out) return SGEMV_EINVAL;
  if (N < 1 || K < 256 || K % 256 != 0 || (nk != 1 && nk != 2)) return SGEMV_EINVAL;
  if ((int64_t)N * K * nk / 4 >= ((int64_t)1 << 31)) return SGEMV_ESIZE;
  int g_min = 1 << 30, g_max = 0;
  int64_t n_groups = 0;
  for (int32_t n = 0; n < N; ++n) {
    int g = group_size[n];
    if (!valid_group(g, K)) return SGEMV_EINVAL;
    g_min = std::min(g_min, g);
    g_max = std::max(g_max, g);
    n_groups += K / g;
  }
  const int cpc = cols_per_chunk(nk);
  const int32_t C = K * nk / 128;
  if (rt == 0 && tpr == 0) {
    // default: 256-lane workgroups, 32 lanes per row (two rows per wave), or
    // 64 when a row has more than 128 chunks (at most 4 chunks per lane)
    tpr = C > 128 ? 64 : 32;
    while (tpr > 4 && tpr / 2 >= C) tpr /= 2;
    rt = 256 / tpr;
  }
  if (!layout_params_ok(K, C, cpc, tpr, rt, g_max)) return SGEMV_ESIZE;
  std::vector<int32_t> perm;
  std::vector<Tile> tiles;
  order_and_tiles(group_size, N, rt, perm, tiles);
  sgemv_desc d;
  memset(&d, 0, sizeof d);
  d.N = N; d.K = K; d.nk = nk; d.rt = rt; d.tpr = tpr;
  d.n_tiles = (int32_t)tiles.size();
  d.g_min = g_min; d.g_max = g_max;
  for (int32_t n = 0; n < N; ++n) d.class_rows[ilog2(group_size[n] / 32)] += 1;
  d.kept = (int64_t)N * K * nk / 4;
  d.vals_bytes = d.kept / 2;
  d.offs_bytes = d.kept / 4;
  d.n_groups = n_groups;
  d.off_tiles = 0;
  d.off_perm = align_up(16 * (int64_t)d.n_tiles);
  d.off_vals = align_up(d.off_perm + 4 * (int64_t)N);
  d.off_offs = align_up(d.off_vals + 16 * (int64_t)N * C);
  d.off_sz = align_up(d.off_offs + 8 * (int64_t)N * C);
  d.blob_bytes = align_up(d.off_sz + 4 * n_groups);
  *out = d;
  return SGEMV_OK;
}

extern "C" int sgemv_layout(const sgemv_desc* d, const uint8_t* vals, const uint8_t* offs,
                            const uint16_t* scale, const uint16_t* zero, const int32_t* gptr,
                            void* blob_v) {
  if (!d || !vals || !offs || !scale || !zero || !gptr || !blob_v) return SGEMV_EINVAL;
  const int32_t N = d->N, K = d->K, nk = d->nk;
  if (N < 1 || K < 256 || K % 256 || (nk != 1 && nk != 2)) return SGEMV_EINVAL;
  // group sizes from the ragged row pointer of the scale/zero arrays
  std::vector<int32_t> gs(N);
  if (gptr[0] != 0) return SGEMV_EINVAL;
  for (int32_t n = 0; n < N; ++n) {
    int32_t ng = gptr[n + 1] - gptr[n];
    if (ng <= 0 || K % ng) return SGEMV_EINVAL;
    gs[n] = K / ng;
    if (!valid_group(gs[n], K)) return SGEMV_EINVAL;
  }
  sgemv_desc chk;
  int rc = sgemv_describe(N, K, nk, gs.data(), d->rt, d->tpr, &chk);
  if (rc) return rc;
  if (memcmp(&chk, d, sizeof chk) != 0) return SGEMV_ESIZE;
  const int cpc = cols_per_chunk(nk);
  const int32_t C = K * nk / 128, tpr = d->tpr, kpr = K * nk / 4;
  const int32_t I = (C + tpr - 1) / tpr;
  std::vector<int32_t> perm;
  std::vector<Tile> tiles;
  order_and_tiles(gs.data(), N, d->rt, perm, tiles);
  uint8_t* blob = (uint8_t*)blob_v;
  memset(blob, 0, (size_t)d->blob_bytes);
  int32_t* tab = (int32_t*)(blob + d->off_tiles);
  int32_t* pm = (int32_t*)(blob + d->off_perm);
  uint32_t* vb = (uint32_t*)(blob + d->off_vals);
  uint32_t* ob = (uint32_t*)(blob + d->off_offs);
  uint32_t* szb = (uint32_t*)(blob + d->off_sz);
  for (int32_t i = 0; i < N; ++i) pm[i] = perm[i];
  int64_t sz_base = 0;
  for (size_t t = 0; t < tiles.size(); ++t) {
    const Tile& T = tiles[t];
    tab[4 * t + 0] = T.row0;
    tab[4 * t + 1] = T.nr;
    tab[4 * t + 2] = T.g;
    tab[4 * t + 3] = (int32_t)sz_base;
    for (int32_t r = 0; r < T.nr; ++r) {
      const int32_t n = perm[T.row0 + r];
      const uint8_t* vrow = vals + (int64_t)n * (kpr / 2);
      const uint8_t* orow = offs + (int64_t)n * (kpr / 4);
      for (int32_t c = 0; c < C; ++c) {
        const int32_t i = c / tpr, kl = c % tpr;
        const int32_t cnt = (i == I - 1) ? C - (I - 1) * tpr : tpr;
        const int64_t s_rel = (int64_t)i * T.nr * tpr + (int64_t)r * cnt + kl;
        const int64_t slot = (int64_t)T.row0 * C + s_rel;
        const int64_t e0 = (int64_t)c * kChunkElems;
        for (int dw = 0; dw < 4; ++dw) {
          uint32_t word = 0;
          for (int k = 0; k < 8; ++k) {
            int m = (k < 4) ? 2 * k : 2 * (k - 4) + 1;
            int64_t j = e0 + 8 * dw + m;
            uint32_t code = (vrow[j >> 1] >> (4 * (j & 1))) & 0xFu;
            word |= code << (4 * k);
          }
          vb[4 * slot + dw] = word;
        }
        for (int D = 0; D < 2; ++D) {
          uint32_t word = 0;
          for (int q = 0; q < 4; ++q)
            for (int b = 0; b < 4; ++b) {
              int64_t j = e0 + 16 * D + 4 * q + b;
              uint32_t o = (orow[j >> 2] >> (2 * (j & 3))) & 3u;
              word |= o << (8 * b + 2 * q);
            }
          ob[2 * slot + D] = word;
        }
        const int per = std::max(1, cpc / T.g);
        for (int j = 0; j < per; ++j) {
          int64_t src = gptr[n] + ((int64_t)c * cpc) / T.g + j;
          int64_t dst = sz_base + (s_rel * cpc) / T.g + j;
          szb[dst] = (uint32_t)scale[src] | ((uint32_t)zero[src] << 16);
        }
      }
    }
    sz_base += (int64_t)T.nr * C * cpc / T.g;
  }
  if (sz_base != d->n_groups) return SGEMV_ESIZE;
  return SGEMV_OK;
}

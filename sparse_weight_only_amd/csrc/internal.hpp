// Internal helpers shared by the host packer, the layout builder and the
// kernel launcher (product side only).
#pragma once
#include <stdint.h>
#include <string.h>

#include "../../include/sgemv.h"

namespace sgemv {

constexpr int kChunkElems = 32;            // kept elements per chunk (16 B codes, 8 B offsets)
constexpr int kMaxChunksPerThread = 8;     // register budget of the kernels
constexpr int64_t kAlign = 256;            // blob section alignment

inline int cols_per_chunk(int nk) { return 128 / nk; }          // 64 at 2:4, 128 at 1:4
inline int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool valid_group(int g, int K) { return (g == 32 || g == 64 || g == 128 || g == 256) && K % g == 0; }
inline int ilog2(int v) { int l = 0; while ((1 << l) < v) ++l; return l; }

// IEEE 754 binary64 -> binary16, round to nearest, ties to even, in one step.
inline uint16_t f64_to_f16(double x) {
  uint64_t b;
  memcpy(&b, &x, 8);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  uint64_t ab = b & 0x7FFFFFFFFFFFFFFFull;
  if (ab >= 0x7FF0000000000000ull) return (uint16_t)(sign | (ab > 0x7FF0000000000000ull ? 0x7E00u : 0x7C00u));
  int e = (int)(ab >> 52) - 1023;
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  if (e < -25) return sign;                         // below half the smallest subnormal
  uint64_t sig = (1ull << 52) | (ab & ((1ull << 52) - 1));
  if (e >= -14) {                                   // normal range: keep 10 fraction bits
    uint64_t q = sig >> 42, rem = sig & ((1ull << 42) - 1), half = 1ull << 41;
    if (rem > half || (rem == half && (q & 1))) ++q;
    int E = e + 15;
    if (q == 2048) { q = 1024; ++E; }
    if (E >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (E << 10) | (int)(q - 1024));
  }
  int shift = 28 - e;                               // subnormal: quantum 2^-24
  uint64_t q = sig >> shift, rem = sig & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  return (uint16_t)(sign | q);                      // q == 1024 is the smallest normal
}

// binary16 -> binary64 (exact).
inline double f16_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = (double)m * (1.0 / 16777216.0);
  else if (e == 31) v = m ? __builtin_nan("") : __builtin_inf();
  else {
    v = (double)(1024 + m);
    int sh = e - 25;
    while (sh > 0) { v *= 2.0; --sh; }
    while (sh < 0) { v *= 0.5; ++sh; }
  }
  return s ? -v : v;
}

inline bool f16_finite(uint16_t h) { return ((h >> 10) & 31) != 31; }

// Kernel geometry of a layout: a tile of rt rows with tpr lanes per row is
// one workgroup of min(256, rt*tpr) lanes, each lane owning rpl rows.
struct Geometry { int wg, rpl, iters, imax, xmax; };
inline int bucket(int n) { return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 8; }
inline Geometry geometry(int32_t K, int32_t C, int32_t tpr, int32_t rt) {
  Geometry g;
  const int32_t slots = rt * tpr;
  g.wg = slots < 256 ? slots : 256;
  g.rpl = slots / g.wg;
  g.iters = (C + tpr - 1) / tpr;
  g.imax = bucket(g.iters);
  g.xmax = ((K / 8 + g.wg - 1) / g.wg) <= 2 ? 2 : 8;
  return g;
}

// Layout parameters the kernels accept: tpr lanes per row (a power of two in
// [4, 64], so a row's lanes sit in one wave); rt*tpr a power of two in
// [64, 1024] giving 1, 2 or 4 rows per lane; at most 8 chunks per row-lane and
// 8 chunks per lane in all; at most 8 x blocks of 8 columns staged per lane;
// chunks that share a scale word owned by the same iteration.
inline bool layout_params_ok(int32_t K, int32_t C, int cpc, int32_t tpr, int32_t rt, int g_max) {
  if (tpr < 4 || tpr > 64 || (tpr & (tpr - 1))) return false;
  const int32_t slots = rt * tpr;
  if (rt < 1 || slots < 64 || slots > 1024 || (slots & (slots - 1))) return false;
  const Geometry g = geometry(K, C, tpr, rt);
  if (g.iters > kMaxChunksPerThread || g.rpl * g.imax > kMaxChunksPerThread) return false;
  if ((K / 8 + g.wg - 1) / g.wg > 8) return false;
  if (g_max > cpc) {
    const int share = g_max / cpc;   // chunks sharing one scale/zero word
    if (tpr % share || C % share) return false;
  }
  return true;
}

}  // namespace sgemv

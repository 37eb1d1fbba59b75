// Internal helpers shared by the host packer, the layout builder and the
// kernel launcher (product side only).
#pragma once
#include <stdint.h>
#include <string.h>

#include "../../include/sgemv.h"

namespace sgemv {

constexpr int64_t kAlign = 256;            // blob section alignment

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

// Dense columns per column chunk; a chunk of one row is split into 4 pieces
// of 64 columns, one per lane block of the matrix-core instruction.
constexpr int kChunkCols = 256;
constexpr int kBlockRows = 16;             // rows per row block (matrix-core tile height)
constexpr int kMaxChunks = 128;            // K <= 32768
constexpr int kMaxWaves = 16;              // waves per workgroup
constexpr int kMaxChunksPerWave = 8;       // register budget of the kernel

inline int bucket(int n) { return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 8; }

// Bytes of one piece (one row, 64 dense columns) in the code and offset sections.
// nk = 4 is the dense ablation: every element kept, no offsets stored.
inline bool valid_nk(int nk) { return nk == 1 || nk == 2 || nk == 4; }
// Bytes of one lane's piece in the code section: 16 (1:4, with its offset
// dword after the 8 bytes of codes), 32 (2:4) or 64 (dense) nibbles; in the
// offset section: 8 at 2:4, none otherwise (the FP16-valued form keeps
// 4 * nk bytes of offsets in a section of its own).
inline int piece_code_bytes(int nk) { return nk == 1 ? 12 : 8 * nk; }
inline int piece_offs_bytes(int nk) { return nk == 2 ? 8 : 0; }
inline int piece_offs16_bytes(int nk) { return 4 * nk; }
inline int piece_value16_bytes(int nk) { return 32 * nk; }                // FP16-valued form

// Launch geometry for (chunks per row, row blocks, batch): how the column
// chunks of a row block are split over the waves of its workgroup and how
// many chunks of x are staged in LDS at once.
struct Launch { int waves, cpw, crem, imax, phase, xloads, xmax, rb; int64_t lds; };

// Wave w takes chunks [w * cpw - max(0, w - crem), ...), cpw of them if
// w < crem, else cpw - 1 (fewer at the end of the row): the waves' ranges
// are contiguous. The most chunks any of the 4 SIMDs of a workgroup gets,
// waves being placed on SIMD w % 4.
inline int simd_max_chunks(int C, int W, int cpw, int crem) {
  int per[4] = {0, 0, 0, 0};
  for (int w = 0; w < W; ++w) {
    const int c0 = w * cpw - (w > crem ? w - crem : 0);
    const int cmax = cpw - (w >= crem ? 1 : 0);
    const int n = C - c0 < cmax ? (C - c0 > 0 ? C - c0 : 0) : cmax;
    per[w & 3] += n;
  }
  int m = per[0];
  for (int k = 1; k < 4; ++k) m = per[k] > m ? per[k] : m;
  return m;
}
inline Launch launch_geometry(int C, int T, int B) {
  Launch L;
  L.rb = 1;
  // up to 4 vectors, two chunks per wave where that keeps the workgroup
  // within 16 waves: a wave with fewer loads to issue starts computing
  // sooner, which hides more of the dequantisation under the data phase.
  // Otherwise (and for larger batches, whose x slices dominate) four.
  int cpw = (B <= 4 && (C + 1) / 2 <= kMaxWaves) ? 2 : 4;
  // smaller slices when the layer has few row blocks, so the grid has
  // enough waves to cover the chip (256 CUs x 4 SIMDs, two waves each)
  while (cpw > 1 && (int64_t)T * ((C + cpw - 1) / cpw) < 2048) cpw /= 2;
  // one vector: one step further below 4096 waves, where the workgroup
  // stays within 16 waves: 4096 x 4096 layers (256 row blocks) as 16 waves
  // of one chunk took 3.62-3.64 us per call against 3.73-3.75 us as 8 waves
  // of two, and the 224-GEMV decoder sequence 961 us against 974 us (several
  // vectors keep the previous geometry: not measured)
  if (B == 1 && cpw > 1 && (int64_t)T * ((C + cpw - 1) / cpw) < 4096 && (C + cpw / 2 - 1) / (cpw / 2) <= kMaxWaves)
    cpw /= 2;
  if ((C + cpw - 1) / cpw > kMaxWaves) cpw = (C + kMaxWaves - 1) / kMaxWaves;
  L.cpw = cpw;
  L.waves = (C + cpw - 1) / cpw;
  L.crem = L.waves;   // every wave takes cpw chunks, the last one what is left
  // The dequantisation of a workgroup is bounded by its busiest SIMD. One
  // more wave, with the chunks split evenly (C % W waves take cpw, the
  // others cpw - 1), when that lowers the most chunks on a SIMD at the same
  // cpw: 43 chunks (K = 11008) as 11 waves of 4 put 12 chunks on a SIMD,
  // 12 waves (7 of 4, 5 of 3) put 11. Measured on the 11008 -> 4096 layers:
  // 0.11-0.13 us off a call at one vector, 0.1-0.45 us off at 4 and 16
  // vectors, 0.15 us more at 8 vectors at 1:4.
  if (L.waves < kMaxWaves) {
    const int W = L.waves + 1, rem = C % W, c2 = C / W + (rem ? 1 : 0);
    if (c2 == cpw && simd_max_chunks(C, W, cpw, rem ? rem : W) < simd_max_chunks(C, L.waves, cpw, L.crem)) {
      L.waves = W;
      L.crem = rem ? rem : W;
    }
  }
  L.imax = bucket(cpw);
  // x of phase chunks staged at once: B * phase <= 16 keeps the staging at
  // most 8 16-byte loads per lane
  // (a power of two: the kernel splits x units with a shift)
  int ph = 1;
  while (ph * 2 <= cpw && B * ph * 2 <= 16) ph *= 2;
  if (ph < cpw && B * cpw <= 16 && (cpw & (cpw - 1)) == 0) ph = cpw;
  L.phase = ph;
  L.xloads = (B * ph * 32 + 63) / 64;
  L.xmax = bucket(L.xloads);
  // per wave: B rows of x, each ph * 512 bytes plus 16 bytes of padding
  // (the one-vector kernel of the INT4 form leaves the padding unused)
  L.lds = (int64_t)L.waves * B * (ph * 512 + 16) + (int64_t)B * kBlockRows * kMaxWaves * 4;
  return L;
}

// Several vectors on a layer with many row blocks: rb row blocks per
// workgroup, so that each wave loads its x slices once for all rb blocks (the
// x traffic from L2 falls rb-fold; at 16 vectors the x of a 4096-column layer
// is 128 KiB per workgroup, five times the weights of one row block). The
// weights of rb x 2 pieces are held in registers, and the partial sums keep
// one slot per wave. Measured on the 11008 x 4096 layers (688 row blocks):
// 4 blocks per workgroup take 15 % off a call at 16 vectors and 7 % at 8, and
// add 10 % at 4 (2 blocks: no better at 8, worse at 16). So: rb = 4 from 8
// vectors on, where K <= 4096 (at most 8 waves of two chunks) and the merged
// grid still has 160 or more workgroups; rb = 1 otherwise.
inline int pick_row_blocks(int C, int T, int B) {
  return B >= 8 && C <= 16 && (int64_t)T >= 4 * 160 ? 4 : 1;
}
constexpr int kMaxWavesRb = 8;             // waves per workgroup with several row blocks (256 VGPRs a lane)
inline Launch launch_geometry_rb(int C, int T, int B, int rb) {
  Launch L = launch_geometry(C, T, B);
  if (rb <= 1) return L;
  // at most 8 waves, at least two chunks per wave
  int cpw = (C + kMaxWavesRb - 1) / kMaxWavesRb;
  if (cpw < 2) cpw = 2;
  L.rb = rb;
  L.cpw = cpw;
  L.waves = (C + cpw - 1) / cpw;
  L.crem = L.waves;
  L.imax = bucket(cpw);
  int ph = 1;
  while (ph * 2 <= cpw && B * ph * 2 <= 16) ph *= 2;
  L.phase = ph;
  L.xloads = (B * ph * 32 + 63) / 64;
  L.xmax = bucket(L.xloads);
  // x slices as above; partial sums: one slot per wave for every (vector,
  // block, row); the blocks' original row indices
  L.lds = (int64_t)L.waves * B * (ph * 512 + 16) + (int64_t)L.waves * rb * B * kBlockRows * 4 + (int64_t)rb * kBlockRows * 4;
  return L;
}

}  // namespace sgemv

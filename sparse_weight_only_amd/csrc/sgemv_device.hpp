// Device code of the SparseGemv kernels for gfx950 (MI355X, CDNA4, wave64).
//
// y = W' x for an N:M-sparse (2:4 or 1:4 along K) INT4 weight matrix with
// per-group FP16 scale and zero, FP16 activations and FP32 accumulation: the
// custom weight-only GEMV with mixed sparsity of the page "Efficient LLM ad
// generation via model compression and parallel verification" (translation
// of arXiv 2605.11582), §1 (second contribution item) and §3.3 "Revised
// kernel". That section stops before describing its kernel; the design here
// is our own for CDNA4.
//
// One workgroup per tile of rt rows of one group size; tpr lanes per row
// split the row's 32-element chunks round-robin (chunk c -> lane c % tpr,
// iteration c / tpr), so that a row's lanes are consecutive in one wave.
//  1. every lane issues all of its weight loads first: a 16-byte code load,
//     an 8-byte offset load and a 4/8/16-byte scale|zero load per chunk,
//     coalesced across the workgroup by the kernel layout;
//  2. the workgroup stages x into LDS as byte planes (per 8 columns: 8 low
//     bytes, then 8 high bytes), one 16-byte pad after every chunk's columns
//     so that neighbouring lanes start in different banks;
//  3. per 4 kept elements: the 2-bit offsets become v_perm byte selectors
//     that pick the matching x halves out of the planes; nibbles become FP16
//     (q - z) exactly via the 0x6400 exponent trick; v_dot2_f32_f16
//     accumulates in FP32; the FP16 scale multiplies each group's partial;
//  4. a DPP reduction over the row's lanes; the row's last lane writes y in
//     FP16 (round to nearest even) at the row's original position.
// The products (q - z) * x are exact in FP32, so the only roundings are the
// FP32 accumulation and the final FP16 conversion.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemv_dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __fp16 hp16x2 __attribute__((ext_vector_type(2)));

struct KParams {
  const int32_t* tiles;  // [n_tiles][4] = row0, nr, g, sz_base
  const int32_t* perm;   // [N] original row of each sorted row
  const u32x4* vals;     // [slots] 16-byte code chunks
  const u32x2* offs;     // [slots] 8-byte offset chunks
  const uint32_t* sz;    // [n_groups] scale | zero << 16
  const u32x4* x;        // [B][K/8]
  uint16_t* y;           // [B][N]
  int32_t N, K, C, B;
  int32_t tpr_log2;
  int32_t phase_iters;   // chunk iterations whose x columns are staged at once
  int32_t pass_log2;     // workgroups per tile = 1 << pass_log2 (batched kernels)
  int32_t rt;            // rows per tile
  int32_t cls_tile[5];   // first tile of each group-size class (32, 64, 128, 256), then n_tiles
  int32_t cls_row[5];    // first sorted row of each class, then N
  int32_t cls_sz[4];     // first scale|zero word of each class
};

// Tile geometry from the class table (no dependent load of the blob's tile table).
struct TileGeo { int row0, nr, g, sz_base; };
__device__ __forceinline__ TileGeo tile_geo(const KParams& p, int tile) {
  // class c = last class whose first tile is <= tile; the flags are monotone,
  // so telescoping sums pick the class's values without an indexed lookup
  const int f1 = tile >= p.cls_tile[1], f2 = tile >= p.cls_tile[2], f3 = tile >= p.cls_tile[3];
  const int c = f1 + f2 + f3;
  auto pick = [&](const int32_t* a) {
    return a[0] + f1 * (a[1] - a[0]) + f2 * (a[2] - a[1]) + f3 * (a[3] - a[2]);
  };
  const int ct = pick(p.cls_tile), cr = pick(p.cls_row), cz = pick(p.cls_sz), end = pick(p.cls_row + 1);
  TileGeo t;
  t.g = 32 << c;
  t.row0 = cr + (tile - ct) * p.rt;
  t.nr = end - t.row0 < p.rt ? end - t.row0 : p.rt;
  t.sz_base = cz + (t.row0 - cr) * (p.K >> (5 + c));
  return t;
}

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// (a & m) | c in one v_and_or_b32 (m in an SGPR, c in a VGPR: one constant-bus read).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
  return r;
}

__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

__device__ __forceinline__ float dot2(f16x2 a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(hp16x2, a), __builtin_bit_cast(hp16x2, b), c, false);
}

// Constants kept in VGPRs so that v_and_or_b32 can take them.
struct Consts {
  uint32_t magic;     // 0x64006400: two FP16 1024.0
  uint32_t sel_or;    // +4 added to the selector bytes of the second group (2:4) or odd elements (1:4)
};

// FP16 (q - z) pairs of one code dword: (e0,e1), (e2,e3), (e4,e5), (e6,e7).
// 0x6400 | n is the FP16 value 1024 + n; 0x6400 | (n << 4) is 1024 + 16 n.
struct Deq { f16x2 w01, w23, w45, w67; };
__device__ __forceinline__ Deq dequant_dword(uint32_t v, f16x2 zc1, f16x2 zc2, const Consts& k) {
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  Deq d;
  const uint32_t v8 = v >> 8;
  d.w01 = as_f16x2(and_or(v, 0x000F000Fu, k.magic)) + zc1;                                  // n - z
  d.w23 = __builtin_elementwise_fma(as_f16x2(and_or(v, 0x00F000F0u, k.magic)), sixteenth, zc2);  // (1024+16n)/16 - 64 - z
  d.w45 = as_f16x2(and_or(v8, 0x000F000Fu, k.magic)) + zc1;
  d.w67 = __builtin_elementwise_fma(as_f16x2(and_or(v8, 0x00F000F0u, k.magic)), sixteenth, zc2);
  return d;
}

__device__ __forceinline__ void zero_consts(uint32_t szw, f16x2& zc1, f16x2& zc2, float& sf) {
  const _Float16 z = __builtin_bit_cast(_Float16, (uint16_t)(szw >> 16));
  const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)(szw & 0xFFFFu));
  const _Float16 a = (_Float16)-1024.0f - z;  // exact: integers up to 1039
  const _Float16 b = (_Float16)-64.0f - z;
  zc1 = f16x2{a, a};
  zc2 = f16x2{b, b};
  sf = (float)s;
}

// Byte selectors of quad qq (4 consecutive kept elements of the chunk):
// offsets of its elements in the four bytes, +4 where the element's x lives
// in the second 4-column half of the 8-column plane block.
__device__ __forceinline__ uint32_t quad_selector(const u32x2 o, int qq, const Consts& k) {
  const uint32_t w = (qq < 4) ? o.x : o.y;
  const int sh = 2 * (qq & 3);
  return and_or(sh ? (w >> sh) : w, 0x03030303u, k.sel_or);
}

// x halves of the kept elements of one 2:4 quad (groups 2qq, 2qq+1 of the
// chunk, both inside the 8-column plane block X).
__device__ __forceinline__ void xsel_2of4(const u32x4 X, uint32_t M, uint32_t& xab, uint32_t& xcd) {
  const uint32_t lo = perm_b32(X.y, X.x, M);
  const uint32_t hi = perm_b32(X.w, X.z, M);
  xab = perm_b32(hi, lo, 0x05010400u);
  xcd = perm_b32(hi, lo, 0x07030602u);
}

// x halves of one 1:4 quad (4 groups, 16 columns: plane blocks X and Y).
__device__ __forceinline__ void xsel_1of4(const u32x4 X, const u32x4 Y, uint32_t M, uint32_t& xab, uint32_t& xcd) {
  const uint32_t lo = perm_b32(X.y, X.x, M);
  const uint32_t hi = perm_b32(X.w, X.z, M);
  xab = perm_b32(hi, lo, 0x05010400u);
  const uint32_t lo2 = perm_b32(Y.y, Y.x, M);
  const uint32_t hi2 = perm_b32(Y.w, Y.z, M);
  xcd = perm_b32(hi2, lo2, 0x07030602u);
}

// One chunk (32 kept elements) of one row against B activation vectors
// (x planes of the chunk at xc, ldsb blocks apart per vector).
template <int NK, int G, int BMAX, int SPC>
__device__ __forceinline__ void chunk_compute(const u32x4 v, const u32x2 o, const uint32_t (&s)[SPC],
                                              const u32x4* __restrict__ xc, int ldsb, int B,
                                              float (&tot)[BMAX], const Consts& k) {
  constexpr int CPC = 128 / NK;
  constexpr int QPG = (G >= CPC) ? 8 : (8 * G) / CPC;  // quads (4 kept elements) per scale group
#pragma unroll
  for (int q0 = 0; q0 < 8; q0 += QPG) {
    f16x2 zc1, zc2;
    float sf;
    zero_consts(s[(G >= CPC) ? 0 : q0 / QPG], zc1, zc2, sf);
    float acc[BMAX];
#pragma unroll
    for (int b = 0; b < BMAX; ++b) acc[b] = 0.0f;
#pragma unroll
    for (int qq = q0; qq < q0 + QPG; qq += 2) {
      const Deq d = dequant_dword(v[qq >> 1], zc1, zc2, k);
      const uint32_t MA = quad_selector(o, qq, k);
      const uint32_t MB = quad_selector(o, qq + 1, k);
#pragma unroll
      for (int b = 0; b < BMAX; ++b) {
        if (BMAX == 1 || b < B) {
          const u32x4* xb = xc + b * ldsb;
          uint32_t xab, xcd, xef, xgh;
          if constexpr (NK == 2) {
            xsel_2of4(xb[qq], MA, xab, xcd);
            xsel_2of4(xb[qq + 1], MB, xef, xgh);
          } else {
            xsel_1of4(xb[2 * qq], xb[2 * qq + 1], MA, xab, xcd);
            xsel_1of4(xb[2 * qq + 2], xb[2 * qq + 3], MB, xef, xgh);
          }
          float a = acc[b];
          a = dot2(d.w01, xab, a);
          a = dot2(d.w23, xcd, a);
          a = dot2(d.w45, xef, a);
          a = dot2(d.w67, xgh, a);
          acc[b] = a;
        }
      }
    }
#pragma unroll
    for (int b = 0; b < BMAX; ++b) tot[b] = __builtin_fmaf(sf, acc[b], tot[b]);
  }
}

// Stage x columns [col0, col0 + ncols) of every batch vector into LDS planes.
template <int NK>
__device__ __forceinline__ void stage_x(const KParams& p, u32x4* xs, int col0, int ncols, int ldsb,
                                        int tid, int nthreads) {
  constexpr int CPC = 128 / NK, BPC = CPC / 8, LSTRIDE = BPC + 1;
  const int nblk = ncols >> 3;
  const int kb = p.K >> 3;
  for (int m = tid; m < p.B * nblk; m += nthreads) {
    const int b = m / nblk, blk = m - b * nblk;
    const int col = col0 + (blk << 3);
    if (col < p.K) {
      const u32x4 xv = p.x[b * kb + (col >> 3)];
      u32x4 pl;
      pl.x = perm_b32(xv.y, xv.x, 0x06040200u);  // low bytes of columns 0..3
      pl.y = perm_b32(xv.w, xv.z, 0x06040200u);  // low bytes of columns 4..7
      pl.z = perm_b32(xv.y, xv.x, 0x07050301u);  // high bytes of columns 0..3
      pl.w = perm_b32(xv.w, xv.z, 0x07050301u);  // high bytes of columns 4..7
      xs[b * ldsb + (blk / BPC) * LSTRIDE + (blk % BPC)] = pl;
    }
  }
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over groups of 2^tpr_log2 consecutive lanes with DPP; the group's last
// lane ends up holding the group's total.
__device__ __forceinline__ float row_reduce(float a, int tpr_log2) {
  if (tpr_log2 >= 1) a += dpp_f32<0xB1, 0xF>(a);   // quad_perm [1,0,3,2]
  if (tpr_log2 >= 2) a += dpp_f32<0x4E, 0xF>(a);   // quad_perm [2,3,0,1]
  if (tpr_log2 >= 3) a += dpp_f32<0x141, 0xF>(a);  // row_half_mirror
  if (tpr_log2 >= 4) a += dpp_f32<0x140, 0xF>(a);  // row_mirror
  if (tpr_log2 >= 5) a += dpp_f32<0x142, 0xA>(a);  // row_bcast:15 into rows 1 and 3
  if (tpr_log2 >= 6) a += dpp_f32<0x143, 0xC>(a);  // row_bcast:31 into rows 2 and 3
  return a;
}

// Thread role inside a tile: the row r, its k-lane kl and how many chunks it owns.
struct Role {
  int r, kl, nch, I, rem, TPR;
  bool active;
};

__device__ __forceinline__ Role make_role(const KParams& p, int vt, int nr) {
  Role o;
  o.TPR = 1 << p.tpr_log2;
  o.r = vt >> p.tpr_log2;
  o.kl = vt & (o.TPR - 1);
  o.active = o.r < nr;
  o.I = (p.C + o.TPR - 1) >> p.tpr_log2;
  o.rem = p.C - (o.I - 1) * o.TPR;
  o.nch = o.active ? (o.kl < o.rem ? o.I : o.I - 1) : 0;
  return o;
}

// Loads of one chunk slot: codes, offsets and its scale|zero words.
template <int SPC, int SHARE>
__device__ __forceinline__ void load_chunk(const KParams& p, int64_t slot0, int s_rel, int sz_base,
                                           u32x4& v, u32x2& o, uint32_t (&s)[SPC]) {
  v = __builtin_nontemporal_load(p.vals + slot0 + s_rel);
  o = __builtin_nontemporal_load(p.offs + slot0 + s_rel);
  const uint32_t* sp = p.sz + sz_base + (SPC > 1 ? s_rel * SPC : s_rel / SHARE);
  if constexpr (SPC == 4) {
    const u32x4 w = __builtin_nontemporal_load((const u32x4*)sp);
    s[0] = w.x; s[1] = w.y; s[2] = w.z; s[3] = w.w;
  } else if constexpr (SPC == 2) {
    const u32x2 w = __builtin_nontemporal_load((const u32x2*)sp);
    s[0] = w.x; s[1] = w.y;
  } else {
    s[0] = __builtin_nontemporal_load(sp);
  }
}

// One tile (or one pass of a tile) at batch <= BMAX with up to MAXCH chunks per lane.
template <int NK, int G, int BMAX, int MAXCH>
__device__ __forceinline__ void tile_body(const KParams& p, u32x4* xs, int row0, int nr, int sz_base, int vt) {
  constexpr int CPC = 128 / NK;
  constexpr int LSTRIDE = CPC / 8 + 1;
  constexpr int SPC = (G >= CPC) ? 1 : CPC / G;   // scale words per chunk
  constexpr int SHARE = (G > CPC) ? G / CPC : 1;  // chunks per scale word
  const Role ro = make_role(p, vt, nr);
  const int64_t slot0 = (int64_t)row0 * p.C;
  Consts k;
  k.magic = 0x64006400u;
  k.sel_or = NK == 2 ? 0x04040000u : 0x04000400u;

  const int yrow = p.perm[row0 + (ro.active ? ro.r : 0)];
  u32x4 v[MAXCH];
  u32x2 o[MAXCH];
  uint32_t s[MAXCH][SPC];
#pragma unroll
  for (int i = 0; i < MAXCH; ++i) {
    if (i < ro.nch) {
      const int cnt = (i == ro.I - 1) ? ro.rem : ro.TPR;
      load_chunk<SPC, SHARE>(p, slot0, i * nr * ro.TPR + ro.r * cnt + ro.kl, sz_base, v[i], o[i], s[i]);
    }
  }

  const int PI = p.phase_iters;
  const int ldsb = PI * ro.TPR * LSTRIDE;  // LDS blocks per batch vector
  const int phase_cols = PI * ro.TPR * CPC;
  const int tid = threadIdx.x, nthr = blockDim.x;
  stage_x<NK>(p, xs, 0, phase_cols, ldsb, tid, nthr);
  __syncthreads();

  float tot[BMAX];
#pragma unroll
  for (int b = 0; b < BMAX; ++b) tot[b] = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXCH; ++i) {
    const int ip = (MAXCH == 1) ? 0 : i % PI;
    if (MAXCH > 1 && i > 0 && ip == 0 && i < ro.I) {  // uniform across the workgroup
      __syncthreads();
      stage_x<NK>(p, xs, (i / PI) * phase_cols, phase_cols, ldsb, tid, nthr);
      __syncthreads();
    }
    if (i < ro.nch) {
      const u32x4* xc = xs + (ip * ro.TPR + ro.kl) * LSTRIDE;
      chunk_compute<NK, G, BMAX, SPC>(v[i], o[i], s[i], xc, ldsb, p.B, tot, k);
    }
  }

#pragma unroll
  for (int b = 0; b < BMAX; ++b) {
    if (BMAX == 1 || b < p.B) {
      const float a = row_reduce(tot[b], p.tpr_log2);
      if (ro.active && ro.kl == ro.TPR - 1) p.y[(int64_t)b * p.N + yrow] = __builtin_bit_cast(uint16_t, (_Float16)a);
    }
  }
}

// Raw buffer loads: 32-bit lane offsets from a per-workgroup base held in
// SGPRs; offsets at or beyond the range return zeros without touching memory.
constexpr int kBufferWord3 = 0x00020000;   // raw 32-bit buffer, gfx9-family layout
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}
// CPOL: 0 = default caching, 2 = non-temporal (the weights are read once).
constexpr int kCached = 0, kStream = 2;
template <int CPOL = kCached>
__device__ __forceinline__ u32x4 bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL));
}
template <int CPOL = kCached>
__device__ __forceinline__ u32x2 bload2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CPOL));
}
template <int CPOL = kCached>
__device__ __forceinline__ uint32_t bload1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CPOL);
}

// Batch-1 tile. A workgroup of nthr lanes covers rt = RPL * nthr / tpr rows:
// lane (lane_row, kl) handles rows lane_row + j * nthr / tpr, j < RPL, and
// chunks kl, kl + tpr, ... (< IMAX per row) of each. x is staged once per
// workgroup; its loads are issued before the weight loads so that the LDS
// staging and the barrier do not wait for the weights (vector loads complete
// in issue order). Every load is unconditional (lanes without work read out
// of range and get zeros), so the number of loads in flight is static and
// each chunk is consumed as soon as its own loads have landed.
template <int NK, int G, int RPL, int IMAX, int XMAX>
__device__ __forceinline__ void tile_b1(const KParams& p, u32x4* xs, int row0, int nr, int sz_base) {
  constexpr int CPC = 128 / NK, BPC = CPC / 8, LSTRIDE = BPC + 1;
  constexpr int SPC = (G >= CPC) ? 1 : CPC / G;
  constexpr int SHARE = (G > CPC) ? G / CPC : 1;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int tl = p.tpr_log2, TPR = 1 << tl;
  const int lane_row = tid >> tl, kl = tid & (TPR - 1);
  const int rows_per_pass = nthr >> tl;
  const int C = p.C;
  const int I = (C + TPR - 1) >> tl;
  const int rem = C - (I - 1) * TPR;
  Consts k;
  k.magic = 0x64006400u;
  k.sel_or = NK == 2 ? 0x04040000u : 0x04000400u;

  // per-workgroup buffer windows
  const uint32_t tile_slots = (uint32_t)nr * (uint32_t)C;
  const int64_t slot0 = (int64_t)row0 * C;
  const auto rx = make_rsrc(p.x, (uint32_t)p.K * 2u);
  const auto rv = make_rsrc(p.vals + slot0, tile_slots * 16u);
  const auto ro = make_rsrc(p.offs + slot0, tile_slots * 8u);
  const auto rs = make_rsrc(p.sz + sz_base, tile_slots * (uint32_t)CPC / (uint32_t)G * 4u);
  const auto rp = make_rsrc(p.perm + row0, (uint32_t)nr * 4u);

  // 1. x loads (16 bytes = 8 columns each)
  const int nblk = p.K >> 3;
  u32x4 xv[XMAX];
#pragma unroll
  for (int j = 0; j < XMAX; ++j) xv[j] = bload4(rx, (uint32_t)(tid + j * nthr) * 16u);
  __builtin_amdgcn_sched_barrier(0);
  // 2. row indices and weight loads
  uint32_t yrow[RPL];
  bool has[RPL][IMAX];
  u32x4 v[RPL][IMAX];
  u32x2 o[RPL][IMAX];
  uint32_t s[RPL][IMAX][SPC];
#pragma unroll
  for (int j = 0; j < RPL; ++j) {
    const int r = lane_row + j * rows_per_pass;
    const bool row_ok = r < nr;
    yrow[j] = bload1(rp, row_ok ? (uint32_t)r * 4u : kOutOfRange);
#pragma unroll
    for (int i = 0; i < IMAX; ++i) {
      const bool ok = row_ok && (i < I - 1 || (i == I - 1 && kl < rem));
      has[j][i] = ok;
      const int cnt = (i == I - 1) ? rem : TPR;
      const uint32_t s_rel = (uint32_t)(i * nr * TPR + r * cnt + kl);
      v[j][i] = bload4<kStream>(rv, ok ? s_rel * 16u : kOutOfRange);
      o[j][i] = bload2<kStream>(ro, ok ? s_rel * 8u : kOutOfRange);
      const uint32_t soff = ok ? (SPC > 1 ? s_rel * SPC : s_rel / SHARE) * 4u : kOutOfRange;
      if constexpr (SPC == 4) {
        const u32x4 w = bload4<kStream>(rs, soff);
        s[j][i][0] = w.x; s[j][i][1] = w.y; s[j][i][2] = w.z; s[j][i][3] = w.w;
      } else if constexpr (SPC == 2) {
        const u32x2 w = bload2<kStream>(rs, soff);
        s[j][i][0] = w.x; s[j][i][1] = w.y;
      } else {
        s[j][i][0] = bload1<kStream>(rs, soff);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // 3. x planes into LDS (low bytes of 8 columns, then their high bytes)
#pragma unroll
  for (int j = 0; j < XMAX; ++j) {
    const int m = tid + j * nthr;
    if (XMAX == 1 || m < nblk) {
      u32x4 pl;
      pl.x = perm_b32(xv[j].y, xv[j].x, 0x06040200u);
      pl.y = perm_b32(xv[j].w, xv[j].z, 0x06040200u);
      pl.z = perm_b32(xv[j].y, xv[j].x, 0x07050301u);
      pl.w = perm_b32(xv[j].w, xv[j].z, 0x07050301u);
      xs[(m / BPC) * LSTRIDE + (m % BPC)] = pl;
    }
  }
  __syncthreads();
  // 4. compute row by row, chunk by chunk as the loads land
#pragma unroll
  for (int j = 0; j < RPL; ++j) {
    const int r = lane_row + j * rows_per_pass;
    float tot[1] = {0.0f};
#pragma unroll
    for (int i = 0; i < IMAX; ++i) {
      if (has[j][i]) {   // the LDS beyond the last chunk's columns holds no x
        const u32x4* xc = xs + (i * TPR + kl) * LSTRIDE;
        chunk_compute<NK, G, 1, SPC>(v[j][i], o[j][i], s[j][i], xc, 0, 1, tot, k);
      }
    }
    const float a = row_reduce(tot[0], tl);
    if (r < nr && kl == TPR - 1) p.y[yrow[j]] = __builtin_bit_cast(uint16_t, (_Float16)a);
  }
}

// Batch-1 kernel: one workgroup per tile.
template <int NK, int RPL, int IMAX, int XMAX>
__global__ __launch_bounds__(256) void sgemv_b1_kernel(KParams p) {
  extern __shared__ u32x4 xs[];
  if ((int)blockIdx.x >= p.cls_tile[4]) return;   // no such tile (uniform per workgroup)
  const TileGeo t = tile_geo(p, blockIdx.x);
  switch (t.g) {
    case 32: tile_b1<NK, 32, RPL, IMAX, XMAX>(p, xs, t.row0, t.nr, t.sz_base); break;
    case 64: tile_b1<NK, 64, RPL, IMAX, XMAX>(p, xs, t.row0, t.nr, t.sz_base); break;
    case 128: tile_b1<NK, 128, RPL, IMAX, XMAX>(p, xs, t.row0, t.nr, t.sz_base); break;
    default: tile_b1<NK, 256, RPL, IMAX, XMAX>(p, xs, t.row0, t.nr, t.sz_base); break;
  }
}

// Beam-batch kernel (B = 2..16): 256-thread workgroups; a tile whose layout
// uses more threads is split into 1 << pass_log2 workgroups, each taking a
// contiguous block of the tile's (row, k-lane) slots. Batch vectors are taken
// 4 at a time so that their x planes fit in LDS; each group of 4 re-reads
// the workgroup's weights, which are then still in L2.
template <int NK>
__global__ __launch_bounds__(256) void sgemv_bn_kernel(KParams p) {
  extern __shared__ u32x4 xs[];
  const int pass = blockIdx.x & ((1 << p.pass_log2) - 1);
  if ((int)(blockIdx.x >> p.pass_log2) >= p.cls_tile[4]) return;   // no such tile
  const TileGeo t = tile_geo(p, blockIdx.x >> p.pass_log2);
  const int row0 = t.row0, nr = t.nr, g = t.g, sz_base = t.sz_base;
  const int vt = threadIdx.x + 256 * pass;
  for (int b0 = 0; b0 < p.B; b0 += 4) {
    KParams q = p;
    q.x = p.x + (int64_t)b0 * (p.K >> 3);
    q.y = p.y + (int64_t)b0 * p.N;
    q.B = p.B - b0 < 4 ? p.B - b0 : 4;
    if (b0 > 0) __syncthreads();
    switch (g) {
      case 32: tile_body<NK, 32, 4, 8>(q, xs, row0, nr, sz_base, vt); break;
      case 64: tile_body<NK, 64, 4, 8>(q, xs, row0, nr, sz_base, vt); break;
      case 128: tile_body<NK, 128, 4, 8>(q, xs, row0, nr, sz_base, vt); break;
      default: tile_body<NK, 256, 4, 8>(q, xs, row0, nr, sz_base, vt); break;
    }
  }
}

typedef void (*KernelFn)(KParams);

}  // namespace sgemv_dev

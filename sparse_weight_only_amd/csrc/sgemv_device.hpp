// Device code of the SparseGemv kernel for gfx950 (MI355X, CDNA4, wave64).
//
// y = W' x for an N:M-sparse (2:4 or 1:4 along K) INT4 weight matrix with
// per-group FP16 scale and zero, FP16 activations and FP32 accumulation: the
// custom weight-only GEMV with mixed sparsity of the page "Efficient
// large-model ad applications through model compression and parallel
// verification" (English gloss of its Chinese title; a translation of arXiv
// 2605.11582), §1 (second contribution item) and §3.3 "Revised
// kernel". That section stops before describing its kernel; the design here
// is our own for CDNA4.
//
// The 2-of-4 sparse matrix-core instruction v_smfmac_f32_16x16x64_f16 does
// the selection of x and the dot product: its A operand is 16 rows x 64
// dense columns given as 2 values per group of 4 columns plus their 2-bit
// in-group indices, which is exactly the 2bit-CSR encoding of a 2:4 row.
// Per lane (row r = lane % 16, column block q = lane / 16) and instruction:
// 8 A values (4 groups of 4 columns), a 16-bit index field, and 16 x values
// of the B operand (column b = lane % 16 is batch vector b).
//
// One workgroup per row block (16 rows sorted by group size); its W waves
// split the row's K/256 column chunks into contiguous ranges, cpw chunks for
// waves w < crem and cpw - 1 after (fewer at the end of the row). Per wave:
//  1. loads, all issued up front and in this order: the wave's x slice
//     (16-byte loads, cached), then codes, offsets and scale|zero words of
//     every chunk (non-temporal: the weights are read once; at 1:4 a lane's
//     codes and offsets are one 12-byte piece, read by one load); lanes
//     without work read out of range and get zeros without touching memory;
//  2. the x slice goes to this wave's own LDS region (no barrier with other
//     waves: a wave waits only for its own loads);
//  3. per 64-column step: codes -> FP16 (q - z) exactly (0x6400 exponent
//     trick), times the FP16 scale -> the A operand; 1:4 rows put each kept
//     value in one slot of its group and 0 in the other; the offsets are the
//     index field as stored; two ds_read_b128 give the B operand; one
//     v_smfmac accumulates 16 rows x 16 columns in FP32;
//  4. the waves' partial sums meet in LDS; 16*B lanes add them in wave order
//     and write y in FP16 (round to nearest even) at the rows' original
//     positions.
// Large batches stage x in phases of `phase` chunks, prefetching the next
// phase's slice while the current one is computed.
//
// Variants of the same block body (template parameters):
//  - NK = 4: the dense INT4 ablation, each 16-column step as two 2-of-4
//    operands with constant index fields (positions (0,1) and (2,3));
//  - V16: the FP16-valued form, the stored values are the A operand (2:4) or
//    fill its slots 0, 2, 5, 7 (1:4); no scale/zero;
//  - ONE: exactly one vector (no x padding, slot-major partial sums);
//  - the group kernels run the body for the row blocks of up to 32 layers.
// A second body (sgemv_block_rb) computes RB row blocks per workgroup for
// batches of several vectors, loading each x slice once for all of them.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sgemv_dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16 __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));

struct KParams {
  const uint8_t* blob;   // kernel-layout blob
  const uint16_t* x;     // [B][K] FP16
  uint16_t* y;           // [B][N] FP16
  uint32_t blob_bytes;
  uint32_t off_codes, off_offs, off_perm, off_sz;
  int32_t N, K, B, C;    // C = K / 256 column chunks
  int32_t cpw;           // column chunks per wave (at most)
  int32_t crem;          // waves w < crem take cpw chunks, the later ones cpw - 1
  int32_t phase;         // chunks whose x slice is staged at once
  int32_t T;             // row blocks (= workgroups)
  int32_t cls_row[5];    // first sorted row of group size 32, 64, 128, 256, then N
  int32_t waves;         // waves per workgroup (the launch's block size / 64)
};

// Raw buffer loads: 32-bit lane offsets from a per-workgroup base held in
// SGPRs; offsets at or beyond the range return zeros without touching memory.
constexpr int kBufferWord3 = 0x00020000;   // raw 32-bit buffer, gfx9-family layout
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}
// CPOL: 0 = default caching, 2 = non-temporal (the weights are read once).
constexpr int kCached = 0, kStream = 2;
// soff is a wave-uniform offset added to every lane's: kOutOfRange there turns
// off the whole load for the wave (offset + 2^31 stays below 2^32 and beyond
// any buffer here) without a per-lane select.
template <int CPOL>
__device__ __forceinline__ u32x4 bload4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, CPOL));
}
template <int CPOL>
__device__ __forceinline__ u32x2 bload2(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, CPOL));
}
template <int CPOL>
__device__ __forceinline__ uint32_t bload1(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, CPOL);
}
// A 1:4 piece: 12 bytes, its 2 code dwords and its offset dword.
struct Piece14 { u32x2 cv; uint32_t ov; };
template <int CPOL>
__device__ __forceinline__ Piece14 bload_piece14(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
  typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
  const u32x3 v = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(r, off, soff, CPOL));
  return Piece14{u32x2{v.x, v.y}, v.z};
}

// A VGPR holding c whose value the compiler cannot see, so that (a & m) | c
// becomes one v_and_or_b32 (m in an SGPR, c in this VGPR). A single VALU move
// at kernel start, before any matrix-core instruction.
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
  return r;
}

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

template <int ABID>
__device__ __forceinline__ f4 smfmac(h8 a, h16 b, f4 c, uint32_t idx) {
  return __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, b, c, (int)idx, 0, ABID);
}

// Per-lane constants of one scale|zero word: (s, s), (s, 0), (0, s),
// -(1024 + z), -(64 + z).
struct Deq { h2 s, s_lo, s_hi, c1, c16; };
__device__ __forceinline__ Deq deq_consts(uint32_t szw) {
  const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)(szw & 0xFFFFu));
  const _Float16 z = __builtin_bit_cast(_Float16, (uint16_t)(szw >> 16));
  const _Float16 a = (_Float16)-1024.0f - z, b = (_Float16)-64.0f - z;   // exact: integers <= 1039
  Deq d;
  d.s = h2{s, s};
  d.s_lo = h2{s, (_Float16)0.0f};
  d.s_hi = h2{(_Float16)0.0f, s};
  d.c1 = h2{a, a};
  d.c16 = h2{b, b};
  return d;
}

// FP16 pairs (q0 - z) * s, (q1 - z) * s of two nibbles placed by the mask:
// 0x000F000F gives 1024 + q (subtract 1024 + z); 0x00F000F0 gives 1024 + 16 q
// (times 1/16, subtract 64 + z). (q - z) is exact; the product is rounded once.
__device__ __forceinline__ uint32_t deq_lo(uint32_t w, uint32_t magic, const Deq& d) {
  return as_u32((as_h2((w & 0x000F000Fu) | magic) + d.c1) * d.s);
}
__device__ __forceinline__ uint32_t deq_hi(uint32_t w, uint32_t magic, const Deq& d) {
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  return as_u32(__builtin_elementwise_fma(as_h2((w & 0x00F000F0u) | magic), sixteenth, d.c16) * d.s);
}

// Number of scale|zero words per column chunk of the sorted rows before row
// i (0 <= i <= N): sum over classes k of (8 >> k) * (rows of class k before
// i), the rows of class k before i being min(max(i, c_k), c_{k+1}) - c_k
// (c = cls_row, ascending). The constant parts sum to 4 c_1 + 2 c_2 + c_3;
// all of it is integer work on the scalar unit.
__device__ __forceinline__ int words_before(const KParams& p, int i) {
  const int m0 = min(i, p.cls_row[1]);
  const int m1 = min(max(i, p.cls_row[1]), p.cls_row[2]);
  const int m2 = min(max(i, p.cls_row[2]), p.cls_row[3]);
  const int m3 = min(max(i, p.cls_row[3]), p.cls_row[4]);
  return (m0 << 3) + (m1 << 2) + (m2 << 1) + m3 - (4 * p.cls_row[1] + 2 * p.cls_row[2] + p.cls_row[3]);
}

// Class (0..3) of sorted row i: the number of class starts c_1..c_3 at or
// before it, each test as the sign bit of c_k - 1 - i (integer arithmetic
// the scalar unit keeps for a wave-uniform i).
__device__ __forceinline__ int class_of(const KParams& p, int i) {
  return (int)(((uint32_t)(p.cls_row[1] - 1 - i) >> 31) + ((uint32_t)(p.cls_row[2] - 1 - i) >> 31) +
               ((uint32_t)(p.cls_row[3] - 1 - i) >> 31));
}

typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));

// Row block rb of the layer p, computed by the whole workgroup. V16: the
// FP16-valued form (the kept values themselves, no groups, no scale/zero).
template <int NK, int IMAX, int XMAX, bool V16 = false, bool ONE = false>
__device__ __forceinline__ void sgemv_block(const KParams& p, const int rb) {
  static_assert(!V16 || NK == 1 || NK == 2, "FP16 values exist at 2:4 and 1:4");
  // waves issue their loads at raised priority, so that a wave still issuing
  // is not held back by the dequantisation of waves whose data has arrived.
  // Measured: 0.15 us off the four MLP layers at one vector, 0.3-0.5 us off
  // the 11008 -> 4096 layers at 16 vectors; at 2-8 vectors it was neutral
  // or slower, so there the priority stays normal.
  const bool raise = ONE || (!V16 && p.B >= 16);
  if constexpr (ONE) __builtin_amdgcn_s_setprio(2);
  else if (raise) __builtin_amdgcn_s_setprio(2);
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int CB = V16 ? 32 * NK : 8 * NK, OB = 4 * NK;   // bytes of one piece's values and offsets
  // the wave index is the same on every lane: keep it (and what follows
  // from it) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = p.waves;   // = blockDim.x / 64, from the arguments loaded at the start
  const int r = lane & 15, q = lane >> 4;
  const int B = p.B, PH = p.phase;
  const auto rbuf = make_rsrc(p.blob, p.blob_bytes);
  const auto rx = make_rsrc(p.x, (uint32_t)(B * p.K * 2));
  // chunks of this wave: [c0, c0 + ncw), contiguous over the waves
  const int c0 = w * p.cpw - (w > p.crem ? w - p.crem : 0);
  const int cw_max = p.cpw - (w >= p.crem ? 1 : 0);
  const int ncw = p.C - c0 < cw_max ? (p.C - c0 > 0 ? p.C - c0 : 0) : cw_max;

  // this lane's sorted row, its group size 32 << cls and its scale|zero words
  const int row = rb * 16 + r;
  const int cls = (row >= p.cls_row[1]) + (row >= p.cls_row[2]) + (row >= p.cls_row[3]);
  const int glog = 5 + cls;
  const int wb0 = words_before(p, rb * 16);
  const uint32_t rec_words = (uint32_t)(words_before(p, rb * 16 + 16) - wb0);
  // a block whose 16 rows share one group size (all but at most three blocks
  // of a layer) holds 256/g words per row, row after row
  const int cls_first = class_of(p, rb * 16);
  const bool one_class = rec_words == (uint32_t)(16 * (8 >> cls_first));
  const uint32_t sz_row = one_class ? (uint32_t)(r * (8 >> cls_first)) : (uint32_t)(words_before(p, row) - wb0);
  const uint32_t sz_lane = sz_row + (uint32_t)((64 * q) >> glog);
  const uint32_t sz_block = (uint32_t)wb0 * (uint32_t)p.C;
  const bool g32 = cls == 0;

  // 0. original index of row tid % 16 of the block, for the lanes that write y
  const uint32_t orow = bload1<kCached>(rbuf, p.off_perm + (uint32_t)(rb * 16 + (tid & 15)) * 4u);

  // 1. x slice of the first phase: B rows x (PH * 256) columns, 16 bytes per
  // load; PH is a power of two, so a unit's row and column are a shift and a mask
  const int span16 = PH * 32;
  const int span_log = 5 + (31 - __builtin_clz((unsigned)PH));
  u32x4 xv[XMAX];
  auto issue_x = [&](int first) {   // chunks c0 + first .. c0 + first + PH - 1
    const int lim = (ncw - first < PH ? ncw - first : PH) * 32;
#pragma unroll
    for (int j = 0; j < XMAX; ++j) {
      const int u = lane + 64 * j, b = u >> span_log, cu = u & (span16 - 1);
      const bool ok = b < B && cu < lim;
      xv[j] = bload4<kCached>(rx, ok ? (__umul24((uint32_t)b, (uint32_t)p.K) + (uint32_t)((c0 + first) * 256 + cu * 8)) * 2u
                                     : kOutOfRange);
    }
  };
  issue_x(0);
  __builtin_amdgcn_sched_barrier(0);

  // weights of every chunk of the wave
  typedef typename std::conditional<
      V16, typename std::conditional<NK == 2, u32x16, u32x8>::type,
      typename std::conditional<NK == 4, u32x8, typename std::conditional<NK == 2, u32x4, u32x2>::type>::type>::type CodeT;
  typedef typename std::conditional<NK == 2, u32x2, uint32_t>::type OffT;
  CodeT cv[IMAX];
  OffT ov[IMAX];
  u32x2 sv[IMAX];
#pragma unroll
  for (int i = 0; i < IMAX; ++i) {
    const int c = c0 + i;
    const uint32_t off = i < ncw ? 0u : kOutOfRange;   // wave-uniform: chunk c exists
    const uint32_t rec = (uint32_t)(rb * p.C + c) * 64u + lane;
    // scale|zero: padding rows of a last, partial block read whatever words
    // follow (or zeros past the blob); their sums are never stored
    const uint32_t so = p.off_sz + (sz_block + (uint32_t)c * rec_words + sz_lane) * 4u;
    // records of 64 lanes x CB bytes stored as 16-byte slices: slice k of all
    // lanes, then slice k + 1 (each load below reads 1 KiB contiguously)
    const uint32_t slice0 = p.off_codes + (rec - lane) * CB + lane * 16u;
    if constexpr (V16) {
      // FP16 values: 64 (2:4) or 32 (1:4) bytes per lane and chunk
      const u32x4 v0 = bload4<kStream>(rbuf, slice0, off);
      const u32x4 v1 = bload4<kStream>(rbuf, slice0 + 1024u, off);
      if constexpr (NK == 2) {
        const u32x4 v2 = bload4<kStream>(rbuf, slice0 + 2048u, off);
        const u32x4 v3 = bload4<kStream>(rbuf, slice0 + 3072u, off);
        const u32x8 lo = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        const u32x8 hi = __builtin_shufflevector(v2, v3, 0, 1, 2, 3, 4, 5, 6, 7);
        cv[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
        ov[i] = bload2<kStream>(rbuf, p.off_offs + rec * OB, off);
      } else {
        cv[i] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        ov[i] = bload1<kStream>(rbuf, p.off_offs + rec * OB, off);
      }
    } else if constexpr (NK == 4) {
      // dense ablation: 32 bytes of codes, no offsets
      const u32x4 lo = bload4<kStream>(rbuf, slice0, off);
      const u32x4 hi = bload4<kStream>(rbuf, slice0 + 1024u, off);
      cv[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      ov[i] = 0u;
    } else if constexpr (NK == 2) {
      cv[i] = bload4<kStream>(rbuf, p.off_codes + rec * CB, off);
      ov[i] = bload2<kStream>(rbuf, p.off_offs + rec * OB, off);
    } else {
      const Piece14 pc = bload_piece14<kStream>(rbuf, p.off_codes + rec * 12u, off);
      cv[i] = pc.cv;
      ov[i] = pc.ov;
    }
    if constexpr (!V16) sv[i] = bload2<kStream>(rbuf, so, off);
    else sv[i] = u32x2{0u, 0u};
    // with two chunks a wave, every wave's first chunk is requested before
    // any second one, so that the last wave served has one chunk, not two,
    // left to compute once its data is in. Measured: 0.07-0.1 us off each
    // 4096 -> 11008 layer at one vector, neutral at 4 vectors; with four
    // chunks a wave (12 waves) the same barrier made the call slower.
    if (i == 0 && IMAX == 2) __builtin_amdgcn_s_barrier();
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (ONE) __builtin_amdgcn_s_setprio(0);
  else if (raise) __builtin_amdgcn_s_setprio(0);

  // x slice of the wave: B rows of span16 16-byte units; with several
  // vectors each row is padded by one unit, so that the 16 batch columns of
  // a B-operand read fall in different LDS banks (ONE: the kernel for one
  // vector, whose lanes all read row 0, a broadcast)
  constexpr int xpad = ONE ? 0 : 1;
  const int xrow_units = span16 + xpad;
  _Float16* xs = reinterpret_cast<_Float16*>(smem) + w * (B * xrow_units * 8);
  // partial sums of the waves, 16 slots per (b, row): for one vector
  // part[b][row][wave] (the final sum reads 4 x 16 bytes per entry), for
  // several part[wave][b][row] (a lane stores its 4 rows with one
  // conflict-free 16-byte write; the 16 lanes of a batch would otherwise hit
  // one bank). Slots of waves this workgroup does not have hold +0, so that
  // the final sum reads all 16 slots without a test per slot.
  constexpr bool slot_major = ONE;
  float* part = reinterpret_cast<float*>(smem + W * B * xrow_units * 16);
  if constexpr (slot_major) {
    // 256 entries (row, slot): one pass when the workgroup has 4+ waves
    if (W >= 4) {
      if (tid < 256 && (tid & 15) >= W) part[tid] = 0.f;
    } else {
      for (int e = tid; e < 256; e += 64 * W)
        if ((e & 15) >= W) part[e] = 0.f;
    }
  } else {
    for (int e = tid; e < (16 - W) * B * 4; e += 64 * W)
      reinterpret_cast<f4*>(part)[W * B * 4 + e] = f4{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t magic = opaque_vgpr(0x64006400u);
  const int bcol = (lane & 15) < B ? (lane & 15) : 0;
  const _Float16* xrow = xs + __umul24((uint32_t)bcol, (uint32_t)(xrow_units * 8)) + 64 * (q >> 1) + 8 * (q & 1);
  f4 acc = {0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int i = 0; i < IMAX; ++i) {
    if (i >= ncw) break;
    const int slot = i % PH;
    if (slot == 0) {
      // 2. stage this phase's x slice in the wave's LDS region, prefetch the next
#pragma unroll
      for (int j = 0; j < XMAX; ++j) {
        const int u = lane + 64 * j;
        if (u < B * span16) reinterpret_cast<u32x4*>(xs)[u + ((u >> span_log) & -xpad)] = xv[j];   // row b at b * xrow_units
      }
      __builtin_amdgcn_wave_barrier();
      if (i + PH < ncw) issue_x(i + PH);
    }
    const _Float16* xc = xrow + 256 * slot;
    // scale|zero of columns 0..31 and 32..63 of this lane's piece (two groups
    // at group size 32, one otherwise)
    const Deq d0 = deq_consts(sv[i].x);
    const Deq d1 = deq_consts(g32 ? sv[i].y : sv[i].x);
    uint32_t idx2 = 0;
    if constexpr (NK == 1) idx2 = ((ov[i] & 0x33333333u) << 2) | ((ov[i] >> 2) & 0x33333333u);
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const Deq& d = t < 2 ? d0 : d1;
      const h8 blo = *reinterpret_cast<const h8*>(xc + 16 * t);
      const h8 bhi = *reinterpret_cast<const h8*>(xc + 16 * t + 128);
      const h16 Bop = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      if constexpr (V16) {
        // FP16 values: at 2:4 the 8 values of step t are the operand as
        // stored; at 1:4 the 4 values go to slots 0, 2, 5, 7 (0 elsewhere),
        // as the dequantised 1:4 operand
        uint32_t a0, a1, a2, a3, idx;
        if constexpr (NK == 2) {
          a0 = cv[i][4 * t]; a1 = cv[i][4 * t + 1]; a2 = cv[i][4 * t + 2]; a3 = cv[i][4 * t + 3];
          idx = ov[i][t >> 1];
        } else {
          const uint32_t e01 = cv[i][2 * t], e23 = cv[i][2 * t + 1];
          a0 = e01 & 0xFFFFu; a1 = e01 >> 16; a2 = e23 << 16; a3 = e23 & 0xFFFF0000u;
          idx = t < 2 ? ov[i] : idx2;
        }
        const h2 A0 = as_h2(a0), A1 = as_h2(a1), A2 = as_h2(a2), A3 = as_h2(a3);
        const h8 A = {A0.x, A0.y, A1.x, A1.y, A2.x, A2.y, A3.x, A3.y};
        if (t & 1) acc = smfmac<1>(A, Bop, acc, idx);
        else acc = smfmac<0>(A, Bop, acc, idx);
        continue;
      }
      if constexpr (NK == 4) {
        // dense ablation: the 4 groups of step t as two 2-of-4 operands with
        // constant index fields, in-group positions (0, 1) and (2, 3)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t cw = cv[i][2 * t + h], c8 = cw >> 8;
          const h2 A0 = as_h2(deq_lo(cw, magic, d)), A1 = as_h2(deq_hi(cw, magic, d));
          const h2 A2 = as_h2(deq_lo(c8, magic, d)), A3 = as_h2(deq_hi(c8, magic, d));
          const h8 A = {A0.x, A0.y, A1.x, A1.y, A2.x, A2.y, A3.x, A3.y};
          acc = smfmac<0>(A, Bop, acc, h ? 0xEEEEEEEEu : 0x44444444u);
        }
        continue;
      }
      uint32_t a0, a1, a2, a3, idx;
      if constexpr (NK == 2) {
        // step t: code dword t = 8 kept elements, 2 per group of 4 columns
        const uint32_t cw = cv[i][t], c8 = cw >> 8;
        a0 = deq_lo(cw, magic, d);
        a1 = deq_hi(cw, magic, d);
        a2 = deq_lo(c8, magic, d);
        a3 = deq_hi(c8, magic, d);
        idx = ov[i][t >> 1];
      } else {
        // step t: 4 kept elements (one per group) in slots 0, 2, 5, 7; the
        // other slot of each group holds 0: the scale pair (s, 0) or (0, s)
        // keeps one half of the exact (q - z) pair
        const uint32_t cw = (t & 1) ? (cv[i][t >> 1] >> 8) : cv[i][t >> 1];
        const h2 q02 = as_h2((cw & 0x000F000Fu) | magic) + d.c1;
        const h2 q13 = __builtin_elementwise_fma(as_h2((cw & 0x00F000F0u) | magic), sixteenth, d.c16);
        a0 = as_u32(q02 * d.s_lo);
        a2 = as_u32(q02 * d.s_hi);
        a1 = as_u32(q13 * d.s_lo);
        a3 = as_u32(q13 * d.s_hi);
        idx = t < 2 ? ov[i] : idx2;
      }
      const h2 A0 = as_h2(a0), A1 = as_h2(a1), A2 = as_h2(a2), A3 = as_h2(a3);
      const h8 A = {A0.x, A0.y, A1.x, A1.y, A2.x, A2.y, A3.x, A3.y};
      if (t & 1) acc = smfmac<1>(A, Bop, acc, idx);
      else acc = smfmac<0>(A, Bop, acc, idx);
    }
  }

  // 4. partial sums of the waves: lane (b = lane % 16, q) holds rows
  // 4q .. 4q + 3 of column b
  if ((lane & 15) < B) {
    if constexpr (slot_major) {
      float* pp = part + ((lane & 15) * 16 + 4 * q) * 16 + w;
      pp[0] = acc.x;
      pp[16] = acc.y;
      pp[32] = acc.z;
      pp[48] = acc.w;
    } else {
      reinterpret_cast<f4*>(part)[(w * B + (lane & 15)) * 4 + q] = acc;
    }
  }
  __syncthreads();
  // entries e = 16 b + row; the block size is a multiple of 16, so every
  // entry of this lane has row tid % 16; the waves are added in order (one
  // vector: the 16 entries of lanes 0..15, no loop)
  for (int e = tid; ONE ? e < 16 : e < 16 * B; e += ONE ? 1024 : 64 * W) {
    float vv[16];
    if constexpr (slot_major) {
      const f4* pv = reinterpret_cast<const f4*>(part + e * 16);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f4 v4 = pv[k];
        vv[4 * k] = v4.x; vv[4 * k + 1] = v4.y; vv[4 * k + 2] = v4.z; vv[4 * k + 3] = v4.w;
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) vv[v] = part[v * B * 16 + e];   // (wave v, b, row) = v * 16B + e
    }
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) s += vv[v];   // slots of absent waves hold +0
    const int b = e >> 4;
    const int n = (int)orow;
    // B * N < 2^31 (the blob size bounds N), so 32-bit indexing is enough
    if (n >= 0 && n < p.N) p.y[(uint32_t)(b * p.N + n)] = __builtin_bit_cast(uint16_t, (_Float16)s);
  }
}

// Row blocks rb0 .. rb0 + RB - 1 of the layer p (INT4 form, 2:4 or 1:4,
// several vectors), computed by the whole workgroup. The steps are those of
// sgemv_block; what differs: each wave holds the weights of RB x IMAX pieces
// in registers and uses every x operand it reads from LDS for the RB blocks,
// so the x slice of a chunk is loaded from L2 once per RB blocks; the
// partial sums keep one slot per wave (part[wave][b][block][row]) and are
// added in a loop over the waves; the blocks' original row indices go
// through LDS. Blocks at or beyond T (the last workgroup) read zeros and
// store nothing.
template <int NK, int IMAX, int XMAX, int RB>
__device__ __forceinline__ void sgemv_block_rb(const KParams& p, const int rb0) {
  static_assert(NK == 1 || NK == 2, "sparse INT4 forms");
  static_assert(RB == 2 || RB == 4, "row blocks per workgroup");
  constexpr int RBLOG = RB == 4 ? 2 : 1;
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int CB = 8 * NK, OB = 4 * NK;   // bytes of one piece's codes and offsets
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = p.waves;   // = blockDim.x / 64, from the arguments loaded at the start
  const int r = lane & 15, q = lane >> 4;
  const int B = p.B, PH = p.phase;
  const auto rbuf = make_rsrc(p.blob, p.blob_bytes);
  const auto rx = make_rsrc(p.x, (uint32_t)(B * p.K * 2));
  // chunks of this wave: [c0, c0 + ncw), contiguous over the waves
  const int c0 = w * p.cpw - (w > p.crem ? w - p.crem : 0);
  const int cw_max = p.cpw - (w >= p.crem ? 1 : 0);
  const int ncw = p.C - c0 < cw_max ? (p.C - c0 > 0 ? p.C - c0 : 0) : cw_max;

  // 0. original index of row tid of the RB blocks (lanes tid < 16 RB)
  const uint32_t orow = tid < 16 * RB && rb0 * 16 + tid < 16 * p.T
                            ? bload1<kCached>(rbuf, p.off_perm + (uint32_t)(rb0 * 16 + tid) * 4u)
                            : 0xFFFFFFFFu;

  // 1. x slice of the first phase (as in sgemv_block)
  const int span16 = PH * 32;
  const int span_log = 5 + (31 - __builtin_clz((unsigned)PH));
  u32x4 xv[XMAX];
  auto issue_x = [&](int first) {
    const int lim = (ncw - first < PH ? ncw - first : PH) * 32;
#pragma unroll
    for (int j = 0; j < XMAX; ++j) {
      const int u = lane + 64 * j, b = u >> span_log, cu = u & (span16 - 1);
      const bool ok = b < B && cu < lim;
      xv[j] = bload4<kCached>(rx, ok ? (__umul24((uint32_t)b, (uint32_t)p.K) + (uint32_t)((c0 + first) * 256 + cu * 8)) * 2u
                                     : kOutOfRange);
    }
  };
  issue_x(0);
  __builtin_amdgcn_sched_barrier(0);

  // per block: this lane's group size class and scale|zero words (as in
  // sgemv_block); then the weights of every (block, chunk) of the wave
  typedef typename std::conditional<NK == 2, u32x4, u32x2>::type CodeT;
  typedef typename std::conditional<NK == 2, u32x2, uint32_t>::type OffT;
  bool g32[RB];
  CodeT cv[RB][IMAX];
  OffT ov[RB][IMAX];
  u32x2 sv[RB][IMAX];
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int rb = rb0 + j;
    const uint32_t blk_off = rb < p.T ? 0u : kOutOfRange;   // wave-uniform
    const int row = rb * 16 + r;
    const int cls = (row >= p.cls_row[1]) + (row >= p.cls_row[2]) + (row >= p.cls_row[3]);
    const int wb0 = words_before(p, rb * 16);
    const uint32_t rec_words = (uint32_t)(words_before(p, rb * 16 + 16) - wb0);
    const int cls_first = class_of(p, rb * 16);
    const bool one_class = rec_words == (uint32_t)(16 * (8 >> cls_first));
    const uint32_t sz_row = one_class ? (uint32_t)(r * (8 >> cls_first)) : (uint32_t)(words_before(p, row) - wb0);
    const uint32_t sz_lane = sz_row + (uint32_t)((64 * q) >> (5 + cls));
    const uint32_t sz_block = (uint32_t)wb0 * (uint32_t)p.C;
    g32[j] = cls == 0;
#pragma unroll
    for (int i = 0; i < IMAX; ++i) {
      const int c = c0 + i;
      const uint32_t off = i < ncw ? blk_off : kOutOfRange;
      const uint32_t rec = (uint32_t)(rb * p.C + c) * 64u + lane;
      const uint32_t so = p.off_sz + (sz_block + (uint32_t)c * rec_words + sz_lane) * 4u;
      if constexpr (NK == 2) {
        cv[j][i] = bload4<kStream>(rbuf, p.off_codes + rec * CB, off);
        ov[j][i] = bload2<kStream>(rbuf, p.off_offs + rec * OB, off);
      } else {
        const Piece14 pc = bload_piece14<kStream>(rbuf, p.off_codes + rec * 12u, off);
        cv[j][i] = pc.cv;
        ov[j][i] = pc.ov;
      }
      sv[j][i] = bload2<kStream>(rbuf, so, off);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // x slice of the wave in LDS, rows padded by one 16-byte unit (as in
  // sgemv_block); partial sums part[wave][b][block][row]; original rows
  const int xrow_units = span16 + 1;
  _Float16* xs = reinterpret_cast<_Float16*>(smem) + w * (B * xrow_units * 8);
  float* part = reinterpret_cast<float*>(smem + W * B * xrow_units * 16);
  int* perm_s = reinterpret_cast<int*>(part + W * RB * B * 16);
  const uint32_t magic = opaque_vgpr(0x64006400u);
  const int bcol = (lane & 15) < B ? (lane & 15) : 0;
  const _Float16* xrow = xs + __umul24((uint32_t)bcol, (uint32_t)(xrow_units * 8)) + 64 * (q >> 1) + 8 * (q & 1);
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  f4 acc[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int i = 0; i < IMAX; ++i) {
    if (i >= ncw) break;
    const int slot = i % PH;
    if (slot == 0) {
      // 2. stage this phase's x slice, prefetch the next
#pragma unroll
      for (int j = 0; j < XMAX; ++j) {
        const int u = lane + 64 * j;
        if (u < B * span16) reinterpret_cast<u32x4*>(xs)[u + (u >> span_log)] = xv[j];   // row b at b * xrow_units
      }
      __builtin_amdgcn_wave_barrier();
      if (i + PH < ncw) issue_x(i + PH);
    }
    const _Float16* xc = xrow + 256 * slot;
    Deq d0[RB], d1[RB];
    uint32_t idx2[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      d0[j] = deq_consts(sv[j][i].x);
      d1[j] = deq_consts(g32[j] ? sv[j][i].y : sv[j][i].x);
      idx2[j] = 0u;
      if constexpr (NK == 1) idx2[j] = ((ov[j][i] & 0x33333333u) << 2) | ((ov[j][i] >> 2) & 0x33333333u);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // 3. the x operand of step t, once for the RB blocks
      const h8 blo = *reinterpret_cast<const h8*>(xc + 16 * t);
      const h8 bhi = *reinterpret_cast<const h8*>(xc + 16 * t + 128);
      const h16 Bop = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const Deq& d = t < 2 ? d0[j] : d1[j];
        uint32_t a0, a1, a2, a3, idx;
        if constexpr (NK == 2) {
          const uint32_t cw = cv[j][i][t], c8 = cw >> 8;
          a0 = deq_lo(cw, magic, d);
          a1 = deq_hi(cw, magic, d);
          a2 = deq_lo(c8, magic, d);
          a3 = deq_hi(c8, magic, d);
          idx = ov[j][i][t >> 1];
        } else {
          const uint32_t cw = (t & 1) ? (cv[j][i][t >> 1] >> 8) : cv[j][i][t >> 1];
          const h2 q02 = as_h2((cw & 0x000F000Fu) | magic) + d.c1;
          const h2 q13 = __builtin_elementwise_fma(as_h2((cw & 0x00F000F0u) | magic), sixteenth, d.c16);
          a0 = as_u32(q02 * d.s_lo);
          a2 = as_u32(q02 * d.s_hi);
          a1 = as_u32(q13 * d.s_lo);
          a3 = as_u32(q13 * d.s_hi);
          idx = t < 2 ? ov[j][i] : idx2[j];
        }
        const h2 A0 = as_h2(a0), A1 = as_h2(a1), A2 = as_h2(a2), A3 = as_h2(a3);
        const h8 A = {A0.x, A0.y, A1.x, A1.y, A2.x, A2.y, A3.x, A3.y};
        if (t & 1) acc[j] = smfmac<1>(A, Bop, acc[j], idx);
        else acc[j] = smfmac<0>(A, Bop, acc[j], idx);
      }
    }
  }

  // 4. partial sums: lane (b, q) stores rows 4q .. 4q + 3 of each block
  if ((lane & 15) < B) {
#pragma unroll
    for (int j = 0; j < RB; ++j) reinterpret_cast<f4*>(part)[((w * B + (lane & 15)) * RB + j) * 4 + q] = acc[j];
  }
  if (tid < 16 * RB) perm_s[tid] = (int)orow;
  __syncthreads();
  // entries e = (b * RB + j) * 16 + row, the waves added in order
  for (int e = tid; e < 16 * B * RB; e += 64 * W) {
    float s = 0.f;
    for (int v = 0; v < W; ++v) s += part[v * B * RB * 16 + e];
    const int b = (e >> 4) >> RBLOG, j = (e >> 4) & (RB - 1);
    const int n = perm_s[j * 16 + (e & 15)];
    // B * N < 2^31 (the blob size bounds N), so 32-bit indexing is enough
    if (n >= 0 && n < p.N) p.y[(uint32_t)(b * p.N + n)] = __builtin_bit_cast(uint16_t, (_Float16)s);
  }
}

// The fields a wave needs before its first loads, passed as 14 leading
// scalar argument dwords that gfx950 preloads into scalar registers at wave
// launch (kernel-argument preloading, enabled at build time); the rest of the
// parameter block, needed only at the end, is loaded from memory. cpw, crem,
// phase and B are packed one byte each; the codes section starts the blob.
#define SGEMV_LEAD_ARGS                                                                                 \
  const uint8_t *blob, const uint16_t *x, uint32_t blob_bytes, uint32_t off_offs, uint32_t off_perm, \
      uint32_t off_sz, int32_t K, uint32_t packed, int32_t cls1, int32_t cls2, int32_t cls3, int32_t cls4
__device__ __forceinline__ KParams lead_params(const uint8_t* blob, const uint16_t* x, uint32_t blob_bytes,
                                               uint32_t off_offs, uint32_t off_perm, uint32_t off_sz, int32_t K,
                                               uint32_t packed, int32_t cls1, int32_t cls2, int32_t cls3,
                                               int32_t cls4, const KParams& rest) {
  KParams p = rest;
  p.blob = blob;
  p.x = x;
  p.blob_bytes = blob_bytes;
  p.off_codes = 0;
  p.off_offs = off_offs;
  p.off_perm = off_perm;
  p.off_sz = off_sz;
  p.K = K;
  p.C = K >> 8;
  p.cpw = (int32_t)(packed & 0xFFu);
  p.crem = (int32_t)((packed >> 8) & 0xFFu);
  p.phase = (int32_t)((packed >> 16) & 0xFFu);
  p.B = (int32_t)(packed >> 24);
  p.cls_row[0] = 0;
  p.cls_row[1] = cls1;
  p.cls_row[2] = cls2;
  p.cls_row[3] = cls3;
  p.cls_row[4] = cls4;
  return p;
}
#define SGEMV_LEAD_PARAMS(rest) \
  lead_params(blob, x, blob_bytes, off_offs, off_perm, off_sz, K, packed, cls1, cls2, cls3, cls4, rest)

// One launch, one layer: workgroup b computes row block b. The launcher
// makes the grid exactly T workgroups, so there is no bound test: testing
// blockIdx against T would make every wave wait for that kernel argument
// before loading the others (measured: 0.1 us per call, 0.7 us per
// four-layer step at one vector). A workgroup past T would only read zeros
// or bytes inside the blob and store nothing (its rows are padding).
template <int NK, int IMAX, int XMAX>
__global__ __launch_bounds__(1024) void sgemv_kernel(SGEMV_LEAD_ARGS, KParams rest) {
  sgemv_block<NK, IMAX, XMAX>(SGEMV_LEAD_PARAMS(rest), (int)blockIdx.x);
}
// The same for exactly one vector (B = 1).
template <int NK, int IMAX, int XMAX>
__global__ __launch_bounds__(1024) void sgemv_b1_kernel(SGEMV_LEAD_ARGS, KParams rest) {
  sgemv_block<NK, IMAX, XMAX, false, true>(SGEMV_LEAD_PARAMS(rest), (int)blockIdx.x);
}
// Several vectors, RB row blocks per workgroup: workgroup b computes row
// blocks RB*b .. RB*b + RB - 1. At most 8 waves, so that the weights of
// RB x IMAX pieces stay in registers.
template <int NK, int IMAX, int XMAX, int RB>
__global__ __launch_bounds__(512) void sgemv_rb_kernel(KParams p) {
  sgemv_block_rb<NK, IMAX, XMAX, RB>(p, (int)blockIdx.x * RB);   // grid: ceil(T / RB), no bound test
}
template <int NK, int IMAX, int XMAX>
__global__ __launch_bounds__(1024) void sgemv_f16_kernel(SGEMV_LEAD_ARGS, KParams rest) {
  sgemv_block<NK, IMAX, XMAX, true>(SGEMV_LEAD_PARAMS(rest), (int)blockIdx.x);   // grid: T, no bound test
}

// One launch, several independent layers with the same N:M choice, batch and
// chunks per wave: workgroup b computes row block b - first_block[i] of layer
// i, the layer whose block range holds b. Layers with fewer chunks than the
// workgroup's waves cover leave the extra waves idle (they add zeros).
constexpr int kMaxGroup = 32;
struct GParams {
  int32_t count;
  int32_t first_block[kMaxGroup + 1];   // prefix of the layers' row blocks; INT32_MAX past count
  KParams t[kMaxGroup];
};
static_assert(sizeof(GParams) <= 4096, "kernel arguments are limited to 4 KiB");

// Layer of workgroup b (the grid is exactly first_block[count] workgroups).
// The entries past count hold INT32_MAX, so the first three boundaries are
// tested without waiting for count: groups of up to 4 layers (those of a
// decoder step) find their layer with one round of argument loads before
// loading the layer's parameters; larger groups continue in a loop. Each
// test is the sign bit of first_block[j] - 1 - b (no overflow: b >= 0).
template <int NK, int IMAX, int XMAX, bool V16, bool ONE = false>
__device__ __forceinline__ void group_block(const GParams& g) {
  const int b = (int)blockIdx.x;
  const int fb1 = g.first_block[1], fb2 = g.first_block[2], fb3 = g.first_block[3];
  const int s1 = (int)((uint32_t)(fb1 - 1 - b) >> 31), s2 = (int)((uint32_t)(fb2 - 1 - b) >> 31),
            s3 = (int)((uint32_t)(fb3 - 1 - b) >> 31);
  int i = s1 + s2 + s3;
  int base = s3 ? fb3 : s2 ? fb2 : s1 ? fb1 : 0;   // first block of layer i
  if (i == 3) {
    while (i + 1 < g.count && b >= g.first_block[i + 1]) ++i;
    base = g.first_block[i];
  }
  sgemv_block<NK, IMAX, XMAX, V16, ONE>(g.t[i], b - base);
}
template <int NK, int IMAX, int XMAX>
__global__ __launch_bounds__(1024) void sgemv_b1_group_kernel(GParams g) {
  group_block<NK, IMAX, XMAX, false, true>(g);
}
template <int NK, int IMAX, int XMAX>
__global__ __launch_bounds__(1024) void sgemv_group_kernel(GParams g) {
  group_block<NK, IMAX, XMAX, false>(g);
}
template <int NK, int IMAX, int XMAX>
__global__ __launch_bounds__(1024) void sgemv_f16_group_kernel(GParams g) {
  group_block<NK, IMAX, XMAX, true>(g);
}

}  // namespace sgemv_dev

// Device code of the task-list launch: many independent batch-1 GEMVs
// y_i = W'_i x_i (INT4 form, 2:4 or 1:4 per task) in one kernel.
//
// Per-token decoding runs every projection of every layer as a GEMV on one
// vector (the page "Efficient large-model ad applications through model
// compression and parallel verification", §1 "our core idea"); a 7B-shaped
// decoder step is 224 of them, 4-19 MB each. One launch per GEMV pays the
// dispatch, ramp-up and drain of a kernel every few microseconds. Here up to
// kListMax of them are one launch, and each wave streams whole rows:
//  - the workgroups of a task are few enough to be resident together; each
//    task gets a number of them in proportion to its bytes;
//  - a workgroup stages its task's x (all K columns) and the original row
//    indices of its row blocks in LDS once, then its waves work alone (no
//    barrier after that): wave w takes a contiguous run of the workgroup's
//    row blocks and walks them chunk by chunk (256 columns of 16 rows),
//    keeping the loads of the next kListDepth - 1 chunks in flight while it
//    computes one, so that each wave streams its weights without waiting
//    for a round trip per block;
//  - per chunk the steps are those of the single-layer kernel at one vector:
//    codes -> FP16 (code - zero) * scale, and 4 steps of the 2-of-4 sparse
//    matrix-core instruction, which selects x and accumulates in FP32; a
//    row's sum runs over its chunks in order in one accumulator (no partial
//    sums to combine); after the last chunk the lanes of column 0 round it
//    to FP16 into LDS, and once the wave's blocks are done its lanes store
//    y at the rows' original positions.
#pragma once
#include "sgemv_device.hpp"

namespace sgemv_dev {

// One task of a list launch (72 bytes; up to kListMax of them travel in the
// kernel arguments, which are limited to 4 KiB).
struct ListTask {
  const uint8_t* blob;     // kernel-layout blob
  const uint16_t* x;       // [K] FP16
  uint16_t* y;             // [N] FP16
  uint32_t blob_bytes, off_offs, off_perm, off_sz;
  int32_t N, cls1, cls2, cls3;   // rows; first sorted row of group size 64, 128, 256
  uint32_t c_nk;           // column chunks (low 16 bits) | nk << 16
  int32_t n_wg;            // workgroups of the task
  int32_t q, r;            // row blocks per workgroup: workgroup j takes q + (j < r) of them
};
constexpr int kListMax = 48;
constexpr int kListWaves = 8;          // waves per workgroup
constexpr int kListDepth = 4;          // chunks per wave in flight (8 took 20 % longer: fewer waves fit)
constexpr int kListMaxBlocks = 256;    // row blocks per workgroup (their row indices are staged in LDS)
struct ListParams {
  int32_t count;           // tasks
  int32_t pad[3];
  ListTask t[kListMax];
};
static_assert(sizeof(ListTask) == 72, "task layout");
static_assert(sizeof(ListParams) <= 4096, "kernel arguments are limited to 4 KiB");

// One grid row of a table launch (the task table sits in device memory, so
// a launch can hold any number of tasks): workgroup (i, row) is workgroup
// j0 + i of the row's task. A task whose share is wider than a row spans
// consecutive rows.
struct ListRow {
  ListTask t;
  int32_t j0;
  int32_t pad;
};
static_assert(sizeof(ListRow) == 80, "table row layout");

// The loads of one chunk of one wave: codes, offsets and scale|zero words.
template <int NK>
struct ChunkRegs {
  typedef typename std::conditional<NK == 2, u32x4, u32x2>::type CodeT;
  typedef typename std::conditional<NK == 2, u32x2, uint32_t>::type OffT;
  CodeT cv;
  OffT ov;
  u32x2 sv;
};

// Where the next chunk to load lies: record index g = block * C + chunk
// (codes and offsets are laid out record after record, so g advances by one
// per chunk, across blocks), the block's scale|zero base and words per
// chunk, and this lane's offset in them (set at each block's first chunk).
struct IssueCursor {
  int blk, chunk, g;
  uint32_t sz_base, sz_step, sz_lane;
};

__device__ __forceinline__ void cursor_block(IssueCursor& ic, const KParams& p, int r, int q) {
  const int rb = ic.blk;
  const int row = rb * 16 + r;
  const int cls = (row >= p.cls_row[1]) + (row >= p.cls_row[2]) + (row >= p.cls_row[3]);
  const int wb0 = words_before(p, rb * 16);
  const uint32_t rec_words = (uint32_t)(words_before(p, rb * 16 + 16) - wb0);
  const int cls_first = class_of(p, rb * 16);
  const bool one_class = rec_words == (uint32_t)(16 * (8 >> cls_first));
  const uint32_t sz_row = one_class ? (uint32_t)(r * (8 >> cls_first)) : (uint32_t)(words_before(p, row) - wb0);
  ic.sz_lane = (sz_row + (uint32_t)((64 * q) >> (5 + cls))) * 4u;
  ic.sz_base = p.off_sz + (uint32_t)wb0 * (uint32_t)p.C * 4u;
  ic.sz_step = rec_words * 4u;
}

template <int NK>
__device__ __forceinline__ void issue_chunk(ChunkRegs<NK>& R, const KParams& p, __amdgpu_buffer_rsrc_t rbuf,
                                            const IssueCursor& ic, bool ok, uint32_t lane_codes, uint32_t lane_offs) {
  constexpr uint32_t CB = 8 * NK, OB = 4 * NK;
  const uint32_t out = ok ? 0u : kOutOfRange;   // wave-uniform: past the wave's last chunk, read zeros
  const uint32_t g = (uint32_t)ic.g;
  if constexpr (NK == 2) {
    R.cv = bload4<kStream>(rbuf, lane_codes, g * 64u * CB + out);
    R.ov = bload2<kStream>(rbuf, lane_offs, p.off_offs + g * 64u * OB + out);
  } else {
    const Piece14 pc = bload_piece14<kStream>(rbuf, lane_codes, g * 64u * 12u + out);
    R.cv = pc.cv;
    R.ov = pc.ov;
  }
  R.sv = bload2<kStream>(rbuf, ic.sz_lane, ic.sz_base + (uint32_t)ic.chunk * ic.sz_step + out);
}

// One chunk's 16 x 16 tile accumulated into acc (column 0 is the vector's).
template <int NK>
__device__ __forceinline__ f4 chunk_mac(const ChunkRegs<NK>& R, const _Float16* xc, bool g32, uint32_t magic,
                                        f4 acc) {
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const Deq d0 = deq_consts(R.sv.x);
  const Deq d1 = deq_consts(g32 ? R.sv.y : R.sv.x);
  uint32_t idx2 = 0;
  if constexpr (NK == 1) idx2 = ((R.ov & 0x33333333u) << 2) | ((R.ov >> 2) & 0x33333333u);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const Deq& d = t < 2 ? d0 : d1;
    const h8 blo = *reinterpret_cast<const h8*>(xc + 16 * t);
    const h8 bhi = *reinterpret_cast<const h8*>(xc + 16 * t + 128);
    const h16 Bop = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    uint32_t a0, a1, a2, a3, idx;
    if constexpr (NK == 2) {
      const uint32_t cw = R.cv[t], c8 = cw >> 8;
      a0 = deq_lo(cw, magic, d);
      a1 = deq_hi(cw, magic, d);
      a2 = deq_lo(c8, magic, d);
      a3 = deq_hi(c8, magic, d);
      idx = R.ov[t >> 1];
    } else {
      const uint32_t cw = (t & 1) ? (R.cv[t >> 1] >> 8) : R.cv[t >> 1];
      const h2 q02 = as_h2((cw & 0x000F000Fu) | magic) + d.c1;
      const h2 q13 = __builtin_elementwise_fma(as_h2((cw & 0x00F000F0u) | magic), sixteenth, d.c16);
      a0 = as_u32(q02 * d.s_lo);
      a2 = as_u32(q02 * d.s_hi);
      a1 = as_u32(q13 * d.s_lo);
      a3 = as_u32(q13 * d.s_hi);
      idx = t < 2 ? R.ov : idx2;
    }
    const h2 A0 = as_h2(a0), A1 = as_h2(a1), A2 = as_h2(a2), A3 = as_h2(a3);
    const h8 A = {A0.x, A0.y, A1.x, A1.y, A2.x, A2.y, A3.x, A3.y};
    if (t & 1) acc = smfmac<1>(A, Bop, acc, idx);
    else acc = smfmac<0>(A, Bop, acc, idx);
  }
  return acc;
}

__device__ __forceinline__ void cursor_next(IssueCursor& ic, const KParams& p, int r, int q) {
  ++ic.g;
  if (++ic.chunk == p.C) {
    ic.chunk = 0;
    ++ic.blk;
    cursor_block(ic, p, r, q);
  }
}

// Row blocks [B0, B0 + nbw) of the task p, computed by one workgroup.
template <int NK>
__device__ __forceinline__ void list_stream(const KParams& p, int B0, int nbw) {
  constexpr int W = kListWaves, D = kListDepth;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int C = p.C;
  const auto rbuf = make_rsrc(p.blob, p.blob_bytes);
  const auto rx = make_rsrc(p.x, (uint32_t)(C * 512));

  // 1. LDS: x (C * 512 bytes), then the original row indices of the
  // workgroup's blocks (64 bytes a block), then the blocks' FP16 results (32
  // bytes a block). x and the row indices go from memory straight to LDS
  // (the buffer-to-LDS form of the load: lane l of a wave writes its 16
  // bytes at the wave's LDS address + 16 l, no registers involved), and the
  // waves issue the loads of their first chunks before the barrier waits for
  // them, so that the staging and the first weights share one round trip.
  typedef __attribute__((address_space(3))) void* LdsPtr;
  _Float16* xs = reinterpret_cast<_Float16*>(smem);
  int* ps = reinterpret_cast<int*>(smem + C * 512);
  uint16_t* ys = reinterpret_cast<uint16_t*>(ps + nbw * 16);
  for (int u0 = 64 * w; u0 < C * 32; u0 += 64 * W)
    if (u0 + lane < C * 32)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (LdsPtr)(smem + u0 * 16), 16, (uint32_t)(u0 + lane) * 16u, 0, 0,
                                               kCached);
  for (int u0 = 64 * w; u0 < nbw * 4; u0 += 64 * W)
    if (u0 + lane < nbw * 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rbuf, (LdsPtr)(smem + C * 512 + u0 * 16), 16,
                                               p.off_perm + (uint32_t)(B0 * 64 + (u0 + lane) * 16), 0, 0, kCached);

  // 2. this wave's blocks: a contiguous run, nbw / W each, the first
  // nbw % W waves one more
  const int qq = nbw / W, rr = nbw % W;
  const int b0 = B0 + w * qq + (w < rr ? w : rr);
  const int nb = qq + (w < rr ? 1 : 0);
  const int total = nb * C;

  // a lane's piece: 16 bytes of codes (2:4) or 12 of codes and offsets (1:4)
  const uint32_t lane_codes = (uint32_t)lane * (NK == 2 ? 16u : 12u), lane_offs = (uint32_t)lane * (4u * NK);
  IssueCursor ic;
  ic.blk = b0;
  ic.chunk = 0;
  ic.g = b0 * C;
  cursor_block(ic, p, r, q);
  ChunkRegs<NK> R[D];
  __builtin_amdgcn_s_setprio(2);
#pragma unroll
  for (int s = 0; s < D; ++s) {
    issue_chunk<NK>(R[s], p, rbuf, ic, s < total, lane_codes, lane_offs);
    cursor_next(ic, p, r, q);
  }
  __builtin_amdgcn_s_setprio(0);
  __syncthreads();
  if (nb == 0) return;

  const uint32_t magic = opaque_vgpr(0x64006400u);
  const _Float16* xlane = xs + 64 * (q >> 1) + 8 * (q & 1);
  int cb = b0, cc = 0;
  bool g32 = cb * 16 + r < p.cls_row[1];
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  // every pass issues the loads of all D slots (past the end they read
  // zeros), so that every path through it leaves the same loads in flight
  // and each wait counts only the loads issued after its slot's
  for (int k = 0; k < total; k += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const bool live = k + s < total;
      if (live) acc = chunk_mac<NK>(R[s], xlane + 256 * cc, g32, magic, acc);
      // the slot is free again: load the chunk D ahead into it
      __builtin_amdgcn_s_setprio(2);
      issue_chunk<NK>(R[s], p, rbuf, ic, k + s + D < total, lane_codes, lane_offs);
      __builtin_amdgcn_s_setprio(0);
      cursor_next(ic, p, r, q);
      if (live && ++cc == C) {
        // block cb done: lane (column 0, q) holds rows 4q .. 4q + 3, kept
        // in LDS until the wave's last block (a store here would make every
        // wait for the loads in flight wait for it too)
        if (r == 0) {
          const h2 lo = {(_Float16)acc.x, (_Float16)acc.y}, hi = {(_Float16)acc.z, (_Float16)acc.w};
          *reinterpret_cast<u32x2*>(ys + (cb - B0) * 16 + 4 * q) = u32x2{as_u32(lo), as_u32(hi)};
        }
        cc = 0;
        ++cb;
        g32 = cb * 16 + r < p.cls_row[1];
        acc = f4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  // 3. y of the wave's rows at their original positions
  __builtin_amdgcn_wave_barrier();
  for (int e = lane; e < nb * 16; e += 64) {
    const int i = (b0 - B0) * 16 + e;
    const int n = ps[i];
    if (n >= 0 && n < p.N) p.y[n] = ys[i];
  }
}

// Workgroup j of task T, which takes row blocks [j q + min(j, r), ... + q +
// (j < r)); workgroups with j >= n_wg of their task have no work and end at
// once.
__device__ __forceinline__ void list_task(const ListTask& T, const int j) {
  if (j >= T.n_wg) return;
  const int B0 = j * T.q + (j < T.r ? j : T.r);
  const int nbw = T.q + (j < T.r ? 1 : 0);
  KParams p;
  p.blob = T.blob;
  p.x = T.x;
  p.y = T.y;
  p.blob_bytes = T.blob_bytes;
  p.off_codes = 0;
  p.off_offs = T.off_offs;
  p.off_perm = T.off_perm;
  p.off_sz = T.off_sz;
  p.N = T.N;
  p.C = (int32_t)(T.c_nk & 0xFFFFu);
  p.K = p.C * 256;
  p.B = 1;
  p.cls_row[0] = 0;
  p.cls_row[1] = T.cls1;
  p.cls_row[2] = T.cls2;
  p.cls_row[3] = T.cls3;
  p.cls_row[4] = T.N;
  if ((T.c_nk >> 16) == 2) list_stream<2>(p, B0, nbw);
  else list_stream<1>(p, B0, nbw);
}

// Workgroup (j, t) of the grid (max_t n_wg, count) of a kernel-argument
// launch: workgroup j of task t.
__device__ __forceinline__ void list_block(const ListParams& g) {
  list_task(g.t[blockIdx.y], (int)blockIdx.x);
}

typedef void (*ListFn)(ListParams);
ListFn get_list_kernel();
typedef void (*ListTableFn)(const ListRow*);
ListTableFn get_list_table_kernel();

}  // namespace sgemv_dev

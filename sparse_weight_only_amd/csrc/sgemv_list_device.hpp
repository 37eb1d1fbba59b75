// Device code of the task-list launch: many independent batch-1 GEMVs
// y_i = W'_i x_i (INT4 form, 2:4 or 1:4 per task) in one kernel, each
// workgroup walking a run of row blocks of one task.
//
// Per-token decoding runs every projection of every layer as a GEMV on one
// vector (the page "Efficient large-model ad applications through model
// compression and parallel verification", §1 "our core idea"); a 7B-shaped
// decoder step is 224 of them, 4-19 MB each. One launch per GEMV pays the
// dispatch, ramp-up and drain of a kernel every few microseconds. Here the
// whole list is one launch: the workgroups are few enough to be resident
// together, each task gets a number of them in proportion to its bytes, and
// each workgroup computes a contiguous run of the task's row blocks, issuing
// the loads of block b + 1 before computing block b, so that its weights
// stream while the previous block is dequantised and reduced.
//
// The steps per row block are those of the single-layer kernel (sgemv_block
// with one vector): the W waves split the row's column chunks into
// contiguous ranges; per 64-column step the codes become FP16 (code - zero)
// * scale, and the 2-of-4 sparse matrix-core instruction selects x and
// accumulates in FP32; the waves' partial sums meet in LDS and are added in
// wave order; y is rounded to FP16. What differs: the x slice of a wave is
// staged in LDS once per workgroup (the task, hence x, is fixed for it); the
// partial sums alternate between two LDS areas, so one barrier per block
// suffices.
#pragma once
#include "sgemv_device.hpp"

namespace sgemv_dev {

// One task of a list launch (76 bytes; up to kListMax of them travel in the
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
struct ListParams {
  int32_t count;           // tasks
  int32_t wlog;            // log2 of the waves per workgroup (3: 8 waves, 4: 16)
  int32_t pad[2];
  ListTask t[kListMax];
};
static_assert(sizeof(ListParams) <= 4096, "kernel arguments are limited to 4 KiB");

// Registers of one row block's weights for one wave: codes, offsets and
// scale|zero words of up to IMAX chunks, and the original row index of row
// lane % 16 of the block.
template <int NK, int IMAX>
struct BlockRegs {
  typedef typename std::conditional<NK == 2, u32x4, u32x2>::type CodeT;
  typedef typename std::conditional<NK == 2, u32x2, uint32_t>::type OffT;
  CodeT cv[IMAX];
  OffT ov[IMAX];
  u32x2 sv[IMAX];
  uint32_t orow;
  bool g32;
};

// Issue the loads of row block rb (rb_ok false: the same instructions read
// zeros without touching memory, so that every block issues the same loads
// and the waits before a block's compute count the next block's loads).
template <int NK, int IMAX>
__device__ __forceinline__ void list_load_block(BlockRegs<NK, IMAX>& R, const KParams& p, __amdgpu_buffer_rsrc_t rbuf,
                                                int rb, bool rb_ok, int c0, int ncw, int lane, int r, int q) {
  constexpr int CB = 8 * NK, OB = 4 * NK;
  const int row = rb * 16 + r;
  const int cls = (row >= p.cls_row[1]) + (row >= p.cls_row[2]) + (row >= p.cls_row[3]);
  const int wb0 = words_before(p, rb * 16);
  const uint32_t rec_words = (uint32_t)(words_before(p, rb * 16 + 16) - wb0);
  const int cls_first = class_of(p, rb * 16);
  const bool one_class = rec_words == (uint32_t)(16 * (8 >> cls_first));
  const uint32_t sz_row = one_class ? (uint32_t)(r * (8 >> cls_first)) : (uint32_t)(words_before(p, row) - wb0);
  const uint32_t sz_lane = sz_row + (uint32_t)((64 * q) >> (5 + cls));
  const uint32_t sz_block = (uint32_t)wb0 * (uint32_t)p.C;
  R.g32 = cls == 0;
  const uint32_t boff = rb_ok ? 0u : kOutOfRange;   // wave-uniform
  R.orow = bload1<kCached>(rbuf, p.off_perm + (uint32_t)(rb * 16 + (lane & 15)) * 4u, boff);
#pragma unroll
  for (int i = 0; i < IMAX; ++i) {
    const int c = c0 + i;
    const uint32_t off = i < ncw ? boff : kOutOfRange;
    const uint32_t rec = (uint32_t)(rb * p.C + c) * 64u + lane;
    const uint32_t so = p.off_sz + (sz_block + (uint32_t)c * rec_words + sz_lane) * 4u;
    if constexpr (NK == 2) {
      R.cv[i] = bload4<kStream>(rbuf, p.off_codes + rec * CB, off);
      R.ov[i] = bload2<kStream>(rbuf, p.off_offs + rec * OB, off);
    } else {
      R.cv[i] = bload2<kStream>(rbuf, p.off_codes + rec * CB, off);
      R.ov[i] = bload1<kStream>(rbuf, p.off_offs + rec * OB, off);
    }
    R.sv[i] = bload2<kStream>(rbuf, so, off);
  }
}

// The 16 x 16 partial tile of one wave for one row block (column 0 is the
// vector's): 4 matrix-core steps per chunk, as in sgemv_block at one vector.
template <int NK, int IMAX>
__device__ __forceinline__ f4 list_compute_block(const BlockRegs<NK, IMAX>& R, const _Float16* xrow, int ncw,
                                                 uint32_t magic) {
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < IMAX; ++i) {
    if (i >= ncw) break;
    const _Float16* xc = xrow + 256 * i;
    const Deq d0 = deq_consts(R.sv[i].x);
    const Deq d1 = deq_consts(R.g32 ? R.sv[i].y : R.sv[i].x);
    uint32_t idx2 = 0;
    if constexpr (NK == 1) idx2 = ((R.ov[i] & 0x33333333u) << 2) | ((R.ov[i] >> 2) & 0x33333333u);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const Deq& d = t < 2 ? d0 : d1;
      const h8 blo = *reinterpret_cast<const h8*>(xc + 16 * t);
      const h8 bhi = *reinterpret_cast<const h8*>(xc + 16 * t + 128);
      const h16 Bop = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      uint32_t a0, a1, a2, a3, idx;
      if constexpr (NK == 2) {
        const uint32_t cw = R.cv[i][t], c8 = cw >> 8;
        a0 = deq_lo(cw, magic, d);
        a1 = deq_hi(cw, magic, d);
        a2 = deq_lo(c8, magic, d);
        a3 = deq_hi(c8, magic, d);
        idx = R.ov[i][t >> 1];
      } else {
        const uint32_t cw = (t & 1) ? (R.cv[i][t >> 1] >> 8) : R.cv[i][t >> 1];
        const h2 q02 = as_h2((cw & 0x000F000Fu) | magic) + d.c1;
        const h2 q13 = __builtin_elementwise_fma(as_h2((cw & 0x00F000F0u) | magic), sixteenth, d.c16);
        a0 = as_u32(q02 * d.s_lo);
        a2 = as_u32(q02 * d.s_hi);
        a1 = as_u32(q13 * d.s_lo);
        a3 = as_u32(q13 * d.s_hi);
        idx = t < 2 ? R.ov[i] : idx2;
      }
      const h2 A0 = as_h2(a0), A1 = as_h2(a1), A2 = as_h2(a2), A3 = as_h2(a3);
      const h8 A = {A0.x, A0.y, A1.x, A1.y, A2.x, A2.y, A3.x, A3.y};
      if (t & 1) acc = smfmac<1>(A, Bop, acc, idx);
      else acc = smfmac<0>(A, Bop, acc, idx);
    }
  }
  return acc;
}

// Compute one row block from its registers, meet the waves' partial sums in
// the LDS area pa (part[row][wave]), and let lanes 0..15 of wave 0 add them
// in wave order and store y. One barrier: the next block uses the other area.
template <int NK, int IMAX>
__device__ __forceinline__ void list_finish_block(const BlockRegs<NK, IMAX>& R, const KParams& p, const _Float16* xrow,
                                                  int ncw, uint32_t magic, float* pa, int tid, int lane, int w, int q) {
  const f4 acc = list_compute_block<NK, IMAX>(R, xrow, ncw, magic);
  if ((lane & 15) == 0) {
    float* pp = pa + (4 * q) * 16 + w;
    pp[0] = acc.x;
    pp[16] = acc.y;
    pp[32] = acc.z;
    pp[48] = acc.w;
  }
  __syncthreads();
  if (tid < 16) {
    const f4* pv = reinterpret_cast<const f4*>(pa + tid * 16);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f4 v4 = pv[k];
      s += v4.x;
      s += v4.y;
      s += v4.z;
      s += v4.w;
    }
    const int n = (int)R.orow;
    if (n >= 0 && n < p.N) p.y[n] = __builtin_bit_cast(uint16_t, (_Float16)s);
  }
}

// Row blocks [b0, b1) of the task p, computed by the whole workgroup of W =
// 1 << wlog waves. Chunk split over the waves as in sgemv_block: the first
// crem waves take cpw chunks, the others cpw - 1 (fewer at the row end).
template <int NK, int IMAX, int XMAX>
__device__ __forceinline__ void list_run(const KParams& p, int b0, int b1, int wlog) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = 1 << wlog;
  const int r = lane & 15, q = lane >> 4;
  const int C = p.C;
  const int cpw = (C + W - 1) >> wlog;
  const int crem = C - W * (cpw - 1);
  const int c0 = w * cpw - (w > crem ? w - crem : 0);
  const int cw_max = cpw - (w >= crem ? 1 : 0);
  const int ncw = C - c0 < cw_max ? (C - c0 > 0 ? C - c0 : 0) : cw_max;
  const auto rbuf = make_rsrc(p.blob, p.blob_bytes);
  const auto rx = make_rsrc(p.x, (uint32_t)(C * 512));

  __builtin_amdgcn_s_setprio(2);
  // x slice of the wave: ncw chunks of 256 values, 16 bytes per load
  u32x4 xv[XMAX];
#pragma unroll
  for (int j = 0; j < XMAX; ++j) {
    const int u = lane + 64 * j;
    xv[j] = bload4<kCached>(rx, u < ncw * 32 ? (uint32_t)(c0 * 512 + u * 16) : kOutOfRange);
  }
  BlockRegs<NK, IMAX> cur;
  list_load_block<NK, IMAX>(cur, p, rbuf, b0, true, c0, ncw, lane, r, q);
  __builtin_amdgcn_s_setprio(0);

  // LDS: the waves' x slices (IMAX * 512 bytes each), then two areas of
  // partial sums part[row][wave] (16 x 16 floats each)
  _Float16* xs = reinterpret_cast<_Float16*>(smem) + w * (IMAX * 256);
  float* part = reinterpret_cast<float*>(smem + W * IMAX * 512);
#pragma unroll
  for (int j = 0; j < XMAX; ++j) {
    const int u = lane + 64 * j;
    if (u < IMAX * 32) reinterpret_cast<u32x4*>(xs)[u] = xv[j];
  }
  // slots of waves the workgroup does not have hold +0 (both areas)
  for (int e = tid; e < 512; e += 64 * W)
    if ((e & 15) >= W) part[e] = 0.f;
  __builtin_amdgcn_wave_barrier();
  const uint32_t magic = opaque_vgpr(0x64006400u);
  const _Float16* xrow = xs + 64 * (q >> 1) + 8 * (q & 1);

  // Two register sets alternate (no copies between them, which would make
  // the wave wait for the loads in flight): block b computes from one set
  // while the loads of block b + 1 fill the other.
  BlockRegs<NK, IMAX> nxt;
  for (int b = b0; b < b1; b += 2) {
    __builtin_amdgcn_s_setprio(2);
    list_load_block<NK, IMAX>(nxt, p, rbuf, b + 1, b + 1 < b1, c0, ncw, lane, r, q);
    __builtin_amdgcn_s_setprio(0);
    list_finish_block<NK, IMAX>(cur, p, xrow, ncw, magic, part + ((b - b0) & 1) * 256, tid, lane, w, q);
    if (b + 1 >= b1) break;
    __builtin_amdgcn_s_setprio(2);
    list_load_block<NK, IMAX>(cur, p, rbuf, b + 2, b + 2 < b1, c0, ncw, lane, r, q);
    __builtin_amdgcn_s_setprio(0);
    list_finish_block<NK, IMAX>(nxt, p, xrow, ncw, magic, part + ((b + 1 - b0) & 1) * 256, tid, lane, w, q);
  }
}

// Workgroup (j, t) of the grid (max_t n_wg, count): workgroup j of task t,
// which takes row blocks [j q + min(j, r), ... + q + (j < r)); workgroups
// with j >= n_wg of their task have no work and end at once.
template <int IMAX, int XMAX>
__device__ __forceinline__ void list_block(const ListParams& g) {
  const int t = (int)blockIdx.y, j = (int)blockIdx.x;
  const ListTask& T = g.t[t];
  if (j >= T.n_wg) return;
  const int b0 = j * T.q + (j < T.r ? j : T.r);
  const int b1 = b0 + T.q + (j < T.r ? 1 : 0);
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
  if ((T.c_nk >> 16) == 2) list_run<2, IMAX, XMAX>(p, b0, b1, g.wlog);
  else list_run<1, IMAX, XMAX>(p, b0, b1, g.wlog);
}

template <int IMAX, int XMAX>
__global__ __launch_bounds__(1024) void sgemv_list_kernel(ListParams g) {
  list_block<IMAX, XMAX>(g);
}

typedef void (*ListFn)(ListParams);
ListFn get_list_kernel(int imax);

}  // namespace sgemv_dev

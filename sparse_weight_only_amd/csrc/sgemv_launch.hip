// sgemv_run: host-side checks and the launch of the SparseGemv kernels.
#include <hip/hip_runtime.h>

#include "internal.hpp"
#include "kernels.hpp"
#include "sgemv_device.hpp"

using namespace sgemv;
using sgemv_dev::KParams;
using sgemv_dev::KernelFn;

namespace {

bool desc_consistent(const sgemv_desc* d) {
  if (d->N < 1 || d->K < 256 || d->K % 256 || (d->nk != 1 && d->nk != 2)) return false;
  if ((int64_t)d->N * d->K * d->nk / 4 >= ((int64_t)1 << 31)) return false;
  const int32_t C = d->K * d->nk / 128;
  if (!layout_params_ok(d->K, C, cols_per_chunk(d->nk), d->tpr, d->rt, d->g_max)) return false;
  if (d->n_tiles < 1 || d->n_tiles > d->N) return false;
  int64_t rows = 0, tiles = 0, groups = 0;
  for (int c = 0; c < 4; ++c) {
    if (d->class_rows[c] < 0) return false;
    rows += d->class_rows[c];
    tiles += (d->class_rows[c] + d->rt - 1) / d->rt;
    groups += (int64_t)d->class_rows[c] * (d->K / (32 << c));
  }
  if (rows != d->N || tiles != d->n_tiles || groups != d->n_groups || d->reserved != 0) return false;
  if (!valid_group(d->g_min, d->K) || !valid_group(d->g_max, d->K) || d->g_min > d->g_max) return false;
  if (d->kept != (int64_t)d->N * d->K * d->nk / 4) return false;
  if (d->vals_bytes != d->kept / 2 || d->offs_bytes != d->kept / 4) return false;
  if (d->n_groups < (int64_t)d->N * (d->K / d->g_max) || d->n_groups > (int64_t)d->N * (d->K / d->g_min)) return false;
  if (d->off_tiles != 0 || d->off_perm != align_up(16 * (int64_t)d->n_tiles)) return false;
  if (d->off_vals != align_up(d->off_perm + 4 * (int64_t)d->N)) return false;
  if (d->off_offs != align_up(d->off_vals + 16 * (int64_t)d->N * C)) return false;
  if (d->off_sz != align_up(d->off_offs + 8 * (int64_t)d->N * C)) return false;
  if (d->blob_bytes != align_up(d->off_sz + 4 * d->n_groups)) return false;
  return true;
}

}  // namespace

namespace {

// What sgemv_run launches for a descriptor and batch: pure host arithmetic.
int make_plan(const sgemv_desc* d, int32_t B, sgemv_plan_t* pl) {
  if (!d || !pl) return SGEMV_EINVAL;
  if (B < 1 || B > 16) return SGEMV_EINVAL;
  if (!desc_consistent(d)) return SGEMV_ESIZE;
  const int cpc = cols_per_chunk(d->nk);
  const int32_t C = d->K * d->nk / 128;
  const Geometry geo = geometry(d->K, C, d->tpr, d->rt);
  const int wg_layout = d->rt * d->tpr;
  sgemv_plan_t q;
  memset(&q, 0, sizeof q);
  q.batched = B > 1;
  if (B == 1) {
    // one workgroup per tile; each lane owns geo.rpl rows of the tile
    q.block = geo.wg;
    q.pass_log2 = 0;
    q.rows_per_lane = geo.rpl;
  } else {
    // 256-lane workgroups; a tile with more (row, lane) slots is split in passes
    q.block = std::min(wg_layout, sgemv_dev::kBatchedThreads);
    q.pass_log2 = ilog2(wg_layout / q.block);
    q.rows_per_lane = 1;
  }
  q.grid = (int64_t)d->n_tiles << q.pass_log2;
  q.chunks_per_row_lane = geo.iters;
  // x columns staged per phase: whole chunk iterations of all lanes, for up to
  // 4 batch vectors at a time
  const int bstage = B == 1 ? 1 : std::min<int>(B, sgemv_dev::kBatchGroup);
  const int64_t per_iter = (int64_t)bstage * d->tpr * (cpc / 8 + 1) * 16;
  const int64_t budget = (B == 1) ? 160 * 1024 : 65536;   // batch 1 stages all of x at once
  int32_t pi = geo.iters;
  while (pi > 1 && per_iter * pi > budget) --pi;
  q.lds_bytes = per_iter * pi;
  q.phase_iters = pi;
  if (q.lds_bytes > 160 * 1024) return SGEMV_ESIZE;
  if (B == 1 && pi != geo.iters) return SGEMV_ESIZE;
  *pl = q;
  return SGEMV_OK;
}

}  // namespace

extern "C" int sgemv_plan(const sgemv_desc* d, int32_t B, sgemv_plan_t* out) { return make_plan(d, B, out); }

extern "C" int sgemv_run(const sgemv_desc* d, const void* blob_dev, const void* x_dev, void* y_dev,
                         int32_t B, void* hip_stream) {
  if (!d || !blob_dev || !x_dev || !y_dev) return SGEMV_EINVAL;
  sgemv_plan_t pl;
  const int rc = make_plan(d, B, &pl);
  if (rc) return rc;
  if (((uintptr_t)blob_dev % 256) || ((uintptr_t)x_dev % 16) || ((uintptr_t)y_dev % 2)) return SGEMV_EALIGN;
  const int32_t C = d->K * d->nk / 128;
  const Geometry geo = geometry(d->K, C, d->tpr, d->rt);
  const uint8_t* blob = (const uint8_t*)blob_dev;
  KParams p;
  p.tiles = (const int32_t*)(blob + d->off_tiles);
  p.perm = (const int32_t*)(blob + d->off_perm);
  p.vals = (const sgemv_dev::u32x4*)(blob + d->off_vals);
  p.offs = (const sgemv_dev::u32x2*)(blob + d->off_offs);
  p.sz = (const uint32_t*)(blob + d->off_sz);
  p.x = (const sgemv_dev::u32x4*)x_dev;
  p.y = (uint16_t*)y_dev;
  p.N = d->N; p.K = d->K; p.C = C; p.B = B;
  p.tpr_log2 = ilog2(d->tpr);
  p.phase_iters = pl.phase_iters;
  p.pass_log2 = pl.pass_log2;
  p.rt = d->rt;
  {
    int32_t t = 0, r = 0, z = 0;
    for (int c = 0; c < 4; ++c) {
      p.cls_tile[c] = t; p.cls_row[c] = r; p.cls_sz[c] = z;
      t += (d->class_rows[c] + d->rt - 1) / d->rt;
      r += d->class_rows[c];
      z += d->class_rows[c] * (d->K / (32 << c));
    }
    p.cls_tile[4] = t; p.cls_row[4] = r;
  }
  KernelFn fn = (B == 1) ? sgemv_dev::get_b1(d->nk, geo.rpl, geo.imax, geo.xmax) : sgemv_dev::get_bn(d->nk);
  if (!fn) return SGEMV_ESIZE;
  if (pl.lds_bytes > 65536) {
    if (hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)pl.lds_bytes) != hipSuccess)
      return SGEMV_EHIP;
  }
  hipLaunchKernelGGL(fn, dim3((uint32_t)pl.grid), dim3(pl.block), (uint32_t)pl.lds_bytes, (hipStream_t)hip_stream, p);
  if (hipGetLastError() != hipSuccess) return SGEMV_EHIP;
  return SGEMV_OK;
}

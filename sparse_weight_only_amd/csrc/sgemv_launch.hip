// sgemv_plan / sgemv_run: host-side checks and the launch of the SparseGemv kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "internal.hpp"
#include "kernels.hpp"
#include "sgemv_device.hpp"
#include "sgemv_list_device.hpp"

using namespace sgemv;
using sgemv_dev::GParams;
using sgemv_dev::GroupFn;
using sgemv_dev::kMaxGroup;
static_assert(sgemv_dev::kMaxGroup == SGEMV_MAX_GROUP, "group size limit");
static_assert(sgemv_dev::kListMax == SGEMV_LIST_MAX, "list size limit");
using sgemv_dev::KernelFn;
using sgemv_dev::KParams;

namespace {

// The descriptor must be one that sgemv_describe (or sgemv_describe_fp16) can produce.
bool desc_consistent(const sgemv_desc* d) {
  if (d->value_format == 1) {
    sgemv_desc chk;
    return sgemv_describe_fp16(d->N, d->K, d->nk, &chk) == SGEMV_OK && memcmp(&chk, d, sizeof chk) == 0;
  }
  if (d->N < 1 || d->K < kChunkCols || d->K % kChunkCols || !valid_nk(d->nk)) return false;
  const int32_t C = d->K / kChunkCols, T = (d->N + kBlockRows - 1) / kBlockRows;
  if (C > kMaxChunks || d->chunks != C || d->n_blocks != T || d->value_format != 0) return false;
  int64_t rows = 0, groups = 0;
  for (int c = 0; c < 4; ++c) {
    if (d->class_rows[c] < 0) return false;
    rows += d->class_rows[c];
    groups += (int64_t)d->class_rows[c] * (d->K / (32 << c));
  }
  if (rows != d->N || groups != d->n_groups) return false;
  if (!valid_group(d->g_min, d->K) || !valid_group(d->g_max, d->K) || d->g_min > d->g_max) return false;
  if (d->class_rows[ilog2(d->g_min / 32)] == 0 || d->class_rows[ilog2(d->g_max / 32)] == 0) return false;
  if (d->kept != (int64_t)d->N * d->K * d->nk / 4) return false;
  if (d->vals_bytes != d->kept / 2 || d->offs_bytes != (d->nk == 4 ? 0 : d->kept / 4)) return false;
  const int64_t records = (int64_t)T * C * 64;
  if (d->off_codes != 0 || d->off_offs != align_up(records * piece_code_bytes(d->nk))) return false;
  if (d->off_perm != align_up(d->off_offs + records * piece_offs_bytes(d->nk))) return false;
  if (d->off_sz != align_up(d->off_perm + 4 * (int64_t)T * kBlockRows)) return false;
  if (d->blob_bytes != align_up(d->off_sz + 4 * d->n_groups + 8) || d->blob_bytes >= ((int64_t)1 << 31)) return false;
  return true;
}

// What sgemv_run launches for a descriptor and batch: pure host arithmetic.
int make_plan(const sgemv_desc* d, int32_t B, sgemv_plan_t* pl, Launch* geo) {
  if (!d || !pl) return SGEMV_EINVAL;
  if (B < 1 || B > 16) return SGEMV_EINVAL;
  if (!desc_consistent(d)) return SGEMV_ESIZE;
  // several row blocks per workgroup: INT4 sparse forms only
  const int rb = d->value_format == 0 && d->nk != 4 ? pick_row_blocks(d->chunks, d->n_blocks, B) : 1;
  const Launch L = launch_geometry_rb(d->chunks, d->n_blocks, B, rb);
  if (L.waves < 1 || L.waves > kMaxWaves || L.cpw > kMaxChunksPerWave || L.xloads > 8) return SGEMV_ESIZE;
  if (L.lds > 160 * 1024 || (L.phase & (L.phase - 1)) != 0) return SGEMV_ESIZE;
  if (L.rb > 1 && (L.rb * L.imax > kMaxChunksPerWave || L.waves > kMaxWavesRb)) return SGEMV_ESIZE;
  sgemv_plan_t q;
  memset(&q, 0, sizeof q);
  q.grid = (d->n_blocks + L.rb - 1) / L.rb;
  q.row_blocks = L.rb;
  q.lds_bytes = L.lds;
  q.block = 64 * L.waves;
  q.waves = L.waves;
  q.chunks_per_wave = L.cpw;
  q.full_waves = L.crem;
  q.phase_chunks = L.phase;
  q.x_loads = L.xloads;
  *pl = q;
  if (geo) *geo = L;
  return SGEMV_OK;
}

// Kernel parameters of one layer under a launch geometry.
KParams make_params(const sgemv_desc* d, const void* blob, const void* x, void* y, int32_t B, const Launch& L) {
  KParams p;
  p.blob = (const uint8_t*)blob;
  p.x = (const uint16_t*)x;
  p.y = (uint16_t*)y;
  p.blob_bytes = (uint32_t)d->blob_bytes;
  p.off_codes = (uint32_t)d->off_codes;
  p.off_offs = (uint32_t)d->off_offs;
  p.off_perm = (uint32_t)d->off_perm;
  p.off_sz = (uint32_t)d->off_sz;
  p.N = d->N; p.K = d->K; p.B = B; p.C = d->chunks;
  p.cpw = L.cpw;
  p.crem = L.crem;
  p.phase = L.phase;
  p.T = d->n_blocks;
  p.cls_row[0] = 0;
  for (int c = 0; c < 4; ++c) p.cls_row[c + 1] = p.cls_row[c] + d->class_rows[c];
  p.waves = L.waves;
  return p;
}

// Dynamic LDS beyond 64 KiB needs the kernel's limit raised. The runtime
// keeps the attribute per kernel and device, so it is set once for each
// (kernel, device) pair, to the full 160 KiB, and remembered here.
int ensure_lds(const void* fn, int64_t lds_bytes) {
  if (lds_bytes <= 65536) return SGEMV_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SGEMV_EHIP;
  static std::mutex mu;
  static std::vector<std::pair<const void*, int>> raised;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& e : raised)
    if (e.first == fn && e.second == dev) return SGEMV_OK;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess) return SGEMV_EHIP;
  raised.emplace_back(fn, dev);
  return SGEMV_OK;
}

bool aligned(const void* blob, const void* x, const void* y) {
  return !(((uintptr_t)blob % 256) || ((uintptr_t)x % 16) || ((uintptr_t)y % 2));
}

// What sgemv_run_group launches: one geometry for the widest layer and the
// summed row blocks; pure host arithmetic.
int make_group_plan(const sgemv_task* tasks, int32_t count, int32_t B, sgemv_plan_t* pl, Launch* geo) {
  if (!tasks || !pl) return SGEMV_EINVAL;
  if (count < 1 || count > kMaxGroup || B < 1 || B > 16) return SGEMV_EINVAL;
  int64_t blocks = 0;
  int32_t cmax = 0;
  for (int32_t i = 0; i < count; ++i) {
    const sgemv_desc* d = tasks[i].desc;
    if (!d) return SGEMV_EINVAL;
    if (!desc_consistent(d)) return SGEMV_ESIZE;
    if (d->nk != tasks[0].desc->nk || d->value_format != tasks[0].desc->value_format) return SGEMV_EINVAL;
    blocks += d->n_blocks;
    cmax = d->chunks > cmax ? d->chunks : cmax;
  }
  if (blocks > ((int64_t)1 << 30)) return SGEMV_ESIZE;
  const Launch L = launch_geometry(cmax, (int32_t)blocks, B);
  if (L.waves < 1 || L.waves > kMaxWaves || L.cpw > kMaxChunksPerWave || L.xloads > 8) return SGEMV_ESIZE;
  if (L.lds > 160 * 1024 || (L.phase & (L.phase - 1)) != 0) return SGEMV_ESIZE;
  sgemv_plan_t q;
  memset(&q, 0, sizeof q);
  q.grid = blocks;
  q.row_blocks = 1;
  q.lds_bytes = L.lds;
  q.block = 64 * L.waves;
  q.waves = L.waves;
  q.chunks_per_wave = L.cpw;
  q.full_waves = L.crem;
  q.phase_chunks = L.phase;
  q.x_loads = L.xloads;
  *pl = q;
  if (geo) *geo = L;
  return SGEMV_OK;
}

// The task-list launch (one vector, INT4 form): the workgroups' count and
// each task's share of them. Pure host arithmetic.
//  - workgroups of 8 waves, at most 6 per compute unit of the 256 on MI355X
//    (12 when the layers differ in shape or N:M choice, below)
//    (3 are resident at once with 72 VGPRs a lane; the others wait and take
//    the place of those that finish first, which evens out the work of
//    unequal runs), and each task's workgroups hold at least 8 of its row
//    blocks where it has that many (one run per wave). Measured on the
//    224-GEMV decoder as 6 launches: 2 per compute unit (all resident) took
//    483 us with 8 chunks in flight a wave; 4 chunks with 4 and 6 per unit
//    took 402-406 and 398-399 us, 8 per unit with 4 waves a workgroup 398 us;
//  - each task gets workgroups in proportion to its algorithmic bytes (at
//    least one, and enough that none takes more than 256 row blocks; largest
//    remainders first), and its workgroup j computes a contiguous run of
//    q + (j < r) row blocks, split over its waves. The launch grid is
//    (largest share, tasks), its rows ordered by the bytes of their longest
//    wave, longest first; workgroups past their task's share end at once.
//    Measured on the decoder sequence: 378-389 us longest first against
//    399-408 us in task order (three interleaved rounds). Splitting in
//    units of 8 blocks, so that a workgroup's waves get the same number of
//    blocks, was slower (386-395 us): the workgroups of a layer then differ
//    by a whole unit.
//  - a table launch (the task table in device memory, any number of tasks)
//    has kListWgPerCU x 256 workgroups (doubled for mixed shapes) per
//    kListMax tasks or part of it, so that each task gets the share it
//    would get in a launch of kListMax tasks.
constexpr int kListCUs = 256;
constexpr int kListWgPerCU = 6;
struct ListPlan { int waves, grid, gx, max_blocks; int64_t lds; };
int make_list_plan(const sgemv_task* tasks, int32_t count, int32_t B, int32_t max_count, ListPlan* lp,
                   std::vector<sgemv_dev::ListTask>* out) {
  using sgemv_dev::kListMaxBlocks;
  using sgemv_dev::kListWaves;
  if (!tasks || !lp) return SGEMV_EINVAL;
  if (count < 1 || count > max_count || B != 1) return SGEMV_EINVAL;
  int cmax = 0;
  double total = 0.0;
  std::vector<double> cost(count);
  std::vector<int> lo(count), hi(count);
  int need = 0;
  for (int32_t i = 0; i < count; ++i) {
    const sgemv_desc* d = tasks[i].desc;
    if (!d) return SGEMV_EINVAL;
    if (!desc_consistent(d)) return SGEMV_ESIZE;
    if (d->value_format != 0 || (d->nk != 1 && d->nk != 2)) return SGEMV_EINVAL;
    cmax = d->chunks > cmax ? d->chunks : cmax;
    cost[i] = (double)(d->vals_bytes + d->offs_bytes + 4 * d->n_groups + 2 * (int64_t)d->K + 2 * (int64_t)d->N);
    total += cost[i];
    const int T = d->n_blocks;
    lo[i] = (T + kListMaxBlocks - 1) / kListMaxBlocks;           // at most 256 blocks a workgroup
    hi[i] = T / kListWaves > lo[i] ? T / kListWaves : lo[i];      // at least one block a wave, where possible
    need += lo[i];
  }
  ListPlan L;
  L.waves = kListWaves;
  // layers of different shapes or N:M choices: twice as many (smaller)
  // workgroups, which even out the end of the launch where the layers'
  // workgroups differ in length. Measured on the decoder sequence (three
  // interleaved rounds): sequence order 360-363 us against 373-387 us,
  // grouped by shape 338-340 us against 343-349 us; 12 per CU for every
  // list made the lists of one shape slower.
  bool mixed = false;
  for (int32_t i = 1; i < count; ++i)
    mixed |= tasks[i].desc->chunks != tasks[0].desc->chunks || tasks[i].desc->n_blocks != tasks[0].desc->n_blocks ||
             tasks[i].desc->nk != tasks[0].desc->nk;
  int grid = kListCUs * kListWgPerCU * (mixed ? 2 : 1) * ((count + sgemv_dev::kListMax - 1) / sgemv_dev::kListMax);
  if (grid < need) grid = need;
  std::vector<int> n(count);
  std::vector<std::pair<double, int>> rem;
  int used = 0;
  for (int32_t i = 0; i < count; ++i) {
    const double share = grid * cost[i] / total;
    int k = (int)share;
    k = k < lo[i] ? lo[i] : k > hi[i] ? hi[i] : k;
    n[i] = k;
    used += k;
    rem.emplace_back(share - k, i);
  }
  std::stable_sort(rem.begin(), rem.end(), [](const std::pair<double, int>& a, const std::pair<double, int>& b) {
    return a.first > b.first;
  });
  for (size_t k = 0; used < grid && k < rem.size(); ++k) {
    const int i = rem[k].second;
    if (n[i] < hi[i]) { ++n[i]; ++used; }
  }
  L.grid = used;
  L.gx = 0;
  L.max_blocks = 0;
  if (out) out->assign(count, sgemv_dev::ListTask{});
  // grid rows in order of the longest wave's bytes, longest first: the
  // workgroups are dispatched row after row, so the long ones start first
  // and the short ones fill the end of the launch
  std::vector<std::pair<double, int>> order(count);
  for (int32_t i = 0; i < count; ++i) {
    const int T = tasks[i].desc->n_blocks, mb = T / n[i] + (T % n[i] ? 1 : 0);
    order[i] = {-(double)((mb + kListWaves - 1) / kListWaves) * cost[i] / T, i};
  }
  std::stable_sort(order.begin(), order.end(),
                   [](const std::pair<double, int>& a, const std::pair<double, int>& b) { return a.first < b.first; });
  for (int32_t k = 0; k < count; ++k) {
    const int i = order[k].second;
    const sgemv_desc* d = tasks[i].desc;
    const int q = d->n_blocks / n[i], r = d->n_blocks % n[i];
    const int mb = q + (r ? 1 : 0);
    L.max_blocks = mb > L.max_blocks ? mb : L.max_blocks;
    L.gx = n[i] > L.gx ? n[i] : L.gx;
    if (out) {
      sgemv_dev::ListTask& t = (*out)[k];
      t.blob = (const uint8_t*)tasks[i].blob_dev;
      t.x = (const uint16_t*)tasks[i].x_dev;
      t.y = (uint16_t*)tasks[i].y_dev;
      t.blob_bytes = (uint32_t)d->blob_bytes;
      t.off_offs = (uint32_t)d->off_offs;
      t.off_perm = (uint32_t)d->off_perm;
      t.off_sz = (uint32_t)d->off_sz;
      t.N = d->N;
      t.cls1 = d->class_rows[0];
      t.cls2 = t.cls1 + d->class_rows[1];
      t.cls3 = t.cls2 + d->class_rows[2];
      t.c_nk = (uint32_t)d->chunks | ((uint32_t)d->nk << 16);
      t.n_wg = n[i];
      t.q = q;
      t.r = r;
    }
  }
  if (L.max_blocks > kListMaxBlocks) return SGEMV_ESIZE;
  // x of the widest task, and the row indices and FP16 results of the most
  // blocks a workgroup takes
  L.lds = (int64_t)cmax * 512 + (int64_t)L.max_blocks * (64 + 32);
  if (L.lds > 160 * 1024) return SGEMV_ESIZE;
  *lp = L;
  return SGEMV_OK;
}

// Grid rows of a table launch: a task whose share is wider than a row spans
// consecutive rows (workgroups past the share in its last row end at once).
constexpr int kListRowWidth = 32;

bool list_pointers_ok(const sgemv_task* tasks, int32_t count, int* rc) {
  for (int32_t i = 0; i < count; ++i) {
    const sgemv_task& t = tasks[i];
    if (!t.blob_dev || !t.x_dev || !t.y_dev) { *rc = SGEMV_EINVAL; return false; }
    if (!aligned(t.blob_dev, t.x_dev, t.y_dev)) { *rc = SGEMV_EALIGN; return false; }
  }
  return true;
}

}  // namespace

extern "C" int sgemv_plan_list(const sgemv_task* tasks, int32_t count, int32_t B, sgemv_plan_t* out) {
  if (!out) return SGEMV_EINVAL;
  ListPlan L;
  const int rc = make_list_plan(tasks, count, B, sgemv_dev::kListMax, &L, nullptr);
  if (rc) return rc;
  sgemv_plan_t q;
  memset(&q, 0, sizeof q);
  q.grid = L.grid;
  q.row_blocks = L.max_blocks;
  q.lds_bytes = L.lds;
  q.block = 64 * L.waves;
  q.waves = L.waves;
  q.chunks_per_wave = 0;
  q.full_waves = L.waves;
  q.phase_chunks = 0;
  q.x_loads = 0;
  *out = q;
  return SGEMV_OK;
}

extern "C" int sgemv_run_list(const sgemv_task* tasks, int32_t count, int32_t B, void* hip_stream) {
  ListPlan L;
  std::vector<sgemv_dev::ListTask> order;
  int rc = make_list_plan(tasks, count, B, sgemv_dev::kListMax, &L, &order);
  if (rc) return rc;
  if (!list_pointers_ok(tasks, count, &rc)) return rc;
  sgemv_dev::ListParams g;
  memset(&g, 0, sizeof g);
  g.count = count;
  std::copy(order.begin(), order.end(), g.t);
  sgemv_dev::ListFn fn = sgemv_dev::get_list_kernel();
  (void)hipGetLastError();
  if (ensure_lds((const void*)fn, L.lds)) return SGEMV_EHIP;
  // grid (largest task share, tasks): workgroup (j, t) is task t's j-th
  hipLaunchKernelGGL(fn, dim3((uint32_t)L.gx, (uint32_t)count), dim3(64 * L.waves), (uint32_t)L.lds,
                     (hipStream_t)hip_stream, g);
  if (hipGetLastError() != hipSuccess) return SGEMV_EHIP;
  return SGEMV_OK;
}

extern "C" int sgemv_list_table(const sgemv_task* tasks, int32_t count, int32_t B, void* table_host,
                                int64_t table_bytes, sgemv_list_launch* out) {
  if (!out) return SGEMV_EINVAL;
  ListPlan L;
  std::vector<sgemv_dev::ListTask> order;
  int rc = make_list_plan(tasks, count, B, SGEMV_LIST_TABLE_MAX, &L, &order);
  if (rc) return rc;
  if (!list_pointers_ok(tasks, count, &rc)) return rc;
  const int width = L.gx < kListRowWidth ? L.gx : kListRowWidth;
  std::vector<sgemv_dev::ListRow> rows;
  for (const sgemv_dev::ListTask& t : order)
    for (int j0 = 0; j0 < t.n_wg; j0 += width) {
      sgemv_dev::ListRow row;
      memset(&row, 0, sizeof row);
      row.t = t;
      row.j0 = j0;
      rows.push_back(row);
    }
  if (rows.size() > 65535) return SGEMV_ESIZE;   // grid rows
  sgemv_list_launch q;
  memset(&q, 0, sizeof q);
  q.table_bytes = (int64_t)(rows.size() * sizeof(sgemv_dev::ListRow));
  q.lds_bytes = L.lds;
  q.workgroups = L.grid;
  q.rows = (int32_t)rows.size();
  q.row_width = width;
  q.tasks = count;
  q.block = 64 * L.waves;
  *out = q;
  if (!table_host) return SGEMV_OK;
  if (table_bytes < q.table_bytes) return SGEMV_ESIZE;
  memcpy(table_host, rows.data(), (size_t)q.table_bytes);
  return SGEMV_OK;
}

extern "C" int sgemv_run_list_table(const void* table_dev, const sgemv_list_launch* launch, void* hip_stream) {
  if (!table_dev || !launch) return SGEMV_EINVAL;
  const sgemv_list_launch& q = *launch;
  if (q.rows < 1 || q.rows > 65535 || q.row_width < 1 || q.row_width > kListRowWidth ||
      q.block != 64 * sgemv_dev::kListWaves || q.lds_bytes < 0 || q.lds_bytes > 160 * 1024 ||
      q.table_bytes != (int64_t)q.rows * (int64_t)sizeof(sgemv_dev::ListRow))
    return SGEMV_EINVAL;
  if ((uintptr_t)table_dev % 16) return SGEMV_EALIGN;
  sgemv_dev::ListTableFn fn = sgemv_dev::get_list_table_kernel();
  (void)hipGetLastError();
  if (ensure_lds((const void*)fn, q.lds_bytes)) return SGEMV_EHIP;
  hipLaunchKernelGGL(fn, dim3((uint32_t)q.row_width, (uint32_t)q.rows), dim3((uint32_t)q.block), (uint32_t)q.lds_bytes,
                     (hipStream_t)hip_stream, (const sgemv_dev::ListRow*)table_dev);
  if (hipGetLastError() != hipSuccess) return SGEMV_EHIP;
  return SGEMV_OK;
}

extern "C" int sgemv_plan(const sgemv_desc* d, int32_t B, sgemv_plan_t* out) {
  return make_plan(d, B, out, nullptr);
}

extern "C" int sgemv_run(const sgemv_desc* d, const void* blob_dev, const void* x_dev, void* y_dev,
                         int32_t B, void* hip_stream) {
  if (!d || !blob_dev || !x_dev || !y_dev) return SGEMV_EINVAL;
  sgemv_plan_t pl;
  Launch L;
  const int rc = make_plan(d, B, &pl, &L);
  if (rc) return rc;
  if (!aligned(blob_dev, x_dev, y_dev)) return SGEMV_EALIGN;
  const KParams p = make_params(d, blob_dev, x_dev, y_dev, B, L);
  if (L.rb == 1) {
    // one layer, one row block per workgroup: the fields needed first go as
    // leading scalar arguments, which the hardware preloads into registers
    sgemv_dev::LeadFn f1 = d->value_format == 1       ? sgemv_dev::get_f16_kernel(d->nk, L.imax, L.xmax)
                           : (B == 1 && d->nk != 4)   ? sgemv_dev::get_b1_kernel(d->nk, L.imax, L.xmax)
                                                      : sgemv_dev::get_kernel(d->nk, L.imax, L.xmax);
    if (!f1 || L.cpw > 255 || L.crem > 255 || L.phase > 255 || p.off_codes != 0) return SGEMV_ESIZE;
    (void)hipGetLastError();   // a stale error of an earlier call must not be reported as this launch's
    if (ensure_lds((const void*)f1, pl.lds_bytes)) return SGEMV_EHIP;
    const uint32_t packed = (uint32_t)L.cpw | ((uint32_t)L.crem << 8) | ((uint32_t)L.phase << 16) | ((uint32_t)B << 24);
    hipLaunchKernelGGL(f1, dim3((uint32_t)pl.grid), dim3(pl.block), (uint32_t)pl.lds_bytes, (hipStream_t)hip_stream,
                       p.blob, p.x, p.blob_bytes, p.off_offs, p.off_perm, p.off_sz, p.K, packed,
                       p.cls_row[1], p.cls_row[2], p.cls_row[3], p.cls_row[4], p);
    if (hipGetLastError() != hipSuccess) return SGEMV_EHIP;
    return SGEMV_OK;
  }
  KernelFn fn = sgemv_dev::get_rb_kernel(d->nk, L.imax, L.xmax, L.rb);
  if (!fn) return SGEMV_ESIZE;
  (void)hipGetLastError();
  if (ensure_lds((const void*)fn, pl.lds_bytes)) return SGEMV_EHIP;
  hipLaunchKernelGGL(fn, dim3((uint32_t)pl.grid), dim3(pl.block), (uint32_t)pl.lds_bytes, (hipStream_t)hip_stream, p);
  if (hipGetLastError() != hipSuccess) return SGEMV_EHIP;
  return SGEMV_OK;
}

extern "C" int sgemv_plan_group(const sgemv_task* tasks, int32_t count, int32_t B, sgemv_plan_t* out) {
  return make_group_plan(tasks, count, B, out, nullptr);
}

extern "C" int sgemv_run_group(const sgemv_task* tasks, int32_t count, int32_t B, void* hip_stream) {
  sgemv_plan_t pl;
  Launch L;
  const int rc = make_group_plan(tasks, count, B, &pl, &L);
  if (rc) return rc;
  GParams g;
  memset(&g, 0, sizeof g);
  g.count = count;
  for (int j = 0; j <= kMaxGroup; ++j) g.first_block[j] = INT32_MAX;   // the kernel's layer search relies on it
  g.first_block[0] = 0;
  for (int32_t i = 0; i < count; ++i) {
    const sgemv_task& t = tasks[i];
    if (!t.blob_dev || !t.x_dev || !t.y_dev) return SGEMV_EINVAL;
    if (!aligned(t.blob_dev, t.x_dev, t.y_dev)) return SGEMV_EALIGN;
    g.t[i] = make_params(t.desc, t.blob_dev, t.x_dev, t.y_dev, B, L);
    g.first_block[i + 1] = g.first_block[i] + t.desc->n_blocks;
  }
  const int nk0 = tasks[0].desc->nk;
  GroupFn fn = tasks[0].desc->value_format == 1 ? sgemv_dev::get_f16_group_kernel(nk0, L.imax, L.xmax)
              : (B == 1 && nk0 != 4)             ? sgemv_dev::get_b1_group_kernel(nk0, L.imax, L.xmax)
                                                 : sgemv_dev::get_group_kernel(nk0, L.imax, L.xmax);
  if (!fn) return SGEMV_ESIZE;
  (void)hipGetLastError();
  if (ensure_lds((const void*)fn, pl.lds_bytes)) return SGEMV_EHIP;
  hipLaunchKernelGGL(fn, dim3((uint32_t)pl.grid), dim3(pl.block), (uint32_t)pl.lds_bytes, (hipStream_t)hip_stream, g);
  if (hipGetLastError() != hipSuccess) return SGEMV_EHIP;
  return SGEMV_OK;
}

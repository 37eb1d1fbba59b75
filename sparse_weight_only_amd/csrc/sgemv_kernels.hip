// SparseGemv kernels for gfx950 (MI355X) and the sgemv_run launcher.
//
// y = W' x for an N:M-sparse (2:4 or 1:4 along K) INT4 weight matrix with
// per-group FP16 scale and zero, FP16 activations and FP32 accumulation: the
// custom weight-only GEMV with mixed sparsity of the page "Efficient LLM ad
// generation via model compression and parallel verification" (translation
// of arXiv 2605.11582), §1 (second contribution item) and §3.3 "Revised
// kernel". That section is cut off before the kernel design; the design here
// is our own for CDNA4.
//
// Design (one workgroup per tile of rt rows of one group size; tpr threads
// per row split the row's 32-element chunks round-robin):
//  1. every thread issues all of its weight loads up front: one 16-byte code
//     load, one 8-byte offset load and one 4/8/16-byte scale|zero load per
//     chunk, coalesced across the workgroup by the kernel layout;
//  2. meanwhile the workgroup stages x into LDS as byte planes (per 8 columns:
//     8 low bytes then 8 high bytes), with one 16-byte pad per chunk so that
//     neighbouring k-lanes read different banks;
//  3. per 4 kept elements: 2-bit offsets -> v_perm byte selectors, which pick
//     the matching x halves out of the planes; nibbles -> FP16 (q - z) exactly
//     via the 0x6400 exponent trick; v_dot2_f32_f16 accumulates in FP32; the
//     FP16 scale multiplies the FP32 partial of each group;
//  4. butterfly reduction over the row's tpr lanes; lane 0 writes y in FP16
//     (round to nearest even) to the row's original position.
// The per-element products (q - z) * x are exact in FP32, so the only
// rounding is the FP32 accumulation and the final FP16 conversion.
#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace {

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
};

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ float dot2(f16x2 a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(hp16x2, a), __builtin_bit_cast(hp16x2, b), c, false);
}

// FP16 (q - z) pairs of one code dword: (e0,e1), (e2,e3), (e4,e5), (e6,e7).
// 0x6400 | n is the FP16 value 1024 + n; 0x6400 | (n << 4) is 1024 + 16 n.
struct Deq { f16x2 w01, w23, w45, w67; };
__device__ __forceinline__ Deq dequant_dword(uint32_t v, f16x2 zc1, f16x2 zc2) {
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  Deq d;
  d.w01 = as_f16x2((v & 0x000F000Fu) | 0x64006400u) + zc1;              // n - z
  d.w23 = as_f16x2((v & 0x00F000F0u) | 0x64006400u) * sixteenth + zc2;  // (1024 + 16 n)/16 - 64 - z
  const uint32_t v8 = v >> 8;
  d.w45 = as_f16x2((v8 & 0x000F000Fu) | 0x64006400u) + zc1;
  d.w67 = as_f16x2((v8 & 0x00F000F0u) | 0x64006400u) * sixteenth + zc2;
  return d;
}

__device__ __forceinline__ void zero_consts(uint32_t szw, f16x2& zc1, f16x2& zc2, float& sf) {
  const _Float16 z = __builtin_bit_cast(_Float16, (uint16_t)(szw >> 16));
  const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)(szw & 0xFFFFu));
  const _Float16 a = (_Float16)-1024.0f - z;   // exact: integers up to 1039
  const _Float16 b = (_Float16)-64.0f - z;
  zc1 = f16x2{a, a};
  zc2 = f16x2{b, b};
  sf = (float)s;
}

// x halves for the kept elements of one 2:4 quad (groups 2qq, 2qq+1 of the
// chunk; one 16-byte plane block X covering its 8 columns).
__device__ __forceinline__ void xsel_2of4(const u32x4 X, uint32_t M, uint32_t& xab, uint32_t& xcd) {
  const uint32_t lo = perm_b32(X.y, X.x, M);
  const uint32_t hi = perm_b32(X.w, X.z, M);
  xab = perm_b32(hi, lo, 0x05010400u);
  xcd = perm_b32(hi, lo, 0x07030602u);
}

// x halves for one 1:4 quad (4 groups, 16 columns, plane blocks X and Y).
__device__ __forceinline__ void xsel_1of4(const u32x4 X, const u32x4 Y, uint32_t M, uint32_t& xab, uint32_t& xcd) {
  const uint32_t lo = perm_b32(X.y, X.x, M);
  const uint32_t hi = perm_b32(X.w, X.z, M);
  xab = perm_b32(hi, lo, 0x05010400u);
  const uint32_t lo2 = perm_b32(Y.y, Y.x, M);
  const uint32_t hi2 = perm_b32(Y.w, Y.z, M);
  xcd = perm_b32(hi2, lo2, 0x07030602u);
}

template <int NK>
__device__ __forceinline__ uint32_t quad_selector(const u32x2 o, int qq) {
  const uint32_t w = (qq < 4) ? o.x : o.y;
  const uint32_t m = (w >> (2 * (qq & 3))) & 0x03030303u;
  return NK == 2 ? (m | 0x04040000u) : (m | 0x04000400u);
}

// One chunk (32 kept elements) of one row against B activation vectors.
template <int NK, int G, int BMAX, int SPC>
__device__ __forceinline__ void chunk_compute(const u32x4 v, const u32x2 o, const uint32_t (&s)[SPC],
                                              const u32x4* __restrict__ xc, int ldsb, int B, float (&tot)[BMAX]) {
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
      const Deq d = dequant_dword(v[qq >> 1], zc1, zc2);
      const uint32_t MA = quad_selector<NK>(o, qq);
      const uint32_t MB = quad_selector<NK>(o, qq + 1);
#pragma unroll
      for (int b = 0; b < BMAX; ++b) {
        if (b < B) {
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
    for (int b = 0; b < BMAX; ++b) tot[b] += sf * acc[b];
  }
}

// Stage x columns [col0, col0 + ncols) of every batch vector into LDS planes.
template <int NK>
__device__ __forceinline__ void stage_x(const KParams& p, u32x4* xs, int col0, int ncols, int ldsb) {
  constexpr int CPC = 128 / NK, BPC = CPC / 8, LSTRIDE = BPC + 1;
  const int nblk = ncols >> 3;
  const int kb = p.K >> 3;
  for (int m = threadIdx.x; m < p.B * nblk; m += blockDim.x) {
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

template <int NK, int G, int BMAX, int MAXCH>
__device__ __forceinline__ void tile_body(const KParams& p, u32x4* xs, int row0, int nr, int sz_base) {
  constexpr int CPC = 128 / NK;
  constexpr int LSTRIDE = CPC / 8 + 1;
  constexpr int SPC = (G >= CPC) ? 1 : CPC / G;    // scale words per chunk
  constexpr int SHARE = (G > CPC) ? G / CPC : 1;   // chunks per scale word
  const int t = threadIdx.x;
  const int tpr_log2 = p.tpr_log2, TPR = 1 << tpr_log2;
  const int r = t >> tpr_log2, kl = t & (TPR - 1);
  const bool active = r < nr;
  const int C = p.C;
  const int I = (C + TPR - 1) >> tpr_log2;
  const int rem = C - (I - 1) * TPR;
  const int nch = active ? (kl < rem ? I : I - 1) : 0;
  const int64_t slot0 = (int64_t)row0 * C;

  u32x4 v[MAXCH];
  u32x2 o[MAXCH];
  uint32_t s[MAXCH][SPC];
#pragma unroll
  for (int i = 0; i < MAXCH; ++i) {
    if (i < nch) {
      const int cnt = (i == I - 1) ? rem : TPR;
      const int s_rel = i * nr * TPR + r * cnt + kl;
      v[i] = __builtin_nontemporal_load(p.vals + slot0 + s_rel);
      o[i] = __builtin_nontemporal_load(p.offs + slot0 + s_rel);
      const uint32_t* sp = p.sz + sz_base + (SPC > 1 ? s_rel * SPC : s_rel / SHARE);
      if constexpr (SPC == 4) {
        const u32x4 w = __builtin_nontemporal_load((const u32x4*)sp);
        s[i][0] = w.x; s[i][1] = w.y; s[i][2] = w.z; s[i][3] = w.w;
      } else if constexpr (SPC == 2) {
        const u32x2 w = __builtin_nontemporal_load((const u32x2*)sp);
        s[i][0] = w.x; s[i][1] = w.y;
      } else {
        s[i][0] = __builtin_nontemporal_load(sp);
      }
    }
  }

  const int PI = p.phase_iters;
  const int ldsb = PI * TPR * LSTRIDE;             // LDS blocks per batch vector
  const int phase_cols = PI * TPR * CPC;
  stage_x<NK>(p, xs, 0, phase_cols, ldsb);
  __syncthreads();

  float tot[BMAX];
#pragma unroll
  for (int b = 0; b < BMAX; ++b) tot[b] = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXCH; ++i) {
    const int ip = i % PI;
    if (i > 0 && ip == 0 && i < I) {   // uniform across the workgroup
      __syncthreads();
      stage_x<NK>(p, xs, (i / PI) * phase_cols, phase_cols, ldsb);
      __syncthreads();
    }
    if (i < nch) {
      const u32x4* xc = xs + (ip * TPR + kl) * LSTRIDE;
      chunk_compute<NK, G, BMAX, SPC>(v[i], o[i], s[i], xc, ldsb, p.B, tot);
    }
  }

  const int yrow = active ? p.perm[row0 + r] : 0;
#pragma unroll
  for (int b = 0; b < BMAX; ++b) {
    if (b < p.B) {
      float a = tot[b];
      for (int m = TPR >> 1; m >= 1; m >>= 1) a += __shfl_xor(a, m, 64);
      if (active && kl == 0) p.y[(int64_t)b * p.N + yrow] = __builtin_bit_cast(uint16_t, (_Float16)a);
    }
  }
}

template <int NK, int BMAX, int MAXCH>
__global__ __launch_bounds__(256) void sgemv_kernel(KParams p) {
  extern __shared__ u32x4 xs[];
  const int* te = p.tiles + 4 * blockIdx.x;
  const int row0 = te[0], nr = te[1], g = te[2], sz_base = te[3];
  switch (g) {
    case 32: tile_body<NK, 32, BMAX, MAXCH>(p, xs, row0, nr, sz_base); break;
    case 64: tile_body<NK, 64, BMAX, MAXCH>(p, xs, row0, nr, sz_base); break;
    case 128: tile_body<NK, 128, BMAX, MAXCH>(p, xs, row0, nr, sz_base); break;
    default: tile_body<NK, 256, BMAX, MAXCH>(p, xs, row0, nr, sz_base); break;
  }
}

typedef void (*KernelFn)(KParams);

template <int NK, int BMAX>
KernelFn pick_maxch(int I) {
  if (I <= 4) return sgemv_kernel<NK, BMAX, 4>;
  if (I <= 8) return sgemv_kernel<NK, BMAX, 8>;
  return sgemv_kernel<NK, BMAX, 16>;
}

template <int NK>
KernelFn pick(int B, int I) {
  if (B == 1) return pick_maxch<NK, 1>(I);
  if (B <= 4) return sgemv_kernel<NK, 4, 16>;
  if (B <= 8) return sgemv_kernel<NK, 8, 16>;
  return sgemv_kernel<NK, 16, 16>;
}

bool desc_consistent(const sgemv_desc* d) {
  using namespace sgemv;
  if (d->N < 1 || d->K < 256 || d->K % 256 || (d->nk != 1 && d->nk != 2)) return false;
  if (d->tpr < 4 || d->tpr > 64 || (d->tpr & (d->tpr - 1))) return false;
  const int wg = d->rt * d->tpr;
  if (d->rt < 1 || (wg != 64 && wg != 128 && wg != 256)) return false;
  const int32_t C = d->K * d->nk / 128;
  if ((C + d->tpr - 1) / d->tpr > kMaxChunksPerThread) return false;
  if (d->n_tiles < 1 || d->n_tiles > d->N) return false;
  if (!valid_group(d->g_min, d->K) || !valid_group(d->g_max, d->K)) return false;
  if (d->kept != (int64_t)d->N * d->K * d->nk / 4) return false;
  if (d->n_groups < (int64_t)d->N * (d->K / d->g_max) || d->n_groups > (int64_t)d->N * (d->K / d->g_min)) return false;
  if (d->off_tiles != 0 || d->off_perm != align_up(16 * (int64_t)d->n_tiles)) return false;
  if (d->off_vals != align_up(d->off_perm + 4 * (int64_t)d->N)) return false;
  if (d->off_offs != align_up(d->off_vals + 16 * (int64_t)d->N * C)) return false;
  if (d->off_sz != align_up(d->off_offs + 8 * (int64_t)d->N * C)) return false;
  if (d->blob_bytes != align_up(d->off_sz + 4 * d->n_groups)) return false;
  return true;
}

}  // namespace

extern "C" int sgemv_run(const sgemv_desc* d, const void* blob_dev, const void* x_dev, void* y_dev,
                         int32_t B, void* hip_stream) {
  using namespace sgemv;
  if (!d || !blob_dev || !x_dev || !y_dev) return SGEMV_EINVAL;
  if (B < 1 || B > 16) return SGEMV_EINVAL;
  if (!desc_consistent(d)) return SGEMV_ESIZE;
  if (((uintptr_t)blob_dev % 256) || ((uintptr_t)x_dev % 16) || ((uintptr_t)y_dev % 2)) return SGEMV_EALIGN;
  const int cpc = cols_per_chunk(d->nk);
  const int32_t C = d->K * d->nk / 128;
  const int32_t I = (C + d->tpr - 1) / d->tpr;
  const int64_t per_iter = (int64_t)B * d->tpr * (cpc / 8 + 1) * 16;   // LDS bytes per staged iteration
  int32_t pi = I;
  while (pi > 1 && per_iter * pi > 65536) --pi;
  const int64_t lds = per_iter * pi;
  if (lds > 160 * 1024) return SGEMV_ESIZE;
  const uint8_t* blob = (const uint8_t*)blob_dev;
  KParams p;
  p.tiles = (const int32_t*)(blob + d->off_tiles);
  p.perm = (const int32_t*)(blob + d->off_perm);
  p.vals = (const u32x4*)(blob + d->off_vals);
  p.offs = (const u32x2*)(blob + d->off_offs);
  p.sz = (const uint32_t*)(blob + d->off_sz);
  p.x = (const u32x4*)x_dev;
  p.y = (uint16_t*)y_dev;
  p.N = d->N; p.K = d->K; p.C = C; p.B = B;
  p.tpr_log2 = ilog2(d->tpr);
  p.phase_iters = pi;
  KernelFn fn = d->nk == 2 ? pick<2>(B, I) : pick<1>(B, I);
  if (lds > 65536) {
    if (hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return SGEMV_EHIP;
  }
  hipStream_t stream = (hipStream_t)hip_stream;
  hipLaunchKernelGGL(fn, dim3(d->n_tiles), dim3(d->rt * d->tpr), (uint32_t)lds, stream, p);
  if (hipGetLastError() != hipSuccess) return SGEMV_EHIP;
  return SGEMV_OK;
}

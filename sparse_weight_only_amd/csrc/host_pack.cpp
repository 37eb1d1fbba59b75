// Host packer: N:M pruning, adaptive group choice, asymmetric INT4 group
// quantisation and the canonical 2bit-CSR arrays.
//
// Follows the page "Efficient large-model ad applications through model
// compression and parallel verification" (English gloss of its Chinese title;
// a translation of arXiv 2605.11582): §3.2
// "Sparsification" (layer-wise N:M, 2:4 or 1:4; the activation-aware
// importance of eq. (3), first term, in sgemv_prune), §3.2 "Adaptive group
// quantization" (finer groups for sensitive channels; sensitivity from the
// first term of eq. (3)), §1 "our core idea" (FP16 -> INT4 weight-only) and
// the first contribution item (index-compressed 2bit-CSR; sgemv_pack_fp16
// keeps the kept values in FP16, the form before INT4). Build with
// -ffp-contract=off: every FP64 operation is rounded on its own.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "internal.hpp"

using namespace sgemv;

namespace {

bool shape_ok(int32_t N, int32_t K, int32_t nk) {
  if (N < 1 || K < 256 || K % 256 != 0 || !valid_nk(nk)) return false;
  return (int64_t)N * K * nk / 4 < ((int64_t)1 << 31);
}

// Kept offsets of one group of 4 (ascending): the nk largest |w|, lower
// column first among equal magnitudes (-0 equals +0).
inline void select_kept(const uint16_t* g4, int nk, int* out) {
  if (nk == 4) {                  // dense ablation: every element
    for (int p = 0; p < 4; ++p) out[p] = p;
    return;
  }
  uint16_t mag[4];
  for (int p = 0; p < 4; ++p) mag[p] = (uint16_t)(g4[p] & 0x7FFFu);   // finite: ordered like |w|
  int first = 0;
  for (int p = 1; p < 4; ++p)
    if (mag[p] > mag[first]) first = p;
  if (nk == 1) { out[0] = first; return; }
  int second = -1;
  for (int p = 0; p < 4; ++p) {
    if (p == first) continue;
    if (second < 0 || mag[p] > mag[second]) second = p;
  }
  out[0] = std::min(first, second);
  out[1] = std::max(first, second);
}

bool all_finite(const uint16_t* a, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!f16_finite(a[i])) return false;
  return true;
}

int64_t fine_count(int32_t N, double frac) {
  int64_t num = (int64_t)nearbyint(frac * 1000000.0);   // half to even, like Python's round
  return ((int64_t)N * num + 999999) / 1000000;
}

// Quantise m kept values (FP16 bits, ascending column) of one group.
void quantize_group(const uint16_t* v16, int m, uint16_t* scale16, uint16_t* zero16, uint8_t* q) {
  double vmin = 0, vmax = 0;
  for (int i = 0; i < m; ++i) {
    double v = f16_to_f64(v16[i]);
    if (i == 0 || v < vmin) vmin = v;
    if (i == 0 || v > vmax) vmax = v;
  }
  double lo = vmin < 0.0 ? vmin : 0.0;
  double hi = vmax > 0.0 ? vmax : 0.0;
  if (hi == lo) {
    *scale16 = 0x3C00;  // 1.0
    *zero16 = 0;
    for (int i = 0; i < m; ++i) q[i] = 0;
    return;
  }
  double t = (hi - lo) / 15.0;
  uint16_t s16 = f64_to_f16(t);
  if (f16_to_f64(s16) < 5.9604644775390625e-08) s16 = 0x0001;   // 2^-24
  double s = f16_to_f64(s16);
  double z = nearbyint(-lo / s);
  if (z < 0.0) z = 0.0;
  if (z > 15.0) z = 15.0;
  z = z + 0.0;                                                      // never -0
  for (int i = 0; i < m; ++i) {
    double c = nearbyint(f16_to_f64(v16[i]) / s) + z;
    if (c < 0.0) c = 0.0;
    if (c > 15.0) c = 15.0;
    q[i] = (uint8_t)c;
  }
  *scale16 = s16;
  *zero16 = f64_to_f16(z);
}

// Column scales c_k = sqrt(sum_t xcal[t][k]^2), sequential over t in FP64.
std::vector<double> column_norms(const uint16_t* xcal, int32_t T, int32_t K) {
  std::vector<double> c(K, 0.0);
  for (int32_t k = 0; k < K; ++k) {
    double s = 0.0;
    for (int32_t t = 0; t < T; ++t) {
      double x = f16_to_f64(xcal[(int64_t)t * K + k]);
      s = s + x * x;
    }
    c[k] = sqrt(s);
  }
  return c;
}

}  // namespace

extern "C" int sgemv_prune(const uint16_t* w, int32_t N, int32_t K, int32_t nk,
                           const uint16_t* xcal, int32_t T, uint16_t* w_out) {
  if (!w || !w_out || !shape_ok(N, K, nk) || nk == 4) return SGEMV_EINVAL;
  if (xcal && T < 1) return SGEMV_EINVAL;
  if (!all_finite(w, (int64_t)N * K)) return SGEMV_EINVAL;
  if (xcal && !all_finite(xcal, (int64_t)T * K)) return SGEMV_EINVAL;
  const std::vector<double> c = xcal ? column_norms(xcal, T, K) : std::vector<double>(K, 1.0);
  for (int32_t n = 0; n < N; ++n) {
    const uint16_t* row = w + (int64_t)n * K;
    uint16_t* out = w_out + (int64_t)n * K;
    for (int32_t j = 0; j < K / 4; ++j) {
      double sc[4];
      for (int p = 0; p < 4; ++p) sc[p] = fabs(f16_to_f64(row[4 * j + p])) * c[4 * j + p];
      // the nk largest scores; a later column replaces an earlier one only
      // when strictly larger, so ties go to the lower column
      int first = 0;
      for (int p = 1; p < 4; ++p)
        if (sc[p] > sc[first]) first = p;
      int second = -1;
      if (nk == 2)
        for (int p = 0; p < 4; ++p) {
          if (p == first) continue;
          if (second < 0 || sc[p] > sc[second]) second = p;
        }
      for (int p = 0; p < 4; ++p) out[4 * j + p] = (p == first || p == second) ? row[4 * j + p] : (uint16_t)0;
    }
  }
  return SGEMV_OK;
}

extern "C" int sgemv_select_groups(const uint16_t* w, int32_t N, int32_t K, int32_t nk,
                                   const uint16_t* xcal, int32_t T, double frac_fine,
                                   int32_t g_fine, int32_t g_coarse, int32_t* group_size_out) {
  if (!w || !xcal || !group_size_out || !shape_ok(N, K, nk) || T < 1) return SGEMV_EINVAL;
  if (!(frac_fine >= 0.0 && frac_fine <= 1.0)) return SGEMV_EINVAL;
  if (!valid_group(g_fine, K) || !valid_group(g_coarse, K)) return SGEMV_EINVAL;
  if (!all_finite(w, (int64_t)N * K) || !all_finite(xcal, (int64_t)T * K)) return SGEMV_EINVAL;
  const std::vector<double> c = column_norms(xcal, T, K);
  std::vector<double> S(N, 0.0);
  for (int32_t n = 0; n < N; ++n) {
    const uint16_t* row = w + (int64_t)n * K;
    double s = 0.0;
    for (int32_t j = 0; j < K / 4; ++j) {
      int kept[4];
      select_kept(row + 4 * j, nk, kept);
      // columns in ascending order; pruned columns add +0 and are skipped
      for (int i = 0; i < nk; ++i) {
        int k = 4 * j + kept[i];
        s = s + fabs(f16_to_f64(row[k])) * c[k];
      }
    }
    S[n] = s;
  }
  std::vector<int32_t> order(N);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return S[a] > S[b]; });
  int64_t cnt = fine_count(N, frac_fine);
  for (int32_t n = 0; n < N; ++n) group_size_out[n] = g_coarse;
  for (int64_t i = 0; i < cnt && i < N; ++i) group_size_out[order[i]] = g_fine;
  return SGEMV_OK;
}

extern "C" int sgemv_pack(const uint16_t* w, int32_t N, int32_t K, int32_t nk,
                          const int32_t* group_size, uint8_t* vals, uint8_t* offs,
                          uint16_t* scale, uint16_t* zero, int32_t* gptr, int32_t* rowptr) {
  if (!w || !group_size || !vals || (!offs && nk != 4) || !scale || !zero || !gptr || !rowptr) return SGEMV_EINVAL;
  if (!shape_ok(N, K, nk)) return SGEMV_EINVAL;
  for (int32_t n = 0; n < N; ++n)
    if (!valid_group(group_size[n], K)) return SGEMV_EINVAL;
  if (!all_finite(w, (int64_t)N * K)) return SGEMV_EINVAL;
  const int kpr = K * nk / 4;
  std::vector<uint16_t> kv(kpr);
  std::vector<uint8_t> ko(kpr), q(kpr);
  int64_t gbase = 0;
  for (int32_t n = 0; n < N; ++n) {
    const uint16_t* row = w + (int64_t)n * K;
    for (int32_t j = 0; j < K / 4; ++j) {
      int kept[4];
      select_kept(row + 4 * j, nk, kept);
      for (int i = 0; i < nk; ++i) {
        kv[j * nk + i] = row[4 * j + kept[i]];
        ko[j * nk + i] = (uint8_t)kept[i];
      }
    }
    const int g = group_size[n];
    const int m = g * nk / 4;                 // kept values per group
    gptr[n] = (int32_t)gbase;
    for (int32_t gi = 0; gi < K / g; ++gi)
      quantize_group(&kv[gi * m], m, &scale[gbase + gi], &zero[gbase + gi], &q[gi * m]);
    gbase += K / g;
    uint8_t* vrow = vals + (int64_t)n * (kpr / 2);
    for (int j = 0; j < kpr / 2; ++j) vrow[j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
    if (nk == 4) {                            // dense: no offsets
      rowptr[n] = (int32_t)((int64_t)n * kpr);
      continue;
    }
    uint8_t* orow = offs + (int64_t)n * (kpr / 4);
    for (int j = 0; j < kpr / 4; ++j)
      orow[j] = (uint8_t)(ko[4 * j] | (ko[4 * j + 1] << 2) | (ko[4 * j + 2] << 4) | (ko[4 * j + 3] << 6));
    rowptr[n] = (int32_t)((int64_t)n * kpr);
  }
  gptr[N] = (int32_t)gbase;
  rowptr[N] = (int32_t)((int64_t)N * kpr);
  return SGEMV_OK;
}

extern "C" int sgemv_pack_fp16(const uint16_t* w, int32_t N, int32_t K, int32_t nk,
                               uint16_t* vals16, uint8_t* offs, int32_t* rowptr) {
  if (!w || !vals16 || !offs || !rowptr || !shape_ok(N, K, nk) || nk == 4) return SGEMV_EINVAL;
  if (!all_finite(w, (int64_t)N * K)) return SGEMV_EINVAL;
  const int kpr = K * nk / 4;
  std::vector<uint8_t> ko(kpr);
  for (int32_t n = 0; n < N; ++n) {
    const uint16_t* row = w + (int64_t)n * K;
    uint16_t* vrow = vals16 + (int64_t)n * kpr;
    for (int32_t j = 0; j < K / 4; ++j) {
      int kept[4];
      select_kept(row + 4 * j, nk, kept);
      for (int i = 0; i < nk; ++i) {
        vrow[j * nk + i] = row[4 * j + kept[i]];
        ko[j * nk + i] = (uint8_t)kept[i];
      }
    }
    uint8_t* orow = offs + (int64_t)n * (kpr / 4);
    for (int j = 0; j < kpr / 4; ++j)
      orow[j] = (uint8_t)(ko[4 * j] | (ko[4 * j + 1] << 2) | (ko[4 * j + 2] << 4) | (ko[4 * j + 3] << 6));
    rowptr[n] = (int32_t)((int64_t)n * kpr);
  }
  rowptr[N] = (int32_t)((int64_t)N * kpr);
  return SGEMV_OK;
}

extern "C" const char* sgemv_strerror(int code) {
  switch (code) {
    case SGEMV_OK: return "ok";
    case SGEMV_EINVAL: return "invalid argument (shape, N:M choice, group size, batch, null pointer or non-finite value)";
    case SGEMV_ESIZE: return "inconsistent descriptor or size beyond the kernels' limits";
    case SGEMV_EALIGN: return "device pointer not aligned as required";
    case SGEMV_EHIP: return "HIP runtime error at launch";
    default: return "unknown status code";
  }
}

extern "C" int sgemv_f64_to_f16(const double* in, uint16_t* out, int64_t n) {
  if (n < 0 || (n > 0 && (!in || !out))) return SGEMV_EINVAL;
  for (int64_t i = 0; i < n; ++i) out[i] = f64_to_f16(in[i]);
  return SGEMV_OK;
}

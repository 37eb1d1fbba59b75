// Kernel selection shared by the instantiation units and the launcher.
#pragma once

namespace sgemv_dev {

struct KParams;
typedef void (*KernelFn)(KParams);

// Chunks per lane are rounded up to a compiled bucket (1, 2, 4 or 8); the
// bucket's workgroup limit is wg_limit() of internal.hpp.
inline int maxch_bucket(int ch) { return ch <= 1 ? 1 : ch <= 2 ? 2 : ch <= 4 ? 4 : 8; }
constexpr int kBatchedThreads = 256;  // workgroup size of the beam-batch kernels

// x blocks (16 bytes) each lane of a batch-1 workgroup stages: 1, 2, 4 or 8.
inline int xmax_bucket(int per_lane) { return per_lane <= 1 ? 1 : per_lane <= 2 ? 2 : per_lane <= 4 ? 4 : 8; }

KernelFn get_b1_nk1_c1(int xmax);
KernelFn get_b1_nk1_c2(int xmax);
KernelFn get_b1_nk1_c4(int xmax);
KernelFn get_b1_nk1_c8(int xmax);
KernelFn get_b1_nk2_c1(int xmax);
KernelFn get_b1_nk2_c2(int xmax);
KernelFn get_b1_nk2_c4(int xmax);
KernelFn get_b1_nk2_c8(int xmax);

inline KernelFn get_b1(int nk, int maxch, int xmax) {
  if (nk == 2) {
    switch (maxch) {
      case 1: return get_b1_nk2_c1(xmax);
      case 2: return get_b1_nk2_c2(xmax);
      case 4: return get_b1_nk2_c4(xmax);
      default: return get_b1_nk2_c8(xmax);
    }
  }
  switch (maxch) {
    case 1: return get_b1_nk1_c1(xmax);
    case 2: return get_b1_nk1_c2(xmax);
    case 4: return get_b1_nk1_c4(xmax);
    default: return get_b1_nk1_c8(xmax);
  }
}
KernelFn get_bn(int nk);
constexpr int kBatchGroup = 4;        // batch vectors staged in LDS together

}  // namespace sgemv_dev

// Kernel selection shared by the instantiation units and the launcher.
#pragma once

namespace sgemv_dev {

struct KParams;
typedef void (*KernelFn)(KParams);

constexpr int kBatchedThreads = 256;  // workgroup size of the beam-batch kernels

KernelFn get_b1_nk1_r1(int imax, int xmax);
KernelFn get_b1_nk1_r2(int imax, int xmax);
KernelFn get_b1_nk1_r4(int imax, int xmax);
KernelFn get_b1_nk2_r1(int imax, int xmax);
KernelFn get_b1_nk2_r2(int imax, int xmax);
KernelFn get_b1_nk2_r4(int imax, int xmax);

// Batch-1 kernel for rows-per-lane rpl, chunk bucket imax and x blocks per lane xmax (2 or 8).
inline KernelFn get_b1(int nk, int rpl, int imax, int xmax) {
  if (nk == 2) return rpl == 1 ? get_b1_nk2_r1(imax, xmax) : rpl == 2 ? get_b1_nk2_r2(imax, xmax) : get_b1_nk2_r4(imax, xmax);
  return rpl == 1 ? get_b1_nk1_r1(imax, xmax) : rpl == 2 ? get_b1_nk1_r2(imax, xmax) : get_b1_nk1_r4(imax, xmax);
}
KernelFn get_bn(int nk);
constexpr int kBatchGroup = 4;        // batch vectors staged in LDS together

}  // namespace sgemv_dev

// Kernel selection shared by the instantiation units and the launcher.
#pragma once
#include <stdint.h>

namespace sgemv_dev {

struct KParams;
struct GParams;
typedef void (*KernelFn)(KParams);
// Single-layer kernels: 14 leading scalar argument dwords (preloaded into
// registers at wave launch), then the parameter block.
typedef void (*LeadFn)(const uint8_t*, const uint16_t*, uint32_t, uint32_t, uint32_t, uint32_t, int32_t, uint32_t,
                       int32_t, int32_t, int32_t, int32_t, KParams);
typedef void (*GroupFn)(GParams);

// Kernel for nk kept per 4, up to imax chunks per wave and xmax 16-byte x
// loads per lane and phase (each in {1, 2, 4, 8}); nullptr otherwise.
LeadFn get_kernel_nk1(int imax, int xmax);
LeadFn get_kernel_nk2(int imax, int xmax);
LeadFn get_kernel_nk4(int imax, int xmax);
inline LeadFn get_kernel(int nk, int imax, int xmax) {
  return nk == 2 ? get_kernel_nk2(imax, xmax) : nk == 1 ? get_kernel_nk1(imax, xmax)
       : nk == 4 ? get_kernel_nk4(imax, xmax) : nullptr;
}
// The same for the several-layer launch.
GroupFn get_group_kernel_nk1(int imax, int xmax);
GroupFn get_group_kernel_nk2(int imax, int xmax);
GroupFn get_group_kernel_nk4(int imax, int xmax);
inline GroupFn get_group_kernel(int nk, int imax, int xmax) {
  return nk == 2 ? get_group_kernel_nk2(imax, xmax) : nk == 1 ? get_group_kernel_nk1(imax, xmax)
       : nk == 4 ? get_group_kernel_nk4(imax, xmax) : nullptr;
}

// Kernels for exactly one vector (INT4 form, nk 1 or 2; xmax 1, 2 or 4):
// the fields needed first as leading scalar arguments (preloaded into
// registers), then the parameter block.
typedef LeadFn B1Fn;
B1Fn get_b1_kernel_nk1(int imax, int xmax);
B1Fn get_b1_kernel_nk2(int imax, int xmax);
GroupFn get_b1_group_kernel_nk1(int imax, int xmax);
GroupFn get_b1_group_kernel_nk2(int imax, int xmax);
inline B1Fn get_b1_kernel(int nk, int imax, int xmax) {
  return nk == 2 ? get_b1_kernel_nk2(imax, xmax) : nk == 1 ? get_b1_kernel_nk1(imax, xmax) : nullptr;
}
inline GroupFn get_b1_group_kernel(int nk, int imax, int xmax) {
  return nk == 2 ? get_b1_group_kernel_nk2(imax, xmax) : nk == 1 ? get_b1_group_kernel_nk1(imax, xmax) : nullptr;
}

// Several vectors, rb row blocks per workgroup (INT4 form, nk 1 or 2; rb 4,
// imax 2, xmax 8).
KernelFn get_rb_kernel(int nk, int imax, int xmax, int rb);

// The FP16-valued form (nk 1 or 2).
LeadFn get_f16_kernel(int nk, int imax, int xmax);
GroupFn get_f16_group_kernel(int nk, int imax, int xmax);

}  // namespace sgemv_dev

// Instantiations of the SparseGemv kernel for the FP16-valued form (2:4 and
// 1:4, the kept values stored as FP16: no groups, no scale or zero).
#include "kernels.hpp"
#include "sgemv_device.hpp"

namespace sgemv_dev {

namespace {
template <int NK, int IMAX>
LeadFn by_xmax(int xmax) {
  switch (xmax) {
    case 1: return sgemv_f16_kernel<NK, IMAX, 1>;
    case 2: return sgemv_f16_kernel<NK, IMAX, 2>;
    case 4: return sgemv_f16_kernel<NK, IMAX, 4>;
    case 8: return sgemv_f16_kernel<NK, IMAX, 8>;
    default: return nullptr;
  }
}
template <int NK, int IMAX>
GroupFn group_by_xmax(int xmax) {
  switch (xmax) {
    case 1: return sgemv_f16_group_kernel<NK, IMAX, 1>;
    case 2: return sgemv_f16_group_kernel<NK, IMAX, 2>;
    case 4: return sgemv_f16_group_kernel<NK, IMAX, 4>;
    case 8: return sgemv_f16_group_kernel<NK, IMAX, 8>;
    default: return nullptr;
  }
}
template <int NK>
LeadFn by_imax(int imax, int xmax) {
  switch (imax) {
    case 1: return by_xmax<NK, 1>(xmax);
    case 2: return by_xmax<NK, 2>(xmax);
    case 4: return by_xmax<NK, 4>(xmax);
    case 8: return by_xmax<NK, 8>(xmax);
    default: return nullptr;
  }
}
template <int NK>
GroupFn group_by_imax(int imax, int xmax) {
  switch (imax) {
    case 1: return group_by_xmax<NK, 1>(xmax);
    case 2: return group_by_xmax<NK, 2>(xmax);
    case 4: return group_by_xmax<NK, 4>(xmax);
    case 8: return group_by_xmax<NK, 8>(xmax);
    default: return nullptr;
  }
}
}  // namespace

LeadFn get_f16_kernel(int nk, int imax, int xmax) {
  return nk == 2 ? by_imax<2>(imax, xmax) : nk == 1 ? by_imax<1>(imax, xmax) : nullptr;
}

GroupFn get_f16_group_kernel(int nk, int imax, int xmax) {
  return nk == 2 ? group_by_imax<2>(imax, xmax) : nk == 1 ? group_by_imax<1>(imax, xmax) : nullptr;
}

}  // namespace sgemv_dev

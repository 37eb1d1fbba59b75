// Instantiations of the SparseGemv kernel for 2:4 sparsity.
#include "kernels.hpp"
#include "sgemv_device.hpp"

namespace sgemv_dev {

namespace {
template <int IMAX>
LeadFn by_xmax(int xmax) {
  switch (xmax) {
    case 1: return sgemv_kernel<2, IMAX, 1>;
    case 2: return sgemv_kernel<2, IMAX, 2>;
    case 4: return sgemv_kernel<2, IMAX, 4>;
    case 8: return sgemv_kernel<2, IMAX, 8>;
    default: return nullptr;
  }
}
template <int IMAX>
GroupFn group_by_xmax(int xmax) {
  switch (xmax) {
    case 1: return sgemv_group_kernel<2, IMAX, 1>;
    case 2: return sgemv_group_kernel<2, IMAX, 2>;
    case 4: return sgemv_group_kernel<2, IMAX, 4>;
    case 8: return sgemv_group_kernel<2, IMAX, 8>;
    default: return nullptr;
  }
}
template <int IMAX>
B1Fn b1_by_xmax(int xmax) {
  switch (xmax) {
    case 1: return sgemv_b1_kernel<2, IMAX, 1>;
    case 2: return sgemv_b1_kernel<2, IMAX, 2>;
    case 4: return sgemv_b1_kernel<2, IMAX, 4>;
    default: return nullptr;
  }
}
template <int IMAX>
GroupFn b1_group_by_xmax(int xmax) {
  switch (xmax) {
    case 1: return sgemv_b1_group_kernel<2, IMAX, 1>;
    case 2: return sgemv_b1_group_kernel<2, IMAX, 2>;
    case 4: return sgemv_b1_group_kernel<2, IMAX, 4>;
    default: return nullptr;
  }
}
}  // namespace

B1Fn get_b1_kernel_nk2(int imax, int xmax) {
  switch (imax) {
    case 1: return b1_by_xmax<1>(xmax);
    case 2: return b1_by_xmax<2>(xmax);
    case 4: return b1_by_xmax<4>(xmax);
    case 8: return b1_by_xmax<8>(xmax);
    default: return nullptr;
  }
}

GroupFn get_b1_group_kernel_nk2(int imax, int xmax) {
  switch (imax) {
    case 1: return b1_group_by_xmax<1>(xmax);
    case 2: return b1_group_by_xmax<2>(xmax);
    case 4: return b1_group_by_xmax<4>(xmax);
    case 8: return b1_group_by_xmax<8>(xmax);
    default: return nullptr;
  }
}

LeadFn get_kernel_nk2(int imax, int xmax) {
  switch (imax) {
    case 1: return by_xmax<1>(xmax);
    case 2: return by_xmax<2>(xmax);
    case 4: return by_xmax<4>(xmax);
    case 8: return by_xmax<8>(xmax);
    default: return nullptr;
  }
}

GroupFn get_group_kernel_nk2(int imax, int xmax) {
  switch (imax) {
    case 1: return group_by_xmax<1>(xmax);
    case 2: return group_by_xmax<2>(xmax);
    case 4: return group_by_xmax<4>(xmax);
    case 8: return group_by_xmax<8>(xmax);
    default: return nullptr;
  }
}

}  // namespace sgemv_dev

// Instantiations of the SparseGemv kernel for the dense INT4 ablation (every
// element kept, no offsets).
#include "kernels.hpp"
#include "sgemv_device.hpp"

namespace sgemv_dev {

namespace {
template <int IMAX>
LeadFn by_xmax(int xmax) {
  switch (xmax) {
    case 1: return sgemv_kernel<4, IMAX, 1>;
    case 2: return sgemv_kernel<4, IMAX, 2>;
    case 4: return sgemv_kernel<4, IMAX, 4>;
    case 8: return sgemv_kernel<4, IMAX, 8>;
    default: return nullptr;
  }
}
template <int IMAX>
GroupFn group_by_xmax(int xmax) {
  switch (xmax) {
    case 1: return sgemv_group_kernel<4, IMAX, 1>;
    case 2: return sgemv_group_kernel<4, IMAX, 2>;
    case 4: return sgemv_group_kernel<4, IMAX, 4>;
    case 8: return sgemv_group_kernel<4, IMAX, 8>;
    default: return nullptr;
  }
}
}  // namespace

LeadFn get_kernel_nk4(int imax, int xmax) {
  switch (imax) {
    case 1: return by_xmax<1>(xmax);
    case 2: return by_xmax<2>(xmax);
    case 4: return by_xmax<4>(xmax);
    case 8: return by_xmax<8>(xmax);
    default: return nullptr;
  }
}

GroupFn get_group_kernel_nk4(int imax, int xmax) {
  switch (imax) {
    case 1: return group_by_xmax<1>(xmax);
    case 2: return group_by_xmax<2>(xmax);
    case 4: return group_by_xmax<4>(xmax);
    case 8: return group_by_xmax<8>(xmax);
    default: return nullptr;
  }
}

}  // namespace sgemv_dev

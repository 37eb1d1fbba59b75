// Batch-1 SparseGemv kernels, 2:4, 2 row(s) per lane (see sgemv_device.hpp).
#include "sgemv_device.hpp"
#include "kernels.hpp"

namespace sgemv_dev {

KernelFn get_b1_nk2_r2(int imax, int xmax) {
  switch (imax) {
    case 1: return xmax == 2 ? sgemv_b1_kernel<2, 2, 1, 2> : sgemv_b1_kernel<2, 2, 1, 8>;
    case 2: return xmax == 2 ? sgemv_b1_kernel<2, 2, 2, 2> : sgemv_b1_kernel<2, 2, 2, 8>;
    case 4: return xmax == 2 ? sgemv_b1_kernel<2, 2, 4, 2> : sgemv_b1_kernel<2, 2, 4, 8>;
    default: return nullptr;
  }
}

}  // namespace sgemv_dev

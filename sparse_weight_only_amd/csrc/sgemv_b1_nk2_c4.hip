// Batch-1 SparseGemv kernels, 2:4, up to 4 chunk(s) per lane (see sgemv_device.hpp).
#include "sgemv_device.hpp"
#include "kernels.hpp"

namespace sgemv_dev {

KernelFn get_b1_nk2_c4(int xmax) {
  switch (xmax) {
    case 1: return sgemv_b1_kernel<2, 4, 1, 512>;
    case 2: return sgemv_b1_kernel<2, 4, 2, 512>;
    case 4: return sgemv_b1_kernel<2, 4, 4, 512>;
    default: return sgemv_b1_kernel<2, 4, 8, 512>;
  }
}

}  // namespace sgemv_dev

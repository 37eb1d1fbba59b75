// Batch-1 SparseGemv kernels, 1:4, up to 8 chunk(s) per lane (see sgemv_device.hpp).
#include "sgemv_device.hpp"
#include "kernels.hpp"

namespace sgemv_dev {

KernelFn get_b1_nk1_c8(int xmax) {
  switch (xmax) {
    case 1: return sgemv_b1_kernel<1, 8, 1, 256>;
    case 2: return sgemv_b1_kernel<1, 8, 2, 256>;
    case 4: return sgemv_b1_kernel<1, 8, 4, 256>;
    default: return sgemv_b1_kernel<1, 8, 8, 256>;
  }
}

}  // namespace sgemv_dev

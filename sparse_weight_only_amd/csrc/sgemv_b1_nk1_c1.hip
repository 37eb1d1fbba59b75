// Batch-1 SparseGemv kernels, 1:4, up to 1 chunk(s) per lane (see sgemv_device.hpp).
#include "sgemv_device.hpp"
#include "kernels.hpp"

namespace sgemv_dev {

KernelFn get_b1_nk1_c1(int xmax) {
  switch (xmax) {
    case 1: return sgemv_b1_kernel<1, 1, 1, 1024>;
    case 2: return sgemv_b1_kernel<1, 1, 2, 1024>;
    case 4: return sgemv_b1_kernel<1, 1, 4, 1024>;
    default: return sgemv_b1_kernel<1, 1, 8, 1024>;
  }
}

}  // namespace sgemv_dev

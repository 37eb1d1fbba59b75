// Beam-batch (B = 2..16) SparseGemv kernel instantiations (see sgemv_device.hpp).
#include "sgemv_device.hpp"
#include "kernels.hpp"

namespace sgemv_dev {

KernelFn get_bn(int nk) { return nk == 2 ? sgemv_bn_kernel<2> : sgemv_bn_kernel<1>; }

}  // namespace sgemv_dev

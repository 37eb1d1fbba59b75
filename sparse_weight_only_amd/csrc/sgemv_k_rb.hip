// Instantiations of the SparseGemv kernel for several vectors with 4 row
// blocks per workgroup (INT4 form, 2:4 and 1:4): two chunks per wave and
// 8 x loads per lane and phase, the only geometry the launcher picks for it.
#include "kernels.hpp"
#include "sgemv_device.hpp"

namespace sgemv_dev {

KernelFn get_rb_kernel(int nk, int imax, int xmax, int rb) {
  if (rb != 4 || imax != 2 || xmax != 8) return nullptr;
  return nk == 2 ? sgemv_rb_kernel<2, 2, 8, 4> : nk == 1 ? sgemv_rb_kernel<1, 2, 8, 4> : nullptr;
}

}  // namespace sgemv_dev

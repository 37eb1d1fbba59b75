// Instantiations of the task-list kernel (one vector, INT4 form, 2:4 and 1:4
// tasks in one launch): up to imax column chunks per wave.
#include "sgemv_list_device.hpp"

namespace sgemv_dev {

ListFn get_list_kernel(int imax) {
  switch (imax) {
    case 1: return sgemv_list_kernel<1, 1>;
    case 2: return sgemv_list_kernel<2, 1>;
    case 3: return sgemv_list_kernel<3, 2>;
    case 4: return sgemv_list_kernel<4, 2>;
    case 6: return sgemv_list_kernel<6, 3>;
    case 8: return sgemv_list_kernel<8, 4>;
    default: return nullptr;
  }
}

}  // namespace sgemv_dev

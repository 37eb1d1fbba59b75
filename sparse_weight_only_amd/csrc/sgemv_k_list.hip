// The task-list kernel (one vector, INT4 form, 2:4 and 1:4 tasks in one launch).
#include "sgemv_list_device.hpp"

namespace sgemv_dev {

__global__ __launch_bounds__(64 * kListWaves) void sgemv_list_kernel(ListParams g) { list_block(g); }

ListFn get_list_kernel() { return sgemv_list_kernel; }

}  // namespace sgemv_dev

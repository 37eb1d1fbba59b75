// The task-list kernel (one vector, INT4 form, 2:4 and 1:4 tasks in one launch).
#include "sgemv_list_device.hpp"

namespace sgemv_dev {

__global__ __launch_bounds__(64 * kListWaves) void sgemv_list_kernel(ListParams g) { list_block(g); }

// the same body with the task table in device memory: grid (row width, rows)
__global__ __launch_bounds__(64 * kListWaves) void sgemv_list_table_kernel(const ListRow* __restrict__ rows) {
  const ListRow& R = rows[blockIdx.y];
  list_task(R.t, R.j0 + (int)blockIdx.x);
}

ListFn get_list_kernel() { return sgemv_list_kernel; }
ListTableFn get_list_table_kernel() { return sgemv_list_table_kernel; }

}  // namespace sgemv_dev

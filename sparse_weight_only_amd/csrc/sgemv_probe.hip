// Measurement probes: an empty kernel and a plain 16-byte-per-lane read, the
// practical ceiling of one launch against which sgemv_run is compared. They
// compute nothing of the method.
#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeLanes = 256;

__global__ void __launch_bounds__(1024) probe_empty_kernel() {}

// One 16-byte non-temporal buffer load per lane; offsets at or beyond
// `bytes` read zeros without touching memory (the last workgroup's tail).
__global__ void __launch_bounds__(kProbeLanes)
    probe_read_kernel(const uint8_t* src, uint32_t bytes, uint32_t* dst, uint32_t store_words, uint32_t magic) {
  const uint32_t gid = blockIdx.x * kProbeLanes + threadIdx.x;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), (short)0, (int)bytes, 0x00020000);
  const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, gid * 16u, 0, 2));
  const uint32_t f = v.x ^ v.y ^ v.z ^ v.w;
  if (gid < store_words) dst[gid] = f;
  else if (f == magic) dst[0] = f;
}

}  // namespace

extern "C" int sgemv_probe_read(const void* src_dev, int64_t bytes, void* dst_dev, int64_t store_bytes,
                                uint32_t magic, void* hip_stream) {
  if (!src_dev || !dst_dev) return SGEMV_EINVAL;
  if (bytes < 16 || bytes % 16 || bytes >= ((int64_t)1 << 31)) return SGEMV_EINVAL;
  if (store_bytes < 0 || store_bytes % 4 || store_bytes > bytes / 4) return SGEMV_EINVAL;
  if ((uintptr_t)src_dev % 256 || (uintptr_t)dst_dev % 4) return SGEMV_EALIGN;
  const uint32_t grid = (uint32_t)((bytes + 16 * kProbeLanes - 1) / (16 * kProbeLanes));
  (void)hipGetLastError();   // report only what this launch raises
  hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(kProbeLanes), 0, (hipStream_t)hip_stream,
                     (const uint8_t*)src_dev, (uint32_t)bytes, (uint32_t*)dst_dev, (uint32_t)(store_bytes / 4), magic);
  return hipGetLastError() == hipSuccess ? SGEMV_OK : SGEMV_EHIP;
}

extern "C" int sgemv_probe_empty(int32_t grid, int32_t block, void* hip_stream) {
  if (grid < 1 || block < 64 || block > 1024 || block % 64) return SGEMV_EINVAL;
  (void)hipGetLastError();
  hipLaunchKernelGGL(probe_empty_kernel, dim3((uint32_t)grid), dim3((uint32_t)block), 0, (hipStream_t)hip_stream);
  return hipGetLastError() == hipSuccess ? SGEMV_OK : SGEMV_EHIP;
}

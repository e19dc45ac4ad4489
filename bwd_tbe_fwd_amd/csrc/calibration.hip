// A plain streaming copy of known size, used to calibrate hardware traffic
// counters (bytes fetched / written beyond L2) against kernels of this library,
// which read and write 16 bytes per lane.
#include "tbe_device.h"
#include "tbe_internal.h"

namespace tbe {
namespace {

__global__ __launch_bounds__(kBlock) void calibration_copy_kernel(const f32x4* __restrict__ src,
                                                                  f32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

}  // namespace
}  // namespace tbe

using namespace tbe;

extern "C" tbe_status tbe_calibration_copy(const void* src, void* dst, int64_t bytes,
                                           tbe_stream_t stream) {
  if (!src || !dst || bytes < 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15) ||
      (reinterpret_cast<uintptr_t>(dst) & 15)) {
    set_error("calibration copy needs 16-byte aligned buffers and a multiple of 16 bytes");
    return TBE_ERR_ARG;
  }
  if (bytes == 0) return TBE_OK;
  const int64_t n16 = bytes / 16;
  const int grid = static_cast<int>(hmax(1, hmin((n16 + kBlock - 1) / kBlock, static_cast<int64_t>(device_cu_count()) * 8)));
  hipLaunchKernelGGL(calibration_copy_kernel, dim3(grid), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                     static_cast<const f32x4*>(src), static_cast<f32x4*>(dst), n16);
  return check_launch("calibration_copy");
}

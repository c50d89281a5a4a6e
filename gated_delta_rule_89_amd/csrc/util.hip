// Small device utilities used by the C ABI.
#include "dev_common.h"
#include "kda_internal.h"

namespace kda {

// dst[i] = src ? src[i] : 0 for i < n.  A kernel rather than a memset node so
// that a captured graph replays it faithfully.
__global__ void copy_or_zero_kernel(float* __restrict__ dst, const float* __restrict__ src, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t stream) {
    if (n <= 0 || dst == src) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                       dst, src, n);
    return hipGetLastError();
}

}  // namespace kda

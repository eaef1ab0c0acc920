// gdr_calib.hip -- a plain device copy (16-byte loads and stores, grid-stride),
// built into its own small library.  It is not part of the gdr C ABI: the
// benchmark runs it under the same hardware counters as the gated delta rule
// kernels to turn counter readings into bytes.
#include <hip/hip_runtime.h>
#include <stddef.h>

__global__ void gdr_calib_copy_kernel(const float4* __restrict__ src, float4* __restrict__ dst,
                                      size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

// Copies `bytes` (a multiple of 16) from src to dst on `stream`; 0 on success.
extern "C" int gdr_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    if (!src || !dst || bytes % 16) return 1;
    hipLaunchKernelGGL(gdr_calib_copy_kernel, dim3(8192), dim3(256), 0, stream,
                       (const float4*)src, (float4*)dst, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

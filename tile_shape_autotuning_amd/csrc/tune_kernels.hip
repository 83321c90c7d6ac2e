// Fill kernel for the autotuner's scratch operands: uniform values in
// [-1, 1) from a counter-based hash of (seed, index), stored as fp32 or bf16.
// Timing on non-trivial values matters: matrix-core power (and so clock)
// depends on the bit patterns fed to it.
#include <hip/hip_runtime.h>

#include "runtime.hpp"

namespace tg {

__device__ __forceinline__ uint32_t mix32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return x;
}

__global__ void fill_uniform_kernel(void* p, int64_t n, int is_bf16, uint32_t seed)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint32_t h = mix32((uint32_t)i ^ mix32(seed + (uint32_t)(i >> 32)));
        const float v = (float)(h >> 8) * (2.0f / 16777216.0f) - 1.0f;
        if (is_bf16)
            static_cast<__bf16*>(p)[i] = static_cast<__bf16>(v);
        else
            static_cast<float*>(p)[i] = v;
    }
}

hipError_t fill_uniform(void* p, int64_t n, int is_bf16, uint32_t seed, hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    const int64_t want = (n + 255) / 256;
    const int blocks = (int)(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(fill_uniform_kernel, dim3(blocks), dim3(256), 0, s, p, n, is_bf16, seed);
    return hipGetLastError();
}

}  // namespace tg

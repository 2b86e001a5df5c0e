// util.hip -- layout transform and device queries.
#include <mutex>

#include "internal.hpp"

namespace dspark {

namespace {

// dst[c, r] = src[r, c] for a rows x cols matrix of 2- or 4-byte elements, through 32 x 32 LDS tiles.
template <typename T>
__global__ void __launch_bounds__(256) transpose_kernel(const T* __restrict__ src, int rows, int cols, T* __restrict__ dst) {
    __shared__ T tile[32][33];
    const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
    for (int y = ty; y < 32; y += 8) {
        const int r = r0 + y, c = c0 + tx;
        if (r < rows && c < cols) tile[y][tx] = src[(size_t)r * cols + c];
    }
    __syncthreads();
    for (int y = ty; y < 32; y += 8) {
        const int c = c0 + y, r = r0 + tx;
        if (r < rows && c < cols) dst[(size_t)c * rows + r] = tile[tx][y];
    }
}

}  // namespace

hipError_t launch_transpose(const void* src, int rows, int cols, int elem_bytes, void* dst, hipStream_t st) {
    const dim3 grid((cols + 31) / 32, (rows + 31) / 32), block(256);
    if (elem_bytes == 2)
        hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, block, 0, st, (const uint16_t*)src, rows, cols, (uint16_t*)dst);
    else
        hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, block, 0, st, (const uint32_t*)src, rows, cols, (uint32_t*)dst);
    return hipGetLastError();
}

int device_cu_count() {
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

}  // namespace dspark

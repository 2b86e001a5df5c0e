// util.hip -- layout transform, a streaming read for measurement, and device queries.
#include <mutex>

#include "internal.hpp"

namespace dspark {

namespace {

// p[0 .. n) = value (a kernel, not a memset, so that the call stays safe to capture in a graph)
__global__ void __launch_bounds__(256) fill_u32_kernel(uint32_t* p, uint32_t value, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = value;
}

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

// Reads a (ordinary 16-byte loads) and then b (non-temporal 16-byte loads) once, grid-stride with UN loads
// per thread in flight, folding the words into a value that is stored only if it equals a constant no read
// can produce by chance in a measurement; the loads cannot be dropped.
template <int UN>
__global__ void __launch_bounds__(1024) stream_read_kernel(const u32x4_t* __restrict__ a, size_t na, const u32x4_t* __restrict__ b,
                                                           size_t nb, uint32_t* sink) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t t0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (size_t i = t0; i < na; i += UN * stride) {
        u32x4_t v[UN];
#pragma unroll
        for (int j = 0; j < UN; ++j) v[j] = (i + j * stride < na) ? a[i + j * stride] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < UN; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    for (size_t i = t0; i < nb; i += UN * stride) {
        u32x4_t v[UN];
#pragma unroll
        for (int j = 0; j < UN; ++j) v[j] = (i + j * stride < nb) ? load_nt_u32x4(b + i + j * stride) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < UN; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

// Launch shape of the streaming read: 16 workgroups of 1024 threads per CU and two loads per thread in
// flight read the round's operands fastest among the shapes measured on MI355X (6.7 to 7.0 TB/s).
hipError_t launch_stream_read(const void* a, size_t a_bytes, const void* b, size_t b_bytes, uint32_t* sink, hipStream_t st) {
    const int grid = 16 * device_cu_count();
    hipLaunchKernelGGL(stream_read_kernel<2>, dim3(grid), dim3(1024), 0, st, (const u32x4_t*)a, a_bytes / 16,
                       (const u32x4_t*)b, b_bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t value, size_t n, hipStream_t st) {
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)(blocks < 1024 ? (blocks ? blocks : 1) : 1024)), dim3(256), 0, st, p,
                       value, n);
    return hipGetLastError();
}

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

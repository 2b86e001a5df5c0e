// schedule.hip -- hardware-aware prefix scheduling of the drafted blocks.
//
// DSpark overview, section "Hardware-aware prefix scheduling": R requests, request r verifies a prefix of
// length l_r of its block; the target batch is B = sum_r (1 + l_r) tokens, the expected committed tokens are
// R + sum over admitted extensions (r, j) of the prefix survival a[r][j], and the objective is
// Theta = (R + sum a) * SPS(B) with SPS the engine's steps-per-second table.  The greedy starts from B = R,
// ranks the extensions by survival (ties: position, then request; survival never increases along a block,
// so every prefix comes before its extension) and admits them while Theta strictly increases.
//
// One workgroup: a bitonic sort of the R K extensions in LDS, fp64 prefix sums of the sorted survivals,
// Theta for every admitted count, the first count whose successor does not increase Theta, and the
// per-request counts of the admitted extensions.  R K <= 4096.
#include "internal.hpp"

namespace dspark {

namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSchedMax = 4096;
constexpr int kSchedPer = kSchedMax / kSchedThreads;

// survival values that are not numbers in [0, 1] count as 0
__device__ __forceinline__ float survival_value(float x) { return (x >= 0.f && x <= 1.f) ? x : 0.f; }

// extension order: survival desc, position j asc, request r asc (ids i = r K + j are unique)
__device__ __forceinline__ bool ext_before(float ka, int ia, float kb, int ib, int K) {
    if (ka != kb) return ka > kb;
    const int ja = ia % K, jb = ib % K;
    if (ja != jb) return ja < jb;
    return ia / K < ib / K;
}

__global__ void __launch_bounds__(kSchedThreads) schedule_kernel(const float* __restrict__ a, const float* __restrict__ sps,
                                                                 int R, int K, int32_t* __restrict__ lengths,
                                                                 float* __restrict__ theta_out) {
    __shared__ float key[kSchedMax];
    __shared__ int id[kSchedMax];
    __shared__ double part[kSchedThreads];
    __shared__ int counts[kSchedMax];
    __shared__ int nstop;
    const int t = threadIdx.x;
    const int n = R * K;
    int np = 1;
    while (np < n) np <<= 1;
    for (int i = t; i < np; i += kSchedThreads) {
        key[i] = i < n ? survival_value(a[i]) : -1.f;  // padding sorts last
        id[i] = i < n ? i : 0x7FFFFFFF;
    }
    for (int i = t; i < R; i += kSchedThreads) counts[i] = 0;
    if (t == 0) nstop = n;
    __syncthreads();
    for (int size = 2; size <= np; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = t; i < np; i += kSchedThreads) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool up = (i & size) == 0;
                    const bool jb = (id[j] == 0x7FFFFFFF) ? false
                                    : (id[i] == 0x7FFFFFFF) ? true
                                                            : ext_before(key[j], id[j], key[i], id[i], K);
                    if (up ? jb : !jb) {
                        const float tk = key[i];
                        const int ti = id[i];
                        key[i] = key[j];
                        id[i] = id[j];
                        key[j] = tk;
                        id[j] = ti;
                    }
                }
            }
            __syncthreads();
        }
    }
    // exclusive prefix sums S_m = sum_{q < m} key[q]: per-thread chunks, then a scan of the chunk sums
    double local[kSchedPer];
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < kSchedPer; ++e) {
        const int m = t * kSchedPer + e;
        local[e] = acc;
        if (m < n) acc += (double)key[m];
    }
    part[t] = acc;
    __syncthreads();
    for (int off = 1; off < kSchedThreads; off <<= 1) {
        const double v = t >= off ? part[t - off] : 0.0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    const double base = t > 0 ? part[t - 1] : 0.0;  // sum of the earlier chunks
    // Theta(m) = (R + S_m) SPS(R + m); the first m < n with Theta(m + 1) <= Theta(m) stops the greedy
#pragma unroll
    for (int e = 0; e < kSchedPer; ++e) {
        const int m = t * kSchedPer + e;
        if (m < n) {
            const double sm = base + local[e];
            const double th0 = ((double)R + sm) * (double)sps[R + m];
            const double th1 = ((double)R + sm + (double)key[m]) * (double)sps[R + m + 1];
            if (!(th1 > th0)) atomicMin(&nstop, m);
        }
    }
    __syncthreads();
    const int ns = nstop;
    for (int m = t; m < ns; m += kSchedThreads) atomicAdd(&counts[id[m] / K], 1);
    __syncthreads();
    for (int r = t; r < R; r += kSchedThreads) lengths[r] = counts[r];
    if (theta_out && t == 0) {
        double s = 0.0;
        for (int m = 0; m < ns; ++m) s += (double)key[m];
        *theta_out = (float)(((double)R + s) * (double)sps[R + ns]);
    }
}

}  // namespace

int schedule_supported(int R, int K) { return R >= 1 && K >= 1 && (long)R * K <= kSchedMax; }

hipError_t launch_schedule(const float* a, const float* sps, int R, int K, int32_t* lengths, float* theta, hipStream_t st) {
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, st, a, sps, R, K, lengths, theta);
    return hipGetLastError();
}

}  // namespace dspark

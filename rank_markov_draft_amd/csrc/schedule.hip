// schedule.hip -- hardware-aware prefix scheduling of the drafted blocks.
//
// DSpark overview, section "Hardware-aware prefix scheduling": R requests, request r verifies a prefix of
// length l_r of its block; the target batch is B = sum_r (1 + l_r) tokens, the expected committed tokens are
// R + sum over admitted extensions (r, j) of the prefix survival a[r][j], and the objective is
// Theta = (R + sum a) * SPS(B) with SPS the engine's steps-per-second table.  The greedy starts from B = R,
// ranks the extensions by survival (ties: position, then request; survival never increases along a block,
// so every prefix comes before its extension) and admits them while Theta strictly increases.
//
// One workgroup: a bitonic sort of the R K extensions (registers, shuffles and LDS), fp64 prefix sums of the sorted survivals,
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

// extension order: survival desc, then position j asc, then request r asc.  Entries carry the tie-break
// key q = j R + r (unique), so the comparison needs no division.
__device__ __forceinline__ bool ext_before(float ka, int qa, float kb, int qb) { return ka != kb ? ka > kb : qa < qb; }

__global__ void __launch_bounds__(kSchedThreads) schedule_kernel(const float* __restrict__ a, const float* __restrict__ sps,
                                                                 int R, int K, int32_t* __restrict__ lengths,
                                                                 float* __restrict__ theta_out) {
    __shared__ float key[kSchedMax];
    __shared__ int id[kSchedMax];
    __shared__ double part[kSchedThreads];
    __shared__ int counts[kSchedMax];
    __shared__ int nstop;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int n = R * K;
    int np = kSchedThreads;  // at least one entry per thread; padding sorts last
    while (np < n) np <<= 1;
    const int E = np / kSchedThreads;  // 1, 2 or 4 entries per thread, thread t holds positions t E .. t E + E - 1
    float kv[kSchedPer];
    int iv[kSchedPer];
#pragma unroll
    for (int e = 0; e < kSchedPer; ++e) {
        const int i = t * E + e;
        kv[e] = (e < E && i < n) ? survival_value(a[i]) : -1.f;
        iv[e] = (e < E && i < n) ? (i % K) * R + i / K : 0x7FFFFFFF;  // i = r K + j  ->  j R + r
    }
    for (int i = t; i < R; i += kSchedThreads) counts[i] = 0;
    if (t == 0) nstop = n;
    // (x, ix) comes before (y, iy); padding (id INT_MAX) after everything
    auto first = [&](float x, int ix, float y, int iy) {
        if (iy == 0x7FFFFFFF) return ix != 0x7FFFFFFF;
        if (ix == 0x7FFFFFFF) return false;
        return ext_before(x, ix, y, iy);
    };
    // Bitonic network in registers: strides inside a thread swap registers, strides inside a wave use
    // shuffles, only strides across waves go through LDS (two barriers each).  In a pair (i, j = i ^ stride)
    // of an ascending block the lower index keeps the element that comes first.
    for (int size = 2; size <= np; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride < E) {
#pragma unroll
                for (int e = 0; e < kSchedPer; ++e) {
                    const int f = e ^ stride;
                    if (e < E && f > e) {
                        const int i = t * E + e;
                        const bool up = (i & size) == 0;
                        const bool ff = first(kv[f], iv[f], kv[e], iv[e]);
                        if (up ? ff : !ff) {
                            const float tk = kv[e];
                            const int ti = iv[e];
                            kv[e] = kv[f];
                            iv[e] = iv[f];
                            kv[f] = tk;
                            iv[f] = ti;
                        }
                    }
                }
            } else if (stride < 64 * E) {
                const int delta = stride / E;
#pragma unroll
                for (int e = 0; e < kSchedPer; ++e) {
                    const float pk = __shfl_xor(kv[e], delta);
                    const int pi = __shfl_xor(iv[e], delta);
                    if (e < E) {
                        const int i = t * E + e;
                        const bool lower = (lane & delta) == 0;
                        const bool up = (i & size) == 0;
                        const bool pf = first(pk, pi, kv[e], iv[e]);
                        if (lower == up ? pf : !pf) {
                            kv[e] = pk;
                            iv[e] = pi;
                        }
                    }
                }
            } else {
                __syncthreads();
#pragma unroll
                for (int e = 0; e < kSchedPer; ++e)
                    if (e < E) {
                        key[t * E + e] = kv[e];
                        id[t * E + e] = iv[e];
                    }
                __syncthreads();
#pragma unroll
                for (int e = 0; e < kSchedPer; ++e)
                    if (e < E) {
                        const int i = t * E + e;
                        const int j = i ^ stride;
                        const float pk = key[j];
                        const int pi = id[j];
                        const bool up = (i & size) == 0;
                        const bool pf = first(pk, pi, kv[e], iv[e]);
                        if ((i < j) == up ? pf : !pf) {
                            kv[e] = pk;
                            iv[e] = pi;
                        }
                    }
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kSchedPer; ++e)
        if (e < E) {
            key[t * E + e] = kv[e];
            id[t * E + e] = iv[e];
        }
    __syncthreads();
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
    for (int m = t; m < ns; m += kSchedThreads) atomicAdd(&counts[id[m] % R], 1);
    __syncthreads();
    for (int r = t; r < R; r += kSchedThreads) lengths[r] = counts[r];
    if (theta_out) {
        // Theta of the admitted set from the prefix sums: the thread whose chunk holds position ns, or the
        // total when every slot is admitted
        if (ns < kSchedMax && ns / kSchedPer == t) {
            const double sn = base + local[ns - t * kSchedPer];
            *theta_out = (float)(((double)R + sn) * (double)sps[R + ns]);
        } else if (ns == kSchedMax && t == 0) {
            *theta_out = (float)(((double)R + part[kSchedThreads - 1]) * (double)sps[R + ns]);
        }
    }
}

}  // namespace

int schedule_supported(int R, int K) { return R >= 1 && K >= 1 && (long)R * K <= kSchedMax; }

hipError_t launch_schedule(const float* a, const float* sps, int R, int K, int32_t* lengths, float* theta, hipStream_t st) {
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, st, a, sps, R, K, lengths, theta);
    return hipGetLastError();
}

}  // namespace dspark

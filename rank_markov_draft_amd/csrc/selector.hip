// selector.hip -- the Selector-style truncated execution of the Markov rule.
//
// "DFlash-2's Selector and DSpark's Markov Head: An Equivalence Observation", section "Where the
// parallelism comes from": (1) fix the candidate sets to the top tokens of the base logits at every
// position, (2) compute the calibrated scores of every adjacent (predecessor, candidate) pair in
// parallel, (3) walk.  Section "What the two methods do" gives the score
// S_t(a, b) = U_t(b) + < A(a) (.) H(h_t), B(b) >.
//
// top-k: one workgroup per row streams the row once (16-byte loads); every thread keeps a sorted
// register list of its best candidates, the lists are merged through LDS by repeated workgroup arg-max.
// Rows with k > 16 (small vocabularies only) are sorted whole in LDS by a bitonic network.
// Pair scores: one workgroup per (row, position, block of 16 predecessors); the 16 gated predecessor
// rows and each block of 16 candidate rows are staged in LDS as fp32, one thread per pair.
// Walk: one wave per row, K serial picks over the precomputed rows.
#include "internal.hpp"

namespace dspark {

namespace {

constexpr int kTkThreads = 256;

// (value desc, id asc); -0.0 == +0.0 because the comparison is on values.
__device__ __forceinline__ bool before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

template <int L>
__device__ __forceinline__ void list_insert(float (&kv)[L], int (&ki)[L], float x, int v) {
    // x beats the current last entry; put it there and bubble it up
    kv[L - 1] = x;
    ki[L - 1] = v;
#pragma unroll
    for (int s = L - 1; s > 0; --s) {
        const bool sw = before(kv[s], ki[s], kv[s - 1], ki[s - 1]);
        const float tv = kv[s];
        const int ti = ki[s];
        kv[s] = sw ? kv[s - 1] : tv;
        ki[s] = sw ? ki[s - 1] : ti;
        kv[s - 1] = sw ? tv : kv[s - 1];
        ki[s - 1] = sw ? ti : ki[s - 1];
    }
}

// Top-k (k <= L) of each row.
template <int L, bool VEC>
__global__ void __launch_bounds__(kTkThreads) topk_kernel(const float* __restrict__ U, int64_t u_stride, int V, int k,
                                                          int32_t* __restrict__ idx, float* __restrict__ val) {
    __shared__ float sk[kTkThreads * L];
    __shared__ int si[kTkThreads * L];
    __shared__ float wk[4];
    __shared__ int wi[4], wt[4];

    const int row = blockIdx.x;
    const float* u = U + (size_t)row * u_stride;
    float kv[L];
    int ki[L];
#pragma unroll
    for (int s = 0; s < L; ++s) {
        kv[s] = -INFINITY;
        ki[s] = 0x7FFFFFFF;
    }
    // every thread scans its ids in increasing order, so an equal value seen later has a larger id
    if (VEC) {
        const int nv = V >> 2;
        for (int q = threadIdx.x; q < nv; q += kTkThreads) {
            const f32x4_t x = load_nt_f32x4(u + 4 * q);
            const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (before(xs[e], 4 * q + e, kv[L - 1], ki[L - 1])) list_insert<L>(kv, ki, xs[e], 4 * q + e);
        }
    } else {
        for (int v = threadIdx.x; v < V; v += kTkThreads) {
            const float x = u[v];
            if (before(x, v, kv[L - 1], ki[L - 1])) list_insert<L>(kv, ki, x, v);
        }
    }
#pragma unroll
    for (int s = 0; s < L; ++s) {
        sk[threadIdx.x * L + s] = kv[s];
        si[threadIdx.x * L + s] = ki[s];
    }
    __syncthreads();
    // k rounds of workgroup arg-max over the heads of the 256 sorted lists
    int head = 0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int out = 0; out < k; ++out) {
        float bk = head < L ? sk[threadIdx.x * L + head] : -INFINITY;
        int bi = head < L ? si[threadIdx.x * L + head] : 0x7FFFFFFF;
        int bt = threadIdx.x;
        for (int off = 32; off > 0; off >>= 1) {
            const float ok_ = __shfl_xor(bk, off);
            const int oi = __shfl_xor(bi, off);
            const int ot = __shfl_xor(bt, off);
            if (before(ok_, oi, bk, bi)) {
                bk = ok_;
                bi = oi;
                bt = ot;
            }
        }
        if (lane == 0) {
            wk[wave] = bk;
            wi[wave] = bi;
            wt[wave] = bt;
        }
        __syncthreads();
        float gk = wk[0];
        int gi = wi[0], gt = wt[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            if (before(wk[w], wi[w], gk, gi)) {
                gk = wk[w];
                gi = wi[w];
                gt = wt[w];
            }
        }
        if (threadIdx.x == gt) ++head;
        if (threadIdx.x == 0) {
            idx[(size_t)row * k + out] = gi;
            if (val) val[(size_t)row * k + out] = gk;
        }
        __syncthreads();
    }
}

// Whole-row bitonic sort in LDS for small vocabularies (V <= 4096), any k <= V.
constexpr int kSortMax = 4096;
__global__ void __launch_bounds__(kTkThreads) topk_sort_kernel(const float* __restrict__ U, int64_t u_stride, int V, int k,
                                                               int32_t* __restrict__ idx, float* __restrict__ val) {
    __shared__ float sv[kSortMax];
    __shared__ int si[kSortMax];
    const int row = blockIdx.x;
    const float* u = U + (size_t)row * u_stride;
    int n = 1;
    while (n < V) n <<= 1;
    for (int i = threadIdx.x; i < n; i += kTkThreads) {
        sv[i] = i < V ? u[i] : -INFINITY;
        si[i] = i < V ? i : 0x7FFFFFFF;
    }
    __syncthreads();
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < n; i += kTkThreads) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool up = (i & size) == 0;  // ascending-in-"before" blocks put the best first
                    const bool jb = before(sv[j], si[j], sv[i], si[i]);
                    if (up ? jb : !jb) {
                        const float tv = sv[i];
                        const int ti = si[i];
                        sv[i] = sv[j];
                        si[i] = si[j];
                        sv[j] = tv;
                        si[j] = ti;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = threadIdx.x; i < k; i += kTkThreads) {
        idx[(size_t)row * k + i] = si[i];
        if (val) val[(size_t)row * k + i] = sv[i];
    }
}

template <typename WT>
__device__ __forceinline__ float wget(const WT* p, size_t i);
template <>
__device__ __forceinline__ float wget<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float wget<uint16_t>(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

constexpr int kPairBlock = 16;
constexpr int kPairChunk = 256;  // rank elements staged per pass

// grid: (B*K, ceil(npred / 16)); scores layout per row b: [topk] anchor row, then (K-1) tables [topk][topk].
template <typename WT>
__global__ void __launch_bounds__(256) pair_score_kernel(SelectorArgs a) {
    __shared__ float ap[kPairBlock][kPairChunk + 1];
    __shared__ float bc[kPairBlock][kPairChunk + 1];
    const WT* A = reinterpret_cast<const WT*>(a.A);
    const WT* Bm = reinterpret_cast<const WT*>(a.Bemb);
    const int bt = blockIdx.x, b = bt / a.K, t = bt % a.K;
    const int npred = (t == 0) ? 1 : a.topk;
    const int i0 = blockIdx.y * kPairBlock;
    if (i0 >= npred) return;
    const int ni = min(kPairBlock, npred - i0);
    const int r = a.r;
    const int32_t* cand_t = a.cand + ((size_t)b * a.K + t) * a.topk;
    const int32_t* cand_p = (t == 0) ? nullptr : a.cand + ((size_t)b * a.K + t - 1) * a.topk;
    const float* Ht = a.H ? a.H + ((size_t)b * a.K + t) * r : nullptr;
    const float* Ut = a.U + ((size_t)b * a.K + t) * a.V;
    float* out = a.scores + (size_t)b * (a.topk + (size_t)(a.K - 1) * a.topk * a.topk) +
                 (t == 0 ? 0 : a.topk + (size_t)(t - 1) * a.topk * a.topk);
    const int ii = threadIdx.x / kPairBlock, jj = threadIdx.x % kPairBlock;
    for (int j0 = 0; j0 < a.topk; j0 += kPairBlock) {
        const int nj = min(kPairBlock, a.topk - j0);
        float acc = 0.f;
        for (int q0 = 0; q0 < r; q0 += kPairChunk) {
            const int nq = min(kPairChunk, r - q0);
            __syncthreads();
            for (int e = threadIdx.x; e < ni * nq; e += 256) {
                const int pi = e / nq, q = e % nq;
                const int pa = (t == 0) ? a.anchor[b] : cand_p[i0 + pi];
                float x = wget<WT>(A, (size_t)pa * r + q0 + q);
                if (Ht) x *= Ht[q0 + q];
                ap[pi][q] = x;
            }
            for (int e = threadIdx.x; e < nj * nq; e += 256) {
                const int cj = e / nq, q = e % nq;
                bc[cj][q] = wget<WT>(Bm, (size_t)cand_t[j0 + cj] * r + q0 + q);
            }
            __syncthreads();
            if (ii < ni && jj < nj)
                for (int q = 0; q < nq; ++q) acc = fmaf(ap[ii][q], bc[jj][q], acc);
        }
        if (ii < ni && jj < nj) out[(size_t)(i0 + ii) * a.topk + j0 + jj] = Ut[cand_t[j0 + jj]] + acc;
    }
}

// One wave per row: K serial picks.
__global__ void __launch_bounds__(64) walk_kernel(SelectorArgs a) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const size_t tstride = a.topk + (size_t)(a.K - 1) * a.topk * a.topk;
    const float* sc = a.scores + (size_t)b * tstride;
    int islot = 0;
    for (int t = 0; t < a.K; ++t) {
        const float* rowp = (t == 0) ? sc : sc + a.topk + ((size_t)(t - 1) * a.topk + islot) * a.topk;
        const int32_t* cand_t = a.cand + ((size_t)b * a.K + t) * a.topk;
        const uint32_t k2 = a.sample ? noise_key2(a.k0, (uint32_t)b, (uint32_t)t) : 0u;
        float bk = -INFINITY, bl = 0.f, m = kMinFinite, s = 0.f;
        int bi = 0x7FFFFFFF, bs = 0;
        for (int j = lane; j < a.topk; j += 64) {
            const float l = rowp[j];
            const int c = cand_t[j];
            const float tt = l * a.inv_t * kLog2e;
            float key = a.sample ? tt + gumbel_log2_units(fmix32(k2 ^ (uint32_t)c)) : l;
            if (beats(key, c, bk, bi)) {
                bk = key;
                bi = c;
                bl = l;
                bs = j;
            }
            lse_merge(m, s, tt, 1.0f);
        }
        for (int off = 32; off > 0; off >>= 1) {
            const float ok_ = __shfl_xor(bk, off);
            const int oi = __shfl_xor(bi, off);
            const float ol = __shfl_xor(bl, off);
            const int os_ = __shfl_xor(bs, off);
            const float om = __shfl_xor(m, off);
            const float oss = __shfl_xor(s, off);
            if (beats(ok_, oi, bk, bi)) {
                bk = ok_;
                bi = oi;
                bl = ol;
                bs = os_;
            }
            lse_merge(m, s, om, oss);
        }
        islot = bs;
        if (lane == 0) {
            a.tokens[(size_t)b * a.K + t] = bi;
            if (a.logprobs) a.logprobs[(size_t)b * a.K + t] = bl * a.inv_t - (m + fast_log2(s)) * kLn2;
        }
    }
}

}  // namespace

size_t topk_workspace_bytes(int, int, int) { return 0; }

hipError_t launch_topk(const float* U, int64_t u_stride, int rows, int V, int topk, int32_t* idx, float* val, void*,
                       hipStream_t st) {
    const bool vec = (V % 4 == 0) && (u_stride % 4 == 0) && ((uintptr_t)U % 16 == 0);
    if (topk <= 16) {
        if (vec) hipLaunchKernelGGL((topk_kernel<16, true>), dim3(rows), dim3(kTkThreads), 0, st, U, u_stride, V, topk, idx, val);
        else hipLaunchKernelGGL((topk_kernel<16, false>), dim3(rows), dim3(kTkThreads), 0, st, U, u_stride, V, topk, idx, val);
    } else if (V <= kSortMax) {
        hipLaunchKernelGGL(topk_sort_kernel, dim3(rows), dim3(kTkThreads), 0, st, U, u_stride, V, topk, idx, val);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int topk_supported(int V, int topk) { return topk >= 1 && topk <= V && (topk <= 16 || V <= kSortMax); }

hipError_t launch_pair_scores(const SelectorArgs& a, hipStream_t st) {
    const dim3 grid(a.B * a.K, (a.topk + kPairBlock - 1) / kPairBlock);
    if (a.bf16) hipLaunchKernelGGL(pair_score_kernel<uint16_t>, grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(pair_score_kernel<float>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_walk(const SelectorArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(walk_kernel, dim3(a.B), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace dspark

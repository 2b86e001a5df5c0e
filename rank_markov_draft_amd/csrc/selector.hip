// selector.hip -- the Selector-style truncated execution of the Markov rule.
//
// "DFlash-2's Selector and DSpark's Markov Head: An Equivalence Observation", section "Where the
// parallelism comes from": (1) fix the candidate sets to the top tokens of the base logits at every
// position, (2) compute the calibrated scores of every adjacent (predecessor, candidate) pair in
// parallel, (3) walk.  Section "What the two methods do" gives the score
// S_t(a, b) = U_t(b) + < A(a) (.) H(h_t), B(b) >.
//
// top-k: one workgroup per row streams the row once (independent 16-byte loads); each wave filters the
// elements against the k-th entry of its exact running list and merges the rare survivors into it.  Rows with
// k > 64 are sorted whole in LDS by a bitonic network (V <= 4096) or radix-selected (k <= 1024).
// Pair scores: bf16 weights with r % 16 == 0 run on the matrix cores (one 32 x 32 table tile per (row,
// position) for k <= 32, a 64 x 64 block per workgroup above); otherwise one workgroup per (row, position, block
// of 16 predecessors) stages the gated predecessor rows and each block of 16 candidate rows in LDS as fp32, one
// thread per pair.  Walk: every table row's pick resolved in parallel (greedy, or the whole-vocabulary draw
// restricted to the candidates), then the path followed; tables larger than the LDS are read from global memory.
#include <algorithm>

#include "internal.hpp"

namespace dspark {

namespace {

constexpr int kTkThreads = 256;

// (value desc, id asc); -0.0 == +0.0 because the comparison is on values.
__device__ __forceinline__ bool before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkUnroll = 4;  // independent 16-byte loads in flight per lane (8 waves per SIMD keep ~128 KB per CU in flight)
constexpr int kTkBuf = 128;                  // candidate slots per wave (a flush at 64 leaves at most 63 + 64 pending)

// Compare-exchange across the wave: this lane and lane ^ j hold two entries; this lane keeps the better one
// (under (value desc, id asc)) when keep_better, else the worse one.
__device__ __forceinline__ void wave_cx(float& v, int& i, int j, bool keep_better) {
    const float ov = __shfl_xor(v, j);
    const int oi = __shfl_xor(i, j);
    if (before(ov, oi, v, i) == keep_better) {
        v = ov;
        i = oi;
    }
}

// Bitonic sort of one entry per lane, best first (lane s ends with rank s).
__device__ __forceinline__ void wave_sort64(float& v, int& i) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) wave_cx(v, i, j, ((lane & j) == 0) == ((lane & k) == 0));
}

// t (a best-first list, one entry per lane) becomes the best 64 of t and c (also sorted best first): the
// better of t[s] and c[63 - s] is a bitonic sequence holding the best 64 of the union, which one bitonic
// merge sorts.
__device__ __forceinline__ void wave_merge64(float& tv, int& ti, float cv, int ci) {
    const int lane = threadIdx.x & 63;
    const float rv = __shfl_xor(cv, 63);
    const int ri = __shfl_xor(ci, 63);
    if (before(rv, ri, tv, ti)) {
        tv = rv;
        ti = ri;
    }
#pragma unroll
    for (int j = 32; j > 0; j >>= 1) wave_cx(tv, ti, j, (lane & j) == 0);
}

// The L-th largest of the wave's 64 lane values (bitonic sort across lanes, ascending, then lane 64 - L).
template <int L>
__device__ __forceinline__ float wave_lth_largest(float t) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const float o = __shfl_xor(t, j);
            const bool up = (lane & k) == 0 || k == 64;  // ascending block (the last merge ascends)
            const bool low = (lane & j) == 0;
            t = (low == up) ? fminf(t, o) : fmaxf(t, o);
        }
    }
    return __shfl(t, 64 - L);
}

// Top-k (k <= L, L = 16, 32 or 64) of each row, one workgroup per row.  Each wave keeps an exact sorted list of
// its best 64 entries (lane s holds rank s) and the list's L-th entry as a threshold; every element is compared
// once against the threshold and the few that beat it are appended to the wave's LDS buffer, which is merged
// into the list once it holds 64: each 64-entry chunk of the buffer by a bitonic sort and one bitonic merge (28
// exchange steps; with L rounds of a six-step wave arg-max instead, 2048 rows of 151936 took 0.22 ms at L = 16
// and 0.52 ms at L = 64, against 0.20 and 0.23 ms so).
// The row is streamed with kTkUnroll independent 16-byte loads per lane, so the scan runs at memory speed; the
// four lists are merged at the end.
template <int L, bool VEC>
__global__ void __launch_bounds__(kTkThreads) __attribute__((amdgpu_waves_per_eu(8))) topk_kernel(const float* __restrict__ U, int64_t u_stride, int V, int k,
                                                          int32_t* __restrict__ idx, float* __restrict__ val) {
    __shared__ float bufv[kTkWaves][kTkBuf];
    __shared__ int bufi[kTkWaves][kTkBuf];
    __shared__ float finv[kTkWaves * 64];
    __shared__ int fini[kTkWaves * 64];
    __shared__ float sthv[kTkWaves];  // each wave's current threshold (its list entry L-1): any of them is a
    __shared__ int sthi[kTkWaves];    // bound for the whole row, so every wave filters with the best of them

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x;
    const float* u = U + (size_t)row * u_stride;
    float* bv = bufv[wave];
    int* bi = bufi[wave];
    float tv = -INFINITY, thv = -INFINITY;  // this lane's list entry; the wave's threshold (list entry L-1)
    int ti = 0x7FFFFFFF, thi = 0x7FFFFFFF;
    int cnt = 0;                            // wave-uniform buffer fill
    if (lane == 0) {
        sthv[wave] = -INFINITY;
        sthi[wave] = 0x7FFFFFFF;
    }
    __syncthreads();

    // An element behind (after, in the order) the L-th entry of any wave's list has L elements of the row ahead
    // of it, so it is not in the row's top L: the waves share their thresholds and filter with the best one.
    auto adopt_shared = [&]() {
#pragma unroll
        for (int w = 0; w < kTkWaves; ++w) {
            const float ov = sthv[w];
            const int oi = sthi[w];
            if (before(ov, oi, thv, thi)) {
                thv = ov;
                thi = oi;
            }
        }
    };
    auto flush = [&]() {
        for (int c0 = 0; c0 < cnt; c0 += 64) {
            const int e = c0 + lane;
            float cv = e < cnt ? bv[e] : -INFINITY;
            int ci = e < cnt ? bi[e] : 0x7FFFFFFF;
            wave_sort64(cv, ci);
            wave_merge64(tv, ti, cv, ci);
        }
        const float nv = __shfl(tv, L - 1);
        const int ni = __shfl(ti, L - 1);
        if (lane == 0) {
            sthv[wave] = nv;
            sthi[wave] = ni;
        }
        if (before(nv, ni, thv, thi)) {
            thv = nv;
            thi = ni;
        }
        if (L > 16) adopt_shared();
        cnt = 0;
    };
    auto offer = [&](float x, int id) {
        const bool p = before(x, id, thv, thi);
        const uint64_t msk = __ballot(p);
        if (msk) {
            if (p) {
                const int slot = cnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(msk >> 32),
                                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)msk, 0u));
                bv[slot] = x;
                bi[slot] = id;
            }
            cnt += __popcll(msk);
            if (cnt >= 64) flush();  // early: each flush tightens the threshold (at 192 pending the scan ran 1-7% longer)
        }
    };
    if (VEC) {
        const int nq = V >> 2;
        const f32x4_t* u4 = reinterpret_cast<const f32x4_t*>(u);
        constexpr int kChunk = kTkThreads * kTkUnroll;  // 16-byte units per chunk of the row
        auto load = [&](int q0, int j) {
            const int q = q0 + j * kTkThreads + (int)threadIdx.x;
            return q < nq ? __builtin_nontemporal_load(u4 + q) : f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        };
        // Prefilter on values alone: an element can enter the list only if it is >= the threshold value (ties
        // are then settled by offer's exact order).  After the first few chunks almost no lane of the wave
        // passes, and one maximum and one ballot cover a load's 4 elements.
        f32x4_t x[kTkUnroll];
#pragma unroll
        for (int j = 0; j < kTkUnroll; ++j) x[j] = load(0, j);
        {
            float mj[kTkUnroll];
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < kTkUnroll; ++j) {
                mj[j] = fmaxf(fmaxf(x[j].x, x[j].y), fmaxf(x[j].z, x[j].w));
                mx = fmaxf(mx, mj[j]);
            }
            // Start the filter at the L-th largest lane maximum of the first chunk: the L lanes at or above it
            // hold L elements at least that large, so no smaller element can enter the wave's top-L.  Equal
            // values still pass (id bound INT_MAX) and are settled exactly.  Without it every element of the
            // first chunk is a candidate and the merges of the start dominate the scan.
            thv = wave_lth_largest<L>(mx);
            thi = 0x7FFFFFFF;
#pragma unroll
            for (int j = 0; j < kTkUnroll; ++j) {
                if (__ballot(mj[j] >= thv)) {
                    const int q = j * kTkThreads + (int)threadIdx.x;
                    const int id = q < nq ? 4 * q : 0x7FFFFFFC;
                    offer(x[j].x, id);
                    offer(x[j].y, id + 1);
                    offer(x[j].z, id + 2);
                    offer(x[j].w, id + 3);
                }
            }
        }
        // The following chunks: a lane's load j of the next chunk is issued as soon as its load j of this chunk
        // has been filtered (and its rare candidates offered), so the wave keeps kTkUnroll loads in flight while
        // it filters (the offers, their order and the thresholds are those of filtering chunk by chunk).  At
        // 2048 rows of 151936 against issuing each chunk's loads after the previous chunk's filter: k = 16 202
        // us either way, k = 64 229 -> 225 us; a plain read of the same rows in this access pattern takes 185
        // us, so the difference to it is not the filter's latency between chunks.  (The offers are written out
        // here rather than in a helper lambda: a lambda the compiler did not inline kept the captured list and
        // threshold in scratch memory, and the scan ran 4.7x slower.)
#pragma unroll
        for (int j = 0; j < kTkUnroll; ++j) x[j] = load(kChunk, j);
        for (int q0 = kChunk; q0 < nq; q0 += kChunk) {
            if (L > 16 && (q0 / kChunk) % 4 == 0) adopt_shared();  // pick up the other waves' progress now and then
#pragma unroll
            for (int j = 0; j < kTkUnroll; ++j) {
                const float m = fmaxf(fmaxf(x[j].x, x[j].y), fmaxf(x[j].z, x[j].w));
                if (__ballot(m >= thv)) {
                    const int q = q0 + j * kTkThreads + (int)threadIdx.x;
                    const int id = q < nq ? 4 * q : 0x7FFFFFFC;
                    offer(x[j].x, id);
                    offer(x[j].y, id + 1);
                    offer(x[j].z, id + 2);
                    offer(x[j].w, id + 3);
                }
                x[j] = load(q0 + kChunk, j);
            }
        }
    } else {
        for (int v0 = 0; v0 < V; v0 += kTkThreads * kTkUnroll) {
            float x[kTkUnroll];
#pragma unroll
            for (int j = 0; j < kTkUnroll; ++j) {
                const int v = v0 + j * kTkThreads + (int)threadIdx.x;
                x[j] = v < V ? u[v] : -INFINITY;
            }
#pragma unroll
            for (int j = 0; j < kTkUnroll; ++j) {
                const int v = v0 + j * kTkThreads + (int)threadIdx.x;
                offer(x[j], v < V ? v : 0x7FFFFFFF);
            }
        }
    }
    if (cnt > 0) flush();
    finv[wave * 64 + lane] = tv;
    fini[wave * 64 + lane] = ti;
    __syncthreads();
    if (wave == 0) {
        // the sorted lists of waves 1..3 merged into wave 0's
        float fv = tv;
        int fi = ti;
#pragma unroll
        for (int w = 1; w < kTkWaves; ++w) wave_merge64(fv, fi, finv[w * 64 + lane], fini[w * 64 + lane]);
        if (lane < k) {
            idx[(size_t)row * k + lane] = fi;
            if (val) val[(size_t)row * k + lane] = fv;
        }
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

// Top-k for 64 < k <= 1024 at any vocabulary size, one workgroup per row, by radix selection on the ordered
// 32-bit key of each value (larger key = larger value, -0 and +0 one key): three counting passes over the
// row fix the k-th largest key K* digit by digit (11, 11 and 10 bits) and how many elements with key K* the
// top-k takes; a fourth pass collects every element with a larger key and, scanning in id order, the lowest
// ids with key K*; the k entries are then sorted in LDS.  The row is read four times: this form serves the
// sizes the one-pass filter does not hold, not the measured ones.
constexpr int kRadixMaxK = 1024;
constexpr int kRadixBins = 2048;

__device__ __forceinline__ uint32_t topk_key(float f) {
    f = f + 0.0f;  // -0 -> +0
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ void __launch_bounds__(kTkThreads) topk_radix_kernel(const float* __restrict__ U, int64_t u_stride, int V,
                                                                int k, int32_t* __restrict__ idx,
                                                                float* __restrict__ val) {
    __shared__ uint32_t hist[kRadixBins];
    __shared__ uint32_t skey[kRadixMaxK];
    __shared__ int sid[kRadixMaxK];
    __shared__ uint32_t s_prefix, s_need, s_nsel, s_taken;
    __shared__ uint32_t s_wsum[kTkWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x;
    const float* u = U + (size_t)row * u_stride;
    if (tid == 0) {
        s_prefix = 0;
        s_need = (uint32_t)k;
    }
    // digit d covers key bits [shift, shift + width); the higher digits are fixed by then
    constexpr int kShift[3] = {21, 10, 0};
    constexpr int kWidth[3] = {11, 11, 10};
    for (int d = 0; d < 3; ++d) {
        const int shift = kShift[d], width = kWidth[d];
        const uint32_t hi_mask = d == 0 ? 0u : ~((1u << (shift + width)) - 1u);
        for (int i = tid; i < kRadixBins; i += kTkThreads) hist[i] = 0;
        __syncthreads();
        const uint32_t prefix = s_prefix;
        for (int v = tid; v < V; v += kTkThreads) {
            const uint32_t key = topk_key(u[v]);
            if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & ((1u << width) - 1u)], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l owns bins nb-1-32l .. nb-32-32l (descending); find the bin where the count from the top
            // reaches need
            const int nb = 1 << width;
            const uint32_t need = s_need;
            uint32_t own = 0;
            for (int j = 0; j < 32; ++j) {
                const int b = nb - 1 - 32 * lane - j;
                if (b >= 0) own += hist[b];
            }
            uint32_t incl = own;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t o = __shfl_up(incl, off);
                if (lane >= off) incl += o;
            }
            const uint32_t excl = incl - own;
            if (excl < need && need <= incl) {
                uint32_t above = excl;
                for (int j = 0; j < 32; ++j) {
                    const int b = nb - 1 - 32 * lane - j;
                    const uint32_t c = hist[b];
                    if (need <= above + c) {
                        s_prefix = prefix | ((uint32_t)b << shift);
                        s_need = need - above;
                        break;
                    }
                    above += c;
                }
            }
        }
        __syncthreads();
    }
    // K* = s_prefix; the top-k holds every key above K* (k - need of them) and the need lowest ids with K*
    const uint32_t kstar = s_prefix, quota = s_need;
    if (tid == 0) {
        s_nsel = 0;
        s_taken = 0;
    }
    __syncthreads();
    for (int v0 = 0; v0 < V; v0 += kTkThreads) {
        const int v = v0 + tid;
        const uint32_t key = v < V ? topk_key(u[v]) : 0u;
        if (v < V && key > kstar) {
            const uint32_t slot = atomicAdd(&s_nsel, 1u);  // < k - quota by the selection above
            if (slot < (uint32_t)kRadixMaxK) {
                skey[slot] = key;
                sid[slot] = v;
            }
        }
        const uint32_t taken = s_taken;  // uniform: written only between the barriers below
        if (taken < quota) {
            const bool eq = v < V && key == kstar;
            const uint64_t m = __ballot(eq);
            const uint32_t rank_in_wave =
                __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (lane == 0) s_wsum[wave] = (uint32_t)__popcll(m);
            __syncthreads();
            uint32_t before_w = 0, total = 0;
            for (int w = 0; w < kTkWaves; ++w) {
                before_w += w < wave ? s_wsum[w] : 0u;
                total += s_wsum[w];
            }
            const uint32_t rank = taken + before_w + rank_in_wave;
            if (eq && rank < quota) {
                // these slots follow the (k - quota) larger keys, whatever order those arrive in
                skey[(k - quota) + rank] = key;
                sid[(k - quota) + rank] = v;
            }
            __syncthreads();
            if (tid == 0) s_taken = taken + total;
        }
        __syncthreads();
    }
    // sort the k entries (key desc, id asc), padded to a power of two
    int n = 1;
    while (n < k) n <<= 1;
    for (int i = k + tid; i < n; i += kTkThreads) {
        skey[i] = 0u;
        sid[i] = 0x7FFFFFFF;
    }
    __syncthreads();
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < n; i += kTkThreads) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool up = (i & size) == 0;
                    const bool jb = skey[j] > skey[i] || (skey[j] == skey[i] && sid[j] < sid[i]);
                    if (up ? jb : !jb) {
                        const uint32_t tk = skey[i];
                        const int ti = sid[i];
                        skey[i] = skey[j];
                        sid[i] = sid[j];
                        skey[j] = tk;
                        sid[j] = ti;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < k; i += kTkThreads) {
        idx[(size_t)row * k + i] = sid[i];
        if (val) val[(size_t)row * k + i] = u[sid[i]];
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
// The block's predecessor and candidate rows are staged as fp32 (gated rows times H), VEC: 16-byte loads,
// several per thread issued together.
template <typename WT, bool VEC>
__global__ void __launch_bounds__(256) pair_score_kernel(SelectorArgs a) {
    constexpr int EV = 16 / (int)sizeof(WT);  // elements per 16-byte load
    constexpr int kReps = 4;                  // loads in flight per thread
    __shared__ float ap[kPairBlock][kPairChunk + 1];
    __shared__ float bc[kPairBlock][kPairChunk + 1];
    __shared__ int rid[2 * kPairBlock];       // predecessor rows, then candidate rows
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
    // blocks of 16 candidates dealt over the grid's third dimension (a loop per workgroup made the blocks of
    // a large top-k one after another: 50 us for three 512 x 512 tables)
    for (int j0 = blockIdx.z * kPairBlock; j0 < a.topk; j0 += gridDim.z * kPairBlock) {
        const int nj = min(kPairBlock, a.topk - j0);
        __syncthreads();
        if ((int)threadIdx.x < ni) rid[threadIdx.x] = (t == 0) ? a.anchor[b] : cand_p[i0 + threadIdx.x];
        if ((int)threadIdx.x >= 64 && (int)threadIdx.x < 64 + nj) rid[kPairBlock + threadIdx.x - 64] = cand_t[j0 + threadIdx.x - 64];
        const float ub = (ii < ni && jj < nj) ? Ut[cand_t[j0 + jj]] : 0.f;
        float acc = 0.f;
        for (int q0 = 0; q0 < r; q0 += kPairChunk) {
            const int nq = min(kPairChunk, r - q0);
            __syncthreads();
            if (VEC) {
                const int nvec = nq / EV;
                const int total = (ni + nj) * nvec;
                for (int e0 = 0; e0 < total; e0 += 256 * kReps) {
                    u32x4_t raw[kReps];
#pragma unroll
                    for (int rep = 0; rep < kReps; ++rep) {
                        const int e = e0 + rep * 256 + (int)threadIdx.x;
                        if (e < total) {
                            const int row = e / nvec, c = e - (e / nvec) * nvec;
                            const WT* src = (row < ni ? A + (size_t)rid[row] * r : Bm + (size_t)rid[kPairBlock + row - ni] * r) + q0 + c * EV;
                            raw[rep] = *reinterpret_cast<const u32x4_t*>(src);
                        }
                    }
#pragma unroll
                    for (int rep = 0; rep < kReps; ++rep) {
                        const int e = e0 + rep * 256 + (int)threadIdx.x;
                        if (e < total) {
                            const int row = e / nvec, c = e - (e / nvec) * nvec;
                            float f[EV];
                            if (sizeof(WT) == 2) {
                                const uint32_t w[4] = {raw[rep].x, raw[rep].y, raw[rep].z, raw[rep].w};
#pragma unroll
                                for (int h = 0; h < 4; ++h) {
                                    f[2 * h] = bf16_to_f32((uint16_t)(w[h] & 0xFFFFu));
                                    f[2 * h + 1] = bf16_to_f32((uint16_t)(w[h] >> 16));
                                }
                            } else {
                                const uint32_t w[4] = {raw[rep].x, raw[rep].y, raw[rep].z, raw[rep].w};
#pragma unroll
                                for (int h = 0; h < EV; ++h) f[h] = __uint_as_float(w[h]);
                            }
                            float* dst = row < ni ? &ap[row][c * EV] : &bc[row - ni][c * EV];
#pragma unroll
                            for (int h = 0; h < EV; ++h) dst[h] = (row < ni && Ht) ? f[h] * Ht[q0 + c * EV + h] : f[h];
                        }
                    }
                }
            } else {
                for (int e = threadIdx.x; e < (ni + nj) * nq; e += 256) {
                    const int row = e / nq, q = e % nq;
                    if (row < ni) {
                        float x = wget<WT>(A, (size_t)rid[row] * r + q0 + q);
                        if (Ht) x *= Ht[q0 + q];
                        ap[row][q] = x;
                    } else {
                        bc[row - ni][q] = wget<WT>(Bm, (size_t)rid[kPairBlock + row - ni] * r + q0 + q);
                    }
                }
            }
            __syncthreads();
            if (ii < ni && jj < nj)
                for (int q = 0; q < nq; ++q) acc = fmaf(ap[ii][q], bc[jj][q], acc);
        }
        if (ii < ni && jj < nj) out[(size_t)(i0 + ii) * a.topk + j0 + jj] = ub + acc;
    }
}

// Pair scores on the matrix cores (bf16 weights, r % 16 == 0, 16-byte aligned rows): one workgroup per
// (row, position, block of 32 predecessors, block of 32 candidates), four waves splitting the rank steps.
// v_mfma_f32_32x32x16_bf16 with A = the (gated) predecessor rows and B = the candidate rows, both loaded
// straight from global memory into operand registers (lane l: row l % 32, rank elements 16 s + 8 (l / 32)
// .. + 7 of step s), no staging.  Gated rows are multiplied by H in fp32 and rounded to bf16, as on the
// Markov path.  The four partial 32x32 tiles are summed through LDS; accumulator i of lane l is predecessor
// 8 (i / 4) + 4 (l / 32) + i % 4 and candidate l % 32.
constexpr int kPairTile = 32;
__global__ void __launch_bounds__(256) pair_score_mfma_kernel(SelectorArgs a) {
    __shared__ float part[4][16][64];
    const uint16_t* A = reinterpret_cast<const uint16_t*>(a.A);
    const uint16_t* Bm = reinterpret_cast<const uint16_t*>(a.Bemb);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bt = blockIdx.x, b = bt / a.K, t = bt % a.K;
    const int npred = (t == 0) ? 1 : a.topk;
    const int i0 = blockIdx.y * kPairTile, j0 = blockIdx.z * kPairTile;
    if (i0 >= npred) return;
    const int ni = min(kPairTile, npred - i0), nj = min(kPairTile, a.topk - j0);
    const int r = a.r;
    const int32_t* cand_t = a.cand + ((size_t)b * a.K + t) * a.topk;
    const int rl = lane & 31, half = lane >> 5;
    const bool pi_ok = rl < ni, cj_ok = rl < nj;
    const int pid = pi_ok ? ((t == 0) ? a.anchor[b] : a.cand[((size_t)b * a.K + t - 1) * a.topk + i0 + rl]) : 0;
    const int cid = cj_ok ? cand_t[j0 + rl] : 0;
    const float* Ht = a.H ? a.H + ((size_t)b * a.K + t) * r : nullptr;
    const uint16_t* arow = A + (size_t)pid * r + 8 * half;
    const uint16_t* brow = Bm + (size_t)cid * r + 8 * half;
    const int nsteps = r / 16;
    f32x16_t acc = {};
    constexpr int kBatch = 4;  // operand loads in flight per lane and operand
    for (int s0 = wave; s0 < nsteps; s0 += 4 * kBatch) {
        u32x4_t ar[kBatch], br[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int st = s0 + 4 * q;
            ar[q] = (st < nsteps && pi_ok) ? *reinterpret_cast<const u32x4_t*>(arow + 16 * st) : u32x4_t{0u, 0u, 0u, 0u};
            br[q] = (st < nsteps && cj_ok) ? *reinterpret_cast<const u32x4_t*>(brow + 16 * st) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int st = s0 + 4 * q;
            if (st < nsteps) {
                u32x4_t av = ar[q];
                if (Ht) {
                    const float* hp = Ht + 16 * st + 8 * half;
                    const uint32_t w[4] = {av.x, av.y, av.z, av.w};
                    uint32_t o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float lo = bf16_to_f32((uint16_t)(w[e] & 0xFFFFu)) * hp[2 * e];
                        const float hi = bf16_to_f32((uint16_t)(w[e] >> 16)) * hp[2 * e + 1];
                        o[e] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
                    }
                    av = u32x4_t{o[0], o[1], o[2], o[3]};
                }
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                             __builtin_bit_cast(bf16x8_t, br[q]), acc, 0, 0, 0);
            }
        }
    }
    // the 16 accumulators of a lane cover predecessors 0 .. 31 of the tile (rows past ni are dropped)
#pragma unroll
    for (int i = 0; i < 16; ++i) part[wave][i][lane] = acc[i];
    __syncthreads();
    if (wave == 0) {
        const float ub = cj_ok ? a.U[((size_t)b * a.K + t) * a.V + cid] : 0.f;
        float* out = a.scores + (size_t)b * (a.topk + (size_t)(a.K - 1) * a.topk * a.topk) +
                     (t == 0 ? 0 : a.topk + (size_t)(t - 1) * a.topk * a.topk);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int pi = 8 * (i / 4) + 4 * half + (i % 4);
            const float v = part[0][i][lane] + part[1][i][lane] + part[2][i][lane] + part[3][i][lane];
            if (pi < ni && cj_ok) out[(size_t)(i0 + pi) * a.topk + j0 + rl] = ub + v;
        }
    }
}

// topk > 32: one workgroup per (row, position, 64 x 64 block of the table).  Every wave computes the whole
// block (four 32 x 32 tiles, each operand fragment used twice) over every fourth rank step, so the block's
// predecessor and candidate rows are read once per workgroup, all in one round of loads at r = 256; the four
// waves' partial sums are added through LDS tile by tile, in wave order.  Operand and accumulator layouts as in pair_score_mfma_kernel.
__global__ void __launch_bounds__(256) pair_score_mfma64_kernel(SelectorArgs a) {
    __shared__ float part[4][16][64];  // one tile's partials of the four waves
    __shared__ float s_ub[64];          // U of the block's candidates
    const uint16_t* A = reinterpret_cast<const uint16_t*>(a.A);
    const uint16_t* Bm = reinterpret_cast<const uint16_t*>(a.Bemb);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bt = blockIdx.x, b = bt / a.K, t = bt % a.K;
    const int npred = (t == 0) ? 1 : a.topk;
    const int i0 = blockIdx.y * 64, j0 = blockIdx.z * 64;
    if (i0 >= npred) return;  // the whole workgroup, before any barrier
    const int ni = min(64, npred - i0), nj = min(64, a.topk - j0);
    const int r = a.r;
    const int32_t* cand_t = a.cand + ((size_t)b * a.K + t) * a.topk;
    const int rl = lane & 31, half = lane >> 5;
    const float* Ht = a.H ? a.H + ((size_t)b * a.K + t) * r : nullptr;
    if (tid < 64) s_ub[tid] = tid < nj ? a.U[((size_t)b * a.K + t) * a.V + cand_t[j0 + tid]] : 0.f;
    const uint16_t* arow[2];
    const uint16_t* brow[2];
    bool pok[2], cok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        pok[h] = 32 * h + rl < ni;
        cok[h] = 32 * h + rl < nj;
        const int pid = pok[h] ? ((t == 0) ? a.anchor[b] : a.cand[((size_t)b * a.K + t - 1) * a.topk + i0 + 32 * h + rl]) : 0;
        const int cid = cok[h] ? cand_t[j0 + 32 * h + rl] : 0;
        arow[h] = A + (size_t)pid * r + 8 * half;
        brow[h] = Bm + (size_t)cid * r + 8 * half;
    }
    const int nsteps = r / 16;
    f32x16_t acc[2][2] = {};
    constexpr int kBatch = 4;  // rank steps per round of loads (four operand loads each)
    for (int s0 = wave; s0 < nsteps; s0 += 4 * kBatch) {
        u32x4_t ar[kBatch][2], br[kBatch][2];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int st = s0 + 4 * q;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                ar[q][h] = (st < nsteps && pok[h]) ? *reinterpret_cast<const u32x4_t*>(arow[h] + 16 * st) : u32x4_t{0u, 0u, 0u, 0u};
                br[q][h] = (st < nsteps && cok[h]) ? *reinterpret_cast<const u32x4_t*>(brow[h] + 16 * st) : u32x4_t{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int st = s0 + 4 * q;
            if (st < nsteps) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (Ht) {
                        const float* hp = Ht + 16 * st + 8 * half;
                        const u32x4_t av = ar[q][h];
                        const uint32_t w[4] = {av.x, av.y, av.z, av.w};
                        uint32_t o[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float lo = bf16_to_f32((uint16_t)(w[e] & 0xFFFFu)) * hp[2 * e];
                            const float hi = bf16_to_f32((uint16_t)(w[e] >> 16)) * hp[2 * e + 1];
                            o[e] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
                        }
                        ar[q][h] = u32x4_t{o[0], o[1], o[2], o[3]};
                    }
                }
#pragma unroll
                for (int hi = 0; hi < 2; ++hi)
#pragma unroll
                    for (int hj = 0; hj < 2; ++hj)
                        acc[hi][hj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ar[q][hi]),
                                                                             __builtin_bit_cast(bf16x8_t, br[q][hj]),
                                                                             acc[hi][hj], 0, 0, 0);
            }
        }
    }
    float* out = a.scores + (size_t)b * (a.topk + (size_t)(a.K - 1) * a.topk * a.topk) +
                 (t == 0 ? 0 : a.topk + (size_t)(t - 1) * a.topk * a.topk);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
#pragma unroll
        for (int hj = 0; hj < 2; ++hj) {
#pragma unroll
            for (int i = 0; i < 16; ++i) part[wave][i][lane] = acc[hi][hj][i];
            __syncthreads();
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int e = tid + 256 * m, L = e & 63, i = e >> 6;
                const float v = part[0][i][L] + part[1][i][L] + part[2][i][L] + part[3][i][L];
                const int pi = 32 * hi + 8 * (i / 4) + 4 * (L / 32) + (i % 4), cj = 32 * hj + (L & 31);
                if (pi < ni && cj < nj) out[(size_t)(i0 + pi) * a.topk + j0 + cj] = s_ub[cj] + v;
            }
            __syncthreads();
        }
    }
}

// Sampling over a candidate set is the draw the whole-vocabulary head makes, restricted to the set: the
// candidates are grouped by vocabulary block (id / 16, aligned blocks of 16 ids); block q's mass S_q (the sum of
// its members' 2^(l c - M), c = log2(e) / T) races with its variate E_q = -log2 u(2 q) (largest S_q / E_q wins,
// ties to the lower block), and inside the winner the id is drawn by inverse CDF over its members in ascending id
// order with target u(2 q + 1) S_q, u(n) the uniform of fmix32(k2 ^ n).  The noise keys on vocabulary blocks,
// never on candidate slots, so a set that holds the whole vocabulary draws what the full head draws.  Members
// are visited in ascending id order through the step's sort permutation.
struct SetDraw {
    int sel;        // position (in ascending id order) of the drawn member
    float total;    // sum of all members' masses
};

// ord[s]: slot of the s-th smallest id; ids[s]: that id; E[s], U2[s]: the race variate and target uniform of its
// block; lmc(slot): l c of a slot; M: max of l c over the set.
template <typename LC>
__device__ __forceinline__ SetDraw draw_set(int n, const int32_t* ord, const int32_t* ids, const float* E,
                                            const float* U2, LC lmc, float M) {
    float total = 0.f, S = 0.f, bS = 0.f, bE = 1.f;
    int beg = 0, bbeg = -1, bend = 0;
    for (int s = 0; s < n; ++s) {
        const float p = fast_exp2(lmc(ord[s]) - M);
        total += p;
        S += p;
        if (s + 1 == n || (ids[s + 1] >> 4) != (ids[s] >> 4)) {  // end of a block's run
            if (S > 0.f && (bbeg < 0 || S * bE > bS * E[s])) {
                bS = S;
                bE = E[s];
                bbeg = beg;
                bend = s + 1;
            }
            S = 0.f;
            beg = s + 1;
        }
    }
    if (bbeg < 0) return SetDraw{0, total};
    const float target = fminf(U2[bbeg] * bS, __uint_as_float(__float_as_uint(bS) - 1u));
    float cum = 0.f;
    int sel = bbeg;
    for (int s = bbeg; s + 1 < bend; ++s) {
        cum += fast_exp2(lmc(ord[s]) - M);
        sel += (cum <= target) ? 1 : 0;
    }
    return SetDraw{sel, total};
}

// One wave per row: K serial picks, reading the row's score tables and candidate ids from global memory (the
// tables too large for the row-parallel walk below even with all of a workgroup's LDS).  In sampling mode the
// step's candidates are ranked by id in LDS and lane 0 makes the draw.
constexpr int kWalkSortMax = 1024;

__global__ void __launch_bounds__(64) walk_kernel(SelectorArgs a) {
    __shared__ int32_t s_ord[kWalkSortMax], s_ids[kWalkSortMax];
    __shared__ float s_E[kWalkSortMax], s_U2[kWalkSortMax];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const size_t tstride = a.topk + (size_t)(a.K - 1) * a.topk * a.topk;
    const float* sc = a.scores + (size_t)b * tstride;
    const int32_t* cands = a.cand + (size_t)b * a.K * a.topk;
    const float c = a.inv_t * kLog2e;
    int islot = 0;
    for (int t = 0; t < a.K; ++t) {
        const float* rowp = (t == 0) ? sc : sc + a.topk + ((size_t)(t - 1) * a.topk + islot) * a.topk;
        const int32_t* cand_t = cands + (size_t)t * a.topk;
        float bk = -INFINITY, bl = 0.f, m = kMinFinite, s = 0.f;
        int bi = 0x7FFFFFFF, bs = 0;
        // unrolled so that a lane's loads of the row are in flight together (same order per lane)
#pragma unroll 8
        for (int j = lane; j < a.topk; j += 64) {
            const float l = rowp[j];
            const int cid = cand_t[j];
            if (beats(l, cid, bk, bi)) {
                bk = l;
                bi = cid;
                bl = l;
                bs = j;
            }
            lse_merge(m, s, l * c, 1.0f);
        }
        // reduce over the lanes that hold candidates (a 16-lane group when topk <= 16)
        const int span = a.topk <= 16 ? 16 : 64;
        for (int off = span >> 1; off > 0; off >>= 1) {
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
        // m is now the largest l c of the set (every lane), bs / bi / bl the greedy pick
        if (a.sample) {
            const uint32_t k2 = noise_key2(a.k0, (uint32_t)b, (uint32_t)t);
            for (int j = lane; j < a.topk; j += 64) {
                const int cid = cand_t[j];
                int rank = 0;
                for (int i = 0; i < a.topk; ++i) rank += cand_t[i] < cid ? 1 : 0;
                const uint32_t q = (uint32_t)cid >> 4;
                s_ord[rank] = j;
                s_ids[rank] = cid;
                s_E[rank] = neg_log2_uniform(fmix32(k2 ^ (2u * q)));
                s_U2[rank] = hash_uniform(fmix32(k2 ^ (2u * q + 1u)));
            }
            __syncthreads();
            if (lane == 0) {
                const SetDraw d = draw_set(a.topk, s_ord, s_ids, s_E, s_U2, [&](int j) { return rowp[j] * c; }, m);
                bs = s_ord[d.sel];
                bi = s_ids[d.sel];
                bl = rowp[bs];
                s = d.total;
            }
            __syncthreads();
        }
        islot = __shfl(bs, 0);
        if (lane == 0) {
            a.tokens[(size_t)b * a.K + t] = bi;
            if (a.logprobs) a.logprobs[(size_t)b * a.K + t] = (bl * c - m - fast_log2(s)) * kLn2;
        }
    }
}

// The walk with every step's choice made in parallel.  A step's pick depends on the path only through the row
// of the pair table it reads (the slot picked one step before); the row's draw (greedy, or the block race with
// noise of row b, step t and the candidates' vocabulary blocks) and its log-sum-exp do not.  So the threads of
// the workgroup take the table rows (the anchor row, then the topk rows of each later table) one per thread, and
// record each row's pick (slot, id, exact log-probability); one thread then follows the path, one LDS read per
// step.  This replaces sixteen dependent cross-lane reductions by one pass over the rows.  The table rows are
// staged in LDS, all at once or, when they exceed it, in chunks of chunk_rows rows (top-64 at K = 16), with a
// pitch of topk + 1 floats, so that the threads' reads of the same column fall in distinct banks.  In sampling
// mode each step's candidates are first ranked by id (one thread per candidate) with their blocks' race
// variates, which every row of that step's table shares.
constexpr int kWalkThreads = 1024;  // 16 waves: the rows of a top-64 table chunk one per thread
constexpr int kWalkLdsMax = 160 * 1024;  // a workgroup's LDS on gfx950

// LDS bytes of everything but the staged table rows
size_t walk_rows_fixed_bytes(int K, int topk) {
    const size_t rows = 1 + (size_t)(K - 1) * topk;
    return 4 * ((size_t)K * topk + 3 * rows + 4 * (size_t)K * topk);
}
size_t walk_rows_row_bytes(int topk) { return 4 * ((size_t)topk + 1); }

// KK: topk fixed at compile time (the loops over a row unrolled, row and column of a staged element by shifts),
// or 0 for any topk.
template <int KK>
__global__ void __launch_bounds__(kWalkThreads) walk_rows_kernel(SelectorArgs a, int chunk_rows) {
    extern __shared__ __attribute__((aligned(16))) float wsh[];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int kk = KK ? KK : a.topk, pitch = kk + 1;
    const int rows = 1 + (a.K - 1) * kk;  // table row `row` holds scores row * kk .. row * kk + kk - 1
    const int tstride = kk + (a.K - 1) * kk * kk;
    const float* sc = a.scores + (size_t)b * tstride;
    const int32_t* cands = a.cand + (size_t)b * a.K * kk;
    int32_t* cs = reinterpret_cast<int32_t*>(wsh);                            // [K][topk] candidate ids
    int32_t* pslot = cs + a.K * kk;                                           // per row: slot of its pick,
    int32_t* pid = pslot + rows;                                              // its id,
    float* plp = reinterpret_cast<float*>(pid + rows);                        // its log-probability
    int32_t* sord = reinterpret_cast<int32_t*>(plp + rows);                   // [K][topk] slots by ascending id,
    int32_t* sids = sord + a.K * kk;                                          // the ids,
    float* sE = reinterpret_cast<float*>(sids + a.K * kk);                    // their blocks' race variates,
    float* sU2 = sE + a.K * kk;                                               // and target uniforms
    float* ss = sU2 + a.K * kk;                                               // [chunk_rows][pitch] table rows
    const float c = a.inv_t * kLog2e;

    for (int e = tid; e < a.K * kk; e += kWalkThreads) cs[e] = cands[e];
    __syncthreads();
    if (a.sample) {
        for (int e = tid; e < a.K * kk; e += kWalkThreads) {
            const int t = e / kk, j = e - t * kk;
            const int32_t* ct = cs + t * kk;
            const int cid = ct[j];
            int rank = 0;
            for (int i = 0; i < kk; ++i) rank += ct[i] < cid ? 1 : 0;
            const uint32_t k2 = noise_key2(a.k0, (uint32_t)b, (uint32_t)t);
            const uint32_t q = (uint32_t)cid >> 4;
            sord[t * kk + rank] = j;
            sids[t * kk + rank] = cid;
            sE[t * kk + rank] = neg_log2_uniform(fmix32(k2 ^ (2u * q)));
            sU2[t * kk + rank] = hash_uniform(fmix32(k2 ^ (2u * q + 1u)));
        }
    }

    for (int r0 = 0; r0 < rows; r0 += chunk_rows) {
        const int nr = min(chunk_rows, rows - r0);
        // stage rows r0 .. r0 + nr - 1 (every thread's loads of a batch are issued before its LDS writes);
        // 16-byte loads when a row is a whole number of them and the tables are 16-byte aligned
        constexpr int kBatch = 16;
        const int e_end = nr * kk;
        const float* src = sc + (size_t)r0 * kk;
        if (KK % 4 == 0 && KK != 0 && ((uintptr_t)sc & 15u) == 0) {
            const f32x4_t* src4 = reinterpret_cast<const f32x4_t*>(src);
            const int q_end = e_end / 4;
            for (int e0 = 0; e0 < q_end; e0 += kBatch * kWalkThreads) {
                f32x4_t v[kBatch];
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    const int e = e0 + q * kWalkThreads + tid;
                    v[q] = e < q_end ? src4[e] : f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    const int e = e0 + q * kWalkThreads + tid;
                    if (e < q_end) {
                        float* d = ss + ((4 * e) / kk) * pitch + (4 * e) % kk;
                        d[0] = v[q].x;
                        d[1] = v[q].y;
                        d[2] = v[q].z;
                        d[3] = v[q].w;
                    }
                }
            }
        } else {
            for (int e0 = 0; e0 < e_end; e0 += kBatch * kWalkThreads) {
                float v[kBatch];
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    const int e = e0 + q * kWalkThreads + tid;
                    v[q] = e < e_end ? src[e] : 0.f;
                }
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    const int e = e0 + q * kWalkThreads + tid;
                    if (e < e_end) ss[(e / kk) * pitch + e % kk] = v[q];
                }
            }
        }
        __syncthreads();

        for (int row = r0 + tid; row < r0 + nr; row += kWalkThreads) {
            const int t = row == 0 ? 0 : 1 + (row - 1) / kk;  // the step whose choice this row makes
            const float* rp = ss + (size_t)(row - r0) * pitch;
            const int32_t* ct = cs + t * kk;
            float bk = -INFINITY, bl = 0.f, M = kMinFinite;
            int bi = 0x7FFFFFFF, bs = 0;
            for (int j = 0; j < kk; ++j) {
                const float l = rp[j];
                const int cid = ct[j];
                if (beats(l, cid, bk, bi)) {
                    bk = l;
                    bi = cid;
                    bl = l;
                    bs = j;
                }
                M = fmaxf(M, l * c);
            }
            float total;
            if (a.sample) {
                const SetDraw d = draw_set(kk, sord + t * kk, sids + t * kk, sE + t * kk, sU2 + t * kk,
                                           [&](int j) { return rp[j] * c; }, M);
                bs = sord[t * kk + d.sel];
                bi = sids[t * kk + d.sel];
                bl = rp[bs];
                total = d.total;
            } else {
                total = 0.f;
                for (int j = 0; j < kk; ++j) total += fast_exp2(rp[j] * c - M);
            }
            pslot[row] = bs;
            pid[row] = bi;
            plp[row] = (bl * c - M - fast_log2(total)) * kLn2;
        }
        __syncthreads();  // the chunk's rows are read before the next chunk overwrites them
    }

    if (tid == 0) {
        int islot = 0;
        for (int t = 0; t < a.K; ++t) {
            const int row = (t == 0) ? 0 : 1 + (t - 1) * kk + islot;
            a.tokens[(size_t)b * a.K + t] = pid[row];
            if (a.logprobs) a.logprobs[(size_t)b * a.K + t] = plp[row];
            islot = pslot[row];
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
    } else if (topk <= 32) {
        if (vec) hipLaunchKernelGGL((topk_kernel<32, true>), dim3(rows), dim3(kTkThreads), 0, st, U, u_stride, V, topk, idx, val);
        else hipLaunchKernelGGL((topk_kernel<32, false>), dim3(rows), dim3(kTkThreads), 0, st, U, u_stride, V, topk, idx, val);
    } else if (topk <= 64) {
        if (vec) hipLaunchKernelGGL((topk_kernel<64, true>), dim3(rows), dim3(kTkThreads), 0, st, U, u_stride, V, topk, idx, val);
        else hipLaunchKernelGGL((topk_kernel<64, false>), dim3(rows), dim3(kTkThreads), 0, st, U, u_stride, V, topk, idx, val);
    } else if (V <= kSortMax) {
        hipLaunchKernelGGL(topk_sort_kernel, dim3(rows), dim3(kTkThreads), 0, st, U, u_stride, V, topk, idx, val);
    } else if (topk <= kRadixMaxK) {
        hipLaunchKernelGGL(topk_radix_kernel, dim3(rows), dim3(kTkThreads), 0, st, U, u_stride, V, topk, idx, val);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int topk_supported(int V, int topk) { return topk >= 1 && topk <= V && (topk <= kRadixMaxK || V <= kSortMax); }

hipError_t launch_pair_scores(const SelectorArgs& a, hipStream_t st) {
    const int nb = (a.topk + kPairBlock - 1) / kPairBlock;
    const dim3 grid(a.B * a.K, nb, nb < 64 ? nb : 64);
    const bool vec = ((uintptr_t)a.A % 16 == 0) && ((uintptr_t)a.Bemb % 16 == 0) && (a.r % (a.bf16 ? 8 : 4) == 0);
    if (a.bf16 && vec && a.r % 16 == 0) {
        if (a.topk <= kPairTile) {
            hipLaunchKernelGGL(pair_score_mfma_kernel, dim3(a.B * a.K, 1, 1), dim3(256), 0, st, a);
        } else {
            const int nt = (a.topk + 63) / 64;
            hipLaunchKernelGGL(pair_score_mfma64_kernel, dim3(a.B * a.K, nt, nt), dim3(256), 0, st, a);
        }
        return hipGetLastError();
    }
    if (a.bf16) {
        if (vec) hipLaunchKernelGGL((pair_score_kernel<uint16_t, true>), grid, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((pair_score_kernel<uint16_t, false>), grid, dim3(256), 0, st, a);
    } else {
        if (vec) hipLaunchKernelGGL((pair_score_kernel<float, true>), grid, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((pair_score_kernel<float, false>), grid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_walk(const SelectorArgs& a, hipStream_t st) {
    // Rows resolved in parallel, the padded tables staged in LDS whole when they fit (160 KB on this part: top-16
    // and top-32 at K = 16), else in chunks of at least a quarter of a workgroup's threads in rows (top-64 at
    // K = 16); otherwise one step at a time from global memory.
    auto allow = [](const void* fn) {
        return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kWalkLdsMax) == hipSuccess
                   ? (size_t)kWalkLdsMax
                   : (size_t)64 * 1024;
    };
    static const size_t lds_cap = std::min(
        std::min(std::min(allow(reinterpret_cast<const void*>(&walk_rows_kernel<0>)),
                          allow(reinterpret_cast<const void*>(&walk_rows_kernel<16>))),
                 allow(reinterpret_cast<const void*>(&walk_rows_kernel<32>))),
        allow(reinterpret_cast<const void*>(&walk_rows_kernel<64>)));
    const size_t fixed = walk_rows_fixed_bytes(a.K, a.topk), per_row = walk_rows_row_bytes(a.topk);
    const size_t rows = 1 + (size_t)(a.K - 1) * a.topk;
    // Chunks of fewer rows than the workgroup has threads would leave most of it idle for every chunk's staging
    // and resolution (top-512 at K = 4 took 1.9 ms so, against 0.02 ms step by step).
    const size_t fit = fixed + per_row <= lds_cap ? (lds_cap - fixed) / per_row : 0;
    if (fit >= rows || fit >= (size_t)kWalkThreads / 4) {
        const size_t chunk = rows < fit ? rows : fit;
        const size_t lds = fixed + chunk * per_row;
        const dim3 g(a.B), blk(kWalkThreads);
        switch (a.topk) {
            case 16: hipLaunchKernelGGL(walk_rows_kernel<16>, g, blk, lds, st, a, (int)chunk); break;
            case 32: hipLaunchKernelGGL(walk_rows_kernel<32>, g, blk, lds, st, a, (int)chunk); break;
            case 64: hipLaunchKernelGGL(walk_rows_kernel<64>, g, blk, lds, st, a, (int)chunk); break;
            default: hipLaunchKernelGGL(walk_rows_kernel<0>, g, blk, lds, st, a, (int)chunk); break;
        }
    } else
        hipLaunchKernelGGL(walk_kernel, dim3(a.B), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace dspark

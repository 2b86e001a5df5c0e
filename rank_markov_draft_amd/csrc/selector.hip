// selector.hip -- the Selector-style truncated execution of the Markov rule.
//
// "DFlash-2's Selector and DSpark's Markov Head: An Equivalence Observation", section "Where the
// parallelism comes from": (1) fix the candidate sets to the top tokens of the base logits at every
// position, (2) compute the calibrated scores of every adjacent (predecessor, candidate) pair in
// parallel, (3) walk.  Section "What the two methods do" gives the score
// S_t(a, b) = U_t(b) + < A(a) (.) H(h_t), B(b) >.
//
// top-k: one workgroup per row streams the row once (independent 16-byte loads); each wave filters the
// elements against the last entry of its exact running top-16 (or top-64) and merges the rare survivors by
// wave arg-max.  Rows with k > 64 (small vocabularies only) are sorted whole in LDS by a bitonic network.
// Pair scores: one workgroup per (row, position, block of 16 predecessors); the 16 gated predecessor
// rows and each block of 16 candidate rows are staged in LDS as fp32 (16-byte loads), one thread per pair.
// Walk: every table row's pick resolved in parallel (greedy, or the whole-vocabulary draw restricted to the
// candidates), then the path followed; tables too large for LDS are walked step by step from global memory.
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
constexpr int kTkBuf = 256;                  // candidate slots per wave
constexpr int kTkSlots = kTkBuf / 64 + 1;    // merge entries per lane: its share of the buffer + one list entry

// Exact top-L (L = 16 or 64) of a wave's list (entry s in lane s, s < L) and the first cnt candidates of its
// buffer: L rounds of wave arg-max under (value desc, id asc).  Entries are distinct (value, id) pairs apart
// from the empty (-inf, INT_MAX) filler, so each round removes exactly the element it emits.
template <int L>
__device__ __forceinline__ void wave_top_merge(const float* bv, const int* bi, int cnt, float& tv, int& ti) {
    const int lane = threadIdx.x & 63;
    float ev[kTkSlots];
    int ei[kTkSlots];
#pragma unroll
    for (int m = 0; m < kTkSlots - 1; ++m) {
        const int e = lane + 64 * m;
        ev[m] = e < cnt ? bv[e] : -INFINITY;
        ei[m] = e < cnt ? bi[e] : 0x7FFFFFFF;
    }
    ev[kTkSlots - 1] = lane < L ? tv : -INFINITY;
    ei[kTkSlots - 1] = lane < L ? ti : 0x7FFFFFFF;
    float nv = -INFINITY;
    int ni = 0x7FFFFFFF;
    for (int out = 0; out < L; ++out) {
        float lv = ev[0];
        int li = ei[0], ls = 0;
#pragma unroll
        for (int m = 1; m < kTkSlots; ++m)
            if (before(ev[m], ei[m], lv, li)) {
                lv = ev[m];
                li = ei[m];
                ls = m;
            }
        float wv = lv;
        int wi = li;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(wv, off);
            const int oi = __shfl_xor(wi, off);
            if (before(ov, oi, wv, wi)) {
                wv = ov;
                wi = oi;
            }
        }
        if (lane == out) {
            nv = wv;
            ni = wi;
        }
        if (lv == wv && li == wi) {
#pragma unroll
            for (int m = 0; m < kTkSlots; ++m)
                if (m == ls) {
                    ev[m] = -INFINITY;
                    ei[m] = 0x7FFFFFFF;
                }
        }
    }
    tv = nv;
    ti = ni;
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

// Top-k (k <= L, L = 16, 32 or 64) of each row, one workgroup per row.  Each wave keeps an exact top-L list (one
// entry per lane 0..L-1) and its L-th entry as a threshold; every element is compared once against the
// threshold and the few that beat it are appended to the wave's LDS buffer, which is merged into the list
// when it fills.  The row is streamed with kTkUnroll independent 16-byte loads per lane, so the scan runs at
// memory speed; the four lists are merged at the end.
template <int L, bool VEC>
__global__ void __launch_bounds__(kTkThreads) __attribute__((amdgpu_waves_per_eu(8))) topk_kernel(const float* __restrict__ U, int64_t u_stride, int V, int k,
                                                          int32_t* __restrict__ idx, float* __restrict__ val) {
    __shared__ float bufv[kTkWaves][kTkBuf];
    __shared__ int bufi[kTkWaves][kTkBuf];
    __shared__ float finv[kTkWaves * L];
    __shared__ int fini[kTkWaves * L];
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
        wave_top_merge<L>(bv, bi, cnt, tv, ti);
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
            if (cnt > kTkBuf - 64) flush();
        }
    };
    if (VEC) {
        const int nq = V >> 2;
        const f32x4_t* u4 = reinterpret_cast<const f32x4_t*>(u);
        for (int q0 = 0; q0 < nq; q0 += kTkThreads * kTkUnroll) {
            f32x4_t x[kTkUnroll];
#pragma unroll
            for (int j = 0; j < kTkUnroll; ++j) {
                const int q = q0 + j * kTkThreads + (int)threadIdx.x;
                x[j] = q < nq ? __builtin_nontemporal_load(u4 + q) : f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            }
            // Prefilter on values alone: an element can enter the list only if it is >= the threshold value
            // (ties are then settled by offer's exact order).  After the first few iterations almost no
            // lane of the wave passes, and one maximum and one ballot cover the lane's 16 elements.
            float mj[kTkUnroll];
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < kTkUnroll; ++j) {
                mj[j] = fmaxf(fmaxf(x[j].x, x[j].y), fmaxf(x[j].z, x[j].w));
                mx = fmaxf(mx, mj[j]);
            }
            if (q0 == 0) {
                // Start the filter at the L-th largest lane maximum of the first chunk: the L lanes at or above
                // it hold L elements at least that large, so no smaller element can enter the wave's top-L.
                // Equal values still pass (id bound INT_MAX) and are settled exactly.  Without it every element
                // of the first chunk is a candidate and the merges of the start dominate the scan.
                thv = wave_lth_largest<L>(mx);
                thi = 0x7FFFFFFF;
            } else if (L > 16 && (q0 / (kTkThreads * kTkUnroll)) % 4 == 0) {
                adopt_shared();  // pick up the other waves' progress now and then
            }
            if (__ballot(mx >= thv)) {
#pragma unroll
                for (int j = 0; j < kTkUnroll; ++j) {
                    if (__ballot(mj[j] >= thv)) {
                        const int q = q0 + j * kTkThreads + (int)threadIdx.x;
                        const int id = q < nq ? 4 * q : 0x7FFFFFFC;
                        offer(x[j].x, id);
                        offer(x[j].y, id + 1);
                        offer(x[j].z, id + 2);
                        offer(x[j].w, id + 3);
                    }
                }
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
    if (lane < L) {
        finv[wave * L + lane] = tv;
        fini[wave * L + lane] = ti;
    }
    __syncthreads();
    if (wave == 0) {
        // the four lists (4 L entries) are merged as buffer entries into an empty list
        float fv = -INFINITY;
        int fi = 0x7FFFFFFF;
        wave_top_merge<L>(finv, fini, kTkWaves * L, fv, fi);
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
    for (int j0 = 0; j0 < a.topk; j0 += kPairBlock) {
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
// step.  This replaces sixteen dependent cross-lane reductions by one pass over the rows.  Rows are staged with
// a pitch of topk + 1 floats, so that the threads' reads of the same column fall in distinct banks.  In
// sampling mode each step's candidates are first ranked by id (one thread per candidate) with their blocks'
// race variates, which every row of that step's table shares.
constexpr int kWalkThreads = 256;
constexpr int kWalkLdsMax = 160 * 1024;  // a workgroup's LDS on gfx950

size_t walk_rows_lds_bytes(int K, int topk) {
    const size_t rows = 1 + (size_t)(K - 1) * topk;
    return 4 * (rows * (topk + 1) + (size_t)K * topk + 3 * rows + 4 * (size_t)K * topk);
}

__global__ void __launch_bounds__(kWalkThreads) walk_rows_kernel(SelectorArgs a) {
    extern __shared__ __attribute__((aligned(16))) float wsh[];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int kk = a.topk, pitch = kk + 1;
    const int rows = 1 + (a.K - 1) * kk;
    const int tstride = kk + (a.K - 1) * kk * kk;
    const float* sc = a.scores + (size_t)b * tstride;
    const int32_t* cands = a.cand + (size_t)b * a.K * kk;
    float* ss = wsh;                                                          // [rows][pitch]
    int32_t* cs = reinterpret_cast<int32_t*>(ss + (size_t)rows * pitch);      // [K][topk] candidate ids
    int32_t* pslot = cs + a.K * kk;                                           // per row: slot of its pick,
    int32_t* pid = pslot + rows;                                              // its id,
    float* plp = reinterpret_cast<float*>(pid + rows);                        // its log-probability
    int32_t* sord = reinterpret_cast<int32_t*>(plp + rows);                   // [K][topk] slots by ascending id,
    int32_t* sids = sord + a.K * kk;                                          // the ids,
    float* sE = reinterpret_cast<float*>(sids + a.K * kk);                    // their blocks' race variates,
    float* sU2 = sE + a.K * kk;                                               // and target uniforms
    const float c = a.inv_t * kLog2e;

    // stage (one round trip: every thread's loads are issued before its LDS writes)
    constexpr int kBatch = 16;
    for (int e0 = 0; e0 < tstride; e0 += kBatch * kWalkThreads) {
        float v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int e = e0 + q * kWalkThreads + tid;
            v[q] = e < tstride ? sc[e] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int e = e0 + q * kWalkThreads + tid;
            if (e < tstride) ss[(e / kk) * pitch + e % kk] = v[q];
        }
    }
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
        __syncthreads();
    }

    for (int row = tid; row < rows; row += kWalkThreads) {
        const int t = row == 0 ? 0 : 1 + (row - 1) / kk;  // the step whose choice this row makes
        const float* rp = ss + (size_t)row * pitch;
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
    __syncthreads();

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
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int topk_supported(int V, int topk) { return topk >= 1 && topk <= V && (topk <= 64 || V <= kSortMax); }

hipError_t launch_pair_scores(const SelectorArgs& a, hipStream_t st) {
    const dim3 grid(a.B * a.K, (a.topk + kPairBlock - 1) / kPairBlock);
    const bool vec = ((uintptr_t)a.A % 16 == 0) && ((uintptr_t)a.Bemb % 16 == 0) && (a.r % (a.bf16 ? 8 : 4) == 0);
    if (a.bf16 && vec && a.r % 16 == 0) {
        const int nt = (a.topk + kPairTile - 1) / kPairTile;
        hipLaunchKernelGGL(pair_score_mfma_kernel, dim3(a.B * a.K, nt, nt), dim3(256), 0, st, a);
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
    // Rows resolved in parallel when the padded tables fit the workgroup's LDS (160 KB on this part: top-16 and
    // top-32 at K = 16); else one step at a time from global memory (top-64 at K = 16).
    static const size_t rows_cap = hipFuncSetAttribute(reinterpret_cast<const void*>(&walk_rows_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kWalkLdsMax) == hipSuccess
                                       ? (size_t)kWalkLdsMax
                                       : (size_t)64 * 1024;
    const size_t rows_lds = walk_rows_lds_bytes(a.K, a.topk);
    if (rows_lds <= rows_cap) hipLaunchKernelGGL(walk_rows_kernel, dim3(a.B), dim3(kWalkThreads), rows_lds, st, a);
    else hipLaunchKernelGGL(walk_kernel, dim3(a.B), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace dspark

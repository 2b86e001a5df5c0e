// gate.hip -- H = sigmoid(h Wg) for every draft position at once.
//
// The equivalence page ("DFlash-2's Selector and DSpark's Markov Head"), section "What the two methods
// do", computes the gate H(h_t) from the current hidden state; the pages give no formula, and this
// library takes a bias-free linear map followed by the logistic sigmoid.  The product is one bf16
// matrix-core GEMM [rows, D] x [D, r] with fp32 accumulation, off the serial draft loop.
//
// Workgroup = eight waves sharing one 32 x 32 output tile; wave w accumulates the 64-wide k steps
// [w n / 8, (w + 1) n / 8) of the n = D / 64 steps (split-K inside the workgroup, summed in a fixed order
// through LDS, so the result is deterministic).  Per k step a wave reads its h block [32 rows x 64 k] with
// eight lanes per 128-byte row segment (whole cache lines; fragment-shaped loads, 32 bytes from each of 32
// rows per instruction, made L2 serve quarter lines) and stages it through LDS for the A fragments, and it
// stages the Wg block [64 k x 32 n] transposed through LDS so that B fragments are k-contiguous too.  The
// next step's loads are issued before the current step's MFMAs.
// The product is small (one workgroup per output tile: 256 at 1024 rows x r = 256) and each step waits on
// memory, so the k range is split eight ways: two waves per SIMD hide each other's waits and each wave's
// chain is short (at rows = 1024, D = 4096, r = 256, event-timed with launch: 21.7 us with four waves, 17.6
// with eight, 20.0 with sixteen; four k steps of loads in flight per wave instead of one: 19.5).  Same-box
// A/B at that shape: the whole-line h loads 21.3 -> 20.7 us.  Not kept: two k steps of loads in flight (21.4
// us); the Wg transpose written as 32-bit (k, k + 1) pairs after a swap between lanes l and l ^ 4 (21.4 us;
// leaving the transpose stores out altogether would save 2.5 us); each workgroup taking its k chunks in a
// rotated order so that the workgroups sharing h rows or Wg columns do not read the same lines at once
// (20.7 us).  What remains is the tiling: the 32 x 32 tiles re-read h once per column block and Wg once per
// row block, about 128 MB of L2 reads for 10.5 MB of operands; the split-K form below (taken when the caller
// gives a workspace) uses 64 x 64 tiles and halves that.
#include <algorithm>

#include "internal.hpp"

namespace dspark {

namespace {

constexpr int kGateWaves = 8;
constexpr int kGateThreads = 64 * kGateWaves;
constexpr int kKStep = 64;                   // k per iteration and wave
constexpr int kBtStride = kKStep + 8;        // bf16 elements per LDS row of the transposed Wg block
constexpr int kAtStride = kKStep + 8;        // bf16 elements per LDS row of the h block

struct GateLoads {
    u32x4_t a[4];  // h[row0 + 8*i + lane/8][k0 + 8*(lane%8) .. +8], i = 0..3
    u32x4_t w[4];  // Wg[k0 + krow][n0 + 8*nch .. +8] for chunk c = lane + 64*q
};

__device__ __forceinline__ void gate_load(GateLoads& L, const uint16_t* __restrict__ h, const uint16_t* __restrict__ Wg,
                                          int rows, int D, int r, int row0, int n0, int k0, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = row0 + 8 * i + (lane >> 3);
        L.a[i] = (row < rows) ? *reinterpret_cast<const u32x4_t*>(h + (size_t)row * D + k0 + 8 * (lane & 7))
                              : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = lane + 64 * q;  // 256 chunks: 64 k-rows x 4 chunks of 8 n
        const int krow = c >> 2, nch = c & 3;
        L.w[q] = *reinterpret_cast<const u32x4_t*>(Wg + (size_t)(k0 + krow) * r + n0 + 8 * nch);
    }
}

__global__ void __launch_bounds__(kGateThreads) gate_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ Wg,
                                                          int rows, int D, int r, float* __restrict__ H) {
    __shared__ __attribute__((aligned(16))) uint16_t bt[kGateWaves][32 * kBtStride];
    __shared__ __attribute__((aligned(16))) uint16_t at[kGateWaves][32 * kAtStride];
    __shared__ float red[kGateWaves - 1][32 * 32];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
    const int row0 = blockIdx.x * 32, n0 = blockIdx.y * 32;
    const int nsteps = D / kKStep;
    const int kbeg = (wave * nsteps / kGateWaves) * kKStep, kend = ((wave + 1) * nsteps / kGateWaves) * kKStep;

    f32x16_t acc = {};
    GateLoads cur, nxt;
    if (kbeg < kend) gate_load(cur, h, Wg, rows, D, r, row0, n0, kbeg, lane);
    uint16_t* my = bt[wave];
    uint16_t* ma = at[wave];
    for (int k0 = kbeg; k0 < kend; k0 += kKStep) {
        if (k0 + kKStep < kend) gate_load(nxt, h, Wg, rows, D, r, row0, n0, k0 + kKStep, lane);
        // the h block into LDS as loaded: ma[row][k]
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4_t*>(ma + (8 * i + (lane >> 3)) * kAtStride + 8 * (lane & 7)) = cur.a[i];
        // transpose the Wg block into LDS: my[n][k]
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = lane + 64 * q;
            const int krow = c >> 2, nch = c & 3;
            const uint32_t wv[4] = {cur.w[q].x, cur.w[q].y, cur.w[q].z, cur.w[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                my[(8 * nch + 2 * e) * kBtStride + krow] = (uint16_t)(wv[e] & 0xFFFFu);
                my[(8 * nch + 2 * e + 1) * kBtStride + krow] = (uint16_t)(wv[e] >> 16);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): LDS writes of this wave done
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(ma + (lane & 31) * kAtStride + 16 * kk + 8 * half);
            const bf16x8_t bf = *reinterpret_cast<const bf16x8_t*>(my + (lane & 31) * kBtStride + 16 * kk + 8 * half);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
        if (k0 + kKStep < kend) cur = nxt;
    }
    // split-K sum in a fixed order: wave 0 + wave 1 + ... + wave 7
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) red[wave - 1][i * 64 + lane] = acc[i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float z = acc[i];
#pragma unroll
            for (int w = 0; w < kGateWaves - 1; ++w) z += red[w][i * 64 + lane];
            const int m = row0 + 8 * (i >> 2) + 4 * half + (i & 3);
            const int n = n0 + (lane & 31);
            if (m < rows) H[(size_t)m * r + n] = 1.0f / (1.0f + __expf(-z));
        }
    }
}

// Split-K form (a workspace is given): 64 x 64 output tiles, so h is re-read once per 64 columns and Wg once
// per 64 rows (half the reads of the 32 x 32 tiles), with the k range split over kSkSplits workgroups per tile to
// keep 256 workgroups at 1024 rows x r = 256.  Eight waves: four 32 x 32 sub-tiles x two halves of the
// workgroup's k slice.  Per 64-wide k step the 256 threads of a k half stage its h block [64 rows x 64 k] and
// Wg block [64 k x 64 n] (transposed to [n][k]) once into a double-buffered LDS stage that its four waves read.
// The two halves are summed in LDS (half 0 + half 1) and each workgroup writes its slice's partial sums; a
// second kernel adds the slices in order (((p0 + p1) + p2) + p3) and applies the sigmoid, so the result is
// deterministic.  At rows 1024, D 4096, r 256 (same box, event-timed with launch): 20.7 us unsplit, 18.4 us
// split (12.9 + 4.0 us of kernel time).  Not kept: two k steps of loads in flight (19.2 us); the slices summed
// by the last of a tile's workgroups to finish (per-tile arrival words) instead of a second launch: 23.2 us
// with the partial sums stored and read at device scope, 62.8 us with a device-wide fence per workgroup
// instead (each wrote back its XCD's L2); the sum as one workgroup per 64 x 64 tile on the split-K grid, so that
// it runs on the XCD that wrote the tile (20.2 against 19.0 us: 64 workgroups are too few).
constexpr int kSkSplits = 4;
constexpr int kSkWaves = 8;
constexpr int kSkThreads = 64 * kSkWaves;

struct SkLoads {
    u32x4_t h[2];  // chunk c = t + 256 i: h[row0 + c / 8][k0 + 8 (c % 8) .. +8]
    u32x4_t w[2];  // chunk c = t + 256 i: Wg[k0 + c / 8][n0 + 8 (c % 8) .. +8]
};

__device__ __forceinline__ void sk_load(SkLoads& L, const uint16_t* __restrict__ h, const uint16_t* __restrict__ Wg,
                                        int rows, int D, int r, int row0, int n0, int k0, int t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = t + 256 * i;
        const int row = row0 + (c >> 3);
        L.h[i] = row < rows ? *reinterpret_cast<const u32x4_t*>(h + (size_t)row * D + k0 + 8 * (c & 7))
                            : u32x4_t{0u, 0u, 0u, 0u};
        L.w[i] = *reinterpret_cast<const u32x4_t*>(Wg + (size_t)(k0 + (c >> 3)) * r + n0 + 8 * (c & 7));
    }
}

__device__ __forceinline__ void sk_store(const SkLoads& L, uint16_t* __restrict__ hb, uint16_t* __restrict__ wb, int t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = t + 256 * i;
        const int row = c >> 3, ch = c & 7;  // h: row, k chunk; Wg: k-row, n chunk
        *reinterpret_cast<u32x4_t*>(hb + row * kAtStride + 8 * ch) = L.h[i];
        const uint32_t wv[4] = {L.w[i].x, L.w[i].y, L.w[i].z, L.w[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wb[(8 * ch + 2 * e) * kBtStride + row] = (uint16_t)(wv[e] & 0xFFFFu);
            wb[(8 * ch + 2 * e + 1) * kBtStride + row] = (uint16_t)(wv[e] >> 16);
        }
    }
}

__global__ void __launch_bounds__(kSkThreads) gate_splitk_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ Wg,
                                                               int rows, int D, int r, float* __restrict__ P) {
    __shared__ __attribute__((aligned(16))) uint16_t hst[2][2][64 * kAtStride];  // [stage][k half][row][k]
    __shared__ __attribute__((aligned(16))) uint16_t wst[2][2][64 * kBtStride];  // [stage][k half][n][k]
    __shared__ float red[4][32 * 32];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
    const int sub = wave & 3, kh = wave >> 2, t = threadIdx.x & 255;
    const int row0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
    const int rs = 32 * (sub & 1), cs = 32 * (sub >> 1);
    const int kslice = D / kSkSplits, khalf = kslice / 2;
    const int kbeg = blockIdx.z * kslice + kh * khalf;
    const int nsteps = khalf / kKStep;

    f32x16_t acc = {};
    SkLoads cur;
    sk_load(cur, h, Wg, rows, D, r, row0, n0, kbeg, t);
    for (int s = 0; s < nsteps; ++s) {
        uint16_t* hb = hst[s & 1][kh];
        uint16_t* wb = wst[s & 1][kh];
        // stage s & 1 was last read at step s - 2, before every wave passed the barrier of step s - 1
        sk_store(cur, hb, wb, t);
        if (s + 1 < nsteps) sk_load(cur, h, Wg, rows, D, r, row0, n0, kbeg + (s + 1) * kKStep, t);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(hb + (rs + (lane & 31)) * kAtStride + 16 * kk + 8 * half);
            const bf16x8_t bf = *reinterpret_cast<const bf16x8_t*>(wb + (cs + (lane & 31)) * kBtStride + 16 * kk + 8 * half);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
        }
    }
    if (kh == 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) red[sub][i * 64 + lane] = acc[i];
    }
    __syncthreads();
    if (kh == 0) {
        float* out = P + (size_t)blockIdx.z * rows * r;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = row0 + rs + 8 * (i >> 2) + 4 * half + (i & 3);
            const int n = n0 + cs + (lane & 31);
            if (m < rows) out[(size_t)m * r + n] = acc[i] + red[sub][i * 64 + lane];
        }
    }
}

// H = sigmoid(((p0 + p1) + p2) + p3), four values per thread (rows * r is a multiple of 64)
__global__ void __launch_bounds__(256) gate_reduce_kernel(const float* __restrict__ P, size_t n, float* __restrict__ H) {
    const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
    for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
        f32x4_t z = *reinterpret_cast<const f32x4_t*>(P + i);
#pragma unroll
        for (int sl = 1; sl < kSkSplits; ++sl) {
            const f32x4_t p = *reinterpret_cast<const f32x4_t*>(P + sl * n + i);
            z.x += p.x;
            z.y += p.y;
            z.z += p.z;
            z.w += p.w;
        }
        *reinterpret_cast<f32x4_t*>(H + i) = f32x4_t{1.0f / (1.0f + __expf(-z.x)), 1.0f / (1.0f + __expf(-z.y)),
                                                     1.0f / (1.0f + __expf(-z.z)), 1.0f / (1.0f + __expf(-z.w))};
    }
}

}  // namespace

size_t gate_splitk_bytes(int rows, int D, int r) {
    if (rows <= 0 || r % 64 != 0 || D % (kSkSplits * 2 * kKStep) != 0) return 0;
    return (size_t)kSkSplits * (size_t)rows * (size_t)r * sizeof(float);
}

hipError_t launch_gate(const uint16_t* h, const uint16_t* Wg, int rows, int D, int r, float* H, void* workspace,
                       size_t workspace_bytes, hipStream_t st) {
    const size_t need = gate_splitk_bytes(rows, D, r);
    if (need > 0 && workspace && workspace_bytes >= need && ((uintptr_t)workspace & 15u) == 0 && ((uintptr_t)H & 15u) == 0) {
        float* P = static_cast<float*>(workspace);
        hipLaunchKernelGGL(gate_splitk_kernel, dim3((rows + 63) / 64, r / 64, kSkSplits), dim3(kSkThreads), 0, st, h, Wg,
                           rows, D, r, P);
        const size_t n = (size_t)rows * r;
        const size_t blocks = std::min<size_t>((n / 4 + 255) / 256, 4096);
        hipLaunchKernelGGL(gate_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, P, n, H);
        return hipGetLastError();
    }
    const dim3 grid((rows + 31) / 32, r / 32), block(kGateThreads);
    hipLaunchKernelGGL(gate_kernel, grid, block, 0, st, h, Wg, rows, D, r, H);
    return hipGetLastError();
}

}  // namespace dspark

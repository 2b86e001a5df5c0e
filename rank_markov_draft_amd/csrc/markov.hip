// markov.hip -- one calibrated position of the Markov head: bias contraction, calibration, pick.
//
// The rule ("DFlash-2's Selector and DSpark's Markov Head: An Equivalence Observation", sections "What
// the two methods do" and "The equivalence"): l_k[b, v] = U_k[b, v] + (W1[a_b] (.) H_k[b])^T W2[:, v],
// followed by a pick over the whole vocabulary (the DSpark overview, "The Markov head") and the exact
// local log-softmax of the picked token ("DSpark: Repair the Joint, Meter the Verify", "Why the
// normalization has to be local").
//
// Matrix-core kernel (bf16 weights, W2 stored [V, r]).  Each workgroup owns a contiguous range of
// 32-wide vocabulary tiles and 128 batch rows; wave w owns rows 32w .. 32w+31.  Per tile the product
// is computed transposed, C[v, b] = sum_j W2t[v, j] X[b, j], with v_mfma_f32_32x32x16_bf16: the W2 tile
// (A operand, shared by the four waves) is staged in LDS, the gathered predecessor rows X (B operand)
// stay in registers for the whole position.  In the 32x32 accumulator a lane holds one batch row
// (b = lane % 32) and 16 vocabulary ids, so the calibration, the streaming log-sum-exp and the running
// arg-max are per-lane scalars, and U_k is read as four 16-byte vectors per lane.  No logits are written.
#include "common.hpp"
#include "internal.hpp"

namespace dspark {

namespace {

constexpr int kThreads = 256;
constexpr int kTileV = 32;
constexpr int kRowsPerWG = 128;

// LDS row stride of a staged W2 tile: r bf16 plus 16 bytes, so that eight consecutive rows read at the
// same column land in distinct 16-byte bank groups.
template <int RK>
struct TileGeom {
    static constexpr int kRowBytes = RK * 32;  // r = 16 * RK bf16
    static constexpr int kStride = kRowBytes + 16;
    static constexpr int kBytes = kTileV * kStride;
    static constexpr int kChunks = kTileV * RK * 2;  // 16-byte chunks per tile
    static constexpr int kChunksPerThread = (kChunks + kThreads - 1) / kThreads;
};

template <int RK>
__device__ __forceinline__ void load_w2_tile(const uint16_t* __restrict__ W2t, int V, int v0, u32x4_t (&reg)[TileGeom<RK>::kChunksPerThread]) {
    using G = TileGeom<RK>;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(W2t + (size_t)v0 * (16 * RK));
#pragma unroll
    for (int q = 0; q < G::kChunksPerThread; ++q) {
        int c = threadIdx.x + q * kThreads;
        int row = c / (2 * RK);
        if (c < G::kChunks && v0 + row < V) {
            reg[q] = load_nt_u32x4(src + c);
        } else {
            reg[q] = u32x4_t{0u, 0u, 0u, 0u};
        }
    }
}

template <int RK>
__device__ __forceinline__ void store_w2_tile(uint8_t* lds, const u32x4_t (&reg)[TileGeom<RK>::kChunksPerThread]) {
    using G = TileGeom<RK>;
#pragma unroll
    for (int q = 0; q < G::kChunksPerThread; ++q) {
        int c = threadIdx.x + q * kThreads;
        if (c < G::kChunks) {
            int row = c / (2 * RK), ch = c % (2 * RK);
            *reinterpret_cast<u32x4_t*>(lds + w2_slot(row) * G::kStride + ch * 16) = reg[q];
        }
    }
}

// U_k values of this lane's row for the 16 accumulator slots of tile v0: slot i <-> v0 + 16*half + i (the W2
// tile is staged in w2_slot order).
template <bool VEC>
__device__ __forceinline__ void load_u_tile(const float* __restrict__ urow, bool valid_b, int V, int v0, int half, float (&u)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        int v = v0 + 16 * half + 4 * q;
        if (VEC) {
            f32x4_t x = {0.f, 0.f, 0.f, 0.f};
            if (valid_b && v < V) x = load_nt_f32x4(urow + v);
            u[4 * q + 0] = x.x;
            u[4 * q + 1] = x.y;
            u[4 * q + 2] = x.z;
            u[4 * q + 3] = x.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) u[4 * q + e] = (valid_b && v + e < V) ? urow[v + e] : 0.f;
        }
    }
}

template <int RK, int MODE, bool GATED, bool VEC_U>
__global__ void __launch_bounds__(kThreads, 2) markov_step_mfma(StepArgs a) {
    constexpr bool SAMPLE = MODE == kModeSample;
    constexpr bool STORE = MODE == kModeStore;
    using G = TileGeom<RK>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][G::kBytes];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int b = blockIdx.y * kRowsPerWG + wave * 32 + (lane & 31);
    const bool valid_b = b < a.B;
    const int r = 16 * RK;

    const int tile_begin = (int)(((long long)blockIdx.x * a.ntiles) / gridDim.x);
    const int tile_end = (int)(((long long)(blockIdx.x + 1) * a.ntiles) / gridDim.x);

    u32x4_t wreg[G::kChunksPerThread];
    float ureg[16];
    const float* urow = a.U + (size_t)(valid_b ? b : 0) * a.u_stride;
    if (tile_begin < tile_end) {
        load_w2_tile<RK>(a.W2t, a.V, tile_begin * kTileV, wreg);
        load_u_tile<VEC_U>(urow, valid_b, a.V, tile_begin * kTileV, half, ureg);
    }

    // Gather the predecessor embedding into B-operand fragments: lane holds X[b, 16*kk + 8*half + 0..7].
    bf16x8_t xf[RK];
    {
        const int p = valid_b ? a.prev[(size_t)b * a.prev_stride] : 0;
        const u32x4_t* wrow = reinterpret_cast<const u32x4_t*>(a.W1 + (size_t)p * r);
#pragma unroll
        for (int kk = 0; kk < RK; ++kk) {
            u32x4_t raw = valid_b ? wrow[2 * kk + half] : u32x4_t{0u, 0u, 0u, 0u};
            if (GATED && valid_b) {
                const float* hrow = a.H + (size_t)b * a.h_stride + 16 * kk + 8 * half;
                f32x4_t h0 = *reinterpret_cast<const f32x4_t*>(hrow);
                f32x4_t h1 = *reinterpret_cast<const f32x4_t*>(hrow + 4);
                float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
                uint32_t w32[4] = {raw.x, raw.y, raw.z, raw.w};
                uint32_t o32[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float lo = bf16_to_f32((uint16_t)(w32[e] & 0xFFFFu)) * hv[2 * e];
                    float hi = bf16_to_f32((uint16_t)(w32[e] >> 16)) * hv[2 * e + 1];
                    o32[e] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
                }
                raw = u32x4_t{o32[0], o32[1], o32[2], o32[3]};
            }
            xf[kk] = __builtin_bit_cast(bf16x8_t, raw);
        }
    }

    uint32_t k2 = 0;
    if (SAMPLE) k2 = noise_key2(a.k0, (uint32_t)b, (uint32_t)a.k);

    float bk = -INFINITY, bl = 0.f, m = kMinFinite, s = 0.f;
    int bi = 0x7FFFFFFF;
    // sampling (two-level exponential race over the lane's aligned 16-id blocks): mass of the best block so
    // far and of the id drawn in it (scaled as s), and the block's race variate
    float bs = 0.f, bE = 1.f, be = 0.f;

    if (tile_begin < tile_end) store_w2_tile<RK>(lds[0], wreg);
    __syncthreads();

    for (int t = tile_begin; t < tile_end; ++t) {
        const int buf = (t - tile_begin) & 1;
        const int v0 = t * kTileV;
        float ucur[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) ucur[i] = ureg[i];
        if (t + 1 < tile_end) {
            load_w2_tile<RK>(a.W2t, a.V, v0 + kTileV, wreg);
            load_u_tile<VEC_U>(urow, valid_b, a.V, v0 + kTileV, half, ureg);
        }

        f32x16_t acc = {};
        const uint8_t* arow = lds[buf] + (lane & 31) * G::kStride + half * 16;
#pragma unroll
        for (int kk = 0; kk < RK; ++kk) {
            bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(arow + kk * 32);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, xf[kk], acc, 0, 0, 0);
        }

        if (STORE) {
            // validation epilogue: write the calibrated logits
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int v = v0 + 16 * half + i;
                if (valid_b && v < a.V) a.logits_out[(size_t)b * a.V + v] = acc[i] + ucur[i];
            }
        } else {
            // calibrate, stream the log-sum-exp, track the arg-max
            float lv[16], tv[16];
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int v = v0 + 16 * half + i;
                const bool ok = valid_b && v < a.V;
                lv[i] = acc[i] + ucur[i];
                tv[i] = ok ? lv[i] * a.c : -INFINITY;
                tmax = fmaxf(tmax, tv[i]);
            }
            const float mn = fmaxf(m, tmax);
            const float scale = fast_exp2(m - mn);
            s *= scale;
            m = mn;
            if (SAMPLE) {
                // the lane's 16 ids are the aligned block q = v0 / 16 + half: its mass, race and drawn id
                bs *= scale;
                be *= scale;
                float e[16], sb = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    e[i] = fast_exp2(tv[i] - m);
                    sb += e[i];
                }
                s += sb;
                float E, target;
                block_race_variates(k2, (uint32_t)(v0 / 16 + half), sb, E, target);
                float cum = 0.f, esel = e[0];
                int sel = 0;
#pragma unroll
                for (int i = 0; i < 15; ++i) {
                    cum += e[i];
                    const bool below = cum <= target;
                    sel += below ? 1 : 0;
                    esel = below ? e[i + 1] : esel;
                }
                if (sb * bE > bs * E) {
                    bs = sb;
                    bE = E;
                    be = esel;
                    bi = v0 + 16 * half + sel;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) s += fast_exp2(tv[i] - m);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int v = v0 + 16 * half + i;
                    const float key = (valid_b && v < a.V) ? lv[i] : -INFINITY;
                    if (key > bk) {
                        bk = key;
                        bi = v;
                        bl = lv[i];
                    }
                }
            }
        }

        if (t + 1 < tile_end) store_w2_tile<RK>(lds[buf ^ 1], wreg);
        __syncthreads();
    }

    if (STORE) return;
    if (SAMPLE && bs > 0.f) {
        // race key log2(S / E) with S in absolute units; the drawn id's logit from its mass
        bk = fast_log2(bs) + m - fast_log2(bE);
        bl = (fast_log2(be) + m) / a.c;
    }
    // lanes l and l + 32 hold the same row
    {
        float ok_ = __shfl_xor(bk, 32);
        int oi = __shfl_xor(bi, 32);
        float ol = __shfl_xor(bl, 32);
        float om = __shfl_xor(m, 32);
        float os = __shfl_xor(s, 32);
        if (beats(ok_, oi, bk, bi)) {
            bk = ok_;
            bi = oi;
            bl = ol;
        }
        lse_merge(m, s, om, os);
    }
    if (half == 0 && valid_b) {
        const size_t o = (size_t)blockIdx.x * a.Bpad + b;
        a.part.key[o] = bk;
        a.part.idx[o] = bi;
        a.part.l[o] = bl;
        a.part.m[o] = m;
        a.part.s[o] = s;
    }
}

// ------------------------------------------------------------------------------------------------
// Vector-ALU kernel: fp32 or bf16 weights, any W2 layout (element (j, v) at W2[j*sj + v*sv]), any r.
// Four batch rows per workgroup; the gathered rows live in LDS as fp32; each thread owns columns.
// ------------------------------------------------------------------------------------------------

constexpr int kValuRows = 4;

template <typename WT>
__device__ __forceinline__ float wload(const WT* p, size_t i);
template <>
__device__ __forceinline__ float wload<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float wload<uint16_t>(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

template <typename WT, int MODE, bool GATED>
__global__ void __launch_bounds__(kThreads) markov_step_valu(StepArgsValu a) {
    constexpr bool SAMPLE = MODE == kModeSample;
    constexpr bool STORE = MODE == kModeStore;
    extern __shared__ float xs[];  // [kValuRows][r]
    const WT* W1 = reinterpret_cast<const WT*>(a.W1);
    const WT* W2 = reinterpret_cast<const WT*>(a.W2);
    const int r = a.r;
    for (int i = threadIdx.x; i < kValuRows * r; i += kThreads) {
        const int rb = i / r, j = i % r;
        const int b = blockIdx.y * kValuRows + rb;
        float x = 0.f;
        if (b < a.B) {
            const int p = a.prev[(size_t)b * a.prev_stride];
            x = wload<WT>(W1, (size_t)p * r + j);
            if (GATED) x *= a.H[(size_t)b * a.h_stride + j];
        }
        xs[i] = x;
    }
    __syncthreads();

    float bk[kValuRows], bl[kValuRows], m[kValuRows], s[kValuRows];
    int bi[kValuRows];
    uint32_t k2[kValuRows];
#pragma unroll
    for (int rb = 0; rb < kValuRows; ++rb) {
        bk[rb] = -INFINITY;
        bl[rb] = 0.f;
        m[rb] = kMinFinite;
        s[rb] = 0.f;
        bi[rb] = 0x7FFFFFFF;
        k2[rb] = SAMPLE ? noise_key2(a.k0, (uint32_t)(blockIdx.y * kValuRows + rb), (uint32_t)a.k) : 0u;
    }
    // Every thread of the workgroup runs the same iterations (the sampling race works on groups of 16 lanes):
    // thread t takes id v0 + t of each 256-id span.
    const int g16 = threadIdx.x & 15;
    for (int v0 = blockIdx.x * kThreads; v0 < a.V; v0 += gridDim.x * kThreads) {
        const int v = v0 + threadIdx.x;
        const bool inr = v < a.V;
        float acc[kValuRows] = {};
        if (inr) {
            for (int j = 0; j < r; ++j) {
                const float w = wload<WT>(W2, (size_t)j * a.sj + (size_t)v * a.sv);
#pragma unroll
                for (int rb = 0; rb < kValuRows; ++rb) acc[rb] = fmaf(xs[rb * r + j], w, acc[rb]);
            }
        }
#pragma unroll
        for (int rb = 0; rb < kValuRows; ++rb) {
            const int b = blockIdx.y * kValuRows + rb;
            if (b >= a.B) continue;  // uniform over the workgroup
            const float l = inr ? acc[rb] + a.U[(size_t)b * a.u_stride + v] : 0.f;
            if (STORE) {
                if (inr) a.logits_out[(size_t)b * a.V + v] = l;
                continue;
            }
            const float t = inr ? l * a.c : -INFINITY;
            const float mn = fmaxf(m[rb], t);
            s[rb] = s[rb] * fast_exp2(m[rb] - mn) + fast_exp2(t - mn);
            m[rb] = mn;
            if (SAMPLE) {
                // Whole-vocabulary draw, block of ids v - g16 .. v - g16 + 15 (16 lanes): block max, masses,
                // inclusive prefix masses in id order, the race variate and the inverse-CDF draw.
                float M = t;
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 16));
                const float e = inr ? fast_exp2(t - M) : 0.f;
                float P = e;
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) {
                    const float y = __shfl_up(P, off, 16);
                    if (g16 >= off) P += y;
                }
                const float S = __shfl(P, 15, 16);
                if (S > 0.f) {
                    float E, target;
                    block_race_variates(k2[rb], (uint32_t)((v - g16) / 16), S, E, target);
                    const unsigned long long below = __ballot(P <= target && g16 < 15);
                    const int sel = __popcll((below >> (threadIdx.x & 48)) & 0x7FFFull);
                    const float key = fast_log2(S) + M - fast_log2(E);
                    const float lsel = __shfl(l, sel, 16);
                    if (key > bk[rb]) {
                        bk[rb] = key;
                        bi[rb] = v - g16 + sel;
                        bl[rb] = lsel;
                    }
                }
            } else if (inr && l > bk[rb]) {
                bk[rb] = l;
                bi[rb] = v;
                bl[rb] = l;
            }
        }
    }
    if (STORE) return;
    // workgroup reduction per row
    __shared__ float rk[kThreads], rl[kThreads], rm[kThreads], rs[kThreads];
    __shared__ int ri[kThreads];
    for (int rb = 0; rb < kValuRows; ++rb) {
        rk[threadIdx.x] = bk[rb];
        ri[threadIdx.x] = bi[rb];
        rl[threadIdx.x] = bl[rb];
        rm[threadIdx.x] = m[rb];
        rs[threadIdx.x] = s[rb];
        __syncthreads();
        for (int w = kThreads / 2; w > 0; w >>= 1) {
            if (threadIdx.x < w) {
                const int o = threadIdx.x + w;
                if (beats(rk[o], ri[o], rk[threadIdx.x], ri[threadIdx.x])) {
                    rk[threadIdx.x] = rk[o];
                    ri[threadIdx.x] = ri[o];
                    rl[threadIdx.x] = rl[o];
                }
                float mm = rm[threadIdx.x], ss = rs[threadIdx.x];
                lse_merge(mm, ss, rm[o], rs[o]);
                rm[threadIdx.x] = mm;
                rs[threadIdx.x] = ss;
            }
            __syncthreads();
        }
        const int b = blockIdx.y * kValuRows + rb;
        if (threadIdx.x == 0 && b < a.B) {
            const size_t o = (size_t)blockIdx.x * a.Bpad + b;
            a.part.key[o] = rk[0];
            a.part.idx[o] = ri[0];
            a.part.l[o] = rl[0];
            a.part.m[o] = rm[0];
            a.part.s[o] = rs[0];
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------------------
// The whole round for small problems (V r <= kValuRoundMaxVR, shapes the matrix-core round kernel does not
// take): one workgroup per kValuRows rows covers the whole vocabulary at every position, so the K positions
// run in one launch, each row's predecessor kept in LDS.  Per position the arithmetic is markov_step_valu's
// over a single vocabulary span; the workgroup's threads are then merged as markov_reduce merges partials.
// ------------------------------------------------------------------------------------------------
template <typename WT, int MODE, bool GATED>
__global__ void __launch_bounds__(kThreads) markov_round_valu(RoundValuArgs a) {
    constexpr bool SAMPLE = MODE == kModeSample;
    extern __shared__ float xs[];  // [kValuRows][r]
    __shared__ int s_prev[kValuRows];
    __shared__ float rk[kThreads / 64], rl[kThreads / 64], rm[kThreads / 64], rs[kThreads / 64];
    __shared__ int ri[kThreads / 64];
    const WT* W1 = reinterpret_cast<const WT*>(a.W1);
    const WT* W2 = reinterpret_cast<const WT*>(a.W2);
    const int r = a.r;
    const int g16 = threadIdx.x & 15;
    const int b0 = blockIdx.x * kValuRows;
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.error) *a.error = 0u;
    if (threadIdx.x < kValuRows)
        s_prev[threadIdx.x] = b0 + (int)threadIdx.x < a.B ? min(max(a.anchor[b0 + threadIdx.x], 0), a.V - 1) : 0;
    __syncthreads();
    for (int k = 0; k < a.K; ++k) {
        for (int i = threadIdx.x; i < kValuRows * r; i += kThreads) {
            const int rb = i / r, j = i % r;
            const int b = b0 + rb;
            float x = 0.f;
            if (b < a.B) {
                x = wload<WT>(W1, (size_t)s_prev[rb] * r + j);
                if (GATED) x *= a.H[((size_t)b * a.K + k) * r + j];
            }
            xs[i] = x;
        }
        __syncthreads();

        float bk[kValuRows], bl[kValuRows], m[kValuRows], s[kValuRows];
        int bi[kValuRows];
        uint32_t k2[kValuRows];
#pragma unroll
        for (int rb = 0; rb < kValuRows; ++rb) {
            bk[rb] = -INFINITY;
            bl[rb] = 0.f;
            m[rb] = kMinFinite;
            s[rb] = 0.f;
            bi[rb] = 0x7FFFFFFF;
            k2[rb] = SAMPLE ? noise_key2(a.k0, (uint32_t)(b0 + rb), (uint32_t)k) : 0u;
        }
        // every thread runs the same iterations (the sampling race works on groups of 16 lanes)
        for (int v0 = 0; v0 < a.V; v0 += kThreads) {
            const int v = v0 + threadIdx.x;
            const bool inr = v < a.V;
            float acc[kValuRows] = {};
            if (inr) {
                // unrolled so that eight W2 loads are in flight at once (one at a time made every step a cache
                // round trip); the accumulation order per row is unchanged
#pragma unroll 8
                for (int j = 0; j < r; ++j) {
                    const float w = wload<WT>(W2, (size_t)j * a.sj + (size_t)v * a.sv);
#pragma unroll
                    for (int rb = 0; rb < kValuRows; ++rb) acc[rb] = fmaf(xs[rb * r + j], w, acc[rb]);
                }
            }
#pragma unroll
            for (int rb = 0; rb < kValuRows; ++rb) {
                const int b = b0 + rb;
                if (b >= a.B) continue;  // uniform over the workgroup
                const float l = inr ? acc[rb] + a.U[((size_t)b * a.K + k) * a.V + v] : 0.f;
                const float t = inr ? l * a.c : -INFINITY;
                const float mn = fmaxf(m[rb], t);
                s[rb] = s[rb] * fast_exp2(m[rb] - mn) + fast_exp2(t - mn);
                m[rb] = mn;
                if (SAMPLE) {
                    float M = t;
#pragma unroll
                    for (int off = 1; off < 16; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 16));
                    const float e = inr ? fast_exp2(t - M) : 0.f;
                    float P = e;
#pragma unroll
                    for (int off = 1; off < 16; off <<= 1) {
                        const float y = __shfl_up(P, off, 16);
                        if (g16 >= off) P += y;
                    }
                    const float S = __shfl(P, 15, 16);
                    if (S > 0.f) {
                        float E, target;
                        block_race_variates(k2[rb], (uint32_t)((v - g16) / 16), S, E, target);
                        const unsigned long long below = __ballot(P <= target && g16 < 15);
                        const int sel = __popcll((below >> (threadIdx.x & 48)) & 0x7FFFull);
                        const float key = fast_log2(S) + M - fast_log2(E);
                        const float lsel = __shfl(l, sel, 16);
                        if (key > bk[rb]) {
                            bk[rb] = key;
                            bi[rb] = v - g16 + sel;
                            bl[rb] = lsel;
                        }
                    }
                } else if (inr && l > bk[rb]) {
                    bk[rb] = l;
                    bi[rb] = v;
                    bl[rb] = l;
                }
            }
        }
        // per row: the wave's lanes merged by shuffles, then the four waves in order through LDS
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int rb = 0; rb < kValuRows; ++rb) {
            if (b0 + rb >= a.B) break;  // uniform over the workgroup
            float kk = bk[rb], ll = bl[rb], mm = m[rb], ss = s[rb];
            int ii = bi[rb];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const float ok_ = __shfl_xor(kk, off);
                const int oi = __shfl_xor(ii, off);
                const float ol = __shfl_xor(ll, off);
                const float om = __shfl_xor(mm, off);
                const float os = __shfl_xor(ss, off);
                if (beats(ok_, oi, kk, ii)) {
                    kk = ok_;
                    ii = oi;
                    ll = ol;
                }
                lse_merge(mm, ss, om, os);
            }
            if (lane == 0) {
                rk[wave] = kk;
                ri[wave] = ii;
                rl[wave] = ll;
                rm[wave] = mm;
                rs[wave] = ss;
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                for (int w = 1; w < kThreads / 64; ++w) {
                    if (beats(rk[w], ri[w], kk, ii)) {
                        kk = rk[w];
                        ii = ri[w];
                        ll = rl[w];
                    }
                    lse_merge(mm, ss, rm[w], rs[w]);
                }
                const size_t o = (size_t)(b0 + rb) * a.K + k;
                a.tokens[o] = ii;
                if (a.logprobs) a.logprobs[o] = ll * a.inv_t - (mm + fast_log2(ss)) * kLn2;
                s_prev[rb] = min(max(ii, 0), a.V - 1);
            }
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Cross-workgroup reduction: one workgroup per row merges the G partials and writes the pick.
// ------------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) markov_reduce(ReduceArgs a) {
    const int b = blockIdx.x;
    float bk = -INFINITY, bl = 0.f, m = kMinFinite, s = 0.f;
    int bi = 0x7FFFFFFF;
    for (int g = threadIdx.x; g < a.G; g += kThreads) {
        const size_t o = (size_t)g * a.Bpad + b;
        const float k = a.part.key[o];
        const int i = a.part.idx[o];
        if (beats(k, i, bk, bi)) {
            bk = k;
            bi = i;
            bl = a.part.l[o];
        }
        lse_merge(m, s, a.part.m[o], a.part.s[o]);
    }
    // wave reduction, then across the four waves through LDS
    for (int off = 32; off > 0; off >>= 1) {
        float ok_ = __shfl_xor(bk, off);
        int oi = __shfl_xor(bi, off);
        float ol = __shfl_xor(bl, off);
        float om = __shfl_xor(m, off);
        float os = __shfl_xor(s, off);
        if (beats(ok_, oi, bk, bi)) {
            bk = ok_;
            bi = oi;
            bl = ol;
        }
        lse_merge(m, s, om, os);
    }
    __shared__ float wk[4], wl[4], wm[4], ws[4];
    __shared__ int wi[4];
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        wk[wave] = bk;
        wi[wave] = bi;
        wl[wave] = bl;
        wm[wave] = m;
        ws[wave] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w) {
            if (beats(wk[w], wi[w], bk, bi)) {
                bk = wk[w];
                bi = wi[w];
                bl = wl[w];
            }
            lse_merge(m, s, wm[w], ws[w]);
        }
        const size_t o = (size_t)b * a.out_stride;
        a.tokens[o] = bi;
        if (a.logprobs) a.logprobs[o] = bl * a.inv_t - (m + fast_log2(s)) * kLn2;
        if (a.best_logit) a.best_logit[o] = bl;
    }
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------------

template <int RK, int MODE>
static void launch_mfma_mode(const StepArgs& a, bool gated, bool vec_u, dim3 grid, hipStream_t st) {
    const dim3 block(kThreads);
    if (gated) {
        if (vec_u) hipLaunchKernelGGL((markov_step_mfma<RK, MODE, true, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((markov_step_mfma<RK, MODE, true, false>), grid, block, 0, st, a);
    } else {
        if (vec_u) hipLaunchKernelGGL((markov_step_mfma<RK, MODE, false, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((markov_step_mfma<RK, MODE, false, false>), grid, block, 0, st, a);
    }
}

template <int RK>
static hipError_t launch_mfma_rk(const StepArgs& a, int mode, bool gated, bool vec_u, dim3 grid, hipStream_t st) {
    if (mode == kModeSample) launch_mfma_mode<RK, kModeSample>(a, gated, vec_u, grid, st);
    else if (mode == kModeStore) launch_mfma_mode<RK, kModeStore>(a, gated, vec_u, grid, st);
    else launch_mfma_mode<RK, kModeGreedy>(a, gated, vec_u, grid, st);
    return hipGetLastError();
}

int mfma_supported_r(int r) { return r % 16 == 0 && r >= 16 && r <= 512 && ((r / 16) & (r / 16 - 1)) == 0; }

hipError_t launch_markov_step_mfma(const StepArgs& a, int mode, bool gated, bool vec_u, int G, hipStream_t st) {
    const dim3 grid(G, (a.B + kRowsPerWG - 1) / kRowsPerWG);
    switch (a.r / 16) {
        case 1: return launch_mfma_rk<1>(a, mode, gated, vec_u, grid, st);
        case 2: return launch_mfma_rk<2>(a, mode, gated, vec_u, grid, st);
        case 4: return launch_mfma_rk<4>(a, mode, gated, vec_u, grid, st);
        case 8: return launch_mfma_rk<8>(a, mode, gated, vec_u, grid, st);
        case 16: return launch_mfma_rk<16>(a, mode, gated, vec_u, grid, st);
        case 32: return launch_mfma_rk<32>(a, mode, gated, vec_u, grid, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename WT, int MODE>
static void launch_valu_mode(const StepArgsValu& a, bool gated, dim3 grid, size_t shm, hipStream_t st) {
    if (gated) hipLaunchKernelGGL((markov_step_valu<WT, MODE, true>), grid, dim3(kThreads), shm, st, a);
    else hipLaunchKernelGGL((markov_step_valu<WT, MODE, false>), grid, dim3(kThreads), shm, st, a);
}

template <typename WT>
static void launch_valu_wt(const StepArgsValu& a, int mode, bool gated, dim3 grid, size_t shm, hipStream_t st) {
    if (mode == kModeSample) launch_valu_mode<WT, kModeSample>(a, gated, grid, shm, st);
    else if (mode == kModeStore) launch_valu_mode<WT, kModeStore>(a, gated, grid, shm, st);
    else launch_valu_mode<WT, kModeGreedy>(a, gated, grid, shm, st);
}

hipError_t launch_markov_step_valu(const StepArgsValu& a, bool bf16, int mode, bool gated, int G, hipStream_t st) {
    const dim3 grid(G, (a.B + kValuRows - 1) / kValuRows);
    const size_t shm = sizeof(float) * kValuRows * a.r;
    if (bf16) launch_valu_wt<uint16_t>(a, mode, gated, grid, shm, st);
    else launch_valu_wt<float>(a, mode, gated, grid, shm, st);
    return hipGetLastError();
}

template <typename WT, int MODE>
static void launch_round_valu_mode(const RoundValuArgs& a, bool gated, dim3 grid, size_t shm, hipStream_t st) {
    if (gated) hipLaunchKernelGGL((markov_round_valu<WT, MODE, true>), grid, dim3(kThreads), shm, st, a);
    else hipLaunchKernelGGL((markov_round_valu<WT, MODE, false>), grid, dim3(kThreads), shm, st, a);
}

hipError_t launch_markov_round_valu(const RoundValuArgs& a, bool bf16, bool sample, bool gated, hipStream_t st) {
    const dim3 grid((a.B + kValuRows - 1) / kValuRows);
    const size_t shm = sizeof(float) * kValuRows * a.r;
    if (bf16) {
        if (sample) launch_round_valu_mode<uint16_t, kModeSample>(a, gated, grid, shm, st);
        else launch_round_valu_mode<uint16_t, kModeGreedy>(a, gated, grid, shm, st);
    } else {
        if (sample) launch_round_valu_mode<float, kModeSample>(a, gated, grid, shm, st);
        else launch_round_valu_mode<float, kModeGreedy>(a, gated, grid, shm, st);
    }
    return hipGetLastError();
}

hipError_t launch_markov_reduce(const ReduceArgs& a, int B, hipStream_t st) {
    hipLaunchKernelGGL(markov_reduce, dim3(B), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace dspark

// markov_round.hip -- a whole Markov-head draft round (all K positions) in one persistent launch.
//
// The rule is the one of markov.hip: for k = 0 .. K-1, l_k[b, v] = U_k[b, v] + (W1[a_b] (.) H_k[b])^T W2[:, v]
// with a_b the token picked at k-1 (the anchor at k = 0), a pick over the whole vocabulary, and the exact
// local log-softmax of the picked token (pages: "DFlash-2's Selector and DSpark's Markov Head", "What the two
// methods do"; the DSpark overview, "The Markov head"; "DSpark: Repair the Joint, Meter the Verify", "Why the
// normalization has to be local").
//
// Design (gfx950):
//  * One workgroup per CU, co-resident (cooperative launch).  Workgroup g owns a fixed contiguous range of
//    32-wide vocabulary tiles for the whole round; wave w owns batch rows 32w .. 32w+31 of each 128-row block.
//  * Four producer waves stream W2 tiles ([32, r] bf16 rows of the [V, r] layout) and U tiles ([128, 32] fp32)
//    with ordinary 16-byte vector loads (kDepth items ahead in registers; on this part they sustain more
//    bandwidth than direct global->LDS loads) into a ring of kNS LDS stages; four consumer waves compute.
//    Producers and consumers hand stages over through LDS counters, with no workgroup barrier per tile.
//    The stream does not depend on the drafted tokens, so it runs ahead across position boundaries.  Stage
//    layouts are XOR-swizzled (and skewed every 8 U rows) so the MFMA operand reads are bank-conflict free.
//  * Per tile: C[v, b] = sum_j W2t[v, j] X[b, j] with v_mfma_f32_32x32x16_bf16 (A = W2 tile from LDS,
//    B = the gathered predecessor rows X, resident in registers for the position).  A lane holds one batch
//    row and 16 vocabulary ids of the accumulator; calibration, the streaming log-sum-exp and the running
//    pick are per-lane scalars.  No logits are written.
//  * Sampling uses the exponential-race form of Gumbel-max: argmax_v p_v / E_v with p_v = 2^(l_v c - m) (the
//    same exponential the log-sum-exp needs) and E_v = -log2 u_v, which is argmax_v (l_v / T + G_v) exactly.
//  * End of a position: one 64-bit atomicMax per row and workgroup on (ordered key, ~id) gives the global
//    pick with ties to the lower id; log-sum-exp partials go to the workspace.  A grid barrier (counter,
//    bounded spin) then releases the next position, whose workgroups gather W1 rows of the new tokens.
//  * A finalize kernel merges the log-sum-exp partials of all positions into tokens and log-probabilities.
#include "common.hpp"
#include "internal.hpp"

namespace dspark {

namespace {

constexpr int kRThreads = 256;
constexpr int kRTileV = 32;
constexpr int kRRows = 128;
constexpr int kUGroupBytes = 8 * 128 + 16;  // 8 U rows of 32 floats + 16-byte skew
constexpr float kNegBig = -1e30f;          // start of a running max; stays finite when scaled by log2(e)/T

template <int RK>
struct Ring {
    static constexpr int kNS = 4;
    static constexpr int kRowBytes = 32 * RK;                 // one W2 row: r = 16 RK bf16
    static constexpr int kW2Bytes = kRTileV * kRowBytes;      // 32 rows
    static constexpr int kUBytes = 16 * kUGroupBytes;         // 128 rows in 16 skewed groups of 8
    static constexpr int kStage = kW2Bytes + kUBytes;
    static constexpr int kSwz = ((2 * RK < 16) ? 2 * RK : 16) - 1;
    // one item = RK W2 units (64 lanes x 16 B) + 16 U units (8 rows x 128 B); producer p takes units p, p + 4, ...
    static constexpr int kUnits = RK + 16;
    static constexpr int kUnitsPerProducer = (kUnits + 3) / 4;
    static constexpr int kDepth = 3;                          // items in flight per producer, in registers
};

constexpr int kConsumers = 4;
constexpr int kProducers = 4;
constexpr int kRoundThreads = 64 * (kConsumers + kProducers);

// vmcnt waits with compile-time counts (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14])
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14)); }

__device__ __forceinline__ uint32_t ordered_key(float f) {
    f = f + 0.0f;  // -0 -> +0, so equal keys compare equal
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lds_load(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_add(uint32_t* p, uint32_t v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

constexpr int kNumCounters = 8;  // the grid barrier counter is spread over 8 cache lines
constexpr int kCounterStride = 32;

template <int RK, int MODE, bool GATED>
__global__ void __launch_bounds__(kRoundThreads, 1) markov_round_kernel(RoundArgs a) {
    using RG = Ring<RK>;
    constexpr bool SAMPLE = MODE == kModeSample;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[RG::kNS * RG::kStage];
    __shared__ uint32_t ready[RG::kNS];  // +1 per producer per filled stage
    __shared__ uint32_t freed[RG::kNS];  // +1 per consumer wave per consumed stage
    __shared__ uint32_t stepdone;        // +1 per consumer wave per finished position
    __shared__ uint32_t released;        // last position whose predecessors are known (set by consumer wave 0)

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int r = 16 * RK;
    const int t0 = (int)(((long long)g * a.ntiles) / G);
    const int t1 = (int)(((long long)(g + 1) * a.ntiles) / G);
    const int ntw = t1 - t0;
    const int nrb = (a.B + kRRows - 1) / kRRows;
    const int per_k = nrb * ntw;
    const int nitems = a.K * per_k;
    const uint32_t spin_limit = a.spin_limit;

    if (threadIdx.x < RG::kNS) {
        ready[threadIdx.x] = 0u;
        freed[threadIdx.x] = 0u;
    }
    if (threadIdx.x == 0) {
        stepdone = 0u;
        released = 0u;
    }
    __syncthreads();

    if (wave >= kConsumers) {
        // ============================================================== producers: stream W2 and U tiles
        // Ordinary 16-byte vector loads into registers, kDepth items ahead, then ds_write into the swizzled
        // stage layout the consumers read.  Unit u of an item: u < RK is W2 rows 2u .. (64 lanes x 16 B of the
        // tile's [32, r] block); u >= RK is U row group u - RK (8 rows x 32 floats).
        const int p = wave - kConsumers;
        constexpr int NU = RG::kUnitsPerProducer;
        constexpr int D = RG::kDepth;
        u32x4_t regs[D][NU];
        auto load = [&](int i, u32x4_t (&dst)[NU]) {
            const int k = i / per_k;
            const int rem = i - k * per_k;
            const int rb = rem / ntw;
            const int t = t0 + (rem - rb * ntw);
            const int v0 = t * kRTileV;
            const float* ub = a.U + (size_t)k * a.u_kstride;
#pragma unroll
            for (int n = 0; n < NU; ++n) {
                const int u = p + 4 * n;
                if (u < RK) {
                    const int P = u * 64 + lane;
                    const int rho = P / (2 * RK), c = P % (2 * RK);
                    const int vrow = min(v0 + rho, a.V - 1);
                    dst[n] = load_nt_u32x4(a.W2t + (size_t)vrow * r + 8 * c);
                } else if (u < RG::kUnits) {
                    const int q = u - RK;
                    const int b = min(rb * kRRows + q * 8 + (lane >> 3), a.B - 1);
                    const int col = min(v0 + 4 * (lane & 7), a.V - 4);
                    dst[n] = load_nt_u32x4(ub + (size_t)b * a.u_stride + col);
                }
            }
        };
        auto store = [&](int i, const u32x4_t (&src)[NU]) {
            uint8_t* st = ring + (i % RG::kNS) * RG::kStage;
#pragma unroll
            for (int n = 0; n < NU; ++n) {
                const int u = p + 4 * n;
                if (u < RK) {
                    const int P = u * 64 + lane;
                    const int rho = P / (2 * RK), c = P % (2 * RK);
                    *reinterpret_cast<u32x4_t*>(st + rho * RG::kRowBytes + 16 * (c ^ (rho & RG::kSwz))) = src[n];
                } else if (u < RG::kUnits) {
                    const int q = u - RK;
                    const int rho8 = lane >> 3, c = lane & 7;
                    *reinterpret_cast<u32x4_t*>(st + RG::kW2Bytes + q * kUGroupBytes + rho8 * 128 + 16 * (c ^ rho8)) = src[n];
                }
            }
        };
        auto publish = [&](int i, const u32x4_t (&src)[NU]) {
            if (i >= RG::kNS) {
                const uint32_t need = (uint32_t)kConsumers * (uint32_t)(i / RG::kNS);
                uint32_t spins = 0;
                while (lds_load(&freed[i % RG::kNS]) < need) {
                    __builtin_amdgcn_s_sleep(1);
                    if (++spins > spin_limit) {
                        __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
            }
            store(i, src);
            wait_lgkmcnt0();
            if (lane == 0) lds_add(&ready[i % RG::kNS], 1u);
        };
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (d < nitems) load(d, regs[d]);
        for (int i0 = 0; i0 < nitems; i0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int i = i0 + d;
                if (i < nitems) {
                    publish(i, regs[d]);
                    if (i + D < nitems) load(i + D, regs[d]);
                }
            }
        }
        return;
    }

    // ================================================================== consumers: contraction and pick
    bf16x8_t xf[RK];
    uint32_t k2 = 0;
    float m = kNegBig, s = 0.f;      // running max of l (natural units) and sum of 2^(l c - m c)
    float bp = 0.f, bE = 1.f;        // sampling: best p = 2^(l c - m c) and its E = -log2 u
    float bl = -INFINITY;            // greedy: best logit
    int bi = 0x7FFFFFFF;
    const float c = a.c;
    const int rho = lane & 31;
    const int rr = wave * 32 + rho;  // this lane's row inside the 128-row block

    auto wait_ready = [&](int i) {
        const uint32_t need = (uint32_t)kProducers * (uint32_t)(i / RG::kNS + 1);
        uint32_t spins = 0;
        while (lds_load(&ready[i % RG::kNS]) < need) {
            __builtin_amdgcn_s_sleep(0);
            if (++spins > spin_limit) {
                __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    };
    // MFMA over the rank for stage i; the operand reads are issued in batches of up to 16 so their
    // LDS latency overlaps, then the MFMAs run back to back.  U values of the lane's row go to u.
    constexpr int kBatch = RK < 16 ? RK : 16;
    auto stage_mma = [&](int i, f32x16_t& acc, float (&u)[16]) {
        const uint8_t* st = ring + (i % RG::kNS) * RG::kStage;
        const uint8_t* arow = st + rho * RG::kRowBytes;
        const uint8_t* urow = st + RG::kW2Bytes + (rr >> 3) * kUGroupBytes + (rr & 7) * 128;
        f32x4_t u4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) u4[q] = *reinterpret_cast<const f32x4_t*>(urow + 16 * ((2 * q + half) ^ (rr & 7)));
        acc = f32x16_t{};
#pragma unroll
        for (int k0 = 0; k0 < RK; k0 += kBatch) {
            bf16x8_t af[kBatch];
#pragma unroll
            for (int kk = 0; kk < kBatch; ++kk)
                af[kk] = *reinterpret_cast<const bf16x8_t*>(arow + 16 * ((2 * (k0 + kk) + half) ^ (rho & RG::kSwz)));
#pragma unroll
            for (int kk = 0; kk < kBatch; ++kk) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk], xf[k0 + kk], acc, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u[4 * q + 0] = u4[q].x;
            u[4 * q + 1] = u4[q].y;
            u[4 * q + 2] = u4[q].z;
            u[4 * q + 3] = u4[q].w;
        }
    };
    // calibration, streaming log-sum-exp and running pick over the 16 ids of one tile
    auto epilogue = [&](const f32x16_t& acc, const float (&u)[16], int t) {
        const int v0 = t * kRTileV;
        const int vl = v0 + 4 * half;  // id of slot i2 = vl + 8 (i2 / 4) + i2 % 4
        float E[16];
        if (SAMPLE) {
            // noise first: it does not depend on the contraction.  fmix32(k2 ^ v) for the ids vl + 8q + o,
            // o = 0..3 (vl + 8q is a multiple of 4, so k2 ^ (vl + 8q + o) = (k2 ^ (vl + 8q)) ^ o and the first
            // xor-shift is shared)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t base = k2 ^ (uint32_t)(vl + 8 * q);
                const uint32_t y = base ^ (base >> 16);
#pragma unroll
                for (int o = 0; o < 4; ++o) {
                    uint32_t h = y ^ (uint32_t)o;
                    h *= 0x85EBCA6Bu;
                    h ^= h >> 13;
                    h *= 0xC2B2AE35u;
                    h ^= h >> 16;
                    const float uu = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, h, 9)) - 0.99999994039535522f;
                    E[4 * q + o] = -fast_log2(uu);  // -log2 u > 0
                }
            }
        }
        float lv[16];
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2) lv[i2] = acc[i2] + u[i2];
        if (v0 + kRTileV > a.V) {
#pragma unroll
            for (int i2 = 0; i2 < 16; ++i2)
                if (vl + 8 * (i2 >> 2) + (i2 & 3) >= a.V) lv[i2] = -INFINITY;
        }
        float cm = fmaxf(fmaxf(lv[0], lv[1]), lv[2]);
#pragma unroll
        for (int i2 = 3; i2 < 15; i2 += 2) cm = fmaxf(fmaxf(cm, lv[i2]), lv[i2 + 1]);
        cm = fmaxf(cm, lv[15]);
        const float mn = fmaxf(m, cm);
        const float scale = fast_exp2((m - mn) * c);
        const float mc = mn * c;
        s *= scale;
        m = mn;
        float e[16];
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2) {
            e[i2] = fast_exp2(fmaf(lv[i2], c, -mc));
            s += e[i2];
        }
        if (SAMPLE) {
            // exponential race: p / E > bp / bE  <=>  l c - log2 E beats the best so far
            bp *= scale;
#pragma unroll
            for (int i2 = 0; i2 < 16; ++i2) {
                const bool better = e[i2] * bE > bp * E[i2];
                bp = better ? e[i2] : bp;
                bE = better ? E[i2] : bE;
                bi = better ? (vl + 8 * (i2 >> 2) + (i2 & 3)) : bi;
            }
        } else {
#pragma unroll
            for (int i2 = 0; i2 < 16; ++i2) {
                const bool better = lv[i2] > bl;
                bl = better ? lv[i2] : bl;
                bi = better ? (vl + 8 * (i2 >> 2) + (i2 & 3)) : bi;
            }
        }
    };

    const int nseg = a.K * nrb;
    for (int seg = 0; seg < nseg; ++seg) {
        const int k = seg / nrb;
        const int rb = seg - k * nrb;
        const int i0 = seg * ntw;
        const int b = rb * kRRows + rr;
        const bool valid_b = b < a.B;
        const bool wave_live = rb * kRRows + wave * 32 < a.B;

        // a new position (or row block): wait for the previous position's picks, then gather X.  Consumer wave 0
        // polls the grid counters; the other consumer waves wait for its LDS flag.
        if (k > 0 && rb == 0) {
            if (wave == 0) {
                const uint32_t target = (uint32_t)G * (uint32_t)k;
                uint32_t spins = 0;
                while (true) {
                    uint32_t tot = 0;
#pragma unroll
                    for (int cc = 0; cc < kNumCounters; ++cc)
                        tot += __hip_atomic_load(a.barrier + kCounterStride * cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (tot >= target) break;
                    __builtin_amdgcn_s_sleep(1);
                    if (++spins > spin_limit) {
                        __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
                if (lane == 0) __hip_atomic_store(&released, (uint32_t)k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            } else {
                uint32_t spins = 0;
                while (lds_load(&released) < (uint32_t)k) {
                    __builtin_amdgcn_s_sleep(0);
                    if (++spins > spin_limit) {
                        __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
            }
        }
        if (wave_live) {
            int pv = 0;
            if (valid_b) {
                if (k == 0) {
                    pv = a.anchor[b];
                } else {
                    const unsigned long long wv = __hip_atomic_load(a.winners + (size_t)(k - 1) * a.Bpad + b,
                                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    pv = (int)(0xFFFFFFFFu - (uint32_t)(wv & 0xFFFFFFFFull));
                    pv = min(max(pv, 0), a.V - 1);
                }
            }
            const u32x4_t* wrow = reinterpret_cast<const u32x4_t*>(a.W1 + (size_t)pv * r);
#pragma unroll
            for (int kk = 0; kk < RK; ++kk) {
                u32x4_t raw = valid_b ? wrow[2 * kk + half] : u32x4_t{0u, 0u, 0u, 0u};
                if (GATED && valid_b) {
                    const float* hrow = a.H + ((size_t)b * a.K + k) * r + 16 * kk + 8 * half;
                    const f32x4_t h0 = *reinterpret_cast<const f32x4_t*>(hrow);
                    const f32x4_t h1 = *reinterpret_cast<const f32x4_t*>(hrow + 4);
                    const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
                    const uint32_t w32[4] = {raw.x, raw.y, raw.z, raw.w};
                    uint32_t o32[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float lo = bf16_to_f32((uint16_t)(w32[e] & 0xFFFFu)) * hv[2 * e];
                        const float hi = bf16_to_f32((uint16_t)(w32[e] >> 16)) * hv[2 * e + 1];
                        o32[e] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
                    }
                    raw = u32x4_t{o32[0], o32[1], o32[2], o32[3]};
                }
                xf[kk] = __builtin_bit_cast(bf16x8_t, raw);
            }
            if (SAMPLE) k2 = noise_key2(a.k0, (uint32_t)b, (uint32_t)k);
        }
        m = kNegBig;
        s = 0.f;
        bp = 0.f;
        bE = 1.f;
        bl = -INFINITY;
        bi = 0x7FFFFFFF;

        // software pipeline over the segment's tiles: the MFMAs of tile tt+1 are issued before the
        // epilogue of tile tt, so the matrix cores work while the vector ALUs finish the previous tile
        f32x16_t acc_cur, acc_nxt;
        float u_cur[16], u_nxt[16];
        wait_ready(i0);
        if (wave_live) stage_mma(i0, acc_cur, u_cur);
        wait_lgkmcnt0();
        if (lane == 0) lds_add(&freed[i0 % RG::kNS], 1u);
        for (int tt = 0; tt < ntw; ++tt) {
            const int i = i0 + tt;
            const bool has_next = tt + 1 < ntw;
            if (has_next) {
                wait_ready(i + 1);
                if (wave_live) stage_mma(i + 1, acc_nxt, u_nxt);
            }
            if (wave_live) epilogue(acc_cur, u_cur, t0 + tt);
            if (has_next) {
                wait_lgkmcnt0();
                if (lane == 0) lds_add(&freed[(i + 1) % RG::kNS], 1u);  // the stage's bytes are in registers now
                acc_cur = acc_nxt;
#pragma unroll
                for (int i2 = 0; i2 < 16; ++i2) u_cur[i2] = u_nxt[i2];
            }
        }

        // end of this position / row block: lane merge, global pick, log-sum-exp partials
        if (wave_live) {
            float key, lbest;
            if (SAMPLE) {
                const float lc = fast_log2(bp) + m * c;  // l_best * c
                key = (bp > 0.f) ? lc - fast_log2(bE) : -INFINITY;
                lbest = lc / c;
            } else {
                key = bl;
                lbest = bl;
            }
            float mc2 = m * c;
            float s2 = s;
            const float okey = __shfl_xor(key, 32);
            const int oi = __shfl_xor(bi, 32);
            const float ol = __shfl_xor(lbest, 32);
            const float omc = __shfl_xor(mc2, 32);
            const float os = __shfl_xor(s2, 32);
            if (beats(okey, oi, key, bi)) {
                key = okey;
                bi = oi;
                lbest = ol;
            }
            lse_merge(mc2, s2, omc, os);
            if (half == 0 && valid_b) {
                const unsigned long long packed =
                    ((unsigned long long)ordered_key(key) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)bi);
                atomicMax(a.winners + (size_t)k * a.Bpad + b, packed);
                const size_t o = ((size_t)k * G + g) * a.Bpad + b;
                a.p_mc[o] = mc2;
                a.p_s[o] = s2;
                a.p_idx[o] = bi;
                a.p_l[o] = lbest;
            }
        }
        if (rb == nrb - 1) {
            // this wave's picks of position k are performed once its memory operations have completed
            wait_vmcnt<0>();
            if (lane == 0) {
                const uint32_t prev = __hip_atomic_fetch_add(&stepdone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (prev == (uint32_t)kConsumers * (uint32_t)(k + 1) - 1u)  // last consumer wave of the workgroup
                    __hip_atomic_fetch_add(a.barrier + kCounterStride * (g % kNumCounters), 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

__global__ void round_init_kernel(unsigned long long* winners, size_t n, uint32_t* counters, uint32_t* error) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) winners[i] = 0ull;
    if (blockIdx.x == 0 && threadIdx.x < kNumCounters) counters[kCounterStride * threadIdx.x] = 0u;
    if (blockIdx.x == 0 && threadIdx.x == 0) *error = 0u;
}

// One wave per (b, k): pick from the winner word, log-sum-exp over the G partials, logit of the pick from the
// partial of the workgroup that owns its id.
__global__ void __launch_bounds__(64) round_finalize_kernel(RoundArgs a, int32_t* tokens, float* logprobs, float inv_t) {
    const int b = blockIdx.x, k = blockIdx.y, lane = threadIdx.x;
    const int G = a.G;
    const unsigned long long wv = a.winners[(size_t)k * a.Bpad + b];
    const int tok = (int)(0xFFFFFFFFu - (uint32_t)(wv & 0xFFFFFFFFull));
    float mc = kMinFinite, s = 0.f, l = 0.f;
    int found = 0;
    for (int gg = lane; gg < G; gg += 64) {
        const size_t o = ((size_t)k * G + gg) * a.Bpad + b;
        lse_merge(mc, s, a.p_mc[o], a.p_s[o]);
        if (a.p_idx[o] == tok) {
            l = a.p_l[o];
            found = 1;
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        const float omc = __shfl_xor(mc, off);
        const float os = __shfl_xor(s, off);
        const float ol = __shfl_xor(l, off);
        const int of = __shfl_xor(found, off);
        lse_merge(mc, s, omc, os);
        if (of && !found) {
            l = ol;
            found = 1;
        }
    }
    if (lane == 0) {
        const bool bad = *a.error != 0u || !found;
        tokens[(size_t)b * a.K + k] = bad ? -1 : tok;
        if (logprobs) logprobs[(size_t)b * a.K + k] = bad ? NAN : l * inv_t - (mc + fast_log2(s)) * kLn2;
    }
}

}  // namespace

int round_supported_r(int r) { return mfma_supported_r(r) && r <= 256; }

int round_lds_bytes(int r) {
    switch (r / 16) {
        case 1: return Ring<1>::kNS * Ring<1>::kStage;
        case 2: return Ring<2>::kNS * Ring<2>::kStage;
        case 4: return Ring<4>::kNS * Ring<4>::kStage;
        case 8: return Ring<8>::kNS * Ring<8>::kStage;
        case 16: return Ring<16>::kNS * Ring<16>::kStage;
        default: return 0;
    }
}

template <int RK, int MODE, bool GATED>
static hipError_t coop_launch(const RoundArgs& a, hipStream_t st) {
    RoundArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&markov_round_kernel<RK, MODE, GATED>), dim3(a.G),
                                      dim3(kRoundThreads), args, 0, st);
}

template <int RK>
static hipError_t launch_round_rk(const RoundArgs& a, bool sample, bool gated, hipStream_t st) {
    if (sample) return gated ? coop_launch<RK, kModeSample, true>(a, st) : coop_launch<RK, kModeSample, false>(a, st);
    return gated ? coop_launch<RK, kModeGreedy, true>(a, st) : coop_launch<RK, kModeGreedy, false>(a, st);
}

template <int RK, int MODE, bool GATED>
static int max_blocks_per_cu() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&markov_round_kernel<RK, MODE, GATED>),
                                                     kRoundThreads, 0) != hipSuccess)
        return 0;
    return n;
}

int round_max_coresident(int r, bool sample, bool gated) {
    int per_cu = 0;
#define DSPARK_OCC(RK_)                                                                                  \
    per_cu = sample ? (gated ? max_blocks_per_cu<RK_, kModeSample, true>() : max_blocks_per_cu<RK_, kModeSample, false>()) \
                    : (gated ? max_blocks_per_cu<RK_, kModeGreedy, true>() : max_blocks_per_cu<RK_, kModeGreedy, false>())
    switch (r / 16) {
        case 1: DSPARK_OCC(1); break;
        case 2: DSPARK_OCC(2); break;
        case 4: DSPARK_OCC(4); break;
        case 8: DSPARK_OCC(8); break;
        case 16: DSPARK_OCC(16); break;
        default: return 0;
    }
#undef DSPARK_OCC
    return per_cu * device_cu_count();
}

hipError_t launch_markov_round(const RoundArgs& a, bool sample, bool gated, int32_t* tokens, float* logprobs,
                               float inv_t, hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
    const size_t nw = (size_t)a.K * a.Bpad;
    hipLaunchKernelGGL(round_init_kernel, dim3(64), dim3(256), 0, st, a.winners, nw, a.barrier, a.error);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_begin) (void)hipEventRecord(ev_begin, st);
    switch (a.r / 16) {
        case 1: e = launch_round_rk<1>(a, sample, gated, st); break;
        case 2: e = launch_round_rk<2>(a, sample, gated, st); break;
        case 4: e = launch_round_rk<4>(a, sample, gated, st); break;
        case 8: e = launch_round_rk<8>(a, sample, gated, st); break;
        case 16: e = launch_round_rk<16>(a, sample, gated, st); break;
        default: return hipErrorInvalidValue;
    }
    if (ev_end) (void)hipEventRecord(ev_end, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(round_finalize_kernel, dim3(a.B, a.K), dim3(64), 0, st, a, tokens, logprobs, inv_t);
    return hipGetLastError();
}

}  // namespace dspark

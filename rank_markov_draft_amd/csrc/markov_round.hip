// markov_round.hip -- a whole Markov-head draft round (all K positions) in one persistent launch.
//
// The rule is the one of markov.hip: for k = 0 .. K-1, l_k[b, v] = U_k[b, v] + (W1[a_b] (.) H_k[b])^T W2[:, v]
// with a_b the token picked at k-1 (the anchor at k = 0), a pick over the whole vocabulary, and the exact
// local log-softmax of the picked token (pages: "DFlash-2's Selector and DSpark's Markov Head", "What the two
// methods do"; the DSpark overview, "The Markov head"; "DSpark: Repair the Joint, Meter the Verify", "Why the
// normalization has to be local").
//
// Design (gfx950):
//  * One workgroup per CU, co-resident (cooperative launch).  Workgroup g owns the 32-wide vocabulary tiles
//    g, g + G, g + 2G, ... for the whole round; wave w owns batch rows 32w .. 32w+31 of each 128-row block.
//  * Four producer waves stream W2 tiles ([32, r] bf16 rows of the [V, r] layout) and U tiles ([128, 32] fp32)
//    with ordinary 16-byte vector loads (kDepth items ahead in registers; on this part they sustain more
//    bandwidth than direct global->LDS loads) into a ring of kNS LDS stages; four consumer waves compute.
//    Producers and consumers hand stages over through LDS counters, with no workgroup barrier per tile.
//    The stream does not depend on the drafted tokens, so it runs ahead across position boundaries.  Stage
//    rows are padded by 16 bytes, so the 16-byte operand reads of 8 consecutive lanes fall in distinct banks
//    and use immediate offsets.
//  * Per tile: C[v, b] = U[b, v] + sum_j W2t[v, j] X[b, j] with v_mfma_f32_32x32x16_bf16 (A = W2 tile from
//    LDS, stored in permuted row slots; B = the gathered predecessor rows X, resident in registers for the
//    position; C seeded with the U tile).  A lane holds one batch row and 16 consecutive vocabulary ids of
//    the accumulator; calibration, the streaming log-sum-exp and the running pick are per-lane scalars.  The
//    MFMAs of tile t + 1 are issued inside the epilogue of tile t.  No logits are written.
//  * Sampling is an exact draw from softmax(l / T) by a two-level exponential race: a lane's 16 ids of a tile
//    form one aligned block whose mass S = sum_v 2^(l_v c - m) (the same exponentials the log-sum-exp needs)
//    races with one exponential variate, and the winning block's id is drawn by inverse CDF, so one hash
//    pair and one logarithm serve 16 ids.
//  * End of a position: one 64-bit atomicMax per row and workgroup on (ordered key, ~id), each row's word on
//    its own cache line, gives the global pick with ties to the lower id; log-sum-exp partials go to the
//    workspace.  A grid barrier then releases the next position, whose workgroups gather W1 rows of the new
//    tokens.  The barrier is a two-level arrival tree (8 group counters, then a top counter) whose last
//    arrival writes 8 copies of a release word: every poll reads one line shared by an eighth of the grid, and
//    the polls do not queue behind the arrivals as they did on counters polled by the whole grid (the
//    boundary took about twice as long so).
//  * A ninth wave per workgroup (the finalizer) clears the pick words and counters at the start of the launch
//    and, one position behind, merges the log-sum-exp partials of its rows into tokens and log-probabilities,
//    so a round is a single launch.
//  * A batch of at most 8 rows takes a small-block form: one U unit per item instead of sixteen and eight ring
//    stages, and (without the gate) two consumer waves that each take every other tile of a position for the
//    same rows, handing their per-row results to wave 0 through LDS, with six producer waves of ten items in
//    flight each (a stream of W2-only items is bound by the bytes in flight).  A batch of 9 .. 64
//    rows takes a half-block form the same way: eight U units per item, five stages, and two sets of two
//    consumer waves taking every other tile, so no consumer wave idles on rows past the batch.
//  * The gated gather X = bf16(W1[a] (.) H) runs in four phases whose loads are all issued before their
//    multiplies, so it costs the pick read and four memory round trips.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace dspark {

namespace {

constexpr int kRTileV = 32;
constexpr int kRRows = 128;
constexpr float kNegBig = -1e30f;  // start of a running max; stays finite when scaled by log2(e)/T

// UR = U units (8 rows each) per item: 16 for a full 128-row block; 8 for a batch of 9 .. 64 rows (a half
// block: the LDS the missing U rows would take holds a fifth stage); 1 for a batch of at most 8 rows, whose
// items are W2 almost only: then the registers and LDS that U rows would take hold more items instead (six in
// flight per producer, eight stages), since a stream of small items is bound by the bytes in flight.
// HL: the gated half block, whose LDS also holds the next position's gate rows, keeps three stages and one more
// item in flight per producer instead.
template <int RK, int UR = 16, bool HL = false>
struct Ring {
    static_assert(UR == 16 || UR == 8 || UR == 1, "full, half or small row block");
    static constexpr int kNS = HL ? 3 : UR == 16 ? 4 : UR == 8 ? 5 : 8;
    static constexpr int kW2Row = 32 * RK + 16;            // one W2 row (r = 16 RK bf16) + 16-byte pad
    static constexpr int kW2Bytes = kRTileV * kW2Row;      // 32 rows
    static constexpr int kURow = 4 * kRTileV + 16;          // one U row of the tile (32 floats) + 16-byte pad
    static constexpr int kUBytes = 8 * UR * kURow;          // 8 UR rows
    static constexpr int kStage = kW2Bytes + kUBytes;
    // one item = RK W2 units (64 lanes x 16 B) + UR U units (8 rows x 128 B); producer p of P takes units p, p + P, ...
    static constexpr int kUnits = RK + UR;
    static constexpr int kDepth = HL ? 4 : UR == 1 ? 6 : 3;  // items in flight per producer, in registers
};

// Waves of a workgroup: consumers, producers and one finalizer, nine in all.  The ungated small block (at most 8
// rows) has little consumer work per item, and its stream of W2-only items is bound by the bytes in flight, so it
// runs two consumer waves and six producers with ten items in flight each (170 KB per CU, against 102 KB with
// four producers of six items).
template <int UR, bool GATED>
struct Waves {
    static constexpr bool kDeep = UR == 1 && !GATED;
    static constexpr int kConsumers = kDeep ? 2 : 4;
    static constexpr int kProducers = kDeep ? 6 : 4;
    static constexpr int kDepth = kDeep ? 10 : 0;  // 0: the ring's own depth
};
constexpr int kRoundThreads = 64 * 9;

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

template <typename T>
__device__ __forceinline__ T agent_load(const T* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void agent_store(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The flag value that names this launch: the call's sequence number mixed with the workspace's epoch.
__device__ __forceinline__ uint64_t launch_tag(const RoundArgs& a, uint32_t ep) {
    return a.seq ^ (0x9E3779B97F4A7C15ull * ((uint64_t)ep + 1ull));
}

// Waits (one lane) until workgroup 0 has cleared this launch's counters; bounded.
__device__ __forceinline__ void wait_cleared(const RoundArgs& a, uint64_t tag) {
    uint32_t spins = 0;
    while (agent_load(a.flag) != tag) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > a.spin_limit) {
            __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
    }
}

// The last position every workgroup has finished, as this workgroup's copy of the release word shows.
__device__ __forceinline__ uint32_t released_position(const RoundArgs& a) {
    return agent_load(a.release + kCounterStride * (blockIdx.x % kBarrierGroups));
}

// The pick word of (position k, row b): the largest of its slots.
__device__ __forceinline__ unsigned long long pick_word(const RoundArgs& a, int k, int b) {
    const unsigned long long* w = a.winners + ((size_t)k * a.Bpad + b) * kWinnerSlots * kWinnerStride;
    unsigned long long v[kWinnerSlots];
#pragma unroll
    for (int s = 0; s < kWinnerSlots; ++s) v[s] = agent_load(w + s * kWinnerStride);
    unsigned long long best = v[0];
#pragma unroll
    for (int s = 1; s < kWinnerSlots; ++s) best = v[s] > best ? v[s] : best;
    return best;
}

// Arrival of this workgroup at the end of position k (one lane of its last consumer wave, after the wave's
// picks are performed).  Returns true for the grid's last arrival, which then releases the position.
__device__ __forceinline__ bool arrive(const RoundArgs& a, int k) {
    const int G = gridDim.x;
    const int grp = (int)blockIdx.x % kBarrierGroups;
    const uint32_t members = (uint32_t)((G - grp + kBarrierGroups - 1) / kBarrierGroups);
    const uint32_t groups = (uint32_t)min(G, kBarrierGroups);
    const uint32_t old = __hip_atomic_fetch_add(a.barrier + kCounterStride * grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old != members * (uint32_t)(k + 1) - 1u) return false;
    const uint32_t o2 = __hip_atomic_fetch_add(a.top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return o2 == groups * (uint32_t)(k + 1) - 1u;
}

// One wave: the confidence of (row b, position k) and the prefix survival ([DSp] "Confidence-scheduled
// verification"): c_k = sigmoid(w_h . h_k + w_m . W1[x_{k-1}]), x_{-1} the anchor; a_k = a_{k-1} c_k.  It
// depends on the tokens before position k only, so it can run as soon as x_{k-1} is known.
// Tokens and survivals of earlier positions are read back with agent-scope loads (they were stored so).
__device__ void confidence_step(const ConfArgs& c, int b, int k) {
    const int lane = threadIdx.x & 63;
    const int prev = (k == 0) ? c.anchor[b] : agent_load(c.tokens + (size_t)b * c.K + k - 1);
    float z = 0.f;
    const uint16_t* hrow = c.h + ((size_t)b * c.K + k) * c.D;
#pragma unroll 8
    for (int d0 = 8 * lane; d0 < c.D; d0 += 512) {
        const u32x4_t q = *reinterpret_cast<const u32x4_t*>(hrow + d0);
        const uint32_t q4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z = fmaf(c.w[d0 + 2 * e], bf16_to_f32((uint16_t)(q4[e] & 0xFFFFu)), z);
            z = fmaf(c.w[d0 + 2 * e + 1], bf16_to_f32((uint16_t)(q4[e] >> 16)), z);
        }
    }
    const bool ok = prev >= 0;  // a token of -1 marks a failed position
    if (ok) {
#pragma unroll 4
        for (int j = lane; j < c.r; j += 64) {
            const float wj = c.w1_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(c.W1)[(size_t)prev * c.r + j])
                                       : static_cast<const float*>(c.W1)[(size_t)prev * c.r + j];
            z = fmaf(c.w[c.D + j], wj, z);
        }
    }
    for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
    if (lane == 0) {
        const float ck = ok ? 1.0f / (1.0f + fast_exp2(-z * kLog2e)) : NAN;
        const float before = (k == 0) ? 1.0f : agent_load(c.survival + (size_t)b * c.K + k - 1);
        c.conf[(size_t)b * c.K + k] = ck;
        agent_store(c.survival + (size_t)b * c.K + k, before * ck);
    }
}

// One wave merges the G partials of (row b, position k): the pick from the winner word wv, the log-sum-exp over
// the partials, the logit of the pick from the partial of the workgroup that owns its id.
__device__ void finalize_with(const RoundArgs& a, int b, int k, unsigned long long wv, bool timed_out) {
    const int lane = threadIdx.x & 63;
    const int G = a.G;
    const int tok = (int)(0xFFFFFFFFu - (uint32_t)(wv & 0xFFFFFFFFull));
    float mc = kMinFinite, s = 0.f, l = 0.f;
    int found = 0;
    for (int gg = lane; gg < G; gg += 64) {
        const size_t o = ((size_t)k * G + gg) * a.Bpad + b;
        lse_merge(mc, s, agent_load(a.p_mc + o), agent_load(a.p_s + o));
        if (agent_load(a.p_idx + o) == tok) {
            l = agent_load(a.p_l + o);
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
        const bool bad = timed_out || agent_load(a.error) != 0u || !found;
        agent_store(a.tokens + (size_t)b * a.K + k, bad ? -1 : tok);
        if (a.logprobs) a.logprobs[(size_t)b * a.K + k] = bad ? NAN : l * a.inv_t - (mc + fast_log2(s)) * kLn2;
    }
}

__device__ void finalize_pair(const RoundArgs& a, int b, int k, bool timed_out) {
    finalize_with(a, b, k, pick_word(a, k, b), timed_out);
}

// STORE (validation only) also writes every tile's calibrated logits to a.logits_out [B, K, V] before its
// epilogue; the contraction and the pick are the same code.
template <int RK, int MODE, bool GATED, int UR, bool STORE = false>
__global__ void __launch_bounds__(kRoundThreads, 1) markov_round_kernel(RoundArgs a) {
    // The gated half block keeps the gate rows of the next position in LDS (filled by the finalizer wave while the
    // current position streams), so the gather after a grid barrier waits on the W1 rows only.
    constexpr int kConsumers = Waves<UR, GATED>::kConsumers;
    constexpr int kProducers = Waves<UR, GATED>::kProducers;
    static_assert(64 * (kConsumers + kProducers + 1) == kRoundThreads, "nine waves");
    constexpr bool HLDS = GATED && UR == 8;
    constexpr int kHPitch = 16 * RK + 4;  // floats per gate row in LDS (16-byte shift per row: no bank conflicts)
    using RG = Ring<RK, UR, HLDS>;
    constexpr bool SAMPLE = MODE == kModeSample;
    // Consumer sets: a small block (at most 8 rows) fills only one wave's 32 rows, so each of its two consumer
    // waves forms a set of its own on the same rows and takes every other tile of a position (slots s, s + 2,
    // ...), handing its per-row results to set 0 through LDS at the end of the position (the greedy maximum and
    // the block race are both maxima over tiles, merged in set order).  A half block (9 .. 64 rows) runs two sets
    // of two waves the same way.  The gated small block keeps one set of four waves: its gather holds more
    // registers, and with the hand-over code it would spill at three waves per SIMD.
    constexpr int SETS = UR == 8 ? 2 : (UR == 1 && !GATED) ? kConsumers : 1;
    constexpr int kRowWaves = kConsumers / SETS;  // consumer waves of one set (32 rows each)
    __shared__ __attribute__((aligned(1024))) uint8_t ring[RG::kNS * RG::kStage];
    __shared__ uint32_t ready[RG::kNS];  // +1 per producer per filled stage
    __shared__ uint32_t freed[RG::kNS];  // +1 per consumer wave per consumed stage
    __shared__ uint32_t stepdone;        // +1 per consumer wave per finished position
    __shared__ uint32_t released;        // last position whose predecessors are known (set by consumer wave 0)
    // HLDS: H[b, j, :] of rows b < 64 for one position j >= 1; hready = positions filled, hdone = consumer-wave
    // gathers of positions >= 1 done (the buffer is refilled once all consumer waves have read it)
    __shared__ __attribute__((aligned(16))) float hbuf[HLDS ? 64 * kHPitch : 4];
    __shared__ uint32_t hready, hdone;
    // sets 1 .. SETS-1 hand their per-row results of a position to set 0 here (double-buffered by segment
    // parity): key, id (bits), logit of the pick, base-2 max and sum of the log-sum-exp
    constexpr int kHand = SETS > 1 ? SETS - 1 : 1;
    __shared__ float mx[SETS > 1 ? 2 : 1][kHand][SETS > 1 ? kRowWaves : 1][5][32];
    __shared__ uint32_t mput[kHand][kRowWaves], mgot[kHand][kRowWaves];  // segments written / read

    const int lane = threadIdx.x & 63;
    // In the half block the wave index is made wave-uniform, so the hand-over slots and counters of the consumer
    // sets and the release address live in scalar registers: held as per-lane values at 168 registers they
    // spilled, and every reload after a position's last tile was a memory round trip under the stream (gated
    // sampling round 0.383 -> 0.353 ms, greedy 0.351 -> 0.348 ms, same-box A/B).  Other forms keep the plain
    // index, which measured faster there (batch-1 sampling 0.245 against 0.247 ms).
    const int wave = UR == 8 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : (int)(threadIdx.x >> 6);
    const int half = lane >> 5;
    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int r = 16 * RK;
    // Tiles are dealt out cyclically: workgroup g takes tiles g, g + G, g + 2G, ...  At any moment the
    // workgroups then read neighbouring 128-byte pieces of each U row (and one contiguous W2 span), which
    // keeps the HBM row buffers open, where contiguous blocks of tiles per workgroup would scatter the reads.
    const int ntw = (a.ntiles - g + G - 1) / G;
    auto tile_of = [&](int j) { return g + G * j; };
    const int nrb = (a.B + kRRows - 1) / kRRows;
    const int per_k = nrb * ntw;
    const int nitems = a.K * per_k;
    const uint32_t spin_limit = a.spin_limit;

    if (threadIdx.x < RG::kNS) {
        ready[threadIdx.x] = 0u;
        freed[threadIdx.x] = 0u;
    }
    if (threadIdx.x < kHand * kRowWaves) {
        (&mput[0][0])[threadIdx.x] = 0u;
        (&mgot[0][0])[threadIdx.x] = 0u;
    }
    if (threadIdx.x == 0) {
        stepdone = 0u;
        released = 0u;
        hready = 0u;
        hdone = 0u;
    }
    // every wave reads the epoch before workgroup 0 can advance it (at the very end of the launch)
    const uint64_t tag = launch_tag(a, agent_load(a.epoch));
    __syncthreads();

    if (wave >= kConsumers + kProducers) {
        // ============================================================== finalizer
        // Workgroup 0 first clears the winner words, the grid counters and the error word, then publishes the
        // call's sequence number; consumers check it before their first atomics.  No other launch is needed.
        if (g == 0) {
            const size_t nw = (size_t)a.K * a.Bpad * kWinnerSlots;
            for (size_t i = lane; i < nw; i += 64) agent_store(a.winners + i * kWinnerStride, 0ull);
            if (lane < kBarrierGroups) {
                agent_store(a.barrier + kCounterStride * lane, 0u);
                agent_store(a.release + kCounterStride * lane, 0u);
            }
            if (lane == 0) {
                agent_store(a.top, 0u);
                agent_store(a.error, 0u);
            }
            wait_vmcnt<0>();
            if (lane == 0) agent_store(a.flag, tag);
        } else if (lane == 0) {
            wait_cleared(a, tag);  // the counters it polls after the last position must be this launch's
        }
        // c_0 needs only the anchor and h_0
        if (a.cf.h)
            for (int b = g; b < a.B; b += G) confidence_step(a.cf, b, 0);
        // Then, position by position, once every workgroup has finished it (this workgroup's release of the
        // next position, or the release word after the last one): tokens and log-probabilities of rows
        // g, g + G, ...  Until the last position this runs while the rest of the workgroup streams and
        // computes, off the serial path.
        for (int k = 0; k < a.K; ++k) {
            if constexpr (HLDS) {
                if (k + 1 < a.K) {
                    // the gate rows of position k + 1, once every consumer wave has gathered position k
                    uint32_t hs = 0;
                    while (lds_load(&hdone) < (uint32_t)(kConsumers * k)) {
                        __builtin_amdgcn_s_sleep(1);
                        if (++hs > spin_limit) {
                            agent_store(a.error, 1u);
                            break;
                        }
                    }
                    constexpr int kQ = 4 * RK;  // 16-byte pieces per row
                    constexpr int kBatch = 16;
                    const int n4 = min(a.B, 64) * kQ;
                    for (int e0 = 0; e0 < n4; e0 += 64 * kBatch) {
                        f32x4_t hv[kBatch];
#pragma unroll
                        for (int q = 0; q < kBatch; ++q) {
                            const int e = e0 + 64 * q + lane;
                            const int b = e / kQ, c4 = e % kQ;
                            hv[q] = e < n4 ? *reinterpret_cast<const f32x4_t*>(a.H + ((size_t)b * a.K + k + 1) * (16 * RK) + 4 * c4)
                                           : f32x4_t{0.f, 0.f, 0.f, 0.f};
                        }
#pragma unroll
                        for (int q = 0; q < kBatch; ++q) {
                            const int e = e0 + 64 * q + lane;
                            if (e < n4) *reinterpret_cast<f32x4_t*>(hbuf + (e / kQ) * kHPitch + 4 * (e % kQ)) = hv[q];
                        }
                    }
                    wait_lgkmcnt0();
                    __asm__ volatile("" ::: "memory");
                    if (lane == 0) lds_add(&hready, 1u);
                }
            }
            bool timed_out = false;
            uint32_t spins = 0;
            if (k + 1 < a.K) {
                while (lds_load(&released) < (uint32_t)(k + 1)) {
                    __builtin_amdgcn_s_sleep(2);
                    if (++spins > spin_limit) {
                        timed_out = true;
                        break;
                    }
                }
            } else {
                while (released_position(a) < (uint32_t)a.K) {
                    __builtin_amdgcn_s_sleep(1);
                    if (++spins > spin_limit) {
                        timed_out = true;
                        break;
                    }
                }
            }
            if (timed_out && lane == 0) agent_store(a.error, 1u);

            // c_{k+1} needs h_{k+1} and x_k only, so it follows the token of position k at once
            for (int b = g; b < a.B; b += G) {
                finalize_pair(a, b, k, timed_out);
                if (a.cf.h && k + 1 < a.K) confidence_step(a.cf, b, k + 1);
            }
        }
        // every workgroup has arrived after its last position, so all have read the epoch: advance it
        if (g == 0 && lane == 0) agent_store(a.epoch, agent_load(a.epoch) + 1u);
        return;
    }
    if (wave >= kConsumers) {
        // ============================================================== producers: stream W2 and U tiles
        // Ordinary 16-byte vector loads into registers, kDepth items ahead, then ds_write into the padded
        // stage layout the consumers read.  Unit u of an item: u < RK is W2 rows 2u .. (64 lanes x 16 B of the
        // tile's [32, r] block); u >= RK is U row group u - RK (8 rows x 32 floats).
        const int p = wave - kConsumers;
        constexpr int NU = (RG::kUnits + kProducers - 1) / kProducers;  // units per producer and item
        constexpr int D = Waves<UR, GATED>::kDepth ? Waves<UR, GATED>::kDepth : RG::kDepth;
        u32x4_t regs[D][NU];
        // Per-lane parts of every unit's global and LDS addresses, computed once: a load then costs one 64-bit
        // add per unit (index arithmetic per item, with its 64-bit multiplies, took issue cycles from the
        // consumer wave on the same SIMD).
        // W2 unit u covers tile rows 64u / (2 RK) + lane / (2 RK), 8 bf16 at column 8 (lane mod 2 RK) (2 RK
        // divides 64); U unit RK + q covers rows 8q + lane / 8, 4 floats at column 4 (lane mod 8).
        static_assert(64 % (2 * RK) == 0, "a W2 unit holds whole rows");
        const int urow = lane >> 3, ucol = 4 * (lane & 7);
        const uint32_t w2lane = 2u * (uint32_t)((lane / (2 * RK)) * r + 8 * (lane % (2 * RK)));
        const uint64_t ulane = 4ull * ((uint64_t)urow * (uint64_t)a.u_stride + (uint64_t)ucol);
        uint32_t soff[NU];   // byte offset in a stage
#pragma unroll
        for (int n = 0; n < NU; ++n) {
            const int u = p + kProducers * n;
            if (u < RK) {
                const int P = u * 64 + lane;
                const int rho = P / (2 * RK), c = P % (2 * RK);
                soff[n] = (uint32_t)(w2_slot(rho) * RG::kW2Row + 16 * c);
            } else {
                soff[n] = (uint32_t)(RG::kW2Bytes + (8 * (u - RK) + urow) * RG::kURow + 16 * (lane & 7));
            }
        }
        // the next item to load: position, row block, tile slot
        int lk = 0, lrb = 0, lj = 0;
        auto load_next = [&](u32x4_t (&dst)[NU]) {
            const int v0 = tile_of(lj) * kRTileV;
            const int b0 = lrb * kRRows;
            if constexpr (UR == 16) {
                if (v0 + kRTileV <= a.V && b0 + kRRows <= a.B) {
                    const uint8_t* w2b = reinterpret_cast<const uint8_t*>(a.W2t + (size_t)v0 * r);
                    const uint8_t* ub = reinterpret_cast<const uint8_t*>(a.U + (size_t)lk * a.u_kstride + (size_t)b0 * a.u_stride + v0);
#pragma unroll
                    for (int n = 0; n < NU; ++n) {
                        const int u = p + kProducers * n;
                        // W2 is re-read every position: a cacheable load lets it stay in the last-level cache
                        if (u < RK)
                            dst[n] = *reinterpret_cast<const u32x4_t*>(w2b + (size_t)(u * (64 / (2 * RK)) * r * 2) + w2lane);
                        else if (u < RG::kUnits)
                            dst[n] = load_nt_u32x4(ub + (size_t)(u - RK) * 32 * (size_t)a.u_stride + ulane);
                    }
                } else {
                    // a tile past the vocabulary's end or a row block past the batch: clamped rows and columns
#pragma unroll
                    for (int n = 0; n < NU; ++n) {
                        const int u = p + kProducers * n;
                        if (u < RK) {
                            const int P = u * 64 + lane;
                            const int vrow = min(v0 + P / (2 * RK), a.V - 1);
                            dst[n] = *reinterpret_cast<const u32x4_t*>(a.W2t + (size_t)vrow * r + 8 * (P % (2 * RK)));
                        } else if (u < RG::kUnits) {
                            const int b = min(b0 + (u - RK) * 8 + urow, a.B - 1);
                            const int col = min(v0 + ucol, a.V - 4);
                            dst[n] = load_nt_u32x4(a.U + (size_t)lk * a.u_kstride + (size_t)b * a.u_stride + col);
                        }
                    }
                }
            } else {
                // small block: W2 units take the precomputed addresses whenever the tile is whole; the U unit
                // (rows 0..7 of the block) clamps its rows to the batch
                const uint8_t* w2b = reinterpret_cast<const uint8_t*>(a.W2t + (size_t)v0 * r);
                const bool vfull = v0 + kRTileV <= a.V;
#pragma unroll
                for (int n = 0; n < NU; ++n) {
                    const int u = p + kProducers * n;
                    if (u < RK) {
                        if (vfull) {
                            dst[n] = *reinterpret_cast<const u32x4_t*>(w2b + (size_t)(u * (64 / (2 * RK)) * r * 2) + w2lane);
                        } else {
                            const int P = u * 64 + lane;
                            const int vrow = min(v0 + P / (2 * RK), a.V - 1);
                            dst[n] = *reinterpret_cast<const u32x4_t*>(a.W2t + (size_t)vrow * r + 8 * (P % (2 * RK)));
                        }
                    } else if (u < RG::kUnits) {
                        const int b = min(b0 + (u - RK) * 8 + urow, a.B - 1);
                        const int col = min(v0 + ucol, a.V - 4);
                        dst[n] = load_nt_u32x4(a.U + (size_t)lk * a.u_kstride + (size_t)b * a.u_stride + col);
                    }
                }
            }
            if (++lj == ntw) {
                lj = 0;
                if (++lrb == nrb) {
                    lrb = 0;
                    ++lk;
                }
            }
        };
        // The 16-byte LDS writes of an item go out in pairs with a short sleep between pairs.  Eight writes in a
        // burst (32 KB per CU per item over the four producers) delay the consumer waves' operand reads on the
        // same CU: a consumer's tile took 0.74 us with the producers writing and 0.42 us without.  The producers
        // mostly wait for a free stage anyway, so spacing the writes costs them nothing (serving round 0.463 ->
        // 0.453 ms mean, with a much shorter tail, in same-box A/B; wider spacing starts to delay the stream).
        auto store = [&](int i, const u32x4_t (&src)[NU]) {
            uint8_t* st = ring + (i % RG::kNS) * RG::kStage;
#pragma unroll
            for (int n = 0; n < NU; ++n) {
                if (p + kProducers * n < RG::kUnits) *reinterpret_cast<u32x4_t*>(st + soff[n]) = src[n];
                if (UR == 16 && n % 2 == 1 && n + 1 < NU) __builtin_amdgcn_s_sleep(3);
            }
        };
        auto publish = [&](int i, const u32x4_t (&src)[NU]) {
            if (i >= RG::kNS) {
                const uint32_t need = (uint32_t)kRowWaves * (uint32_t)(i / RG::kNS);  // one set consumes an item
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
        // The stream runs ahead across position boundaries as far as the ring and the registers allow (kNS + D
        // items).  Holding back the next position's loads until the boundary had passed helped while the grid
        // barrier polled counters that every workgroup shared; with the arrival tree it costs 3%.
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (d < nitems) load_next(regs[d]);
        for (int i0 = 0; i0 < nitems; i0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int i = i0 + d;
                if (i < nitems) {
                    publish(i, regs[d]);
                    if (i + D < nitems) load_next(regs[d]);
                }
            }
        }
        return;
    }

    // ================================================================== consumers: contraction and pick
    bf16x8_t xf[RK];
    uint32_t k2 = 0;
    float m = kNegBig, s = 0.f;  // running max of l (natural units) and sum of 2^(l c - m c)
    // sampling: mass of the lane's best block so far (scaled as s), its race variate E = -log2 u, and the mass
    // of the id drawn inside it
    float bs = 0.f, bE = 1.f, be = 0.f;
    float bl = -INFINITY;        // greedy: best logit
    int bslot = 0, btile = -1;   // best id = 32 btile + 16 half + bslot
    float* store_row = nullptr;  // STORE: this lane's row of the current position in a.logits_out, or null
    const float c = a.c;
    const int rho = lane & 31;
    const int cset = SETS > 1 ? wave / kRowWaves : 0;                    // tile slots cset, cset + SETS, ...
    const int wrow = SETS > 1 ? wave % kRowWaves : wave;
    const int rr = wrow * 32 + rho;                                      // this lane's row of the 128-row block
    const int a_off = rho * RG::kW2Row + 16 * half;                      // its A-operand row in a stage
    // its 16 U values in a stage (a small block holds rows 0..7 only; the rows after them are past the batch)
    const int u_off = RG::kW2Bytes + (UR == 16 ? rr : min(rr, 8 * UR - 1)) * RG::kURow + 64 * half;

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
        __asm__ volatile("" ::: "memory");  // stage reads stay after the wait
    };
    auto release = [&](int i) {
        wait_lgkmcnt0();
        __asm__ volatile("" ::: "memory");  // and before the release
        if (lane == 0) lds_add(&freed[i % RG::kNS], 1u);
    };
    // The U values of stage i seed the accumulator, so the MFMAs produce U + W2^T X directly.
    auto read_u = [&](int i) -> f32x16_t {
        const uint8_t* p = ring + (i % RG::kNS) * RG::kStage + u_off;
        const f32x4_t q0 = *reinterpret_cast<const f32x4_t*>(p);
        const f32x4_t q1 = *reinterpret_cast<const f32x4_t*>(p + 16);
        const f32x4_t q2 = *reinterpret_cast<const f32x4_t*>(p + 32);
        const f32x4_t q3 = *reinterpret_cast<const f32x4_t*>(p + 48);
        const f32x8_t lo = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
        const f32x8_t hi = __builtin_shufflevector(q2, q3, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    };
    // STORE: the lane's 16 logits of tile t (ids 32 t + 16 half + j), ids past the vocabulary left out
    auto store_tile = [&](const f32x16_t& lv, int t) {
        if constexpr (STORE) {
            if (!store_row) return;
            const int v0 = t * kRTileV + 16 * half;
            float* d = store_row + v0;
            if (v0 + 16 <= a.V) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<f32x4_t*>(d + 4 * q) = f32x4_t{lv[4 * q], lv[4 * q + 1], lv[4 * q + 2], lv[4 * q + 3]};
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (v0 + j < a.V) d[j] = lv[j];
            }
        }
    };
    auto frag = [&](int i, int j) -> bf16x8_t {
        return *reinterpret_cast<const bf16x8_t*>(ring + (i % RG::kNS) * RG::kStage + a_off + 32 * j);
    };
    // Start of a tile's epilogue (needs all 16 values): optional tail mask, tile max, running max and rescale.
    // Returns the tile max; mc = m * c afterwards.
    auto tile_head = [&](f32x16_t& lv, int t, auto mask_tail, float& mc) -> float {
        if (decltype(mask_tail)::value) {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (t * kRTileV + 16 * half + j >= a.V) lv[j] = -INFINITY;
        }
        float cm = fmaxf(fmaxf(lv[0], lv[1]), lv[2]);
#pragma unroll
        for (int j = 3; j < 15; j += 2) cm = fmaxf(fmaxf(cm, lv[j]), lv[j + 1]);
        cm = fmaxf(cm, lv[15]);
        const float mn = fmaxf(m, cm);
        const float scale = fast_exp2((m - mn) * c);
        s *= scale;
        if (SAMPLE) {
            bs *= scale;
            be *= scale;
        }
        m = mn;
        mc = mn * c;
        return cm;
    };
    // Greedy pick update of a tile (after its MFMA successor has been issued: it may branch).  A lane's ids
    // ascend with the slot, so the first slot equal to the tile max is the lowest id.
    auto greedy_pick = [&](const f32x16_t& lv, float cm, int t) {
        if (cm > bl) {
            int sl = 15;
#pragma unroll
            for (int j = 14; j >= 0; --j) sl = (lv[j] == cm) ? j : sl;
            bl = cm;
            bslot = sl;
            btile = t;
        }
    };
    auto greedy_elem = [&](const f32x16_t& lv, int j, float mc) { s += fast_exp2(fmaf(lv[j], c, -mc)); };

    // Sampling draws over the whole vocabulary with a two-level exponential race.  A lane's 16 ids of a tile
    // are one aligned block (ids 16 q .. 16 q + 15, q = 2 t + half).  The block's mass S = sum_v 2^(l_v c - m c)
    // races with one variate E = -log2 u(2 q): the block with the largest S / E wins, and inside the winner the
    // id is drawn by inverse CDF with target u(2 q + 1) S, where u(n) is the uniform of hash fmix32(k2 ^ n).
    // The winner is distributed as S / sum S (independent exponential clocks) and the id inside as its share
    // of S, so the draw is exactly softmax(l / T): one hash pair and one logarithm per 16 ids.
    // Pass 1, element j: its mass replaces the logit in lv, and sb accumulates the block mass in slot order.
    auto sample_mass = [&](f32x16_t& lv, int j, float mc, float& sb) {
        lv[j] = fast_exp2(fmaf(lv[j], c, -mc));
        sb += lv[j];
    };
    // The block's race variate and the inverse-CDF target, which stays strictly below the block mass.
    auto sample_block = [&](int t, float sb, float& E, float& target) {
        block_race_variates(k2, 2u * (uint32_t)t + (uint32_t)half, sb, E, target);
    };
    // Pass 2, element j < 15: the drawn slot is the number of inclusive prefixes (same order as sb) at or
    // below the target; esel follows the mass of that slot.
    auto sample_cdf = [&](const f32x16_t& lv, int j, float target, float& cum, int& sel, float& esel) {
        cum += lv[j];
        const bool below = cum <= target;
        sel += below ? 1 : 0;
        esel = below ? lv[j + 1] : esel;
    };
    // The race against the lane's best block: S / E > bs / bE.
    auto sample_update = [&](int t, float sb, float E, int sel, float esel) {
        const bool better = sb * bE > bs * E;
        bs = better ? sb : bs;
        bE = better ? E : bE;
        be = better ? esel : be;
        bslot = better ? sel : bslot;
        btile = better ? t : btile;
    };

    // A tile's epilogue in one straight-line block with the operand reads and the MFMAs of the set's next tile
    // (item in, into nxt), so the matrix cores' dependent accumulation chain runs under the vector ALUs' work.
    auto pipelined = [&](f32x16_t& cur, f32x16_t& nxt, int in, int t) {
        const std::integral_constant<bool, false> kUnmasked{};
        // The next tile's reads first (its U tile and the first two A operands), then the head of this tile's
        // epilogue while they land.  Then 16 steps, each: the A operand two MFMAs ahead, one MFMA and a share
        // of the epilogue's vector work.  The scheduling barriers keep that order: left alone, the scheduler
        // reads each A operand right before its MFMA and stalls the wave on every read.
        nxt = read_u(in);
        bf16x8_t fr[RK];
        fr[0] = frag(in, 0);
        if (RK > 1) fr[1] = frag(in, 1);
        __builtin_amdgcn_sched_barrier(0);
        store_tile(cur, t);
        float mc;
        const float cm = tile_head(cur, t, kUnmasked, mc);
        float sb = 0.f, E = 1.f, target = 0.f, cum = 0.f, esel = 0.f;
        int sel = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j + 2 < RK) fr[j + 2] = frag(in, j + 2);
            if (j < RK) nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[j], xf[j], nxt, 0, 0, 0);
            if (SAMPLE) {
                // steps 0-7: masses of slots 2j, 2j+1; step 8: the block's variates; steps 8-15: inverse CDF
                if (j < 8) {
                    sample_mass(cur, 2 * j, mc, sb);
                    sample_mass(cur, 2 * j + 1, mc, sb);
                } else {
                    if (j == 8) {
                        s += sb;
                        sample_block(t, sb, E, target);
                        esel = cur[0];
                    }
                    sample_cdf(cur, 2 * (j - 8), target, cum, sel, esel);
                    if (j < 15) sample_cdf(cur, 2 * (j - 8) + 1, target, cum, sel, esel);
                    else sample_update(t, sb, E, sel, esel);
                }
            } else {
                greedy_elem(cur, j, mc);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (!SAMPLE) greedy_pick(cur, cm, t);
    };
    auto last = [&](f32x16_t& cur, int t, auto mask_tail) {
        store_tile(cur, t);
        float mc;
        const float cm = tile_head(cur, t, mask_tail, mc);
        if (SAMPLE) {
            float sb = 0.f, E, target, cum = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) sample_mass(cur, j, mc, sb);
            s += sb;
            sample_block(t, sb, E, target);
            float esel = cur[0];
            int sel = 0;
#pragma unroll
            for (int j = 0; j < 15; ++j) sample_cdf(cur, j, target, cum, sel, esel);
            sample_update(t, sb, E, sel, esel);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) greedy_elem(cur, j, mc);
            greedy_pick(cur, cm, t);
        }
    };

    const int nseg = a.K * nrb;
    for (int seg = 0; seg < nseg; ++seg) {
        const int k = seg / nrb;
        const int rb = seg - k * nrb;
        const int i0 = seg * ntw;
        const int b = rb * kRRows + rr;
        const bool valid_b = b < a.B;
        const bool wave_live = rb * kRRows + wrow * 32 < a.B;

        // a new position (or row block): wait for the previous position's picks, then gather X.  Consumer wave 0
        // polls this workgroup's copy of the release word; the other consumer waves wait for its LDS flag.
        if (k > 0 && rb == 0) {
            if (wave == 0) {
                uint32_t spins = 0;
                while (true) {
                    if (released_position(a) >= (uint32_t)k) break;
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
                    const unsigned long long wv = pick_word(a, k - 1, b);
                    pv = (int)(0xFFFFFFFFu - (uint32_t)(wv & 0xFFFFFFFFull));
                    pv = min(max(pv, 0), a.V - 1);
                }
            }
            const u32x4_t* wrow = reinterpret_cast<const u32x4_t*>(a.W1 + (size_t)pv * r);
            if (HLDS && k > 0) {
                // W1 row chunks first (they need only the pick), then the gate row from LDS once it is there
                u32x4_t raw[RK];
#pragma unroll
                for (int q = 0; q < RK; ++q) raw[q] = wrow[2 * q + half];
                uint32_t hs = 0;
                while (lds_load(&hready) < (uint32_t)k) {
                    __builtin_amdgcn_s_sleep(0);
                    if (++hs > spin_limit) {
                        __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
                __asm__ volatile("" ::: "memory");  // gate reads stay after the wait
                const float* hl = hbuf + (valid_b ? b : 0) * kHPitch + 8 * half;
#pragma unroll
                for (int q = 0; q < RK; ++q) {
                    const f32x4_t h0 = *reinterpret_cast<const f32x4_t*>(hl + 16 * q);
                    const f32x4_t h1 = *reinterpret_cast<const f32x4_t*>(hl + 16 * q + 4);
                    const float hf[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
                    const uint32_t w32[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
                    uint32_t o32[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float lo = bf16_to_f32((uint16_t)(w32[e] & 0xFFFFu)) * hf[2 * e];
                        const float hi = bf16_to_f32((uint16_t)(w32[e] >> 16)) * hf[2 * e + 1];
                        o32[e] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
                    }
                    const u32x4_t o = valid_b ? u32x4_t{o32[0], o32[1], o32[2], o32[3]} : u32x4_t{0u, 0u, 0u, 0u};
                    xf[q] = __builtin_bit_cast(bf16x8_t, o);
                }
            } else if constexpr (GATED) {
                // X = bf16(W1[a] * H) in phases of kPh 16-value chunks.  Each phase issues all of its loads (W1
                // row chunks, H chunks) before its multiplies, so the gather costs the pick read and one memory
                // round trip per phase, rather than one per chunk; four phases fit the register budget at
                // r = 256.  Rows past the batch load row 0 and are zeroed.
                constexpr int kPh = RK >= 4 ? RK / 4 : 1;
                const float* hrow = a.H + ((size_t)(valid_b ? b : 0) * a.K + k) * r + 8 * half;
                auto apply = [&](const u32x4_t raw, const f32x4_t h0, const f32x4_t h1) -> bf16x8_t {
                    const float hf[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
                    const uint32_t w32[4] = {raw.x, raw.y, raw.z, raw.w};
                    uint32_t o32[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float lo = bf16_to_f32((uint16_t)(w32[e] & 0xFFFFu)) * hf[2 * e];
                        const float hi = bf16_to_f32((uint16_t)(w32[e] >> 16)) * hf[2 * e + 1];
                        o32[e] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
                    }
                    const u32x4_t o = valid_b ? u32x4_t{o32[0], o32[1], o32[2], o32[3]} : u32x4_t{0u, 0u, 0u, 0u};
                    return __builtin_bit_cast(bf16x8_t, o);
                };
#pragma unroll
                for (int p0 = 0; p0 < RK; p0 += kPh) {
                    u32x4_t raw[kPh];
#pragma unroll
                    for (int q = 0; q < kPh; ++q) raw[q] = wrow[2 * (p0 + q) + half];
                    f32x4_t hv[2 * kPh];
#pragma unroll
                    for (int q = 0; q < kPh; ++q) {
                        hv[2 * q] = *reinterpret_cast<const f32x4_t*>(hrow + 16 * (p0 + q));
                        hv[2 * q + 1] = *reinterpret_cast<const f32x4_t*>(hrow + 16 * (p0 + q) + 4);
                    }
#pragma unroll
                    for (int q = 0; q < kPh; ++q) xf[p0 + q] = apply(raw[q], hv[2 * q], hv[2 * q + 1]);
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < RK; ++kk) {
                    const u32x4_t raw = valid_b ? wrow[2 * kk + half] : u32x4_t{0u, 0u, 0u, 0u};
                    xf[kk] = __builtin_bit_cast(bf16x8_t, raw);
                }
            }
            if (SAMPLE) k2 = noise_key2(a.k0, (uint32_t)b, (uint32_t)k);
        }
        if (HLDS && k > 0 && rb == 0) {
            // this wave's reads of the gate rows are done: the finalizer may refill the buffer
            wait_lgkmcnt0();
            __asm__ volatile("" ::: "memory");
            if (lane == 0) lds_add(&hdone, 1u);
        }
        if constexpr (STORE) store_row = valid_b ? a.logits_out + ((size_t)b * a.K + k) * (size_t)a.V : nullptr;
        m = kNegBig;
        s = 0.f;
        bs = 0.f;
        bE = 1.f;
        be = 0.f;
        bl = -INFINITY;
        bslot = 0;
        btile = -1;

        // Software pipeline over the segment's tiles (with several sets: over the set's tile slots cset,
        // cset + SETS, ...), unrolled by two so the accumulator sets alternate.
        f32x16_t acc_a, acc_b;
        const std::integral_constant<bool, true> kMasked{};
        const std::integral_constant<bool, false> kUnmasked{};
        if constexpr (SETS == 1) {
            wait_ready(i0);
            if (wave_live) {
                acc_a = read_u(i0);
#pragma unroll
                for (int j = 0; j < RK; ++j) acc_a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(i0, j), xf[j], acc_a, 0, 0, 0);
            }
            release(i0);
            int tt = 0;
            for (; tt + 2 < ntw; tt += 2) {
                wait_ready(i0 + tt + 1);
                if (wave_live) pipelined(acc_a, acc_b, i0 + tt + 1, tile_of(tt));
                release(i0 + tt + 1);
                wait_ready(i0 + tt + 2);
                if (wave_live) pipelined(acc_b, acc_a, i0 + tt + 2, tile_of(tt + 1));
                release(i0 + tt + 2);
            }
            // one or two tiles left, the first in acc_a; only the segment's last tile can be the vocabulary's tail
            const bool tail = tile_of(ntw - 1) == a.ntiles - 1 && a.ntiles * kRTileV > a.V;
            if (tt + 1 < ntw) {
                wait_ready(i0 + tt + 1);
                if (wave_live) pipelined(acc_a, acc_b, i0 + tt + 1, tile_of(tt));
                release(i0 + tt + 1);
                if (wave_live) {
                    if (tail) last(acc_b, tile_of(tt + 1), kMasked);
                    else last(acc_b, tile_of(tt + 1), kUnmasked);
                }
            } else if (tt < ntw) {
                if (wave_live) {
                    if (tail) last(acc_a, tile_of(tt), kMasked);
                    else last(acc_a, tile_of(tt), kUnmasked);
                }
            }
        } else {
            const int nts = (ntw - cset + SETS - 1) / SETS;
            auto slot = [&](int u) { return cset + SETS * u; };
            if (nts > 0) {
                wait_ready(i0 + slot(0));
                if (wave_live) {
                    acc_a = read_u(i0 + slot(0));
#pragma unroll
                    for (int j = 0; j < RK; ++j)
                        acc_a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(i0 + slot(0), j), xf[j], acc_a, 0, 0, 0);
                }
                release(i0 + slot(0));
                int u = 0;
                for (; u + 2 < nts; u += 2) {
                    wait_ready(i0 + slot(u + 1));
                    if (wave_live) pipelined(acc_a, acc_b, i0 + slot(u + 1), tile_of(slot(u)));
                    release(i0 + slot(u + 1));
                    wait_ready(i0 + slot(u + 2));
                    if (wave_live) pipelined(acc_b, acc_a, i0 + slot(u + 2), tile_of(slot(u + 1)));
                    release(i0 + slot(u + 2));
                }
                // one or two tiles left, the first in acc_a; only the segment's last slot can be the vocabulary's tail
                const bool tail = slot(nts - 1) == ntw - 1 && tile_of(ntw - 1) == a.ntiles - 1 && a.ntiles * kRTileV > a.V;
                if (u + 1 < nts) {
                    wait_ready(i0 + slot(u + 1));
                    if (wave_live) pipelined(acc_a, acc_b, i0 + slot(u + 1), tile_of(slot(u)));
                    release(i0 + slot(u + 1));
                    if (wave_live) {
                        if (tail) last(acc_b, tile_of(slot(u + 1)), kMasked);
                        else last(acc_b, tile_of(slot(u + 1)), kUnmasked);
                    }
                } else {
                    if (wave_live) {
                        if (tail) last(acc_a, tile_of(slot(u)), kMasked);
                        else last(acc_a, tile_of(slot(u)), kUnmasked);
                    }
                }
            }
        }

        // end of this position / row block: lane merge, merge of the sets, global pick, log-sum-exp partials.
        // With several sets every consumer wave takes part in the hand-over (a set without tiles carries neutral
        // values), so the hand-over counters stay in step.
        if (SETS > 1 || wave_live) {
            int bi = (btile >= 0) ? 32 * btile + 16 * half + bslot : 0x7FFFFFFF;
            float key, lbest;
            if (SAMPLE) {
                // race key log2(S / E) with S in absolute units, and the logit of the drawn id from its mass
                const float mcb = m * c;
                key = (bs > 0.f) ? fast_log2(bs) + mcb - fast_log2(bE) : -INFINITY;
                lbest = (fast_log2(be) + mcb) / c;
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
            if constexpr (SETS > 1) {
                // sets 1 .. SETS-1 hand over; set 0 merges them in set order
                const int mb = seg & 1;
                if (cset > 0) {
                    const int h = cset - 1;
                    uint32_t spins = 0;
                    while (lds_load(&mgot[h][wrow]) + 1u < (uint32_t)seg) {  // set 0 has read this buffer's last use
                        __builtin_amdgcn_s_sleep(0);
                        if (++spins > spin_limit) {
                            __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            break;
                        }
                    }
                    if (half == 0) {
                        float* q = &mx[mb][h][wrow][0][rho];
                        q[0] = key;
                        q[32] = __int_as_float(bi);
                        q[64] = lbest;
                        q[96] = mc2;
                        q[128] = s2;
                    }
                    wait_lgkmcnt0();
                    __asm__ volatile("" ::: "memory");
                    if (lane == 0) lds_add(&mput[h][wrow], 1u);
                } else {
#pragma unroll
                    for (int h = 0; h < SETS - 1; ++h) {
                        uint32_t spins = 0;
                        while (lds_load(&mput[h][wrow]) < (uint32_t)(seg + 1)) {
                            __builtin_amdgcn_s_sleep(0);
                            if (++spins > spin_limit) {
                                __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                break;
                            }
                        }
                        __asm__ volatile("" ::: "memory");
                        const float* q = &mx[mb][h][wrow][0][rho];
                        const float okey2 = q[0];
                        const int oi2 = __float_as_int(q[32]);
                        const float ol2 = q[64];
                        const float omc2 = q[96];
                        const float os2 = q[128];
                        wait_lgkmcnt0();
                        __asm__ volatile("" ::: "memory");
                        if (lane == 0) lds_add(&mgot[h][wrow], 1u);
                        if (beats(okey2, oi2, key, bi)) {
                            key = okey2;
                            bi = oi2;
                            lbest = ol2;
                        }
                        lse_merge(mc2, s2, omc2, os2);
                    }
                }
            }
            // the winner words and counters of this launch are cleared before the first atomics touch them
            if (cset == 0 && seg == 0 && lane == 0) wait_cleared(a, tag);
            if (cset == 0 && half == 0 && valid_b) {
                const unsigned long long packed =
                    ((unsigned long long)ordered_key(key) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)bi);
                atomicMax(a.winners + (((size_t)k * a.Bpad + b) * kWinnerSlots + g % kWinnerSlots) * kWinnerStride, packed);
                const size_t o = ((size_t)k * G + g) * a.Bpad + b;
                // read by other workgroups' finalizers within this launch
                agent_store(a.p_mc + o, mc2);
                agent_store(a.p_s + o, s2);
                agent_store(a.p_idx + o, bi);
                agent_store(a.p_l + o, lbest);
            }
        }
        if (rb == nrb - 1 && cset == 0) {
            // this wave's picks of position k are performed once its memory operations have completed
            wait_vmcnt<0>();
            int last_all = 0;
            if (lane == 0) {
                const uint32_t prev = __hip_atomic_fetch_add(&stepdone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (prev == (uint32_t)kRowWaves * (uint32_t)(k + 1) - 1u)  // last set-0 wave of the workgroup
                    last_all = arrive(a, k) ? 1 : 0;
            }
            // the grid's last arrival writes every copy of the release word
            if (__shfl(last_all, 0) && lane < kBarrierGroups)
                agent_store(a.release + kCounterStride * lane, (uint32_t)(k + 1));
        }
    }
}

// The confidence head after a draft made position by position: one wave per row, positions in order.
__global__ void __launch_bounds__(64) confidence_kernel(ConfArgs c) {
    for (int k = 0; k < c.K; ++k) confidence_step(c, blockIdx.x, k);
}

// ====================================================================================================================
// The resident round: one row (B = 1), r = 256, greedy picks.
//
// A single row's draft with the tiled round streams all of W2 at every position (2 r V bytes, 77.8 MB at V = 151936)
// to compute one row of logits.  Here each lane of ten waves per workgroup holds one vocabulary row of W2 (256 bf16
// in 128 registers) for the whole round, read once at the start; a position then reads only its base logits, the
// previous pick and one W1 row (and gate row), and each lane forms its logit U_k[v] + W2[v] . X with v_dot2 on bf16
// pairs against X broadcast from LDS.  Workgroup g covers the ids [g V / G, (g + 1) V / G), at most 640 of them.
//
// With no stream to overlap, a position is a chain of memory round trips, so the hand-over is kept short: each
// workgroup writes its packed (key, ~id) word for position k into a slot of its own (slot[k][g] in the winner
// array, cleared at the start of the launch; a written word is never zero), and an eleventh wave of every
// workgroup (the pick wave, which holds no W2 row) polls the G slots of position k until all are written and takes
// their maximum, the same pick the tiled round's atomic maximum gives, then hands it to its workgroup through LDS.
// That replaces the atomic maximum, the arrival counters, the release word and the pick read by one store and one
// polled read.  The log-sum-exp partials are written just before the slot word, and each wave waits for all its
// stores at the next position before the workgroup's next slot word, so partials of position k are complete once
// every slot of position k + 1 (or every done word after the last position) is written; the pick wave of
// workgroup 0 merges them then, one position behind.
constexpr int kResWaves = 10;                       // waves holding W2 rows, one id per lane
constexpr int kResThreads = 64 * (kResWaves + 1);   // and the pick wave
constexpr int kResR = 256;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// One wave: waits (bounded) until all G slot words of position k are written, then returns their maximum (0 and
// *timed_out set if the wait gave up).
__device__ unsigned long long resident_slots(const RoundArgs& a, int k, int G, bool* timed_out) {
    constexpr int kPer = 1024 / 64;  // words per lane at the largest grid
    const int lane = threadIdx.x & 63;
    const unsigned long long* row = a.winners + (size_t)k * G;
    uint32_t spins = 0;
    while (true) {
        // every word of a pass is requested before any is examined: one round trip per pass
        unsigned long long wv[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) wv[i] = (lane + 64 * i < G) ? agent_load(row + lane + 64 * i) : ~0ull;
        unsigned long long best = 0ull;
        bool all = true;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const bool used = lane + 64 * i < G;
            all = all && wv[i] != 0ull;
            best = (used && wv[i] > best) ? wv[i] : best;
        }
        if (__all(all)) {
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const unsigned long long o = __shfl_xor(best, off);
                best = o > best ? o : best;
            }
            return best;
        }
        __builtin_amdgcn_s_sleep(1);
        if (++spins > a.spin_limit) {
            *timed_out = true;
            return 0ull;
        }
    }
}

template <bool GATED, bool STORE>
__global__ void __launch_bounds__(kResThreads, 1) markov_resident_kernel(RoundArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t xs[kResWaves][kResR / 2];  // each wave's copy of X (bf16 pairs)
    // per wave and position: best logit, its id, base-2 max and sum of the log-sum-exp (read by the workgroup's last
    // wave to finish the position, which merges them in wave order)
    __shared__ float wkey[kResWaves], wmc[kResWaves], wsum[kResWaves];
    __shared__ int wid[kResWaves];
    // stepdone: waves done per position; donecnt: waves past the last position (a counter of its own, since a wave
    // reaches it without waiting for the others); picked: positions whose pick the pick wave has placed in ptok
    __shared__ uint32_t stepdone, donecnt, picked;
    __shared__ int ptok;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = gridDim.x;
    const int g = blockIdx.x;
    const uint32_t spin_limit = a.spin_limit;
    if (threadIdx.x == 0) {
        stepdone = 0u;
        donecnt = 0u;
        picked = 0u;
        ptok = 0;
    }
    const uint64_t tag = launch_tag(a, agent_load(a.epoch));
    __syncthreads();

    if (wave == kResWaves) {
        // ============================================================== pick wave (and, in workgroup 0, finalizer)
        // Polls the slot words of each position and hands the pick to this workgroup's waves through LDS; the
        // waves that hold W2 rows have no registers to spare for a poll.  In workgroup 0 it then merges the
        // previous position, whose partials are complete now (see above).
        if (g == 0) {
            const size_t nw = (size_t)(a.K + 1) * G;
            for (size_t i = lane; i < nw; i += 64) agent_store(a.winners + i, 0ull);
            if (lane == 0) agent_store(a.error, 0u);
            wait_vmcnt<0>();
            if (lane == 0) agent_store(a.flag, tag);
            if (a.cf.h) confidence_step(a.cf, 0, 0);
        } else if (lane == 0) {
            wait_cleared(a, tag);  // no slot word is read before this launch has cleared it
        }
        unsigned long long prev = 0ull;
        bool prev_to = false;
        // workgroup 0 follows every position and the done words; the others need the picks of 0 .. K - 2 only
        const int kend = g == 0 ? a.K : a.K - 2;
        for (int k = 0; k <= kend; ++k) {
            bool timed_out = false;
            const unsigned long long wv = resident_slots(a, k, G, &timed_out);
            if (timed_out && lane == 0) agent_store(a.error, 1u);
            if (k + 1 < a.K && lane == 0) {
                ptok = (int)(0xFFFFFFFFu - (uint32_t)(wv & 0xFFFFFFFFull));
                __hip_atomic_store(&picked, (uint32_t)(k + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            if (g == 0 && k >= 1) {
                // c_k needs x_{k-1} only, so it follows the token of position k - 1 at once
                finalize_with(a, 0, k - 1, prev, prev_to || timed_out);
                if (a.cf.h && k < a.K) confidence_step(a.cf, 0, k);
            }
            prev = wv;
            prev_to = timed_out;
        }
        // every workgroup has written its done word, so all have read the epoch: advance it
        if (g == 0 && lane == 0) agent_store(a.epoch, agent_load(a.epoch) + 1u);
        return;
    }

    // ================================================================== W2 rows resident in registers
    const int v_lo = (int)(((int64_t)g * a.V) / G);
    const int v_hi = (int)(((int64_t)(g + 1) * a.V) / G);
    const int v = v_lo + 64 * wave + lane;
    const bool live = v < v_hi;
    u32x4_t w[kResR / 8];
    {
        const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(a.W2t + (size_t)(live ? v : v_lo) * kResR);
#pragma unroll
        for (int q = 0; q < kResR / 8; ++q) w[q] = wp[q];
    }
    const float c = a.c;
    float u_next = live ? a.U[v] : 0.f;
    for (int k = 0; k <= a.K; ++k) {
        if (k == a.K) {
            // after the last position: a done word once every wave's stores are complete
            wait_vmcnt<0>();
            int last = 0;
            if (lane == 0)
                last = __hip_atomic_fetch_add(&donecnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) ==
                       (uint32_t)kResWaves - 1u;
            if (lane == 0 && last) agent_store(a.winners + (size_t)k * G + g, 1ull);
            break;
        }
        const float u_cur = u_next;
        // the previous position's pick, from the pick wave through LDS
        int pv;
        if (k == 0) {
            pv = a.anchor[0];
        } else {
            uint32_t spins = 0;
            while (__hip_atomic_load(&picked, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < (uint32_t)k) {
                __builtin_amdgcn_s_sleep(0);
                if (++spins > spin_limit) {
                    __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
            pv = ptok;
        }
        pv = min(max(pv, 0), a.V - 1);
        // X = W1[pv] (gated: bf16(W1[pv] * H[0, k])) into this wave's LDS copy, one 16-byte chunk per lane
        if (lane < kResR / 8) {
            u32x4_t raw = reinterpret_cast<const u32x4_t*>(a.W1 + (size_t)pv * kResR)[lane];
            if constexpr (GATED) {
                const float* hrow = a.H + (size_t)k * kResR + 8 * lane;
                const f32x4_t h0 = *reinterpret_cast<const f32x4_t*>(hrow);
                const f32x4_t h1 = *reinterpret_cast<const f32x4_t*>(hrow + 4);
                const float hf[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
                const uint32_t w32[4] = {raw.x, raw.y, raw.z, raw.w};
                uint32_t o32[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = bf16_to_f32((uint16_t)(w32[e] & 0xFFFFu)) * hf[2 * e];
                    const float hi = bf16_to_f32((uint16_t)(w32[e] >> 16)) * hf[2 * e + 1];
                    o32[e] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
                }
                raw = u32x4_t{o32[0], o32[1], o32[2], o32[3]};
            }
            *reinterpret_cast<u32x4_t*>(&xs[wave][4 * lane]) = raw;
        }
        wait_lgkmcnt0();
        __asm__ volatile("" ::: "memory");  // the wave's X writes land before its reads
        // l = U_k[v] + W2[v] . X, two partial sums added in a fixed order
        float acc0 = u_cur, acc1 = 0.f;
#pragma unroll
        for (int q = 0; q < kResR / 8; ++q) {
            const u32x4_t x = *reinterpret_cast<const u32x4_t*>(&xs[wave][4 * q]);
            acc0 = dot2_bf16(w[q].x, x.x, acc0);
            acc1 = dot2_bf16(w[q].y, x.y, acc1);
            acc0 = dot2_bf16(w[q].z, x.z, acc0);
            acc1 = dot2_bf16(w[q].w, x.w, acc1);
        }
        const float l = acc0 + acc1;
        if constexpr (STORE) {
            if (live) a.logits_out[(size_t)k * a.V + v] = l;
        }
        // the wave's pick (largest logit, lowest id on ties) and log-sum-exp terms
        float bk = live ? l : -INFINITY;
        int bi = live ? v : 0x7FFFFFFF;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ok = __shfl_xor(bk, off);
            const int oi = __shfl_xor(bi, off);
            if (beats(ok, oi, bk, bi)) {
                bk = ok;
                bi = oi;
            }
        }
        const float mc = fmaxf(bk, kNegBig) * c;
        float e = live ? fast_exp2(fmaf(l, c, -mc)) : 0.f;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) e += __shfl_xor(e, off);
        if (k == 0 && lane == 0) wait_cleared(a, tag);  // this launch's slot words are cleared before any is written
        if (lane == 0) {
            wkey[wave] = bk;
            wid[wave] = bi;
            wmc[wave] = mc;
            wsum[wave] = e;
        }
        // this wave's stores of earlier positions (partials, slot word) are complete before the workgroup's next word
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        __asm__ volatile("" ::: "memory");
        int last = 0;
        if (lane == 0)
            last = __hip_atomic_fetch_add(&stepdone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) ==
                   (uint32_t)kResWaves * (uint32_t)(k + 1) - 1u;
        // the next position's base logit, issued after the wait above so that it lands during the hand-over
        if (k + 1 < a.K) {
            const float* ub = a.U + (size_t)(k + 1) * a.u_kstride;  // wave-uniform base, 32-bit lane offset
            u_next = live ? ub[(uint32_t)v] : 0.f;
        }
        if (__shfl(last, 0)) {
            // the workgroup's last wave: merge the waves in order, then the partials and the slot word.  The lane
            // index is formed here (the W2 rows leave no register to keep one across the loop)
            __asm__ volatile("" ::: "memory");
            int ln;
            __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
            const bool has = ln < kResWaves;
            const int j = has ? ln : 0;
            float mk = has ? wkey[j] : -INFINITY;
            int mi = has ? wid[j] : 0x7FFFFFFF;
            float mm = has ? wmc[j] : kNegBig * c;
            float ms = has ? wsum[j] : 0.f;
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                const float ok = __shfl_xor(mk, off);
                const int oi = __shfl_xor(mi, off);
                const float om = __shfl_xor(mm, off);
                const float os = __shfl_xor(ms, off);
                if (beats(ok, oi, mk, mi)) {
                    mk = ok;
                    mi = oi;
                }
                lse_merge(mm, ms, om, os);
            }
            if (lane == 0) {
                const size_t o = ((size_t)k * G + g) * a.Bpad;
                agent_store(a.p_mc + o, mm);
                agent_store(a.p_s + o, ms);
                agent_store(a.p_idx + o, mi);
                agent_store(a.p_l + o, mk);
                const unsigned long long packed =
                    ((unsigned long long)ordered_key(mk) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)mi);
                agent_store(a.winners + (size_t)k * G + g, packed);
            }
        }
    }
}

// ====================================================================================================================
// The matrix-core resident round: at most 64 rows, r = 256, greedy picks, at most 16 vocabulary tiles per
// workgroup (V <= 512 G: 131,072 at 256 CUs), gated or not (the gated workload: B = 64, V = 129,280).
//
// The tiled round streams W2 at every position and stalls at each grid boundary once its ring and registers
// are full.  Here a workgroup's W2 tiles stay in registers for the whole round: eight waves, two per SIMD
// with 256 registers each, each hold the A operands of two 32-id tiles (16 x 8 bf16 per lane and tile, 128
// registers; rows placed by the same slot order as the tiled round, so a lane's accumulator holds 16
// consecutive ids).  Per position only the base logits stream, straight into the accumulators (C operand),
// requested one position ahead as soon as each accumulator's epilogue is done.  X (64 rows, bf16) and the
// next position's gate rows (fp32, loaded with direct global-to-LDS loads) live in LDS; the B operands are read
// from X.  The same v_mfma_f32_32x32x16_bf16 with the same operands as the tiled round, seeded with U, gives
// the same logits.  The end of a position merges the rows over the eight waves in wave order; wave 0 then
// makes the tiled round's pick atomics, partials and arrival, and wave 1 merges the previous position's row
// of this workgroup's (rows g < B) while wave 0 waits for the release.
constexpr int kRmWaves = 4;               // one per SIMD: 512 registers each
constexpr int kRmThreads = 64 * kRmWaves;
constexpr int kRmRows = 64;
constexpr int kRmTiles = 16;              // tiles per workgroup and round
constexpr int kRmTpw = kRmTiles / kRmWaves;  // tiles per wave
constexpr int kRmRpw = kRmRows / kRmWaves;   // X rows gathered per wave
constexpr int kRmXPitch = 2 * kResR + 16;  // bytes per X row in LDS (a 16-byte shift per row: no bank conflicts)
constexpr int kRmHPitch = 4 * kResR + 16;  // bytes per gate row in LDS
typedef __attribute__((address_space(3))) void lds_void_t;

// The tile row held in slot s (the inverse of w2_slot): slot 8a + 4b + c holds row 16b + 4a + c.
__device__ __forceinline__ int w2_row_of_slot(int s) { return 16 * ((s >> 2) & 1) + 4 * (s >> 3) + (s & 3); }

template <bool GATED, bool STORE>
__global__ void __launch_bounds__(kRmThreads, 1) markov_resident_mfma_kernel(RoundArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t xs[kRmRows * kRmXPitch];
    __shared__ __attribute__((aligned(16))) uint8_t hs[GATED ? kRmRows * kRmHPitch : 16];
    __shared__ float mkey[kRmWaves][kRmRows], mmc[kRmWaves][kRmRows], msum[kRmWaves][kRmRows];
    __shared__ int mid[kRmWaves][kRmRows];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5;
    const int rho = lane & 31;
    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int nrb = (a.B + 31) / 32;
    const int ntw = (a.ntiles - g + G - 1) / G;
    const float c = a.c;
    const uint32_t spin_limit = a.spin_limit;
    const uint64_t tag = launch_tag(a, agent_load(a.epoch));
    if (g == 0 && wave == 0) {
        // this launch's pick words and counters, then its tag (read by every workgroup before its first arrival)
        const size_t nw = (size_t)a.K * a.Bpad * kWinnerSlots;
        for (size_t i = lane; i < nw; i += 64) agent_store(a.winners + i * kWinnerStride, 0ull);
        if (lane < kBarrierGroups) {
            agent_store(a.barrier + kCounterStride * lane, 0u);
            agent_store(a.release + kCounterStride * lane, 0u);
        }
        if (lane == 0) {
            agent_store(a.top, 0u);
            agent_store(a.error, 0u);
        }
        wait_vmcnt<0>();
        if (lane == 0) agent_store(a.flag, tag);
    }

    // W2 tiles (slots wave, wave + kRmWaves, ... of this workgroup's tiles g, g + G, ...) as A operands
    bf16x8_t wa[kRmTpw][16];
#pragma unroll
    for (int tt = 0; tt < kRmTpw; ++tt) {
        const int j = wave + kRmWaves * tt;
        const int v = min(32 * (g + G * j) + w2_row_of_slot(rho), a.V - 1);
        const bf16x8_t* wp = reinterpret_cast<const bf16x8_t*>(a.W2t + (size_t)v * kResR + 8 * half);
#pragma unroll
        for (int q = 0; q < 16; ++q) wa[tt][q] = j < ntw ? wp[2 * q] : bf16x8_t{};
    }
    // base logits of (position k, tile slot j, row block rb) in the accumulator layout: row 32 rb + rho, ids
    // 32 t + 16 half .. + 15 (a tail tile's ids past the vocabulary read as 0 and are masked at the epilogue)
    auto load_u = [&](int k, int j, int rb, f32x16_t& dst) {
        const int b = min(32 * rb + rho, a.B - 1);
        const int col = 32 * (g + G * j) + 16 * half;
        const float* up = a.U + (size_t)k * a.u_kstride + (size_t)b * a.u_stride + col;
        f32x4_t q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = col + 4 * i < a.V ? *reinterpret_cast<const f32x4_t*>(up + 4 * i) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dst[4 * i] = q[i].x;
            dst[4 * i + 1] = q[i].y;
            dst[4 * i + 2] = q[i].z;
            dst[4 * i + 3] = q[i].w;
        }
    };
    // the gate rows of position k for this wave's rows, global -> LDS
    auto load_h = [&](int k) {
        if constexpr (GATED) {
#pragma unroll
            for (int i = 0; i < kRmRpw; ++i) {
                const int b = kRmRpw * wave + i;
                if (b < a.B)
                    __builtin_amdgcn_global_load_lds(
                        reinterpret_cast<const void*>(a.H + ((size_t)b * a.K + k) * kResR + 4 * lane),
                        (lds_void_t*)(hs + b * kRmHPitch), 16, 0, 0);
            }
        }
    };
    // X rows of position k (predecessors from the pick words of k - 1, or the anchors), this wave's rows: lane l
    // takes row kRmRpw wave + l / kLpr, kCpl consecutive 16-byte chunks
    constexpr int kLpr = 64 / kRmRpw;       // lanes per row
    constexpr int kCpl = 32 / kLpr;         // chunks per lane (32 chunks of 16 bytes per row)
    auto gather = [&](int k) {
        const int b = kRmRpw * wave + lane / kLpr;
        const bool vb = b < a.B;
        int pv = 0;
        if (vb) {
            if (k == 0) {
                pv = a.anchor[b];
            } else {
                const unsigned long long wv = pick_word(a, k - 1, b);
                pv = (int)(0xFFFFFFFFu - (uint32_t)(wv & 0xFFFFFFFFull));
            }
            pv = min(max(pv, 0), a.V - 1);
        }
        const u32x4_t* wrow = reinterpret_cast<const u32x4_t*>(a.W1 + (size_t)pv * kResR);
        u32x4_t raw[kCpl];
#pragma unroll
        for (int i = 0; i < kCpl; ++i) raw[i] = wrow[kCpl * (lane % kLpr) + i];
#pragma unroll
        for (int i = 0; i < kCpl; ++i) {
            const int ch = kCpl * (lane % kLpr) + i;
            u32x4_t o = raw[i];
            if constexpr (GATED) {
                const float* hl = reinterpret_cast<const float*>(hs + (vb ? b : 0) * kRmHPitch) + 8 * ch;
                const f32x4_t h0 = *reinterpret_cast<const f32x4_t*>(hl);
                const f32x4_t h1 = *reinterpret_cast<const f32x4_t*>(hl + 4);
                const float hf[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
                const uint32_t w32[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
                uint32_t o32[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = bf16_to_f32((uint16_t)(w32[e] & 0xFFFFu)) * hf[2 * e];
                    const float hi = bf16_to_f32((uint16_t)(w32[e] >> 16)) * hf[2 * e + 1];
                    o32[e] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
                }
                o = u32x4_t{o32[0], o32[1], o32[2], o32[3]};
            }
            if (!vb) o = u32x4_t{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4_t*>(xs + b * kRmXPitch + 16 * ch) = o;
        }
    };

    f32x16_t acc[kRmTpw][2];
#pragma unroll
    for (int tt = 0; tt < kRmTpw; ++tt)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
            if (wave + kRmWaves * tt < ntw && rb < nrb) load_u(0, wave + kRmWaves * tt, rb, acc[tt][rb]);
    load_h(0);
    wait_vmcnt<0>();
    __syncthreads();
    gather(0);
    __syncthreads();

    for (int k = 0; k < a.K; ++k) {
        // per row block: running max and sum of the log-sum-exp, best logit and its slot / tile
        float m[2] = {kNegBig, kNegBig}, s[2] = {0.f, 0.f}, bl[2] = {-INFINITY, -INFINITY};
        int bslot[2] = {0, 0}, btile[2] = {-1, -1};
#pragma unroll
        for (int tt = 0; tt < kRmTpw; ++tt) {
            const int j = wave + kRmWaves * tt;
            if (j >= ntw) continue;
            const int t = g + G * j;
            // both row blocks of the tile at once: two independent accumulation chains on the same A operands, so
            // each MFMA issues while the other chain's previous one completes (rows past the batch read zero X)
            {
                const uint8_t* x0 = xs + rho * kRmXPitch + 16 * half;
                const uint8_t* x1 = x0 + 32 * kRmXPitch;
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    acc[tt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[tt][q], *reinterpret_cast<const bf16x8_t*>(x0 + 32 * q), acc[tt][0], 0, 0, 0);
                    acc[tt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[tt][q], *reinterpret_cast<const bf16x8_t*>(x1 + 32 * q), acc[tt][1], 0, 0, 0);
                }
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                if (rb >= nrb) continue;
                f32x16_t& lv = acc[tt][rb];
                const int b = 32 * rb + rho;
                const int v0 = 32 * t + 16 * half;
                if constexpr (STORE) {
                    if (b < a.B) {
                        float* d = a.logits_out + ((size_t)b * a.K + k) * (size_t)a.V + v0;
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            if (v0 + i < a.V) d[i] = lv[i];
                    }
                }
                // greedy epilogue (ids past the vocabulary masked), as in the tiled round
                if (v0 + 16 > a.V) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (v0 + i >= a.V) lv[i] = -INFINITY;
                }
                float cm = lv[0];
#pragma unroll
                for (int i = 1; i < 16; ++i) cm = fmaxf(cm, lv[i]);
                const float mn = fmaxf(m[rb], cm);
                s[rb] *= fast_exp2((m[rb] - mn) * c);
                m[rb] = mn;
                const float mc = mn * c;
#pragma unroll
                for (int i = 0; i < 16; ++i) s[rb] += fast_exp2(fmaf(lv[i], c, -mc));
                if (cm > bl[rb]) {
                    int sl = 15;
#pragma unroll
                    for (int i = 14; i >= 0; --i) sl = (lv[i] == cm) ? i : sl;
                    bl[rb] = cm;
                    bslot[rb] = sl;
                    btile[rb] = t;
                }
                // the accumulator is free: the next position's base logits go into it now
                if (k + 1 < a.K) load_u(k + 1, j, rb, acc[tt][rb]);
            }
        }
        if (k + 1 < a.K) load_h(k + 1);  // every wave has read the gate rows of k (barrier after the gather)
        // this wave's per-row results: the two lanes of a row merged, then into LDS
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            if (rb >= nrb) continue;
            int bi = btile[rb] >= 0 ? 32 * btile[rb] + 16 * half + bslot[rb] : 0x7FFFFFFF;
            float key = bl[rb];
            float mc2 = m[rb] * c, s2 = s[rb];
            const float okey = __shfl_xor(key, 32);
            const int oi = __shfl_xor(bi, 32);
            const float omc = __shfl_xor(mc2, 32);
            const float os = __shfl_xor(s2, 32);
            if (beats(okey, oi, key, bi)) {
                key = okey;
                bi = oi;
            }
            lse_merge(mc2, s2, omc, os);
            if (half == 0) {
                mkey[wave][32 * rb + rho] = key;
                mid[wave][32 * rb + rho] = bi;
                mmc[wave][32 * rb + rho] = mc2;
                msum[wave][32 * rb + rho] = s2;
            }
        }
        __syncthreads();
        if (wave == 0) {
            // one lane per row: the eight waves' results in wave order, then the global pick and partials
            const int b = lane;
            if (b < a.B) {
                float key = mkey[0][b], mc2 = mmc[0][b], s2 = msum[0][b];
                int bi = mid[0][b];
#pragma unroll
                for (int w = 1; w < kRmWaves; ++w) {
                    const float ok = mkey[w][b];
                    const int oi = mid[w][b];
                    if (beats(ok, oi, key, bi)) {
                        key = ok;
                        bi = oi;
                    }
                    lse_merge(mc2, s2, mmc[w][b], msum[w][b]);
                }
                if (k == 0) wait_cleared(a, tag);
                const unsigned long long packed =
                    ((unsigned long long)ordered_key(key) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)bi);
                atomicMax(a.winners + (((size_t)k * a.Bpad + b) * kWinnerSlots + g % kWinnerSlots) * kWinnerStride, packed);
                const size_t o = ((size_t)k * G + g) * a.Bpad + b;
                agent_store(a.p_mc + o, mc2);
                agent_store(a.p_s + o, s2);
                agent_store(a.p_idx + o, bi);
                agent_store(a.p_l + o, key);
            }
            wait_vmcnt<0>();
            int last_all = 0;
            if (lane == 0) last_all = arrive(a, k) ? 1 : 0;
            if (__shfl(last_all, 0) && lane < kBarrierGroups)
                agent_store(a.release + kCounterStride * lane, (uint32_t)(k + 1));
            // the release of position k (the last one's is awaited after the loop)
            if (k + 1 < a.K) {
                uint32_t spins = 0;
                while (released_position(a) < (uint32_t)(k + 1)) {
                    __builtin_amdgcn_s_sleep(1);
                    if (++spins > spin_limit) {
                        __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
            }
        } else if (wave == 1 && k >= 1 && g < a.B) {
            finalize_pair(a, g, k - 1, false);  // released before this position began
        }
        if (k + 1 < a.K) {
            wait_vmcnt<0>();  // this wave's gate rows in LDS (and its base logits in registers)
            __syncthreads();
            gather(k + 1);
            __syncthreads();
        }
    }
    // after the last position: its release, then this workgroup's row of it
    bool timed_out = false;
    if (wave == 1 && g < a.B) {
        uint32_t spins = 0;
        while (released_position(a) < (uint32_t)a.K) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > spin_limit) {
                timed_out = true;
                break;
            }
        }
        if (timed_out && lane == 0) agent_store(a.error, 1u);
        finalize_pair(a, g, a.K - 1, timed_out);
    }
    // every workgroup has arrived after its last position, so all have read the epoch: advance it
    if (g == 0 && wave == 0) {
        uint32_t spins = 0;
        while (released_position(a) < (uint32_t)a.K) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > spin_limit) break;
        }
        if (lane == 0) agent_store(a.epoch, agent_load(a.epoch) + 1u);
    }
}

}  // namespace

hipError_t launch_confidence(const ConfArgs& c, int B, hipStream_t st) {
    hipLaunchKernelGGL(confidence_kernel, dim3(B), dim3(64), 0, st, c);
    return hipGetLastError();
}

int round_supported_r(int r) { return mfma_supported_r(r) && r <= 256; }


template <int RK, int MODE, bool GATED, int UR>
static const void* round_fn(bool store) {
    return store ? reinterpret_cast<const void*>(&markov_round_kernel<RK, MODE, GATED, UR, true>)
                 : reinterpret_cast<const void*>(&markov_round_kernel<RK, MODE, GATED, UR, false>);
}

template <int RK, int MODE, bool GATED>
static const void* round_fn(int form, bool store) {
    return form == kRowsSmall  ? round_fn<RK, MODE, GATED, 1>(store)
           : form == kRowsHalf ? round_fn<RK, MODE, GATED, 8>(store)
                               : round_fn<RK, MODE, GATED, 16>(store);
}

template <int RK>
static const void* round_fn(bool sample, bool gated, int form, bool store) {
    if (sample) return gated ? round_fn<RK, kModeSample, true>(form, store) : round_fn<RK, kModeSample, false>(form, store);
    return gated ? round_fn<RK, kModeGreedy, true>(form, store) : round_fn<RK, kModeGreedy, false>(form, store);
}

static const void* round_fn_r(int r, bool sample, bool gated, int form, bool store) {
    switch (r / 16) {
        case 1: return round_fn<1>(sample, gated, form, store);
        case 2: return round_fn<2>(sample, gated, form, store);
        case 4: return round_fn<4>(sample, gated, form, store);
        case 8: return round_fn<8>(sample, gated, form, store);
        case 16: return round_fn<16>(sample, gated, form, store);
        default: return nullptr;
    }
}

int round_max_coresident(int r, bool sample, bool gated, int form, bool store) {
    const void* fn = round_fn_r(r, sample, gated, form, store);
    int per_cu = 0;
    if (!fn || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kRoundThreads, 0) != hipSuccess) return 0;
    return per_cu * device_cu_count();
}

// The grid is one workgroup per CU (at most the device's co-resident count), so on a device that runs nothing
// else all workgroups are resident together and the grid barrier completes.  An ordinary launch is the default:
// on this part the runtime's cooperative launch, which guarantees co-residency, adds about 20 us per call
// (measured on the serving round, 0.452 against 0.474 ms).  A device shared with kernels that hold CUs for
// long can keep workgroups waiting; the kernel's bounded waits then give up, it exits normally and reports the
// failure in the error word (tokens -1).  `cooperative` selects the guaranteed launch instead.
hipError_t launch_markov_round(const RoundArgs& a, bool sample, bool gated, bool cooperative, hipStream_t st,
                               hipEvent_t ev_begin, hipEvent_t ev_end) {
    const void* fn = round_fn_r(a.r, sample, gated, round_row_form(a.B), a.logits_out != nullptr);
    if (!fn) return hipErrorInvalidValue;
    if (ev_begin) (void)hipEventRecord(ev_begin, st);
    RoundArgs copy = a;
    void* args[] = {&copy};
    const hipError_t e = cooperative ? hipLaunchCooperativeKernel(fn, dim3(a.G), dim3(kRoundThreads), args, 0, st)
                                     : hipLaunchKernel(fn, dim3(a.G), dim3(kRoundThreads), args, 0, st);
    if (ev_end) (void)hipEventRecord(ev_end, st);
    return e;
}

static const void* resident_fn(bool gated, bool store) {
    return gated ? (store ? reinterpret_cast<const void*>(&markov_resident_kernel<true, true>)
                          : reinterpret_cast<const void*>(&markov_resident_kernel<true, false>))
                 : (store ? reinterpret_cast<const void*>(&markov_resident_kernel<false, true>)
                          : reinterpret_cast<const void*>(&markov_resident_kernel<false, false>));
}

int resident_max_coresident(bool gated, bool store) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, resident_fn(gated, store), kResThreads, 0) != hipSuccess) return 0;
    return per_cu * device_cu_count();
}

// The slot words of K + 1 positions live in the winner array ([K][Bpad][kWinnerSlots] words, kWinnerStride apart).
bool resident_supported(int B, int K, int r, bool sample, int V, int G, int Bpad) {
    return B == 1 && r == kResR && !sample && G >= 1 && (int64_t)V <= (int64_t)kResWaves * 64 * G &&
           (int64_t)(K + 1) * G <= (int64_t)K * Bpad * kWinnerSlots * kWinnerStride;
}

static const void* resident_mfma_fn(bool gated, bool store) {
    return gated ? (store ? reinterpret_cast<const void*>(&markov_resident_mfma_kernel<true, true>)
                          : reinterpret_cast<const void*>(&markov_resident_mfma_kernel<true, false>))
                 : (store ? reinterpret_cast<const void*>(&markov_resident_mfma_kernel<false, true>)
                          : reinterpret_cast<const void*>(&markov_resident_mfma_kernel<false, false>));
}

int resident_mfma_max_coresident(bool gated, bool store) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, resident_mfma_fn(gated, store), kRmThreads, 0) != hipSuccess)
        return 0;
    return per_cu * device_cu_count();
}

bool resident_mfma_supported(int B, int r, bool sample, int V, int G) {
    const int64_t ntiles = ((int64_t)V + 31) / 32;
    return B >= 1 && B <= kRmRows && r == kResR && !sample && G >= 1 && (ntiles + G - 1) / G <= kRmTiles;
}

hipError_t launch_markov_resident_mfma(const RoundArgs& a, bool gated, bool cooperative, hipStream_t st,
                                       hipEvent_t ev_begin, hipEvent_t ev_end) {
    if (!resident_mfma_supported(a.B, a.r, false, a.V, a.G) || a.cf.h) return hipErrorInvalidValue;
    const void* fn = resident_mfma_fn(gated, a.logits_out != nullptr);
    if (ev_begin) (void)hipEventRecord(ev_begin, st);
    RoundArgs copy = a;
    void* args[] = {&copy};
    const hipError_t e = cooperative ? hipLaunchCooperativeKernel(fn, dim3(a.G), dim3(kRmThreads), args, 0, st)
                                     : hipLaunchKernel(fn, dim3(a.G), dim3(kRmThreads), args, 0, st);
    if (ev_end) (void)hipEventRecord(ev_end, st);
    return e;
}

// Launched like the tiled round (one workgroup per CU, ordinary launch unless `cooperative`).
hipError_t launch_markov_resident(const RoundArgs& a, bool gated, bool cooperative, hipStream_t st, hipEvent_t ev_begin,
                                  hipEvent_t ev_end) {
    if (!resident_supported(a.B, a.K, a.r, false, a.V, a.G, a.Bpad)) return hipErrorInvalidValue;
    const void* fn = resident_fn(gated, a.logits_out != nullptr);
    if (ev_begin) (void)hipEventRecord(ev_begin, st);
    RoundArgs copy = a;
    void* args[] = {&copy};
    const hipError_t e = cooperative ? hipLaunchCooperativeKernel(fn, dim3(a.G), dim3(kResThreads), args, 0, st)
                                     : hipLaunchKernel(fn, dim3(a.G), dim3(kResThreads), args, 0, st);
    if (ev_end) (void)hipEventRecord(ev_end, st);
    return e;
}

}  // namespace dspark

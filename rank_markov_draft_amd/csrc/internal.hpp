// internal.hpp -- kernel argument blocks and launchers shared between the libdspark translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dspark {

constexpr int kModeGreedy = 0;
constexpr int kModeSample = 1;
constexpr int kModeStore = 2;  // validation: write the calibrated logits instead of picking

// One position of the Markov head, matrix-core kernel (bf16, W2 stored [V, r]).
struct StepArgs {
    const float* U;         // row b at U + b * u_stride
    int64_t u_stride;
    const uint16_t* W1;     // [V, r] bf16 bits
    const uint16_t* W2t;    // [V, r] bf16 bits
    const int32_t* prev;    // predecessor of row b at prev[b * prev_stride]
    int64_t prev_stride;
    const float* H;         // gate row b at H + b * h_stride (gated kernels only)
    int64_t h_stride;
    int B, V, r, k;         // k: position (noise counter)
    uint32_t k0;            // noise key of the seed
    float c;                // log2(e) / T  (T = 1 in greedy mode)
    int ntiles;             // ceil(V / 32)
    Partials part;          // [G][Bpad]
    int Bpad;
    float* logits_out;      // store mode: [B, V]
};

// Same for the vector-ALU kernel; W2 element (j, v) at W2[j * sj + v * sv].
struct StepArgsValu {
    const float* U;
    int64_t u_stride;
    const void* W1;
    const void* W2;
    int64_t sj, sv;
    const int32_t* prev;
    int64_t prev_stride;
    const float* H;
    int64_t h_stride;
    int B, V, r, k;
    uint32_t k0;
    float c;
    Partials part;
    int Bpad;
    float* logits_out;
};

// The whole draft round for small problems on the vector-ALU path (one launch, one workgroup per kValuRows rows
// covering the whole vocabulary at every position).
struct RoundValuArgs {
    const float* U;         // [B, K, V]
    const void* W1;         // [V, r]
    const void* W2;         // [r, V] (sj = V, sv = 1) or [V, r] (sj = 1, sv = r)
    int64_t sj, sv;
    const int32_t* anchor;  // [B]
    const float* H;         // [B, K, r] or null
    int B, K, V, r;
    uint32_t k0;
    float c;                // log2(e) / T
    float inv_t;            // 1 / T (1 in greedy mode)
    int32_t* tokens;        // [B, K]
    float* logprobs;        // [B, K] or null
    uint32_t* error;        // the workspace's error word (cleared: this path has no bounded waits)
};
// Largest V * r the one-launch vector-ALU round takes (each workgroup reads the whole W2 every position).
constexpr size_t kValuRoundMaxVR = 65536;
hipError_t launch_markov_round_valu(const RoundValuArgs& a, bool bf16, bool sample, bool gated, hipStream_t st);

struct ReduceArgs {
    Partials part;
    int G, Bpad;
    float inv_t;            // 1 / T in sampling mode, 1 in greedy mode
    int32_t* tokens;        // row b at tokens[b * out_stride]
    float* logprobs;        // same indexing, or null
    float* best_logit;      // same indexing, or null
    int64_t out_stride;
};

// Confidence head c_k = sigmoid(w_h . h_k + w_m . W1[x_{k-1}]) and prefix survival a_k = prod_{i<=k} c_i.
struct ConfArgs {
    const uint16_t* h;          // [B, K, D] bf16, 16-byte aligned, D % 8 == 0; null: no confidence head
    int D;
    const float* w;             // [D + r]: the h part, then the W1 part
    const void* W1;             // [V, r]
    bool w1_bf16;
    int r, K;
    const int32_t* anchor;      // [B]
    const int32_t* tokens;      // [B, K] drafted tokens (x_{-1} = anchor)
    float* conf;                // [B, K]
    float* survival;            // [B, K]
};
hipError_t launch_confidence(const ConfArgs& c, int B, hipStream_t st);

// A whole draft round in one persistent cooperative launch (bf16, W2 stored [V, r], V % 4 == 0).
struct RoundArgs {
    const float* U;             // U[b, k, v] at U + k * u_kstride + b * u_stride + v
    int64_t u_stride, u_kstride;
    const uint16_t* W1;         // [V, r]
    const uint16_t* W2t;        // [V, r]
    const int32_t* anchor;      // [B]
    const float* H;             // [B, K, r] or null
    int B, K, V, r;
    uint32_t k0;
    float c;                    // log2(e) / T
    int ntiles, G, Bpad;
    unsigned long long* winners;  // [K][Bpad][kWinnerSlots] packed (ordered key, ~id), kWinnerStride words apart
    uint32_t* barrier;          // grid barrier: kBarrierGroups group arrival counters, one cache line each
    uint32_t* top;              // arrivals of whole groups
    uint32_t* release;          // kBarrierGroups copies of the last released position, one cache line each
    uint32_t* error;            // set if a barrier wait timed out
    uint32_t spin_limit;
    uint64_t* flag;             // set by workgroup 0 once it has cleared winners, counters and error
    uint32_t* epoch;            // launches of the workspace so far; advanced at the end of every launch
    uint64_t seq;               // per-call sequence number (never 0); with the epoch it names the launch
    int32_t* tokens;            // [B, K] outputs, written by the kernel's finalizer waves
    ConfArgs cf;                // optional confidence head, also computed by the finalizers
    float* logprobs;            // [B, K] or null
    float inv_t;
    float* p_mc;                // [K][G][Bpad] log-sum-exp partials (base-2 max of l c, sum)
    float* p_s;
    int* p_idx;                 // [K][G][Bpad] best id and its logit per workgroup
    float* p_l;
    float* logits_out;          // validation: [B, K, V] calibrated logits along the drafted path, or null
};
// Each (position, row) pick has kWinnerSlots words (workgroup g updates slot g % kWinnerSlots), each on a
// 128-byte line of its own: every workgroup updates every row once per position, and atomics on one line are
// serialised where they are performed.  A reader takes the largest slot.  More slots shorten the atomics
// of an idle machine (microbenchmark: 1.8 us with one, 1.1 us with two) but under the stream the extra reads
// at the start of the next position cost more (serving round: 2 slots +1%, 4 slots +3% over one).
constexpr int kWinnerStride = 16;
constexpr int kWinnerSlots = 1;
// Grid barrier: workgroup g arrives on group counter g % kBarrierGroups; the last arrival of a group counts
// on the top counter, and the last arrival there writes every copy of the release word, which each workgroup
// polls on a line shared with few others.
constexpr int kBarrierGroups = 8;
constexpr int kCounterStride = 32;  // words between counters (128 bytes)
int round_supported_r(int r);
// Row forms of the round kernel: a batch of at most 8 rows takes the small-block form (one U unit per item,
// deeper stream), 9 .. 64 rows the half-block form (eight U units per item, two sets of consumer waves), more
// rows the full 128-row blocks.
constexpr int kRowsFull = 0, kRowsHalf = 1, kRowsSmall = 2;
inline int round_row_form(int B) { return B <= 8 ? kRowsSmall : B <= 64 ? kRowsHalf : kRowsFull; }
int round_max_coresident(int r, bool sample, bool gated, int form, bool store = false);
hipError_t launch_markov_round(const RoundArgs& a, bool sample, bool gated, bool cooperative, hipStream_t st,
                               hipEvent_t ev_begin, hipEvent_t ev_end);
// The resident round: a single row, r = 256, greedy; each lane keeps one vocabulary row of W2 in registers for the
// whole round (workgroup g covers ids [g V / G, (g + 1) V / G), at most 640).  Same arguments and workspace as the
// tiled round; its per-workgroup pick words of positions 0 .. K use the winner array.
int resident_max_coresident(bool gated, bool store);
bool resident_supported(int B, int K, int r, bool sample, int V, int G, int Bpad);
hipError_t launch_markov_resident(const RoundArgs& a, bool gated, bool cooperative, hipStream_t st, hipEvent_t ev_begin,
                                  hipEvent_t ev_end);
// The matrix-core resident round: at most 64 rows, r = 256, greedy, at most 16 vocabulary tiles per workgroup;
// each workgroup keeps its W2 tiles in registers as matrix-core operands for the whole round.  Same arguments and
// workspace as the tiled round; no confidence head.
int resident_mfma_max_coresident(bool gated, bool store);
bool resident_mfma_supported(int B, int r, bool sample, int V, int G);
hipError_t launch_markov_resident_mfma(const RoundArgs& a, bool gated, bool cooperative, hipStream_t st,
                                       hipEvent_t ev_begin, hipEvent_t ev_end);

int mfma_supported_r(int r);
hipError_t launch_markov_step_mfma(const StepArgs& a, int mode, bool gated, bool vec_u, int G, hipStream_t st);
hipError_t launch_markov_step_valu(const StepArgsValu& a, bool bf16, int mode, bool gated, int G, hipStream_t st);
hipError_t launch_markov_reduce(const ReduceArgs& a, int B, hipStream_t st);

hipError_t launch_transpose(const void* src, int rows, int cols, int elem_bytes, void* dst, hipStream_t st);
hipError_t launch_fill_u32(uint32_t* p, uint32_t value, size_t n, hipStream_t st);
hipError_t launch_stream_read(const void* a, size_t a_bytes, const void* b, size_t b_bytes, uint32_t* sink, hipStream_t st);

// gate: H = sigmoid(h Wg)
// Workspace bytes of the split-K gate for these sizes (0: the single-kernel form serves them).
size_t gate_splitk_bytes(int rows, int D, int r);
// The split-K form when a large enough 16-byte aligned workspace is given (and H is 16-byte aligned), else the
// single kernel.
hipError_t launch_gate(const uint16_t* h, const uint16_t* Wg, int rows, int D, int r, float* H, void* workspace,
                       size_t workspace_bytes, hipStream_t st);

// selector
size_t topk_workspace_bytes(int rows, int V, int topk);
int topk_supported(int V, int topk);
hipError_t launch_topk(const float* U, int64_t u_stride, int rows, int V, int topk, int32_t* idx, float* val,
                       void* ws, hipStream_t st);
struct SelectorArgs {
    const float* U;         // [B, K, V]
    const void* A;          // [V, r]
    const void* Bemb;       // [V, r]
    bool bf16;
    const int32_t* anchor;
    const float* H;         // [B, K, r] or null
    int B, K, V, r, topk;
    bool sample;
    uint32_t k0;
    float inv_t;            // 1/T (sample) or 1
    const int32_t* cand;    // [B, K, topk]
    float* scores;          // [B, topk + (K-1) topk^2]
    int32_t* tokens;
    float* logprobs;
};
hipError_t launch_pair_scores(const SelectorArgs& a, hipStream_t st);
hipError_t launch_walk(const SelectorArgs& a, hipStream_t st);

int device_cu_count();

int schedule_supported(int R, int K);
hipError_t launch_schedule(const float* a, const float* sps, int R, int K, int32_t* lengths, float* theta, hipStream_t st);

}  // namespace dspark

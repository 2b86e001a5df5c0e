// api.hip -- the extern "C" boundary of libdspark: argument checks, workspace carving, dispatch.
#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/dspark.h"
#include "internal.hpp"

namespace dspark {
namespace {

thread_local char g_err[256] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int device_fail(hipError_t e, const char* what) {
    return fail(DSPARK_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxG = 1024;          // upper bound on workgroups along the vocabulary
constexpr uint32_t kDefaultSpinLimit = 1u << 22;  // sleeps before a bounded wait of the round kernel gives up
std::atomic<uint32_t> g_spin_limit{kDefaultSpinLimit};
std::atomic<int> g_cooperative{0};  // whole-round kernel: ordinary launch (0) or cooperative launch (1)
constexpr int kRowPad = 128;         // partials are padded to whole 128-row blocks
constexpr int kMfmaWGPerCU = 2;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
int round_up(int x, int m) { return (x + m - 1) / m * m; }

struct MarkovWs {
    Partials part;  // per-step path: [kMaxG][Bpad]
    int Bpad;
    unsigned long long* winners;  // whole-round path
    uint32_t* counters;
    float* p_mc;
    float* p_s;
    int* p_idx;
    float* p_l;
    void* w2t;  // transposed W2 (only when an [r, V] bf16 W2 is drafted on the matrix-core path)
};

bool mfma_eligible(int wdtype, int r) { return wdtype == DSPARK_BF16 && mfma_supported_r(r); }

size_t step_part_bytes(int B) { return 5 * align256(sizeof(float) * kMaxG * (size_t)round_up(B, kRowPad)); }

int round_gmax() {
    const int n = device_cu_count();
    return n < kMaxG ? n : kMaxG;
}

// grid-barrier group counters (8 cache lines), the error word, the init flag, the epoch, the top counter and
// the 8 release words
constexpr size_t kCounterBytes = 4096;
constexpr int kErrorWord = 256, kFlagWord = 288, kEpochWord = 320, kTopWord = 352, kReleaseWord = 512;
static_assert(kCounterStride * kBarrierGroups <= kErrorWord, "group counters overlap the error word");
static_assert((kReleaseWord + kCounterStride * kBarrierGroups) * 4 <= (int)kCounterBytes, "release words overflow");

// Sequence numbers of whole-round launches: the kernel clears its own counters and marks the clearing with a
// value made from the call's number and the workspace's launch epoch (advanced by every launch, so replays of
// a captured graph, whose arguments are fixed, differ too); a stale flag never matches.  The start is drawn
// from the clock so that two processes sharing memory are unlikely to collide.
uint64_t next_call_seq() {
    static std::atomic<uint64_t> seq{(uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() * 0x9E3779B97F4A7C15ull};
    uint64_t s;
    do s = seq.fetch_add(1, std::memory_order_relaxed) + 1; while (s == 0);
    return s;
}

// winners [K][Bpad][kWinnerSlots] u64 (kWinnerStride words apart), the counters, four [K][Gmax][Bpad] partial arrays
size_t round_region_bytes(int B, int K) {
    const size_t Bpad = (size_t)round_up(B, kRowPad);
    return align256(sizeof(unsigned long long) * (size_t)K * Bpad * kWinnerSlots * kWinnerStride) + kCounterBytes +
           4 * align256(sizeof(float) * (size_t)K * round_gmax() * Bpad);
}

size_t markov_ws_bytes(int B, int K, int V, int r, int wdtype, int w2_layout, bool need_pack) {
    size_t bytes = step_part_bytes(B) + round_region_bytes(B, K);
    if (need_pack && w2_layout == DSPARK_W2_RV && mfma_eligible(wdtype, r)) bytes += align256((size_t)V * r * 2);
    return bytes;
}

MarkovWs carve_markov(void* ws, int B, int K) {
    MarkovWs w{};
    w.Bpad = round_up(B, kRowPad);
    uint8_t* p = (uint8_t*)ws;
    const size_t one = align256(sizeof(float) * kMaxG * (size_t)w.Bpad);
    w.part.key = (float*)p;
    w.part.idx = (int*)(p + one);
    w.part.l = (float*)(p + 2 * one);
    w.part.m = (float*)(p + 3 * one);
    w.part.s = (float*)(p + 4 * one);
    uint8_t* q = p + 5 * one;
    const size_t wn = align256(sizeof(unsigned long long) * (size_t)K * w.Bpad * kWinnerSlots * kWinnerStride);
    w.winners = (unsigned long long*)q;
    w.counters = (uint32_t*)(q + wn);
    const size_t pn = align256(sizeof(float) * (size_t)K * round_gmax() * w.Bpad);
    uint8_t* pp = q + wn + kCounterBytes;
    w.p_mc = (float*)pp;
    w.p_s = (float*)(pp + pn);
    w.p_idx = (int*)(pp + 2 * pn);
    w.p_l = (float*)(pp + 3 * pn);
    w.w2t = pp + 4 * pn;
    return w;
}

int check_common(const void* W1, const void* W2, int wdtype, int w2_layout, int B, int V, int r, int mode,
                 float temperature) {
    if (!W1 || !W2) return fail(DSPARK_EINVAL, "W1 and W2 must not be NULL");
    if (B <= 0 || V <= 0 || r <= 0) return fail(DSPARK_EINVAL, "B, V and r must be positive (B=%d V=%d r=%d)", B, V, r);
    if (wdtype != DSPARK_F32 && wdtype != DSPARK_BF16) return fail(DSPARK_EINVAL, "unknown weight dtype %d", wdtype);
    if (w2_layout != DSPARK_W2_RV && w2_layout != DSPARK_W2_VR) return fail(DSPARK_EINVAL, "unknown W2 layout %d", w2_layout);
    if (mode != DSPARK_GREEDY && mode != DSPARK_SAMPLE) return fail(DSPARK_EINVAL, "unknown mode %d", mode);
    if (mode == DSPARK_SAMPLE && !(temperature > 0.f)) return fail(DSPARK_EINVAL, "temperature must be > 0 when sampling");
    if (r > 1024) return fail(DSPARK_EUNSUPPORTED, "r = %d exceeds 1024", r);
    if (B > 65535 * 4) return fail(DSPARK_EUNSUPPORTED, "B = %d too large", B);
    return DSPARK_OK;
}

// One position: contraction + calibration + pick (or logits store), then the cross-workgroup reduction.
int run_step(const float* Uk, int64_t u_stride, const void* W1, const void* W2, int wdtype, int w2_layout,
             const int32_t* prev, int64_t prev_stride, const float* Hk, int64_t h_stride, int B, int V, int r, int k,
             int mode, uint32_t k0, float temperature, int32_t* tok, float* lp, float* bestl, int64_t out_stride,
             const MarkovWs* ws, float* logits_out, hipStream_t st, hipEvent_t ev_begin = nullptr,
             hipEvent_t ev_end = nullptr) {
    const bool store = logits_out != nullptr;
    const int kmode = store ? kModeStore : (mode == DSPARK_SAMPLE ? kModeSample : kModeGreedy);
    const float teff = (mode == DSPARK_SAMPLE) ? temperature : 1.0f;
    const float c = kLog2e / teff;
    const bool gated = Hk != nullptr;
    const int ncu = device_cu_count();
    const bool use_mfma = mfma_eligible(wdtype, r) && w2_layout == DSPARK_W2_VR && aligned16(W1) && aligned16(W2) &&
                          (!gated || (aligned16(Hk) && h_stride % 4 == 0));
    Partials part{};
    int Bpad = 0;
    if (!store) {
        part = ws->part;
        Bpad = ws->Bpad;
    }
    int G = 0;
    hipError_t e;
    if (use_mfma) {
        StepArgs a{};
        a.U = Uk;
        a.u_stride = u_stride;
        a.W1 = (const uint16_t*)W1;
        a.W2t = (const uint16_t*)W2;
        a.prev = prev;
        a.prev_stride = prev_stride;
        a.H = Hk;
        a.h_stride = h_stride;
        a.B = B;
        a.V = V;
        a.r = r;
        a.k = k;
        a.k0 = k0;
        a.c = c;
        a.ntiles = (V + 31) / 32;
        a.part = part;
        a.Bpad = Bpad;
        a.logits_out = logits_out;
        G = a.ntiles < ncu * kMfmaWGPerCU ? a.ntiles : ncu * kMfmaWGPerCU;
        if (G > kMaxG) G = kMaxG;
        const bool vec_u = (V % 4 == 0) && (u_stride % 4 == 0) && aligned16(Uk);
        if (ev_begin) (void)hipEventRecord(ev_begin, st);
        e = launch_markov_step_mfma(a, kmode, gated, vec_u, G, st);
        if (ev_end) (void)hipEventRecord(ev_end, st);
    } else {
        StepArgsValu a{};
        a.U = Uk;
        a.u_stride = u_stride;
        a.W1 = W1;
        a.W2 = W2;
        a.sj = (w2_layout == DSPARK_W2_RV) ? V : 1;
        a.sv = (w2_layout == DSPARK_W2_RV) ? 1 : r;
        a.prev = prev;
        a.prev_stride = prev_stride;
        a.H = Hk;
        a.h_stride = h_stride;
        a.B = B;
        a.V = V;
        a.r = r;
        a.k = k;
        a.k0 = k0;
        a.c = c;
        a.part = part;
        a.Bpad = Bpad;
        a.logits_out = logits_out;
        const int nblk = (V + 255) / 256;
        G = nblk < ncu * 4 ? nblk : ncu * 4;
        if (G > kMaxG) G = kMaxG;
        if (ev_begin) (void)hipEventRecord(ev_begin, st);
        e = launch_markov_step_valu(a, wdtype == DSPARK_BF16, kmode, gated, G, st);
        if (ev_end) (void)hipEventRecord(ev_end, st);
    }
    if (e != hipSuccess) return device_fail(e, "markov step launch");
    if (store) return DSPARK_OK;
    ReduceArgs ra{};
    ra.part = part;
    ra.G = G;
    ra.Bpad = Bpad;
    ra.inv_t = 1.0f / teff;
    ra.tokens = tok;
    ra.logprobs = lp;
    ra.best_logit = bestl;
    ra.out_stride = out_stride;
    e = launch_markov_reduce(ra, B, st);
    if (e != hipSuccess) return device_fail(e, "markov reduce launch");
    return DSPARK_OK;
}

bool coop_supported() {
    static int cached[64] = {0};  // 0 unknown, 1 yes, 2 no
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    if (cached[dev] == 0) {
        int v = 0;
        cached[dev] = (hipDeviceGetAttribute(&v, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess && v) ? 1 : 2;
    }
    return cached[dev] == 1;
}

int markov_draft_impl(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout, const int32_t* anchor,
                      const float* H, int B, int K, int V, int r, int mode, uint64_t seed, float temperature,
                      int32_t* tokens, float* logprobs, void* workspace, size_t workspace_bytes, void* stream,
                      hipEvent_t* ev, int* kernel_launches, const ConfArgs* cf = nullptr,
                      float* logits_out = nullptr) {
    g_err[0] = 0;
    int rc = check_common(W1, W2, wdtype, w2_layout, B, V, r, mode, temperature);
    if (rc) return rc;
    if (!U || !anchor || !tokens) return fail(DSPARK_EINVAL, "U, anchor and tokens must not be NULL");
    if (K <= 0) return fail(DSPARK_EINVAL, "K must be positive");
    if (B > 65535) return fail(DSPARK_EUNSUPPORTED, "B = %d too large for a draft", B);
    const size_t need = markov_ws_bytes(B, K, V, r, wdtype, w2_layout, true);
    if (!workspace || workspace_bytes < need)
        return fail(DSPARK_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    hipStream_t st = (hipStream_t)stream;
    MarkovWs ws = carve_markov(workspace, B, K);
    const void* W2use = W2;
    int layout = w2_layout;
    if (w2_layout == DSPARK_W2_RV && mfma_eligible(wdtype, r)) {
        hipError_t e = launch_transpose(W2, r, V, 2, ws.w2t, st);
        if (e != hipSuccess) return device_fail(e, "transpose launch");
        W2use = ws.w2t;
        layout = DSPARK_W2_VR;
    }
    const uint32_t k0 = noise_key0(seed);
    const bool sample = mode == DSPARK_SAMPLE;
    const float teff = sample ? temperature : 1.0f;

    // whole round in one persistent launch when the shape allows it
    const bool round_ok = mfma_eligible(wdtype, r) && round_supported_r(r) && layout == DSPARK_W2_VR && aligned16(W1) && aligned16(W2use) &&
                          aligned16(U) && V % 4 == 0 && (!H || aligned16(H)) &&
                          (!g_cooperative.load(std::memory_order_relaxed) || coop_supported());
    if (round_ok) {
        const int ntiles = (V + 31) / 32;
        // a single row at r = 256 (greedy) keeps W2 resident on chip instead of streaming it at every position
        int Gres = 0;
        if (B == 1 && r == 256 && !sample) {
            Gres = resident_max_coresident(H != nullptr, logits_out != nullptr);
            if (Gres > round_gmax()) Gres = round_gmax();
        }
        const bool resident = resident_supported(B, K, r, sample, V, Gres, ws.Bpad);
        // up to 64 rows at r = 256 (greedy) whose W2 tiles fit the workgroups' registers keep them there
        int Grm = 0;
        if (!resident && B <= 64 && r == 256 && !sample && !cf) {
            Grm = resident_mfma_max_coresident(H != nullptr, logits_out != nullptr);
            if (Grm > round_gmax()) Grm = round_gmax();
        }
        const bool resident_mfma = !resident && !cf && resident_mfma_supported(B, r, sample, V, Grm);
        int G = resident ? Gres
                : resident_mfma ? Grm
                                : round_max_coresident(r, sample, H != nullptr, round_row_form(B), logits_out != nullptr);
        if (!resident && !resident_mfma) {
            if (G > round_gmax()) G = round_gmax();
            if (G > ntiles) G = ntiles;
        }
        if (G >= 1) {
            RoundArgs a{};
            a.U = U;
            a.u_stride = (int64_t)K * V;
            a.u_kstride = V;
            a.W1 = (const uint16_t*)W1;
            a.W2t = (const uint16_t*)W2use;
            a.anchor = anchor;
            a.H = H;
            a.B = B;
            a.K = K;
            a.V = V;
            a.r = r;
            a.k0 = k0;
            a.c = kLog2e / teff;
            a.ntiles = ntiles;
            a.G = G;
            a.Bpad = ws.Bpad;
            a.winners = ws.winners;
            a.barrier = ws.counters;
            a.error = ws.counters + kErrorWord;
            a.flag = reinterpret_cast<uint64_t*>(ws.counters + kFlagWord);
            a.epoch = ws.counters + kEpochWord;
            a.top = ws.counters + kTopWord;
            a.release = ws.counters + kReleaseWord;
            a.seq = next_call_seq();
            a.tokens = tokens;
            a.logprobs = logprobs;
            a.inv_t = 1.0f / teff;
            if (cf) a.cf = *cf;
            a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
            a.p_mc = ws.p_mc;
            a.p_s = ws.p_s;
            a.p_idx = ws.p_idx;
            a.p_l = ws.p_l;
            a.logits_out = logits_out;
            const bool coop = g_cooperative.load(std::memory_order_relaxed) != 0;
            hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
            hipError_t e = resident        ? launch_markov_resident(a, H != nullptr, coop, st, e0, e1)
                           : resident_mfma ? launch_markov_resident_mfma(a, H != nullptr, coop, st, e0, e1)
                                           : launch_markov_round(a, sample, H != nullptr, coop, st, e0, e1);
            if (e != hipSuccess) return device_fail(e, "draft round launch");
            if (kernel_launches) *kernel_launches = 1;
            return DSPARK_OK;
        }
    }
    if (logits_out) return fail(DSPARK_EUNSUPPORTED, "this shape does not take the whole-round kernel");
    if ((size_t)V * r <= kValuRoundMaxVR) {
        // a small problem: the whole round in one launch on the vector ALUs (it also clears the error word)
        RoundValuArgs a{};
        a.U = U;
        a.W1 = W1;
        a.W2 = W2use;
        a.sj = (layout == DSPARK_W2_RV) ? V : 1;
        a.sv = (layout == DSPARK_W2_RV) ? 1 : r;
        a.anchor = anchor;
        a.H = H;
        a.B = B;
        a.K = K;
        a.V = V;
        a.r = r;
        a.k0 = k0;
        a.c = kLog2e / teff;
        a.inv_t = 1.0f / teff;
        a.tokens = tokens;
        a.logprobs = logprobs;
        a.error = ws.counters + kErrorWord;
        if (ev) (void)hipEventRecord(ev[0], st);
        hipError_t e = launch_markov_round_valu(a, wdtype == DSPARK_BF16, sample, H != nullptr, st);
        if (ev) (void)hipEventRecord(ev[1], st);
        if (e != hipSuccess) return device_fail(e, "draft round launch");
        if (kernel_launches) *kernel_launches = 1;
        if (cf) {
            e = launch_confidence(*cf, B, st);
            if (e != hipSuccess) return device_fail(e, "confidence launch");
        }
        return DSPARK_OK;
    }
    {
        // this path has no bounded waits: clear the error word so dspark_markov_status reports this call
        hipError_t e = launch_fill_u32(ws.counters + kErrorWord, 0u, 1, st);
        if (e != hipSuccess) return device_fail(e, "error word clear");
    }
    // one launch pair (contraction, reduction) per position
    for (int k = 0; k < K; ++k) {
        const int32_t* prev = (k == 0) ? anchor : tokens + (k - 1);
        const int64_t pstride = (k == 0) ? 1 : K;
        rc = run_step(U + (size_t)k * V, (int64_t)K * V, W1, W2use, wdtype, layout, prev, pstride,
                      H ? H + (size_t)k * r : nullptr, (int64_t)K * r, B, V, r, k, mode, k0, temperature, tokens + k,
                      logprobs ? logprobs + k : nullptr, nullptr, K, &ws, nullptr, st, ev ? ev[2 * k] : nullptr,
                      ev ? ev[2 * k + 1] : nullptr);
        if (rc) return rc;
    }
    if (kernel_launches) *kernel_launches = K;
    if (cf) {
        hipError_t e = launch_confidence(*cf, B, st);
        if (e != hipSuccess) return device_fail(e, "confidence launch");
    }
    return DSPARK_OK;
}

// Scratch of the entry point that allocates nothing (dspark_markov_draft_noalloc): one array per device, held
// until the process ends.  Host code never passes the array's name to a kernel (on the host it is a stand-in,
// not a device address); it resolves the device address once per device with hipGetSymbolAddress and uses
// that pointer.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of this device's scratch array (resolved once per device, with that device current), or
// null with the reason in g_err.
void* scratch_ptr() {
    static std::mutex mu;
    static void* ptrs[64] = {nullptr};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        fail(DSPARK_EDEVICE, "no current device");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            device_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
            return nullptr;
        }
        ptrs[dev] = p;
    }
    return ptrs[dev];
}

}  // namespace
}  // namespace dspark

using namespace dspark;

extern "C" {

int dspark_abi_version(void) { return DSPARK_ABI_VERSION; }

const char* dspark_status_str(int status) {
    switch (status) {
        case DSPARK_OK: return "DSPARK_OK";
        case DSPARK_EINVAL: return "DSPARK_EINVAL";
        case DSPARK_EUNSUPPORTED: return "DSPARK_EUNSUPPORTED";
        case DSPARK_EWORKSPACE: return "DSPARK_EWORKSPACE";
        case DSPARK_EDEVICE: return "DSPARK_EDEVICE";
        default: return "DSPARK_UNKNOWN_STATUS";
    }
}

const char* dspark_last_error(void) { return g_err; }

size_t dspark_markov_workspace_bytes(int B, int K, int V, int r, int wdtype, int w2_layout) {
    if (B <= 0 || K <= 0 || V <= 0 || r <= 0) return 0;
    return markov_ws_bytes(B, K, V, r, wdtype, w2_layout, true);
}

int dspark_pack_w2(const void* src_rv, int V, int r, int wdtype, void* dst_vr, void* stream) {
    g_err[0] = 0;
    if (!src_rv || !dst_vr) return fail(DSPARK_EINVAL, "NULL buffer");
    if (V <= 0 || r <= 0) return fail(DSPARK_EINVAL, "V and r must be positive");
    if (wdtype != DSPARK_F32 && wdtype != DSPARK_BF16) return fail(DSPARK_EINVAL, "unknown weight dtype %d", wdtype);
    hipError_t e = launch_transpose(src_rv, r, V, wdtype == DSPARK_BF16 ? 2 : 4, dst_vr, (hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "transpose launch");
    return DSPARK_OK;
}

int dspark_stream_read(const void* a, size_t a_bytes, const void* b, size_t b_bytes, uint32_t* sink, void* stream) {
    g_err[0] = 0;
    if (!sink || (a_bytes && !a) || (b_bytes && !b)) return fail(DSPARK_EINVAL, "NULL buffer");
    if (a_bytes % 16 || b_bytes % 16) return fail(DSPARK_EINVAL, "sizes must be multiples of 16 bytes");
    if (!aligned16(a) || !aligned16(b)) return fail(DSPARK_EINVAL, "buffers must be 16-byte aligned");
    hipError_t e = launch_stream_read(a, a_bytes, b, b_bytes, sink, (hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "stream read launch");
    return DSPARK_OK;
}

int dspark_markov_draft(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout,
                        const int32_t* anchor, const float* H, int B, int K, int V, int r, int mode, uint64_t seed,
                        float temperature, int32_t* tokens, float* logprobs, void* workspace, size_t workspace_bytes,
                        void* stream) {
    return markov_draft_impl(U, W1, W2, wdtype, w2_layout, anchor, H, B, K, V, r, mode, seed, temperature, tokens,
                             logprobs, workspace, workspace_bytes, stream, nullptr, nullptr);
}

size_t dspark_markov_noalloc_max_bytes(void) { return kScratchBytes; }

int dspark_markov_draft_noalloc(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout,
                                const int32_t* anchor, const float* H, int B, int K, int V, int r, int mode,
                                uint64_t seed, float temperature, int32_t* tokens, float* logprobs, void* stream) {
    g_err[0] = 0;
    int rc = check_common(W1, W2, wdtype, w2_layout, B, V, r, mode, temperature);
    if (rc) return rc;
    if (K <= 0) return fail(DSPARK_EINVAL, "K must be positive");
    if (w2_layout == DSPARK_W2_RV && mfma_eligible(wdtype, r))
        return fail(DSPARK_EUNSUPPORTED, "the allocation-free draft needs W2 as [V, r] (DSPARK_W2_VR) for bf16 weights");
    const size_t need = markov_ws_bytes(B, K, V, r, wdtype, w2_layout, true);
    if (need > kScratchBytes)
        return fail(DSPARK_EUNSUPPORTED, "B=%d K=%d needs %zu bytes of scratch, more than the %zu the library holds", B, K,
                    need, kScratchBytes);
    void* ws = scratch_ptr();
    if (!ws) return DSPARK_EDEVICE;
    return markov_draft_impl(U, W1, W2, wdtype, w2_layout, anchor, H, B, K, V, r, mode, seed, temperature, tokens,
                             logprobs, ws, kScratchBytes, stream, nullptr, nullptr);
}

int dspark_markov_status(const void* workspace, size_t workspace_bytes, int B, int K, void* stream) {
    g_err[0] = 0;
    if (!workspace) return fail(DSPARK_EINVAL, "workspace must not be NULL");
    if (B <= 0 || K <= 0) return fail(DSPARK_EINVAL, "B and K must be positive");
    const MarkovWs ws = carve_markov(const_cast<void*>(workspace), B, K);
    const size_t end = (size_t)((const uint8_t*)(ws.counters + kErrorWord + 1) - (const uint8_t*)workspace);
    if (workspace_bytes < end) return fail(DSPARK_EWORKSPACE, "workspace of %zu bytes too small for B=%d K=%d", workspace_bytes, B, K);
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "hipStreamSynchronize");
    uint32_t err = 0;
    e = hipMemcpy(&err, ws.counters + kErrorWord, sizeof err, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return device_fail(e, "reading the error word");
    if (err) return fail(DSPARK_EDEVICE, "a bounded wait of the whole-round kernel gave up: tokens -1 / NaN where it failed");
    return DSPARK_OK;
}

void dspark_set_cooperative_launch(int on) { g_cooperative.store(on ? 1 : 0, std::memory_order_relaxed); }

void dspark_set_spin_limit(uint32_t sleeps) { g_spin_limit.store(sleeps ? sleeps : kDefaultSpinLimit, std::memory_order_relaxed); }

int dspark_markov_draft_logits(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout,
                               const int32_t* anchor, const float* H, int B, int K, int V, int r, int mode,
                               uint64_t seed, float temperature, int32_t* tokens, float* logprobs, float* logits,
                               void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    if (!logits) return fail(DSPARK_EINVAL, "logits must not be NULL");
    return markov_draft_impl(U, W1, W2, wdtype, w2_layout, anchor, H, B, K, V, r, mode, seed, temperature, tokens,
                             logprobs, workspace, workspace_bytes, stream, nullptr, nullptr, nullptr, logits);
}

int dspark_markov_draft_confidence(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout,
                                   const int32_t* anchor, const float* H, int B, int K, int V, int r, int mode,
                                   uint64_t seed, float temperature, const void* h, int D, const float* conf_w,
                                   int32_t* tokens, float* logprobs, float* conf, float* survival, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    if (!h || !conf_w || !conf || !survival) return fail(DSPARK_EINVAL, "h, conf_w, conf and survival must not be NULL");
    if (D <= 0 || D % 8 != 0) return fail(DSPARK_EUNSUPPORTED, "the confidence head needs D %% 8 == 0 (D=%d)", D);
    if (!aligned16(h)) return fail(DSPARK_EINVAL, "h must be 16-byte aligned");
    ConfArgs c{};
    c.h = (const uint16_t*)h;
    c.D = D;
    c.w = conf_w;
    c.W1 = W1;
    c.w1_bf16 = wdtype == DSPARK_BF16;
    c.r = r;
    c.K = K;
    c.anchor = anchor;
    c.tokens = tokens;
    c.conf = conf;
    c.survival = survival;
    return markov_draft_impl(U, W1, W2, wdtype, w2_layout, anchor, H, B, K, V, r, mode, seed, temperature, tokens,
                             logprobs, workspace, workspace_bytes, stream, nullptr, nullptr, &c);
}

int dspark_markov_draft_timed(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout,
                              const int32_t* anchor, const float* H, int B, int K, int V, int r, int mode,
                              uint64_t seed, float temperature, int32_t* tokens, float* logprobs, void* workspace,
                              size_t workspace_bytes, void* stream, float* kernel_ms, int* kernel_launches,
                              float* round_ms) {
    g_err[0] = 0;
    if (!kernel_ms || !kernel_launches || !round_ms) return fail(DSPARK_EINVAL, "timing outputs must not be NULL");
    if (K <= 0 || K > 4096) return fail(DSPARK_EINVAL, "K must be in [1, 4096] for the timed call");
    std::vector<hipEvent_t> ev(2 * (size_t)K + 2, nullptr);
    for (auto& x : ev) {
        hipError_t e = hipEventCreate(&x);
        if (e != hipSuccess) {
            for (auto& y : ev)
                if (y) (void)hipEventDestroy(y);
            return device_fail(e, "hipEventCreate");
        }
    }
    hipStream_t st = (hipStream_t)stream;
    (void)hipEventRecord(ev[2 * K], st);
    int launches = 0;
    int rc = markov_draft_impl(U, W1, W2, wdtype, w2_layout, anchor, H, B, K, V, r, mode, seed, temperature, tokens,
                               logprobs, workspace, workspace_bytes, stream, ev.data(), &launches);
    (void)hipEventRecord(ev[2 * K + 1], st);
    if (rc == DSPARK_OK) {
        hipError_t e = hipEventSynchronize(ev[2 * K + 1]);
        if (e != hipSuccess) rc = device_fail(e, "hipEventSynchronize");
    }
    if (rc == DSPARK_OK) {
        float total = 0.f;
        for (int i = 0; i < launches; ++i) {
            float t = 0.f;
            (void)hipEventElapsedTime(&t, ev[2 * i], ev[2 * i + 1]);
            total += t;
        }
        *kernel_ms = total;
        *kernel_launches = launches;
        (void)hipEventElapsedTime(round_ms, ev[2 * K], ev[2 * K + 1]);
    }
    for (auto& x : ev) (void)hipEventDestroy(x);
    return rc;
}

int dspark_markov_step(const float* U_k, int64_t u_stride, const void* W1, const void* W2, int wdtype, int w2_layout,
                       const int32_t* prev, const float* H_k, int B, int V, int r, int k, int mode, uint64_t seed,
                       float temperature, int32_t* tok, float* logprob, float* best_logit, void* workspace,
                       size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    int rc = check_common(W1, W2, wdtype, w2_layout, B, V, r, mode, temperature);
    if (rc) return rc;
    if (!U_k || !prev || !tok) return fail(DSPARK_EINVAL, "U_k, prev and tok must not be NULL");
    if (u_stride < V) return fail(DSPARK_EINVAL, "u_stride %lld < V %d", (long long)u_stride, V);
    if (k < 0) return fail(DSPARK_EINVAL, "k must be >= 0");
    const size_t need = markov_ws_bytes(B, 1, V, r, wdtype, w2_layout, true);
    if (!workspace || workspace_bytes < need)
        return fail(DSPARK_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    hipStream_t st = (hipStream_t)stream;
    MarkovWs ws = carve_markov(workspace, B, 1);
    const void* W2use = W2;
    int layout = w2_layout;
    if (w2_layout == DSPARK_W2_RV && mfma_eligible(wdtype, r)) {
        hipError_t e = launch_transpose(W2, r, V, 2, ws.w2t, st);
        if (e != hipSuccess) return device_fail(e, "transpose launch");
        W2use = ws.w2t;
        layout = DSPARK_W2_VR;
    }
    return run_step(U_k, u_stride, W1, W2use, wdtype, layout, prev, 1, H_k, r, B, V, r, k, mode, noise_key0(seed),
                    temperature, tok, logprob, best_logit, 1, &ws, nullptr, st);
}

int dspark_markov_logits(const float* U_k, int64_t u_stride, const void* W1, const void* W2, int wdtype, int w2_layout,
                         const int32_t* prev, const float* H_k, int B, int V, int r, float* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    int rc = check_common(W1, W2, wdtype, w2_layout, B, V, r, DSPARK_GREEDY, 1.0f);
    if (rc) return rc;
    if (!U_k || !prev || !out) return fail(DSPARK_EINVAL, "U_k, prev and out must not be NULL");
    if (u_stride < V) return fail(DSPARK_EINVAL, "u_stride %lld < V %d", (long long)u_stride, V);
    hipStream_t st = (hipStream_t)stream;
    const void* W2use = W2;
    int layout = w2_layout;
    if (w2_layout == DSPARK_W2_RV && mfma_eligible(wdtype, r)) {
        const size_t need = (size_t)V * r * 2;
        if (!workspace || workspace_bytes < need)
            return fail(DSPARK_EWORKSPACE, "workspace of %zu bytes needed for the transposed W2", need);
        hipError_t e = launch_transpose(W2, r, V, 2, workspace, st);
        if (e != hipSuccess) return device_fail(e, "transpose launch");
        W2use = workspace;
        layout = DSPARK_W2_VR;
    }
    return run_step(U_k, u_stride, W1, W2use, wdtype, layout, prev, 1, H_k, r, B, V, r, 0, DSPARK_GREEDY, 0, 1.0f,
                    nullptr, nullptr, nullptr, 1, nullptr, out, st);
}

size_t dspark_gate_workspace_bytes(int rows, int D, int r) {
    if (rows <= 0 || D <= 0 || r <= 0 || D % 256 != 0 || r % 32 != 0) return 0;
    return gate_splitk_bytes(rows, D, r);
}

int dspark_gate(const void* h, const void* Wg, int rows, int D, int r, float* H, void* workspace, size_t workspace_bytes,
                void* stream) {
    g_err[0] = 0;
    if (!h || !Wg || !H) return fail(DSPARK_EINVAL, "NULL buffer");
    if (rows <= 0 || D <= 0 || r <= 0) return fail(DSPARK_EINVAL, "rows, D and r must be positive");
    if (D % 256 != 0 || r % 32 != 0)
        return fail(DSPARK_EUNSUPPORTED, "gate needs D %% 256 == 0 and r %% 32 == 0 (D=%d r=%d)", D, r);
    if (!aligned16(h) || !aligned16(Wg)) return fail(DSPARK_EINVAL, "h and Wg must be 16-byte aligned");
    if (rows > 65535 * 32) return fail(DSPARK_EUNSUPPORTED, "too many rows");
    if (workspace && workspace_bytes < dspark_gate_workspace_bytes(rows, D, r))
        return fail(DSPARK_EINVAL, "gate workspace too small (%zu < %zu bytes)", workspace_bytes,
                    dspark_gate_workspace_bytes(rows, D, r));
    if (workspace && !aligned16(workspace)) return fail(DSPARK_EINVAL, "workspace must be 16-byte aligned");
    hipError_t e = launch_gate((const uint16_t*)h, (const uint16_t*)Wg, rows, D, r, H, workspace, workspace_bytes,
                               (hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "gate launch");
    return DSPARK_OK;
}

size_t dspark_topk_workspace_bytes(int rows, int V, int topk) {
    if (rows <= 0 || V <= 0 || topk <= 0) return 0;
    return 256;  // no scratch is used; a non-zero size keeps the calling convention uniform
}

int dspark_topk(const float* U, int64_t u_stride, int rows, int V, int topk, int32_t* idx, float* val, void* workspace,
                size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    (void)workspace;
    (void)workspace_bytes;
    if (!U || !idx) return fail(DSPARK_EINVAL, "U and idx must not be NULL");
    if (rows <= 0 || V <= 0) return fail(DSPARK_EINVAL, "rows and V must be positive");
    if (u_stride < V) return fail(DSPARK_EINVAL, "u_stride < V");
    if (topk < 1 || topk > V) return fail(DSPARK_EINVAL, "topk %d outside [1, V]", topk);
    if (!topk_supported(V, topk)) return fail(DSPARK_EUNSUPPORTED, "topk > 1024 needs V <= 4096");
    hipError_t e = launch_topk(U, u_stride, rows, V, topk, idx, val, nullptr, (hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "topk launch");
    return DSPARK_OK;
}

int dspark_schedule_prefixes(const float* survival, const float* sps, int R, int K, int32_t* lengths, float* theta,
                             void* stream) {
    g_err[0] = 0;
    if (!survival || !sps || !lengths) return fail(DSPARK_EINVAL, "survival, sps and lengths must not be NULL");
    if (R <= 0 || K <= 0) return fail(DSPARK_EINVAL, "R and K must be positive");
    if (!schedule_supported(R, K)) return fail(DSPARK_EUNSUPPORTED, "R * K = %ld exceeds 4096", (long)R * K);
    hipError_t e = launch_schedule(survival, sps, R, K, lengths, theta, (hipStream_t)stream);
    if (e != hipSuccess) return device_fail(e, "schedule launch");
    return DSPARK_OK;
}

size_t dspark_selector_workspace_bytes(int B, int K, int V, int r, int topk) {
    if (B <= 0 || K <= 0 || V <= 0 || r <= 0 || topk <= 0) return 0;
    const size_t tstride = (size_t)topk + (size_t)(K - 1) * topk * topk;
    return align256(sizeof(int32_t) * (size_t)B * K * topk) + align256(sizeof(float) * (size_t)B * tstride);
}

int dspark_selector_draft(const float* U, const void* A, const void* Bemb, int wdtype, const int32_t* anchor,
                          const float* H, int B, int K, int V, int r, int topk, int mode, uint64_t seed,
                          float temperature, int32_t* tokens, float* logprobs, int32_t* cand, float* scores,
                          void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    if (!U || !A || !Bemb || !anchor || !tokens) return fail(DSPARK_EINVAL, "U, A, Bemb, anchor, tokens must not be NULL");
    if (B <= 0 || K <= 0 || V <= 0 || r <= 0) return fail(DSPARK_EINVAL, "B, K, V and r must be positive");
    if (wdtype != DSPARK_F32 && wdtype != DSPARK_BF16) return fail(DSPARK_EINVAL, "unknown weight dtype %d", wdtype);
    if (mode != DSPARK_GREEDY && mode != DSPARK_SAMPLE) return fail(DSPARK_EINVAL, "unknown mode %d", mode);
    if (mode == DSPARK_SAMPLE && !(temperature > 0.f)) return fail(DSPARK_EINVAL, "temperature must be > 0 when sampling");
    if (topk < 1 || topk > V) return fail(DSPARK_EINVAL, "topk %d outside [1, V]", topk);
    if (!topk_supported(V, topk)) return fail(DSPARK_EUNSUPPORTED, "topk > 1024 needs V <= 4096");
    if (topk > 1024) return fail(DSPARK_EUNSUPPORTED, "the walk takes at most 1024 candidates (topk = %d)", topk);
    if (r > 1024) return fail(DSPARK_EUNSUPPORTED, "r = %d exceeds 1024", r);
    if ((size_t)B * K > 2147483647u) return fail(DSPARK_EUNSUPPORTED, "B * K too large");
    const size_t need = dspark_selector_workspace_bytes(B, K, V, r, topk);
    if (!workspace || workspace_bytes < need)
        return fail(DSPARK_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    hipStream_t st = (hipStream_t)stream;
    uint8_t* p = (uint8_t*)workspace;
    int32_t* cand_ws = (int32_t*)p;
    float* scores_ws = (float*)(p + align256(sizeof(int32_t) * (size_t)B * K * topk));
    SelectorArgs a{};
    a.U = U;
    a.A = A;
    a.Bemb = Bemb;
    a.bf16 = wdtype == DSPARK_BF16;
    a.anchor = anchor;
    a.H = H;
    a.B = B;
    a.K = K;
    a.V = V;
    a.r = r;
    a.topk = topk;
    a.sample = mode == DSPARK_SAMPLE;
    a.k0 = noise_key0(seed);
    a.inv_t = a.sample ? 1.0f / temperature : 1.0f;
    a.cand = cand ? cand : cand_ws;
    a.scores = scores ? scores : scores_ws;
    a.tokens = tokens;
    a.logprobs = logprobs;
    hipError_t e = launch_topk(U, V, B * K, V, topk, const_cast<int32_t*>(a.cand), nullptr, nullptr, st);
    if (e != hipSuccess) return device_fail(e, "topk launch");
    e = launch_pair_scores(a, st);
    if (e != hipSuccess) return device_fail(e, "pair-score launch");
    e = launch_walk(a, st);
    if (e != hipSuccess) return device_fail(e, "walk launch");
    return DSPARK_OK;
}

}  // extern "C"

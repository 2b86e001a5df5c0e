/*
 * dspark.h -- C ABI of libdspark: DSpark's semi-autoregressive draft calibration on one AMD MI355X
 * (gfx950).
 *
 * What the library computes (pages cited by title and section):
 *  - The Markov head.  "DFlash-2's Selector and DSpark's Markov Head: An Equivalence Observation",
 *    section "What the two methods do": logits_k = U_k + W1[a]^T W2 with W1 in R^{V x r},
 *    W2 in R^{r x V} and a the previously sampled token; the DSpark overview, section "The Markov
 *    head": W1 is an embedding lookup and W2 projects back to the vocabulary, one matrix-vector
 *    product per position, positions taken left to right ("Semi-autoregressive generation").
 *  - The gated variant.  Same page, section "The equivalence: remove the gate, recover the Markov
 *    Head": logits_t = U_t + (W1[a] (.) H(h_t))^T W2.
 *  - The Selector execution.  Same page, section "Where the parallelism comes from": keep the top-k
 *    tokens of the base logits at every position, compute the calibrated scores of all k x k
 *    adjacent (predecessor, candidate) pairs in parallel, then walk.
 *  - The drawn token's exact local log-probability.  "DSpark: Repair the Joint, Meter the Verify",
 *    section "Why the normalization has to be local": a softmax over the vocabulary of one position.
 *
 * Conventions for every call below:
 *  - Tensor pointers are DEVICE pointers to row-major, contiguous memory owned by the caller.  The
 *    library never allocates or frees memory inside these calls; scratch memory is the caller's
 *    `workspace`, sized by the matching *_workspace_bytes call.
 *  - Every call enqueues work on `stream` (a hipStream_t passed as void*, NULL = the null stream)
 *    and returns after enqueueing, without synchronising with the device.
 *  - Host-detectable argument errors return before anything is enqueued and leave every output
 *    untouched: DSPARK_EINVAL (NULL required pointer, size <= 0, unknown enum, temperature <= 0 in
 *    sampling mode, top-k out of range), DSPARK_EWORKSPACE (workspace too small or NULL when
 *    needed), DSPARK_EUNSUPPORTED (a shape outside the documented limits).  A failed kernel launch
 *    returns DSPARK_EDEVICE.  dspark_last_error() gives a one-line reason for the calling thread's
 *    last non-OK status.  No C++ exception crosses this boundary.
 *  - Preconditions not checked on the host: token ids (anchor, prev) lie in [0, V); U, H and the
 *    weights are finite.  Violations give unspecified results.
 *  - Token ties: every argmax, race, top-k and walk breaks ties towards the lower vocabulary id.
 *  - Determinism: identical inputs, seed and shapes give bit-identical outputs on one device.
 *  - Calls on one stream run in order; concurrent calls need distinct workspaces.
 *
 * Noise (sampling mode).  The pages fix the distribution (softmax(l / T)), not the generator.  Uniforms come
 * from a counter hash: fmix(x) is the MurmurHash3 32-bit finalisation mix (A. Appleby, public domain);
 * k0 = fmix(lo32(seed) ^ fmix(hi32(seed))), k1 = fmix(k0 ^ b), k2 = fmix(k1 ^ k), h(n) = fmix(k2 ^ n);
 * u(n) = (2 * (h(n) >> 9) + 1) / 2^24.  b is the batch row, k the draft position (0-based).
 *  - A draw over a set of ids (the whole vocabulary for the Markov head, the candidate set for the Selector's
 *    walk) races the set's members grouped in aligned vocabulary blocks of 16 ids: with p_v = exp(l_v / T - M),
 *    block j (ids 16 j .. 16 j + 15 that belong to the set) has mass S_j = sum of its members' p_v and variate
 *    E_j = -ln u(2 j); the block with the largest S_j / E_j wins (equivalently the largest ln S_j + G_j with
 *    G_j = -ln(-ln u(2 j)) a Gumbel variate: a Gumbel-max over blocks; ties to the lower block), and the drawn
 *    id is the first member of the winner, in ascending id order, whose inclusive prefix mass exceeds
 *    u(2 j + 1) S_j.  An exact draw from softmax(l / T) over the set, one hash pair per block rather than one
 *    hash per id; the noise keys on vocabulary blocks, never on candidate slots, so a candidate set holding
 *    the whole vocabulary draws exactly what the full head draws.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSPARK_ABI_VERSION 2

/* status codes */
#define DSPARK_OK 0
#define DSPARK_EINVAL 1
#define DSPARK_EUNSUPPORTED 2
#define DSPARK_EWORKSPACE 3
#define DSPARK_EDEVICE 4

/* weight element types (U, H and all outputs are always fp32 / int32) */
#define DSPARK_F32 0
#define DSPARK_BF16 1 /* raw bfloat16, 2 bytes per element */

/* storage order of W2 */
#define DSPARK_W2_RV 0 /* [r, V]: as the pages write W2 */
#define DSPARK_W2_VR 1 /* [V, r]: W2 transposed, one r-vector per vocabulary id (same layout as Bemb) */

/* pick rule */
#define DSPARK_GREEDY 0 /* argmax of the calibrated logits; temperature ignored (T = 1) */
#define DSPARK_SAMPLE 1 /* an exact sample of softmax(l / T) at temperature T (see Noise) */

/* Version of this ABI (DSPARK_ABI_VERSION of the built library). */
int dspark_abi_version(void);

/* Static string naming a status code. */
const char* dspark_status_str(int status);

/* One-line reason for the calling thread's most recent non-OK status ("" if none). */
const char* dspark_last_error(void);

/* ------------------------------------------------------------------------------------------------ */
/* Markov head                                                                                      */
/* ------------------------------------------------------------------------------------------------ */

/* Workspace bytes dspark_markov_draft / dspark_markov_step need for these sizes (0 on bad sizes). */
size_t dspark_markov_workspace_bytes(int B, int K, int V, int r, int wdtype, int w2_layout);

/*
 * Draft K positions for B rows with the Markov head (the DSpark overview, sections "Semi-autoregressive
 * generation" and "The Markov head"; the equivalence page, section "What the two methods do").
 * For k = 0 .. K-1 and every row b, with a_0 = anchor[b] and a_k = tokens[b, k-1]:
 *     l[v]          = U[b, k, v] + sum_j x[j] * W2[j, v],   x = W1[a_k, :] (.) H[b, k, :]  (H == NULL: x = W1[a_k])
 *     tokens[b, k]  = argmax_v l[v] (GREEDY) or the block-race draw from softmax(l / T) (SAMPLE; see Noise)
 *     logprobs[b,k] = l[tok] / T - log sum_v exp(l[v] / T)   (T = 1 in GREEDY)
 *
 * U        [B, K, V] fp32.
 * W1       [V, r] weights of type wdtype.
 * W2       [r, V] (w2_layout = DSPARK_W2_RV) or [V, r] (DSPARK_W2_VR) of type wdtype.  The bf16 matrix-core
 *          path reads the [V, r] layout; an [r, V] W2 is first transposed into the workspace on every call,
 *          so callers that draft repeatedly should transpose once with dspark_pack_w2.
 * anchor   [B] int32, the token each row's block starts from.
 * H        [B, K, r] fp32 gate values (for example from dspark_gate) or NULL for the ungated head.
 * r        1 .. 1024.  The bf16 matrix-core path needs r % 16 == 0 and r <= 512; other shapes run on a
 *          vector-ALU path of the same results.
 * mode     DSPARK_GREEDY or DSPARK_SAMPLE; seed and temperature (> 0) are used in SAMPLE mode only.
 * tokens   [B, K] int32 output.   logprobs: [B, K] fp32 output or NULL.
 * Accumulation is fp32 over bf16 (or fp32) products; the gated bf16 path rounds x to bf16 (nearest even).
 * Greedy bf16 drafts at r = 256 with a [V, r] W2 keep W2 on chip for the whole round when it fits: one row with
 * V <= 640 x (CU count) (each lane holds one W2 row; dot products summed in two fixed-order halves), and 2 .. 64
 * rows with V <= 512 x (CU count) and no confidence head (each workgroup holds its W2 tiles as matrix-core
 * operands; the same per-tile contraction as the tiled round, rows merged over waves in a fixed order).
 * Device-side failure: the whole-round kernel (one persistent launch per call) waits on other workgroups with
 * bounded spins.  If a wait gives up (it never should on an idle device; a device shared with other work that
 * keeps workgroups from being co-resident could cause it), the kernel still exits normally, writes tokens = -1
 * and logprobs = NaN at the positions it could not finish and sets an error word in the workspace; the call
 * itself has already returned DSPARK_OK.  Callers that must not feed -1 onward check dspark_markov_status.
 */
int dspark_markov_draft(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout,
                        const int32_t* anchor, const float* H, int B, int K, int V, int r, int mode,
                        uint64_t seed, float temperature, int32_t* tokens, float* logprobs, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * dspark_markov_draft for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same computation and kernels, with no workspace
 * argument.  The scratch is a file-scope device array of the library, dspark_markov_noalloc_max_bytes()
 * = 16 MiB per device, held until the process ends; this call neither allocates nor frees.  Every call on a
 * device shares that device's array, so calls that overlap in time on one device (other streams, other host
 * threads) race and give wrong results; calls in order on one stream are safe.  The kernels clear what must
 * start at zero themselves.  Shapes whose workspace (dspark_markov_workspace_bytes) exceeds the array return
 * DSPARK_EUNSUPPORTED (B = 128, K = 16 needs about 11 MB on a 256-CU device), and so does a bf16 W2 stored
 * [r, V] (its transposed copy would not fit: use DSPARK_W2_VR, or dspark_pack_w2 once).  A position that fails
 * on the device is marked as in dspark_markov_draft (tokens -1, logprobs NaN); dspark_markov_status, which reads
 * a caller's workspace, does not apply to this call.
 */
size_t dspark_markov_noalloc_max_bytes(void);
int dspark_markov_draft_noalloc(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout,
                                const int32_t* anchor, const float* H, int B, int K, int V, int r, int mode,
                                uint64_t seed, float temperature, int32_t* tokens, float* logprobs, void* stream);

/*
 * Device-side status of the last dspark_markov_draft* call made with this workspace (and these B, K) on
 * `stream`: waits for the stream (this call synchronises the host), then returns DSPARK_EDEVICE if a bounded
 * wait of the whole-round kernel gave up (tokens -1 and logprobs NaN where it failed), DSPARK_OK otherwise.
 */
int dspark_markov_status(const void* workspace, size_t workspace_bytes, int B, int K, void* stream);

/*
 * Launch of the whole-round kernel, for the calls that follow in this process.  The kernel runs one workgroup
 * per CU and synchronises them at every position, so all must be resident together.  By default (on = 0) it is
 * an ordinary launch: on a device that runs nothing else at the same time every workgroup is resident at once.
 * The runtime's cooperative launch (on = 1) guarantees co-residency even on a shared device, at a cost of
 * about 20 us per call on MI355X.  With the ordinary launch on a device shared with kernels that hold CUs for
 * long, the round's bounded waits can give up: the kernel still exits, and dspark_markov_status reports it.
 */
void dspark_set_cooperative_launch(int on);

/*
 * Testing hook: the number of sleeps after which a bounded wait of the whole-round kernel gives up, for the
 * calls that follow in this process (0 restores the default, 2^22).  A tiny limit forces the failure path of
 * dspark_markov_status without faulting: every wait still ends and the kernel exits normally.
 */
void dspark_set_spin_limit(uint32_t sleeps);

/*
 * Validation call: dspark_markov_draft (same arguments and results) that also writes the calibrated logits of
 * every position along the drafted path, logits[b, k, v] = l[v] with a_k = tokens[b, k-1] (fp32, [B, K, V]),
 * computed by the drafting kernel itself (the whole-round kernel with a store epilogue: the same contraction and
 * the same pick).  Only shapes that take the whole-round kernel (bf16 weights, r % 16 == 0, r <= 256,
 * V % 4 == 0, 16-byte aligned buffers) are accepted; DSPARK_EUNSUPPORTED otherwise.
 */
int dspark_markov_draft_logits(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout,
                               const int32_t* anchor, const float* H, int B, int K, int V, int r, int mode,
                               uint64_t seed, float temperature, int32_t* tokens, float* logprobs, float* logits,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * dspark_markov_draft plus the confidence head and prefix survival of the drafted block (DSpark overview,
 * section "Confidence-scheduled verification"): conf[b, k] = sigmoid(w_h . h[b, k, :] + w_m . W1[x_{k-1}, :])
 * with x_{k-1} the token drafted at position k-1 (the anchor at k = 0), and survival[b, k] = the product of
 * conf[b, 0..k].  h [B, K, D] bf16 (16-byte aligned, D % 8 == 0); conf_w [D + r] fp32, w_h then w_m; conf and
 * survival [B, K] fp32 outputs.  On the whole-round path the head is computed inside the same launch, one
 * position behind the draft; otherwise by one extra launch after it.  fp32 arithmetic; a failed position
 * (token -1) has NaN confidence and survival from there on.  Other arguments, outputs and errors as
 * dspark_markov_draft; DSPARK_EUNSUPPORTED if D % 8 != 0.
 */
int dspark_markov_draft_confidence(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout,
                                   const int32_t* anchor, const float* H, int B, int K, int V, int r, int mode,
                                   uint64_t seed, float temperature, const void* h, int D, const float* conf_w,
                                   int32_t* tokens, float* logprobs, float* conf, float* survival, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Measurement variant of dspark_markov_draft (same arguments and results).  It also records HIP event
 * pairs on `stream` around every launch of the contraction kernel (one launch per round on the persistent
 * path, one per position otherwise) and around the whole call, waits for the call to finish (this call
 * synchronises the host with the stream), and writes to host memory: *kernel_ms, the summed duration of
 * the contraction launches; *kernel_launches, their number; *round_ms, the whole call.  1 <= K <= 4096.
 */
int dspark_markov_draft_timed(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout,
                              const int32_t* anchor, const float* H, int B, int K, int V, int r, int mode,
                              uint64_t seed, float temperature, int32_t* tokens, float* logprobs, void* workspace,
                              size_t workspace_bytes, void* stream, float* kernel_ms, int* kernel_launches,
                              float* round_ms);

/*
 * One position of the same rule with the predecessors supplied by the caller (teacher forcing).
 * U_k      [B, V] fp32 with row b at U_k + b * u_stride (u_stride >= V).
 * prev     [B] int32 predecessors.   H_k: [B, r] fp32 or NULL.   k: the draft position, used only as the
 *          noise counter in SAMPLE mode.
 * tok      [B] int32 output.  logprob, best_logit: [B] fp32 outputs or NULL (best_logit = l[tok]).
 */
int dspark_markov_step(const float* U_k, int64_t u_stride, const void* W1, const void* W2, int wdtype,
                       int w2_layout, const int32_t* prev, const float* H_k, int B, int V, int r, int k, int mode,
                       uint64_t seed, float temperature, int32_t* tok, float* logprob, float* best_logit,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Validation call: the calibrated logits of one position, written out as out[b, v] = l[v] (fp32,
 * [B, V]), computed with the same bias contraction the drafting kernels use.  Arguments as
 * dspark_markov_step.  Needs no workspace for the [V, r] layout; with an [r, V] W2 it needs
 * V * r * (2 or 4) bytes of workspace for the transposed copy.
 */
int dspark_markov_logits(const float* U_k, int64_t u_stride, const void* W1, const void* W2, int wdtype,
                         int w2_layout, const int32_t* prev, const float* H_k, int B, int V, int r, float* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Transpose W2 from [r, V] to [V, r] (element type wdtype): dst[v, j] = src[j, v].  Both device
 * buffers hold V * r elements and must not overlap.
 */
int dspark_pack_w2(const void* src_rv, int V, int r, int wdtype, void* dst_vr, void* stream);

/*
 * Measurement utility, not a step of the method: reads the device buffer a (a_bytes) with ordinary 16-byte
 * loads and then b (b_bytes) with non-temporal ones, once, and writes nothing but possibly one word of sink
 * (a device uint32).  Timing it over the operands of a draft round (W2 and the base logits of each position)
 * gives the rate at which this part streams those bytes, the practical ceiling beside the nominal HBM peak.
 * Sizes must be multiples of 16 and the buffers 16-byte aligned (DSPARK_EINVAL otherwise); a NULL buffer is
 * allowed only with size 0.
 */
int dspark_stream_read(const void* a, size_t a_bytes, const void* b, size_t b_bytes, uint32_t* sink, void* stream);

/* ------------------------------------------------------------------------------------------------ */
/* gate                                                                                             */
/* ------------------------------------------------------------------------------------------------ */

/*
 * H = sigmoid(h Wg): the context gate of the gated head and of the Selector (equivalence page,
 * section "What the two methods do": H(h_t) is computed from the current hidden state; the speculators
 * guide, "Markov Head": the gated variant gates the bias by the backbone hidden state).  The pages give
 * no formula; this library takes a bias-free linear map followed by the logistic sigmoid.
 * h [rows, D] bf16, Wg [D, r] bf16, H [rows, r] fp32 output.  fp32 accumulation.
 * D % 256 == 0 and r % 32 == 0 are required (DSPARK_EUNSUPPORTED otherwise).
 * workspace (device, 16-byte aligned, owned by the caller, contents need not be initialised) may be NULL.  With
 * at least dspark_gate_workspace_bytes(rows, D, r) bytes (a non-zero size) and a 16-byte aligned H, the
 * product runs split over the k range in two launches (partial sums in the workspace, then their fixed-order
 * sum and the sigmoid); otherwise, or with a NULL workspace, in one launch.  Both are deterministic; their
 * results may differ in the last bits (another summation order).  A workspace smaller than that size, or
 * misaligned, is DSPARK_EINVAL.  Calls sharing one workspace must not overlap.
 */
int dspark_gate(const void* h, const void* Wg, int rows, int D, int r, float* H, void* workspace, size_t workspace_bytes,
                void* stream);

/* Workspace bytes of dspark_gate's split-k form for these sizes (0: it does not apply; pass NULL). */
size_t dspark_gate_workspace_bytes(int rows, int D, int r);

/* ------------------------------------------------------------------------------------------------ */
/* Selector-style top-k truncation                                                                  */
/* ------------------------------------------------------------------------------------------------ */

/* Workspace bytes dspark_topk needs (0 on bad sizes). */
size_t dspark_topk_workspace_bytes(int rows, int V, int topk);

/*
 * Top-k of every row of U under the order (value desc, vocabulary id asc); -0.0 and +0.0 compare
 * equal.  (Equivalence page, section "Where the parallelism comes from": the candidate set of a
 * position is the top tokens under the base logits.)
 * U [rows, V] fp32 with row i at U + i * u_stride.  idx [rows, topk] int32 output, val [rows, topk]
 * fp32 output or NULL.  1 <= topk <= V; topk <= 1024 at any V (DSPARK_EUNSUPPORTED for topk > 1024
 * unless V <= 4096, where the row is sorted whole).  topk <= 64 takes one pass over the row; 64 < topk <=
 * 1024 at V > 4096 takes a radix selection that reads the row four times.
 */
int dspark_topk(const float* U, int64_t u_stride, int rows, int V, int topk, int32_t* idx, float* val,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Hardware-aware prefix scheduling of drafted blocks (DSpark overview, section "Hardware-aware prefix
 * scheduling").  R requests with prefix survivals survival[r, j] (j < K; e.g. the survival output of
 * dspark_markov_draft_confidence); sps[B] = the target engine's steps per second at a batch of B tokens,
 * B = 0 .. R (K + 1).  The greedy starts from B = R (no draft token verified), ranks the extensions (r, j) by
 * survival (ties: smaller j, then smaller r; survival never increases along a block, so prefixes come
 * first) and admits them while Theta = (R + sum of admitted survivals) * sps[R + admitted] strictly
 * increases.  lengths [R] int32 output: tokens of each block to verify; theta [1] fp32 output or NULL:
 * Theta of the admitted set.  Survival values outside [0, 1] (or NaN) count as 0.  Device pointers; one
 * workgroup, fp64 sums.  R K <= 4096 (DSPARK_EUNSUPPORTED otherwise).
 */
int dspark_schedule_prefixes(const float* survival, const float* sps, int R, int K, int32_t* lengths, float* theta,
                             void* stream);

/* Workspace bytes dspark_selector_draft needs (0 on bad sizes). */
size_t dspark_selector_workspace_bytes(int B, int K, int V, int r, int topk);

/*
 * Selector execution of the (optionally gated) Markov rule (equivalence page, sections "Where the
 * parallelism comes from" and "Two implications"):
 *  1. cand[b, t, :] = top-k of U[b, t, :];
 *  2. pair scores, all in parallel: the anchor row  S0[b, j] = U[b,0,c_0j] + < A[anchor_b] (.) H[b,0], Bemb[c_0j] >
 *     and for t >= 1  S_t[b, i, j] = U[b,t,c_tj] + < A[c_{t-1,i}] (.) H[b,t], Bemb[c_tj] >;
 *  3. the walk: i_0 = pick over S0[b, :], i_t = pick over S_t[b, i_{t-1}, :]; tokens[b, t] = c_{t, i_t}.
 *     The pick over the k candidates is the argmax (GREEDY) or the draw of Noise restricted to the
 *     candidates (SAMPLE); logprobs[b, t] = log softmax over the walked row of scores / T.
 * U [B, K, V] fp32; A, Bemb [V, r] of type wdtype; anchor [B]; H [B, K, r] fp32 or NULL.
 * topk as for dspark_topk and at most 1024 (DSPARK_EUNSUPPORTED above); r <= 1024 (rows are staged with 16-byte loads when r % 8 == 0 for bf16 or
 * r % 4 == 0 for fp32 and A, Bemb are 16-byte aligned, element by element otherwise).
 * tokens [B, K] int32 output; logprobs [B, K] fp32 or NULL; cand [B, K, topk] int32 or NULL;
 * scores [B, topk + (K-1) * topk * topk] fp32 or NULL (anchor row, then the K-1 tables, row-major i, j).
 */
int dspark_selector_draft(const float* U, const void* A, const void* Bemb, int wdtype, const int32_t* anchor,
                          const float* H, int B, int K, int V, int r, int topk, int mode, uint64_t seed,
                          float temperature, int32_t* tokens, float* logprobs, int32_t* cand, float* scores,
                          void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */

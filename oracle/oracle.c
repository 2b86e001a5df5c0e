/*
 * oracle.c -- plain fp64 CPU reference for DSpark's Markov-head draft calibration and for the
 * Selector-style top-k truncation of the same rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls this file: only the
 * tests, the smoke check and the bench's CPU-baseline leg use it.  It shares no code, header,
 * table or constant with the GPU library; the two meet only through the seeded inputs (made by the
 * separate input generator) and through the published definition of the noise hash below, which
 * each side implements on its own.
 *
 * Every number is computed in IEEE double precision, one plain loop at a time, in the order the
 * defining formula states (sums over the rank index j ascending, vocabulary scans v ascending).
 * Inputs are read exactly: bf16 and fp32 values convert to double without rounding.
 *
 * Sources (pages; cited by title and section):
 *  [MvS]  "DFlash-2's Selector and DSpark's Markov Head: An Equivalence Observation"
 *         (jialefu.github.io) -- sections "What the two methods do", "The equivalence: remove the
 *         gate, recover the Markov Head", "Where the parallelism comes from", "Two implications".
 *  [DSp]  "DSpark" overview (himanshu-arora.com) -- sections "Semi-autoregressive generation",
 *         "The Markov head", "Confidence-scheduled verification", "Hardware-aware prefix scheduling".
 *  [Tut]  "DSpark: Repair the Joint, Meter the Verify" (stable-lab.github.io) -- sections
 *         "Fix 1: A First-Order Markov Head", "Why the normalization has to be local",
 *         "The Trap: A Product of Marginals", "Marginalization, From Scratch".
 *  [vLLM] "DSpark" (docs.vllm.ai speculators user guide) -- "Markov Head", "Key Parameters".
 *
 * Readings where the pages leave a step open (each listed with its reason in the design notes):
 *  - position 1 is conditioned on the anchor token;
 *  - ties in every argmax / top-k go to the lower vocabulary id (never the candidate slot);
 *  - sampling is an exact draw from softmax(l/T) over the set the pick ranges over (the whole vocabulary,
 *    or a candidate set) by one definition: a Gumbel-max race between the set's members grouped in aligned
 *    vocabulary blocks of 16 ids (noise keyed on (seed, row, position, block)), then inverse CDF inside the
 *    winning block; so a candidate set holding every id draws exactly what the whole vocabulary draws;
 *    greedy ignores T;
 *  - the reported log-probability is log softmax(l/T)[token] over the same set the pick ranges over;
 *  - the gate multiplies the predecessor embedding: x = W1[a] (.) H(h_k).
 *
 * Parity status: every exported function is pinned by a CPU test against a value the pages print, a
 * closed form, a special case or brute force; see the test files.  No function here is unpinned.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_W2_RV 0 /* W2 stored [r, V] as on the pages */
#define OR_W2_VR 1 /* W2 stored transposed, [V, r] */
#define OR_GREEDY 0
#define OR_SAMPLE 1

/* ------------------------------------------------------------------------------------------ */
/* exact reads of the stored inputs                                                             */
/* ------------------------------------------------------------------------------------------ */

/* Element i of a weight tensor stored as fp32 or as raw bf16 bits; both widen exactly. */
static double weight_at(const void* p, int dtype, size_t i) {
    if (dtype == OR_F32) return (double)((const float*)p)[i];
    uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* W2[j, v] in either storage order ([MvS] "What the two methods do": W2 is 256 x V). */
static double w2_at(const void* W2, int dtype, int layout, int V, int r, int j, int v) {
    size_t i = (layout == OR_W2_RV) ? (size_t)j * (size_t)V + (size_t)v : (size_t)v * (size_t)r + (size_t)j;
    return weight_at(W2, dtype, i);
}

/* ------------------------------------------------------------------------------------------ */
/* noise: counter-based hash of (seed, row, position, vocabulary id)                            */
/* ------------------------------------------------------------------------------------------ */

/* Finalisation mix of MurmurHash3 (A. Appleby, public domain): xor-shift 16, multiply by
 * 0x85EBCA6B, xor-shift 13, multiply by 0xC2B2AE35, xor-shift 16, all modulo 2^32. */
static uint32_t murmur3_fmix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    h *= 0xC2B2AE35u;
    h ^= h >> 16;
    return h;
}

uint32_t oracle_fmix32(uint32_t h) { return murmur3_fmix32(h); }

/* Threads the parallel loops below use (OpenMP's current maximum), and a setter (n >= 1). */
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* Chained key: k0 from the 64-bit seed, then the row, the position and the vocabulary id are
 * folded in one at a time, each followed by a full finalisation mix. */
uint32_t oracle_noise_bits(uint64_t seed, uint32_t row, uint32_t pos, uint32_t v) {
    uint32_t k0 = murmur3_fmix32((uint32_t)(seed & 0xFFFFFFFFu) ^ murmur3_fmix32((uint32_t)(seed >> 32)));
    uint32_t k1 = murmur3_fmix32(k0 ^ row);
    uint32_t k2 = murmur3_fmix32(k1 ^ pos);
    return murmur3_fmix32(k2 ^ v);
}

/* Uniform in (0,1): the top 23 bits m of the hash give u = (2m + 1) / 2^24, never 0 or 1. */
double oracle_noise_uniform(uint64_t seed, uint32_t row, uint32_t pos, uint32_t v) {
    uint32_t h = oracle_noise_bits(seed, row, pos, v);
    return (2.0 * (double)(h >> 9) + 1.0) / 16777216.0;
}

/* Standard Gumbel variate G = -ln(-ln u) (inverse CDF of exp(-exp(-g))). */
double oracle_gumbel(uint64_t seed, uint32_t row, uint32_t pos, uint32_t v) {
    double u = oracle_noise_uniform(seed, row, pos, v);
    return -log(-log(u));
}

/* Noise of n consecutive vocabulary ids v0 .. v0+n-1 at one (row, position): uniforms and Gumbel
 * variates (either output may be NULL).  Same definitions as above, one call per id. */
void oracle_noise_fill(uint64_t seed, uint32_t row, uint32_t pos, uint32_t v0, int64_t n, double* u, double* g) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        if (u) u[i] = oracle_noise_uniform(seed, row, pos, v0 + (uint32_t)i);
        if (g) g[i] = oracle_gumbel(seed, row, pos, v0 + (uint32_t)i);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* gate  H = sigmoid(h Wg)                                                                      */
/* ------------------------------------------------------------------------------------------ */

/* [MvS] "What the two methods do": the Selector's gate H(h_t) is computed from the current hidden
 * state; [vLLM] "Markov Head": the gated variant gates the bias by the backbone hidden state.  The
 * form is a sigmoid of a linear map with no bias: H[i, j] = 1 / (1 + exp(-sum_d h[i,d] Wg[d,j])).
 * h is [rows, D] bf16, Wg is [D, r] bf16, H is [rows, r]. */
void oracle_gate(const uint16_t* h, const uint16_t* Wg, int rows, int D, int r, double* H) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < rows; ++i) {
        for (int j = 0; j < r; ++j) {
            double z = 0.0;
            for (int d = 0; d < D; ++d)
                z += weight_at(h, OR_BF16, (size_t)i * D + d) * weight_at(Wg, OR_BF16, (size_t)d * r + j);
            H[(size_t)i * r + j] = 1.0 / (1.0 + exp(-z));
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* confidence head and prefix survival                                                          */
/* ------------------------------------------------------------------------------------------ */

/* [DSp] "Confidence-scheduled verification": c_k = sigmoid(w^T [h_k ; W1[x_{k-1}]]) is the probability that
 * position k is accepted given that the prefix so far survived, and the prefix survival is the product
 * a_j = prod_{i <= j} c_i.  x_{k-1} is the token drafted at position k-1; at k = 0 it is the anchor (the
 * predecessor the Markov step uses at that position).  h [B, K, D] bf16; w [D + r] fp32, the h part first,
 * then the W1 part; W1 [V, r] of type wdtype; tokens [B, K].  conf and survival [B, K]. */
void oracle_confidence(const uint16_t* h, int D, const float* w, const void* W1, int wdtype, int r,
                       const int32_t* anchor, const int32_t* tokens, int B, int K, double* conf, double* survival) {
    for (int b = 0; b < B; ++b) {
        double a = 1.0;
        for (int k = 0; k < K; ++k) {
            const int prev = (k == 0) ? anchor[b] : tokens[(size_t)b * K + k - 1];
            double z = 0.0;
            for (int d = 0; d < D; ++d) z += (double)w[d] * weight_at(h, OR_BF16, ((size_t)b * K + k) * D + d);
            for (int j = 0; j < r; ++j) z += (double)w[D + j] * weight_at(W1, wdtype, (size_t)prev * r + j);
            const double c = 1.0 / (1.0 + exp(-z));
            a *= c;
            conf[(size_t)b * K + k] = c;
            survival[(size_t)b * K + k] = a;
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* hardware-aware prefix scheduling                                                             */
/* ------------------------------------------------------------------------------------------ */

/* [DSp] "Hardware-aware prefix scheduling": R requests, request r may verify a prefix of length l_r of its
 * drafted block; the target batch is B = sum_r (1 + l_r) tokens, the expected committed tokens are
 * R + sum_{(r,j) in S} a[r][j] (a = prefix survival), and the objective is
 * Theta(S) = (R + sum a) * SPS(B), SPS the engine's steps-per-second table (sps[B], B = 0 .. R (K + 1)).
 * Survival values that are not finite numbers in [0, 1] count as 0. */
static double survival_value(float x) { return (x >= 0.0f && x <= 1.0f) ? (double)x : 0.0; }

/* Extension order: survival descending, then position j ascending, then request r ascending.  Survival
 * never increases along a request's block, so this order admits every prefix before its extension. */
static const float* g_sched_a;
static int g_sched_K;
static int sched_cmp(const void* pa, const void* pb) {
    const int x = *(const int*)pa, y = *(const int*)pb;
    const double ax = survival_value(g_sched_a[x]), ay = survival_value(g_sched_a[y]);
    if (ax != ay) return ax > ay ? -1 : 1;
    const int jx = x % g_sched_K, jy = y % g_sched_K;
    if (jx != jy) return jx < jy ? -1 : 1;
    return (x / g_sched_K) < (y / g_sched_K) ? -1 : ((x / g_sched_K) > (y / g_sched_K) ? 1 : 0);
}

/* The greedy of the same section: start from B = R (no extension), take extensions in the order above and
 * admit each while Theta strictly increases; stop at the first one that would not.  Writes l_r and returns
 * Theta of the admitted set. */
double oracle_schedule_greedy(const float* a, const float* sps, int R, int K, int32_t* lengths) {
    const int n = R * K;
    int* order = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    for (int i = 0; i < n; ++i) order[i] = i;
    g_sched_a = a;
    g_sched_K = K;
    qsort(order, (size_t)n, sizeof(int), sched_cmp);
    for (int r = 0; r < R; ++r) lengths[r] = 0;
    double tokens = (double)R;
    double theta = tokens * (double)sps[R];
    for (int m = 0; m < n; ++m) {
        const double t2 = (tokens + survival_value(a[order[m]])) * (double)sps[R + m + 1];
        if (!(t2 > theta)) break;
        tokens += survival_value(a[order[m]]);
        theta = t2;
        lengths[order[m] / K] += 1;
    }
    free(order);
    return theta;
}

/* Brute force over every prefix-length vector l in [0, K]^R ((K + 1)^R <= 2^22): the largest Theta and,
 * for the first vector (in lexicographic order) that reaches it, the lengths. */
double oracle_schedule_best(const float* a, const float* sps, int R, int K, int32_t* lengths) {
    if (R <= 0 || K < 0) return -1.0;
    long total = 1;
    for (int r = 0; r < R; ++r) {
        total *= (K + 1);
        if (total > (1L << 22)) return -1.0;
    }
    int* l = (int*)calloc((size_t)R, sizeof(int));
    double best = -INFINITY;
    for (long c = 0; c < total; ++c) {
        long rem = c;
        int count = 0;
        double tokens = (double)R;
        for (int r = R - 1; r >= 0; --r) {
            l[r] = (int)(rem % (K + 1));
            rem /= (K + 1);
        }
        for (int r = 0; r < R; ++r) {
            count += l[r];
            for (int j = 0; j < l[r]; ++j) tokens += survival_value(a[(size_t)r * K + j]);
        }
        const double theta = tokens * (double)sps[R + count];
        if (theta > best) {
            best = theta;
            for (int r = 0; r < R; ++r) lengths[r] = l[r];
        }
    }
    free(l);
    return best;
}

/* ------------------------------------------------------------------------------------------ */
/* one calibrated position                                                                      */
/* ------------------------------------------------------------------------------------------ */

/* Predecessor embedding x[j] = W1[prev, j] * H[j] (H == NULL means the ungated head, H = 1).
 * [MvS] "The equivalence": gated form logits_t = U_t + (W1[a] (.) H(h_t))^T W2. */
static void predecessor_embedding(const void* W1, int dtype, int r, int prev, const double* Hk, double* x) {
    for (int j = 0; j < r; ++j) {
        double w = weight_at(W1, dtype, (size_t)prev * r + j);
        x[j] = Hk ? w * Hk[j] : w;
    }
}

/* Calibrated logit of candidate v: U_k(v) + sum_j x[j] W2[j, v]  ([MvS] "The equivalence",
 * per-candidate form; [DSp] "The Markov head": one matrix-vector product over the vocabulary). */
static double calibrated_logit(const float* Uk, const void* W2, int dtype, int layout, int V, int r,
                               const double* x, int v) {
    double bias = 0.0;
    for (int j = 0; j < r; ++j) bias += x[j] * w2_at(W2, dtype, layout, V, r, j, v);
    return (double)Uk[v] + bias;
}

/* The pick at one position ranges over a set of n logits l[0..n) with distinct vocabulary ids ids[0..n)
 * (ids == NULL: the whole vocabulary, id = slot).  Every sum over the set runs in ascending id order, so a
 * candidate set that holds every id gives, bit for bit, what the whole vocabulary gives.
 *
 * Greedy: the largest l, ties to the lower id.
 * Sampling ([DSp] "DSpark vs DFlash 2": sample from the corrected logits; the pages fix the distribution,
 * softmax(l/T) over the set, not the sampler): a two-level exponential race.  With p_v = exp(l_v/T - M),
 * M = max l/T, the members are grouped by vocabulary block q = id div 16 (aligned blocks of 16 ids; a
 * restricted set may hold only some ids of a block).  Block q has mass S_q = sum of its members' p_v and race
 * key ln S_q + G_q with G_q = -ln(-ln u(seed,row,pos, 2q)), a Gumbel variate of the counter hash: the block
 * with the largest key wins (ties to the lower block), i.e. a Gumbel-max over blocks.  Inside the winner the
 * id is the first member (ascending id) whose inclusive prefix mass exceeds u(seed,row,pos, 2q+1) S_q.  The
 * arg-max of ln S_q + G_q is block q with probability S_q / sum S (Gumbel-max), and the inverse CDF then takes
 * v with probability p_v / S_q: the draw is exactly softmax(l/T) over the set.
 * Log-probability: l/T - LSE at the pick, LSE = M + ln sum_q S_q (greedy: T = 1) ([Tut] "Why the
 * normalization has to be local": the exact probability of the drawn token).
 *
 * Margin (north star's "top-2 margin"; every term moves by at most 2 eps when each key l (greedy) or log-mass
 * l/T (sampling) moves by at most eps): greedy, the gap between the two largest l; sampling, the smallest of
 * the race gap between the two largest block keys and, inside the winner, the log-ratio margins of the two
 * inverse-CDF comparisons: with A the mass before the drawn id, m its mass, C the mass after it and u the
 * target uniform, ln(u (m + C)) - ln((1 - u) A) for "A <= u S" (A > 0) and ln((1 - u)(A + m)) - ln(u C) for
 * "u S < A + m" (C > 0).
 *
 * Reachability of a given id f (the GPU's token, to be checked where it differs from the oracle's): f is
 * reachable when some perturbation of every key / log-mass by at most eps makes the pick f.  Greedy:
 * l_f >= max l - 2 eps.  Sampling: f's block could win the race (its key within 2 eps of the best other
 * block's) and f's interval could hold the target: with A, m, C as above for f, the comparisons
 * (1 - u) A' <= u (m' + C') and u C' < (1 - u)(A' + m') must hold together for some A' in [A e^-eps, A e^eps],
 * C' in [C e^-eps, C e^eps], m' = m e^eps (both are conditions on z = (1 - u) A' - u C', which sweeps an
 * interval).  The two levels are tested separately, which can only widen the accepted set. */
typedef struct {
    int32_t id;
    int slot;
} id_slot;

static int by_id(const void* x, const void* y) {
    const int32_t a = ((const id_slot*)x)->id, b = ((const id_slot*)y)->id;
    return (a > b) - (a < b);
}

/* Slots of the set in ascending id order (ids == NULL: the identity). */
static int* id_order(const int32_t* ids, int n) {
    int* ord = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    if (!ids) {
        for (int s = 0; s < n; ++s) ord[s] = s;
        return ord;
    }
    id_slot* t = (id_slot*)malloc(sizeof(id_slot) * (size_t)(n > 0 ? n : 1));
    for (int s = 0; s < n; ++s) {
        t[s].id = ids[s];
        t[s].slot = s;
    }
    qsort(t, (size_t)n, sizeof(id_slot), by_id);
    for (int s = 0; s < n; ++s) ord[s] = t[s].slot;
    free(t);
    return ord;
}

#define ID_OF(s) (ids ? ids[(s)] : (s))

/* Vocabulary block of an id in the sampling race: aligned blocks of 16 ids. */
static int block_of(int32_t id) { return id / 16; }

/* Result of one pick; reach is set only when a follow id is given (follow_id >= 0). */
typedef struct {
    int slot;          /* slot picked */
    double margin;
    double logprob;    /* log softmax at the pick */
    double lse;
    double lp_follow;  /* log softmax at the follow id (NaN if it is not in the set) */
    int reach;         /* the follow id is the pick or reachable */
} pick_out;

static void choose(const double* l, const int32_t* ids, int n, int mode, uint64_t seed, int row, int pos, double T,
                   int follow_id, double eps, pick_out* out) {
    int* ord = id_order(ids, n);
    const double Teff = (mode == OR_SAMPLE) ? T : 1.0;
    double M = -INFINITY;
    for (int s = 0; s < n; ++s)
        if (l[s] / Teff > M) M = l[s] / Teff;
    /* the follow id's slot, if it is a member */
    int fslot = -1;
    for (int s = 0; s < n && follow_id >= 0; ++s)
        if (ID_OF(s) == follow_id) fslot = s;
    out->reach = 0;
    out->lp_follow = NAN;
    if (mode != OR_SAMPLE) {
        int best = -1;
        double k1 = -INFINITY, k2 = -INFINITY, total = 0.0;
        for (int i = 0; i < n; ++i) {
            const int s = ord[i];
            total += exp(l[s] - M);
            if (best < 0 || l[s] > k1) { /* ascending ids: an equal key keeps the lower id */
                if (best >= 0) k2 = k1;
                k1 = l[s];
                best = s;
            } else if (l[s] > k2) {
                k2 = l[s];
            }
        }
        out->slot = best;
        out->margin = k1 - k2;
        out->lse = M + log(total);
        out->logprob = l[best] - out->lse;
        if (fslot >= 0) {
            out->lp_follow = l[fslot] - out->lse;
            out->reach = (fslot == best) || (l[fslot] >= k1 - 2.0 * eps);
        }
        free(ord);
        return;
    }
    /* sampling: blocks are runs of equal id / 16 in id order */
    double total = 0.0, k1 = -INFINITY, k2 = -INFINITY;
    int J = -1;     /* winning block */
    int Jbeg = 0, Jend = 0;
    double SJ = 0.0;
    double kf = -INFINITY, kf_other = -INFINITY; /* the follow id's block key, and the best key of other blocks */
    int fq = fslot >= 0 ? block_of(ID_OF(fslot)) : -1;
    for (int i0 = 0; i0 < n;) {
        const int q = block_of(ID_OF(ord[i0]));
        int i1 = i0;
        double S = 0.0;
        while (i1 < n && block_of(ID_OF(ord[i1])) == q) S += exp(l[ord[i1++]] / T - M);
        total += S;
        if (S > 0.0) {
            const double key = log(S) + oracle_gumbel(seed, (uint32_t)row, (uint32_t)pos, (uint32_t)(2 * q));
            if (J < 0 || key > k1) {
                k2 = k1;
                k1 = key;
                J = q;
                Jbeg = i0;
                Jend = i1;
                SJ = S;
            } else if (key > k2) {
                k2 = key;
            }
            if (q == fq) kf = key;
            else if (key > kf_other) kf_other = key;
        }
        i0 = i1;
    }
    /* inverse CDF inside the winner, ascending ids */
    const double u = oracle_noise_uniform(seed, (uint32_t)row, (uint32_t)pos, (uint32_t)(2 * J + 1));
    const double target = u * SJ;
    int tok = -1;
    double cum = 0.0, A = 0.0, m = 0.0;
    for (int i = Jbeg; i < Jend && tok < 0; ++i) {
        const double pv = exp(l[ord[i]] / T - M);
        if (cum + pv > target && pv > 0.0) {
            tok = ord[i];
            A = cum;
            m = pv;
        }
        cum += pv;
    }
    if (tok < 0) /* only if rounding put the target at the block's mass: the last member with mass */
        for (int i = Jend - 1; i >= Jbeg && tok < 0; --i)
            if (exp(l[ord[i]] / T - M) > 0.0) {
                tok = ord[i];
                m = exp(l[ord[i]] / T - M);
                A = SJ - m;
            }
    const double C = SJ - A - m > 0.0 ? SJ - A - m : 0.0;
    double margin = (k2 > -INFINITY) ? k1 - k2 : INFINITY;
    if (A > 0.0) {
        const double d = log(u * (m + C)) - log((1.0 - u) * A);
        if (d < margin) margin = d;
    }
    if (C > 0.0) {
        const double d = log((1.0 - u) * (A + m)) - log(u * C);
        if (d < margin) margin = d;
    }
    out->slot = tok;
    out->margin = margin;
    out->lse = M + log(total);
    out->logprob = l[tok] / T - out->lse;
    if (fslot >= 0) {
        out->lp_follow = l[fslot] / T - out->lse;
        if (fslot == tok) {
            out->reach = 1;
        } else {
            /* f's block against the others */
            int race_ok = (kf > -INFINITY) && (kf_other == -INFINITY || kf >= kf_other - 2.0 * eps);
            /* f inside its block */
            double Af = 0.0, mf = 0.0, Cf = 0.0;
            int seen = 0;
            for (int i = 0; i < n; ++i) {
                const int s = ord[i];
                if (block_of(ID_OF(s)) != fq) continue;
                const double pv = exp(l[s] / T - M);
                if (s == fslot) {
                    mf = pv;
                    seen = 1;
                } else if (!seen) {
                    Af += pv;
                } else {
                    Cf += pv;
                }
            }
            const double uf = oracle_noise_uniform(seed, (uint32_t)row, (uint32_t)pos, (uint32_t)(2 * fq + 1));
            const double ep = exp(eps), em = exp(-eps), m1 = mf * ep;
            const double zmin = (1.0 - uf) * Af * em - uf * Cf * ep;
            const double zmax = (1.0 - uf) * Af * ep - uf * Cf * em;
            const int in_ok = mf > 0.0 && zmin <= uf * m1 && zmax > -(1.0 - uf) * m1;
            out->reach = race_ok && in_ok;
        }
    }
    free(ord);
}

#undef ID_OF

/* ------------------------------------------------------------------------------------------ */
/* O-M: full-vocabulary Markov head, K serial positions                                         */
/* ------------------------------------------------------------------------------------------ */

/* [DSp] "Semi-autoregressive generation" / "The Markov head", [Tut] "Fix 1": for k = 0..K-1 the bias
 * W1[prev]^T W2 is added to U_k and a token is picked over the full vocabulary; the token becomes the
 * predecessor of position k+1.  Position 0's predecessor is the anchor.
 *
 * U: [B, K, V] fp32.  W1: [V, r].  W2: [r, V] or [V, r] (layout).  anchor: [B].
 * H: [B, K, r] gate values or NULL.  follow: [B, K] or NULL -- when given, the predecessor of position
 * k > 0 is follow[b, k-1] instead of the oracle's own pick (teacher forcing along a given path).
 * rows: list of nrows row ids to compute (NULL: all B rows).
 * Outputs at [b*K + k]: tokens, logprobs (log softmax at the pick), margins (see choose()), lp_follow (log
 * softmax at follow[b,k], or NULL), best_logit (l at the pick, or NULL), reach (follow[b,k] is the pick or
 * reachable by a perturbation of at most eps, see choose(); or NULL). */
void oracle_markov_draft(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout,
                         const int32_t* anchor, const double* H, int B, int K, int V, int r, int mode,
                         uint64_t seed, double temperature, const int32_t* follow, const int32_t* rows,
                         int nrows, int32_t* tokens, double* logprobs, double* margins, double* lp_follow,
                         double* best_logit, int32_t* reach, double eps) {
    int n = rows ? nrows : B;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ri = 0; ri < n; ++ri) {
        int b = rows ? rows[ri] : ri;
        double* l = (double*)malloc(sizeof(double) * (size_t)V);
        double* x = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
        int prev = anchor[b];
        for (int k = 0; k < K; ++k) {
            const float* Uk = U + ((size_t)b * K + k) * (size_t)V;
            const double* Hk = H ? H + ((size_t)b * K + k) * (size_t)r : NULL;
            predecessor_embedding(W1, wdtype, r, prev, Hk, x);
            for (int v = 0; v < V; ++v) l[v] = calibrated_logit(Uk, W2, wdtype, w2_layout, V, r, x, v);
            size_t o = (size_t)b * K + k;
            pick_out p;
            choose(l, NULL, V, mode, seed, b, k, temperature, follow ? follow[o] : -1, eps, &p);
            tokens[o] = p.slot;
            if (logprobs) logprobs[o] = p.logprob;
            if (margins) margins[o] = p.margin;
            if (best_logit) best_logit[o] = l[p.slot];
            if (follow) {
                if (lp_follow) lp_follow[o] = p.lp_follow;
                if (reach) reach[o] = p.reach;
                prev = (follow[o] >= 0 && follow[o] < V) ? follow[o] : p.slot;
            } else {
                prev = p.slot;
            }
        }
        free(l);
        free(x);
    }
}

/* Calibrated logits of one position for every row, given each row's predecessor:
 * out[b, v] = U_k[b, v] + sum_j x_b[j] W2[j, v] with x_b = W1[prev[b]] (.) H_k[b].
 * Uk rows are u_stride floats apart; H_k is [B, r] or NULL.  rows/nrows select rows (NULL: all);
 * out is indexed [b*V + v]. */
void oracle_markov_logits(const float* Uk, int64_t u_stride, const void* W1, const void* W2, int wdtype,
                          int w2_layout, const int32_t* prev, const double* Hk, int B, int V, int r,
                          const int32_t* rows, int nrows, double* out) {
    int n = rows ? nrows : B;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ri = 0; ri < n; ++ri) {
        int b = rows ? rows[ri] : ri;
        double* x = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
        predecessor_embedding(W1, wdtype, r, prev[b], Hk ? Hk + (size_t)b * r : NULL, x);
        for (int v = 0; v < V; ++v)
            out[(size_t)b * V + v] = calibrated_logit(Uk + (size_t)b * u_stride, W2, wdtype, w2_layout, V, r, x, v);
        free(x);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* O-T: top-k candidates of the base logits                                                     */
/* ------------------------------------------------------------------------------------------ */

/* "a before b" in the candidate order: larger value first, equal values (including -0 == +0) by the
 * lower vocabulary id. */
static int ranks_before(float va, int ia, float vb, int ib) {
    if (va > vb) return 1;
    if (va < vb) return 0;
    return ia < ib;
}

/* First k ids of one row of base logits u[0..V) in the order (value desc, id asc).  One ascending
 * scan keeps the first k of that order seen so far (insertion into a sorted list of length k), which
 * yields exactly the first k of the full sort. */
static void topk_row(const float* u, int V, int k, int32_t* id, float* vv) {
    int have = 0;
    for (int v = 0; v < V; ++v) {
        float x = u[v];
        if (have == k && !ranks_before(x, v, vv[k - 1], id[k - 1])) continue;
        int pos = (have < k) ? have : k - 1;
        while (pos > 0 && ranks_before(x, v, vv[pos - 1], id[pos - 1])) {
            vv[pos] = vv[pos - 1];
            id[pos] = id[pos - 1];
            --pos;
        }
        vv[pos] = x;
        id[pos] = v;
        if (have < k) ++have;
    }
}

/* [MvS] "Where the parallelism comes from": at each position keep the top-k tokens under the base
 * logits.  Definition: sort all V ids by (U desc, id asc) and keep the first k.
 * U: [rows, V] with rows u_stride floats apart.  idx: [rows, k]; val: [rows, k] or NULL.
 * Requires 1 <= k <= V. */
void oracle_topk(const float* U, int64_t u_stride, int rows, int V, int k, int32_t* idx, float* val) {
#pragma omp parallel for schedule(dynamic, 4)
    for (int row = 0; row < rows; ++row) {
        float* vv = (float*)malloc(sizeof(float) * (size_t)k);
        topk_row(U + (size_t)row * u_stride, V, k, idx + (size_t)row * k, vv);
        if (val)
            for (int s = 0; s < k; ++s) val[(size_t)row * k + s] = vv[s];
        free(vv);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* O-R: the Markov head restricted to given candidate sets                                       */
/* ------------------------------------------------------------------------------------------ */

/* The plain definition of what the truncated execution computes: O-M with the vocabulary at position
 * k replaced by the candidate set cand[b, k, 0..topk).  Pick, margin and log-softmax range over that
 * set (choose(), ascending ids).  Same argument meaning as oracle_markov_draft; cand is [B, K, topk].  A
 * follow id that is not a candidate gets lp_follow = NaN and reach = 0 (its predecessor role still holds). */
void oracle_markov_restricted(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout,
                              const int32_t* anchor, const double* H, const int32_t* cand, int B, int K,
                              int V, int r, int topk, int mode, uint64_t seed, double temperature,
                              const int32_t* follow, const int32_t* rows, int nrows, int32_t* tokens,
                              double* logprobs, double* margins, double* lp_follow, int32_t* reach, double eps) {
    int n = rows ? nrows : B;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ri = 0; ri < n; ++ri) {
        int b = rows ? rows[ri] : ri;
        double* l = (double*)malloc(sizeof(double) * (size_t)topk);
        double* x = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
        int prev = anchor[b];
        for (int k = 0; k < K; ++k) {
            const float* Uk = U + ((size_t)b * K + k) * (size_t)V;
            const double* Hk = H ? H + ((size_t)b * K + k) * (size_t)r : NULL;
            const int32_t* c = cand + ((size_t)b * K + k) * (size_t)topk;
            predecessor_embedding(W1, wdtype, r, prev, Hk, x);
            for (int s = 0; s < topk; ++s) l[s] = calibrated_logit(Uk, W2, wdtype, w2_layout, V, r, x, c[s]);
            size_t o = (size_t)b * K + k;
            pick_out p;
            choose(l, c, topk, mode, seed, b, k, temperature, follow ? follow[o] : -1, eps, &p);
            tokens[o] = c[p.slot];
            if (logprobs) logprobs[o] = p.logprob;
            if (margins) margins[o] = p.margin;
            if (follow) {
                if (lp_follow) lp_follow[o] = p.lp_follow;
                if (reach) reach[o] = p.reach;
                prev = (follow[o] >= 0 && follow[o] < V) ? follow[o] : c[p.slot];
            } else {
                prev = c[p.slot];
            }
        }
        free(l);
        free(x);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* O-S: the Selector, step by step                                                              */
/* ------------------------------------------------------------------------------------------ */

/* [MvS] "Where the parallelism comes from", in its order:
 *  1. fix the candidate sets: top-k of U at every position (O-T);
 *  2. precompute every calibration inside those sets: the anchor row
 *       T0[j]      = U_0(c_0j)  + < A[anchor] (.) H_0, Bemb[c_0j] >
 *     and for t = 1..K-1 the k x k table of predecessor i, candidate j
 *       T_t[i][j]  = U_t(c_tj) + < A[c_{t-1,i}] (.) H_t, Bemb[c_tj] >
 *     ([MvS] "What the two methods do": S_t(a,b) = U_t(b) + <A(a) (.) H(h_t), B(b)>);
 *  3. walk: pick over the anchor row, then over row i_{t-1} of each table (choose(): greedy, or the
 *     block race over the candidates, its noise keyed on vocabulary blocks, never on candidate slots).
 * A, Bemb: [V, r].  H: [B, K, r] or NULL.  cand_out: [B, K, topk] or NULL.
 * tables_out: [B, topk + (K-1)*topk*topk] (anchor row, then the tables) or NULL.
 * logprobs: log softmax of the walked row's scores/T at the pick. */
void oracle_selector_draft(const float* U, const void* A, const void* Bemb, int wdtype, const int32_t* anchor,
                           const double* H, int B, int K, int V, int r, int topk, int mode, uint64_t seed,
                           double temperature, const int32_t* rows, int nrows, int32_t* tokens,
                           double* logprobs, double* margins, int32_t* cand_out, double* tables_out) {
    int n = rows ? nrows : B;
    size_t tstride = (size_t)topk + (size_t)(K > 0 ? K - 1 : 0) * topk * topk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ri = 0; ri < n; ++ri) {
        int b = rows ? rows[ri] : ri;
        int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)K * topk);
        double* tab = (double*)malloc(sizeof(double) * tstride);
        double* row = (double*)malloc(sizeof(double) * (size_t)topk);
        /* 1. candidate sets */
        float* cval = (float*)malloc(sizeof(float) * (size_t)topk);
        for (int t = 0; t < K; ++t)
            topk_row(U + ((size_t)b * K + t) * (size_t)V, V, topk, cand + (size_t)t * topk, cval);
        free(cval);
        /* 2. all pair scores */
        for (int t = 0; t < K; ++t) {
            const float* Ut = U + ((size_t)b * K + t) * (size_t)V;
            const double* Ht = H ? H + ((size_t)b * K + t) * (size_t)r : NULL;
            int npred = (t == 0) ? 1 : topk;
            for (int i = 0; i < npred; ++i) {
                int a = (t == 0) ? anchor[b] : cand[(size_t)(t - 1) * topk + i];
                for (int j = 0; j < topk; ++j) {
                    int c = cand[(size_t)t * topk + j];
                    double dot = 0.0;
                    for (int q = 0; q < r; ++q) {
                        double ag = weight_at(A, wdtype, (size_t)a * r + q);
                        if (Ht) ag = ag * Ht[q];
                        dot += ag * weight_at(Bemb, wdtype, (size_t)c * r + q);
                    }
                    size_t o = (t == 0) ? (size_t)j : (size_t)topk + ((size_t)(t - 1) * topk + i) * topk + j;
                    tab[o] = (double)Ut[c] + dot;
                }
            }
        }
        /* 3. the walk */
        int islot = 0;
        for (int t = 0; t < K; ++t) {
            const double* src = (t == 0) ? tab : tab + topk + ((size_t)(t - 1) * topk + islot) * topk;
            for (int j = 0; j < topk; ++j) row[j] = src[j];
            pick_out p;
            choose(row, cand + (size_t)t * topk, topk, mode, seed, b, t, temperature, -1, 0.0, &p);
            islot = p.slot;
            size_t o = (size_t)b * K + t;
            tokens[o] = cand[(size_t)t * topk + islot];
            if (logprobs) logprobs[o] = p.logprob;
            if (margins) margins[o] = p.margin;
        }
        if (cand_out) memcpy(cand_out + (size_t)b * K * topk, cand, sizeof(int32_t) * (size_t)K * topk);
        if (tables_out) memcpy(tables_out + (size_t)b * tstride, tab, sizeof(double) * tstride);
        free(cand);
        free(tab);
        free(row);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* O-B: brute-force enumeration of every path of one row                                        */
/* ------------------------------------------------------------------------------------------ */

/* log q(path) = sum_k [ l_k(t_k | t_{k-1}) / T - LSE_k(t_{k-1}) ] with t_{-1} = anchor, for all V^K
 * paths (path index = sum_k t_k V^(K-1-k)).  [Tut] "Fix 1": the draft distribution is the product of
 * K locally normalised first-order factors.  U: [K, V] (one row), H: [K, r] or NULL.
 * Returns -1 (and computes nothing) unless V <= 64 and V^K <= 2^20. */
int oracle_enumerate_paths(const float* U, const void* W1, const void* W2, int wdtype, int w2_layout,
                           int32_t anchor, const double* H, int K, int V, int r, double temperature,
                           double* logq) {
    if (V <= 0 || V > 64 || K <= 0 || K > 32) return -1;
    double count = pow((double)V, (double)K);
    if (count > 1048576.0) return -1;
    long np = (long)count;
    /* log_cond[k][a][v] = log softmax over v of l_k(v | a)/T, for every predecessor a
     * (position 0 only needs a = anchor). */
    double* lc = (double*)malloc(sizeof(double) * (size_t)K * V * V);
    double* l = (double*)malloc(sizeof(double) * (size_t)V);
    double* x = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
    for (int k = 0; k < K; ++k) {
        for (int a = 0; a < V; ++a) {
            int pred = (k == 0) ? anchor : a;
            predecessor_embedding(W1, wdtype, r, pred, H ? H + (size_t)k * r : NULL, x);
            double M = -INFINITY;
            for (int v = 0; v < V; ++v) {
                l[v] = calibrated_logit(U + (size_t)k * V, W2, wdtype, w2_layout, V, r, x, v) / temperature;
                if (l[v] > M) M = l[v];
            }
            double sum = 0.0;
            for (int v = 0; v < V; ++v) sum += exp(l[v] - M);
            double lse = M + log(sum);
            for (int v = 0; v < V; ++v) lc[((size_t)k * V + a) * V + v] = l[v] - lse;
        }
    }
    for (long p = 0; p < np; ++p) {
        long rem = p;
        int path[32];
        for (int k = K - 1; k >= 0; --k) {
            path[k] = (int)(rem % V);
            rem /= V;
        }
        double s = 0.0;
        for (int k = 0; k < K; ++k) {
            int a = (k == 0) ? 0 : path[k - 1]; /* row index into lc; position 0 was built from the anchor */
            s += lc[((size_t)k * V + a) * V + path[k]];
        }
        logq[p] = s;
    }
    free(lc);
    free(l);
    free(x);
    return 0;
}

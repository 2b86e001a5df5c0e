/*
 * synth.c -- seeded synthetic inputs for the draft-calibration workloads.
 *
 * This module holds no arithmetic of the method itself: it only turns (seed, tensor tag, flat index)
 * into numbers.  Both the GPU tests/bench and the CPU oracle consume its output; neither side's
 * computation lives here.
 *
 * Counter streams: value i of stream (seed, tag) is the i-th output of SplitMix64 (G. Steele, D. Lea,
 * C. Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014) started from the state
 * seed ^ (tag << 56): state_i = state_0 + (i + 1) * 0x9E3779B97F4A7C15, then the output mix.
 * Uniforms take the top 53 bits.  Normal i uses uniforms 2i and 2i+1 through the cosine branch of the
 * Box-Muller transform in double precision.  Every value is therefore a pure function of
 * (seed, tag, index), independent of thread count and chunking.
 *
 * Roundings: double -> fp32 by the C conversion (round to nearest even); fp32 -> bf16 by round to
 * nearest even on the bit pattern.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static const double SYNTH_PI = 3.14159265358979323846;

uint64_t synth_splitmix(uint64_t seed, uint32_t tag, uint64_t i) {
    uint64_t z = (seed ^ ((uint64_t)tag << 56)) + (i + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double uniform53(uint64_t x) { return (double)(x >> 11) * (1.0 / 9007199254740992.0); }

double synth_normal(uint64_t seed, uint32_t tag, uint64_t i) {
    double u1 = uniform53(synth_splitmix(seed, tag, 2 * i));
    double u2 = uniform53(synth_splitmix(seed, tag, 2 * i + 1));
    return sqrt(-2.0 * log(1.0 - u1)) * cos(2.0 * SYNTH_PI * u2);
}

uint16_t synth_f32_to_bf16(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return (uint16_t)((b >> 16) | 0x40u);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

/* out[i] = fp32(sigma * z_i), i in [0, n) */
void synth_normal_f32(uint64_t seed, uint32_t tag, int64_t n, double sigma, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(sigma * synth_normal(seed, tag, (uint64_t)i));
}

/* out[i] = bf16(fp32(sigma * z_i)) as raw bits */
void synth_normal_bf16(uint64_t seed, uint32_t tag, int64_t n, double sigma, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = synth_f32_to_bf16((float)(sigma * synth_normal(seed, tag, (uint64_t)i)));
}

/* Base-logit rows: out[row, v] = fp32(scale * z + boost * [v is hot in this row]).  Each row gets
 * n_hot distinct hot ids, drawn as splitmix(seed, tag_hot, row * 4096 + j) mod V for j = 0, 1, ...
 * skipping repeats (n_hot <= min(V, 256)).  z comes from stream tag_z at flat index row * V + v. */
void synth_logits(uint64_t seed, uint32_t tag_z, uint32_t tag_hot, int64_t rows, int V, int n_hot, double scale,
                  double boost, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        int hot[256];
        int have = 0;
        for (uint64_t j = 0; have < n_hot && j < 4096; ++j) {
            int v = (int)(synth_splitmix(seed, tag_hot, (uint64_t)row * 4096u + j) % (uint64_t)V);
            int dup = 0;
            for (int q = 0; q < have; ++q) dup |= (hot[q] == v);
            if (!dup) hot[have++] = v;
        }
        float* o = out + row * (int64_t)V;
        for (int v = 0; v < V; ++v) {
            double z = synth_normal(seed, tag_z, (uint64_t)(row * (int64_t)V + v));
            double isHot = 0.0;
            for (int q = 0; q < have; ++q) isHot += (hot[q] == v) ? 1.0 : 0.0;
            o[v] = (float)(scale * z + boost * isHot);
        }
    }
}

/* out[i] = splitmix(seed, tag, i) mod V */
void synth_tokens(uint64_t seed, uint32_t tag, int64_t n, int V, int32_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)(synth_splitmix(seed, tag, (uint64_t)i) % (uint64_t)V);
}

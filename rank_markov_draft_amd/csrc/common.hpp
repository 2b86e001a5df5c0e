// common.hpp -- device helpers shared by the libdspark kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Streaming 16-byte loads (non-temporal hint: read once, do not keep in the caches).
__device__ __forceinline__ u32x4_t load_nt_u32x4(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ f32x4_t load_nt_f32x4(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMinFinite = -3.402823466e38f;

// MurmurHash3 32-bit finalisation mix (A. Appleby, public domain).
__host__ __device__ __forceinline__ uint32_t fmix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    h *= 0xC2B2AE35u;
    h ^= h >> 16;
    return h;
}

// Seed part of the noise key chain: fmix(lo32(seed) ^ fmix(hi32(seed))).
__host__ __device__ __forceinline__ uint32_t noise_key0(uint64_t seed) {
    return fmix32((uint32_t)(seed & 0xFFFFFFFFull) ^ fmix32((uint32_t)(seed >> 32)));
}

// Row/position part: fmix(fmix(k0 ^ b) ^ k).
__device__ __forceinline__ uint32_t noise_key2(uint32_t k0, uint32_t b, uint32_t k) {
    return fmix32(fmix32(k0 ^ b) ^ k);
}

// Uniform u = (2 (h >> 9) + 1) / 2^24 of hash h, in (0, 1).  Formed exactly: 1 + m 2^-23 (m = h >> 9) minus
// (1 - 2^-24) has no rounding error.
__device__ __forceinline__ float hash_uniform(uint32_t h) {
    return __uint_as_float((h >> 9) | 0x3F800000u) - 0.99999994039535522f;
}

// -log2 u > 0 for that uniform.  Close to u = 1 the hardware log2 is replaced by the series
// -ln(1 - w) = w + w^2/2 + w^3/3 + w^4/4 with w = 1 - u (exact), whose truncation error is below 2^-26
// relative for w < 2^-7.
__device__ __forceinline__ float neg_log2_uniform(uint32_t h) {
    const uint32_t m = h >> 9;
    const float u = __uint_as_float(m | 0x3F800000u) - 0.99999994039535522f;
    const float w = (float)(2u * (0x7FFFFFu - m) + 1u) * 5.9604644775390625e-8f;  // 1 - u, exact
    const float series = w * (1.0f + w * (0.5f + w * (0.33333334f + w * 0.25f))) * kLog2e;
    return (w < 0.0078125f) ? series : -__builtin_amdgcn_logf(u);
}

// -log2(-ln u) + log2(ln 2) = -log2(-log2 u), i.e. the Gumbel variate G(u) = -ln(-ln u) times log2(e) up to
// the constant -log2(ln 2), for the uniform of hash h.  Only differences of this value enter an argmax, so
// the constant is dropped.  (Gumbel-max over a restricted candidate set.)
__device__ __forceinline__ float gumbel_log2_units(uint32_t h) { return -__builtin_amdgcn_logf(neg_log2_uniform(h)); }

// Whole-vocabulary draw, block q (ids 16 q .. 16 q + 15) of a two-level exponential race: its race variate
// E = -log2 u(2 q) and its inverse-CDF target u(2 q + 1) sb for block mass sb > 0, kept strictly below sb;
// u(n) is the uniform of fmix32(k2 ^ n).  The block with the largest sb / E wins; inside it the drawn id is
// the first whose inclusive prefix mass (slot order) exceeds the target.
__device__ __forceinline__ void block_race_variates(uint32_t k2, uint32_t q, float sb, float& E, float& target) {
    E = neg_log2_uniform(fmix32(k2 ^ (2u * q)));
    const float u2 = hash_uniform(fmix32(k2 ^ (2u * q + 1u)));
    target = fminf(u2 * sb, __uint_as_float(__float_as_uint(sb) - 1u));
}

// Row rho of a staged 32-row W2 tile (vocabulary id v0 + rho) goes to LDS slot w2_slot(rho).  A 32x32x16 MFMA's
// A-operand row m (read by lanes m and m + 32) produces accumulator rows 8 (i / 4) + 4 (lane / 32) + i % 4, so
// with this order accumulator i of a lane holds id v0 + 16 (lane / 32) + i: 16 consecutive ids per lane.
__device__ __forceinline__ int w2_slot(int rho) { return 8 * ((rho & 15) >> 2) + 4 * (rho >> 4) + (rho & 3); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// (key, id) order: larger key first, equal keys by the lower vocabulary id.
__device__ __forceinline__ bool beats(float ka, int ia, float kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

// Merge of two streaming log-sum-exp states (m, s) in base 2: s * 2^m summarises sum 2^t.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
    float mn = fmaxf(m, m2);
    s = s * fast_exp2(m - mn) + s2 * fast_exp2(m2 - mn);
    m = mn;
}

// Per-(row, workgroup) partial result of one position's pick, structure of arrays, each [G][Bpad].
struct Partials {
    float* key;  // best key
    int* idx;    // its vocabulary id
    float* l;    // its calibrated logit
    float* m;    // base-2 running max of l * c
    float* s;    // sum of 2^(l * c - m)
};

}  // namespace dspark

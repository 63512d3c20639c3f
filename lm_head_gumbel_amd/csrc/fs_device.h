// Device helpers of libfs: Philox-4x32-10, the Gumbel transform, packed
// argmax keys, and the bf16 MFMA operand types for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum NoiseStream : uint32_t {
    kStreamToken = 0,        // per-id Gumbel noise
    kStreamGroup = 1,        // per-group Gumbel of the hierarchical resample
    kStreamMerge = 2,        // Bernoulli uniforms of the online merge
    kStreamMultinomial = 3,  // inverse-CDF uniform of the unfused baseline
};

// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11, section 3): ten rounds
// of two 32x32->64-bit products; between rounds the key advances by the Weyl
// constants.  Each 64-bit product is one v_mad_u64_u32 on CDNA.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1,
                       (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0);
    }
    return c;
}

// Standard Gumbel from one 32-bit word, in FP32.  With v = (r + 1/2) 2^-32 and
// u = 1 - v, g = -log(-log u).  The exponential variate e = -log u is formed
// without subtracting nearly equal numbers: for r >= 2^31, u itself comes
// from the complement word (~r + 1/2) 2^-32 and e = -log u; for r < 2^31,
// e = -log1p(-v), as the series v + v^2/2 + v^3/3 + v^4/4 for v < 2^-8
// (truncation below 2^-24 relative) and as -log(1 - v) above (1 - v is then
// rounded by at most 2^-17 relative to e).  Both logarithms use the hardware
// base-2 logarithm (normal inputs only: e and u are at least 2^-33), without
// branches.  |g - exact g| stays within about 1e-5 for every word (measured
// 7.9e-6 over 2.5e7 words).
__device__ __forceinline__ float gumbel_from_word(uint32_t r) {
    constexpr float kLn2 = 0.693147180559945309f;
    const bool low = r < 0x80000000u;
    const float v = fmaf((float)(low ? r : ~r), 0x1p-32f, 0x1p-33f);   // v, or u itself
    const float arg = low ? 1.f - v : v;
    float e = -__builtin_amdgcn_logf(arg) * kLn2;
    const float series = v * fmaf(v, fmaf(v, fmaf(v, 0.25f, 1.f / 3.f), 0.5f), 1.f);
    e = (low && v < 0x1p-8f) ? series : e;
    return -__builtin_amdgcn_logf(e) * kLn2;
}

// Where a call's noise comes from: the Philox key (the call's seed) and the
// decode step, or, when given, one seed per batch row (seeds[b]) and a step
// read from device memory at run time (calls that a graph can replay).
struct NoiseSrc {
    uint32_t k0, k1, step;
    const uint64_t* seeds;      // [B] or null
    const uint32_t* step_ptr;   // or null
};
struct RowKey {
    uint32_t k0, k1, step;
};
__device__ __forceinline__ RowKey row_key(const NoiseSrc& n, int b) {
    RowKey r{n.k0, n.k1, n.step};
    if (n.seeds) {
        const uint64_t s = n.seeds[b];
        r.k0 = (uint32_t)s;
        r.k1 = (uint32_t)(s >> 32);
    }
    if (n.step_ptr) r.step = *n.step_ptr;
    return r;
}

// Uniform on (0, 1) from one word: (r + 1/2) 2^-32, rounded to FP32.
__device__ __forceinline__ float uniform_from_word(uint32_t r) {
    return fmaf((float)r, 0x1p-32f, 0x1p-33f);
}

// Order-preserving map float -> uint32 (larger float, larger key).
__device__ __forceinline__ uint32_t float_to_ordered(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ordered_to_float(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Packed (score, index) key: the maximum key holds the largest score and,
// among equal scores, the lowest index.  Index -1 packs to the low word 0.
__device__ __forceinline__ uint64_t pack_key(float s, int32_t idx) {
    return ((uint64_t)float_to_ordered(s) << 32) | (uint32_t)(~(uint32_t)idx);
}
__device__ __forceinline__ float key_score(uint64_t k) { return ordered_to_float((uint32_t)(k >> 32)); }
__device__ __forceinline__ int32_t key_index(uint64_t k) { return (int32_t)(~(uint32_t)k); }

__device__ __forceinline__ uint64_t key_max(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
    const uint32_t lo = __shfl_xor((uint32_t)v, mask, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), mask, 64);
    return ((uint64_t)hi << 32) | lo;
}

// Online log-sum-exp state: value = mx + log(sm).
struct Lse {
    float mx, sm;
};
__device__ __forceinline__ Lse lse_empty() { return Lse{-INFINITY, 0.f}; }
__device__ __forceinline__ Lse lse_add(Lse a, float x) {
    // Without branches, one exponential for both cases: exp(-|x - mx|) is
    // exp(mx - x) when x is the new maximum and exp(x - mx) otherwise (0 when
    // a is empty).  A masked x (-inf) leaves a as it is.
    const bool ok = x > -INFINITY;
    const float dlt = x - a.mx;
    const float e = __expf(-fabsf(dlt));
    const bool up = dlt > 0.f;
    const float sm = up ? a.sm * e + 1.f : a.sm + e;
    a.sm = ok ? sm : a.sm;
    a.mx = ok && up ? x : a.mx;
    return a;
}
__device__ __forceinline__ Lse lse_merge(Lse a, Lse b) {
    // Without branches: the larger state's sum plus the smaller one's scaled
    // by exp(-|a.mx - b.mx|); an empty state yields the other one.
    const bool ge = a.mx >= b.mx;
    const float e = __expf(-fabsf(a.mx - b.mx));
    const Lse hi = ge ? a : b, lo = ge ? b : a;
    Lse r{hi.mx, hi.sm + lo.sm * e};
    r = a.mx > -INFINITY ? r : b;
    return b.mx > -INFINITY ? r : a;
}
__device__ __forceinline__ float lse_value(Lse a) {
    return (a.mx > -INFINITY) ? a.mx + __logf(a.sm) : -INFINITY;
}

}  // namespace fs

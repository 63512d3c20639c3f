// Exact top-k selection for the top-k truncation variant ("FlashSampling"
// explainer on aitrends.kr, implementation paragraph: top-k candidates per
// tile, then a global top-k merge).  The candidate set is the k valid ids
// with the largest tempered logit x, ties to the lower id; the sample is the
// largest noisy score s = x + Gumbel among them.
//
// Selection works on the order-preserving 32-bit image of x (masked ids map
// to 0, below every valid value): the k-th largest value t is found bit by
// bit from the top by counting the values >= a candidate threshold with wave
// ballots, then the values > t and the first `need` values == t in id order
// are taken.  Every step is a count, so the result does not depend on timing.
#pragma once

#include "fs_device.h"
#include "fs_epilogue.h"
#include "fs_internal.h"

namespace fs {

__device__ __forceinline__ uint32_t topk_order(float x) {
    return x > -INFINITY ? float_to_ordered(x) : 0u;
}

// Set lanes of a wave-wide predicate (the same value in every lane).
__device__ __forceinline__ int wave_count(bool p) { return __popcll(__ballot(p)); }

// Gumbel noise of global id gid in column c (token stream).
__device__ __forceinline__ float token_gumbel(const Stage1Args& a, int col, int gid) {
    const uint4 w4 =
        philox4x32_10(make_uint4((uint32_t)gid >> 2, (uint32_t)col, a.step, kStreamToken), a.k0,
                      a.k1);
    const int q = gid & 3;
    const uint32_t word = q == 0 ? w4.x : q == 1 ? w4.y : q == 2 ? w4.z : w4.w;
    return gumbel_from_word(word);
}

// One wave: the top-k candidates of rows [0, nr) of one column whose x sit
// in LDS at xcol[row] (row r is global id gid0 + r).  Writes a.topk
// candidates (x, s, id) at offset o of a.cx / a.cs / a.cidx, unused slots as
// (-inf, -inf, -1).  sx / sid: 64 entries of per-wave LDS staging.  NR * 64
// must cover nr.
template <int NR>
__device__ void topk_select_column(const Stage1Args& a, const ColCtx& c, const float* xcol,
                                   int nr, int gid0, size_t o, float* sx, int* sid) {
    const int lane = threadIdx.x & 63;
    const int k = a.topk;
    uint32_t u[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int r = lane + 64 * i;
        u[i] = r < nr ? topk_order(xcol[r]) : 0u;
    }
    auto count_ge = [&](uint32_t t) {
        int n = 0;
#pragma unroll
        for (int i = 0; i < NR; ++i) n += wave_count(u[i] >= t);
        return n;
    };

    // select u > t, plus the first `need` of u == t in row order; with at
    // most k valid values that is every valid one (t = 1 lies below them all)
    uint32_t t = 1;
    int need = 0;
    if (count_ge(1) > k) {
        t = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = t | (1u << bit);
            if (count_ge(cand) >= k) t = cand;
        }
        need = k - count_ge(t + 1);   // t <= image of +inf, so t + 1 does not wrap
    }

    // compact the selected (x, id) into the wave's staging area, in row order
    const uint64_t below = (1ull << lane) - 1ull;
    int nsel = 0, ties = 0;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const bool tie = u[i] == t && need > 0;
        const uint64_t tb = __ballot(tie);
        const bool sel = u[i] > t || (tie && ties + __popcll(tb & below) < need);
        ties += __popcll(tb);
        const uint64_t sb = __ballot(sel);
        if (sel) {
            const int pos = nsel + __popcll(sb & below);
            const int r = lane + 64 * i;
            sx[pos] = xcol[r];
            sid[pos] = gid0 + r;
        }
        nsel += __popcll(sb);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

    // noise for the selected only, one candidate per lane
    if (lane < k) {
        float x = -INFINITY, s = -INFINITY;
        int id = -1;
        if (lane < nsel) {
            x = sx[lane];
            id = sid[lane];
            s = c.greedy ? x : x + token_gumbel(a, c.col, id);
        }
        a.cx[o + lane] = x;
        a.cs[o + lane] = s;
        a.cidx[o + lane] = id;
    }
    __builtin_amdgcn_wave_barrier();
}

}  // namespace fs

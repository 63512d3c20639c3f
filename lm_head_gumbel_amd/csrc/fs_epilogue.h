// Epilogue of the stage-1 kernels, shared by all of them: per-column
// temperature and mask, Philox-Gumbel noise for one MFMA lane's four rows,
// folding into a column's running winner and log-mass, the cross-lane column
// reduction and the record writes ("FlashSampling" explainer on aitrends.kr,
// Stage 1 and tensor-parallel paragraphs).
#pragma once

#include "fs_device.h"
#include "fs_internal.h"

namespace fs {

// Per-column constants of the epilogue.
struct ColCtx {
    int col;
    bool ok;
    bool greedy;
    float inv_t;
    const uint32_t* allow_row;
    RowKey key;   // Philox key and step of the column's batch row
};

__device__ __forceinline__ ColCtx col_ctx(const Stage1Args& a, int col) {
    ColCtx c;
    c.col = col;
    c.ok = col < a.B;
    c.greedy = true;
    c.inv_t = 1.f;
    if (c.ok) {
        const float T = a.temp ? a.temp[col] : 1.f;
        c.greedy = (a.flags & kFlagNoNoise) || !(T > 0.f);
        c.inv_t = c.greedy ? 1.f : 1.f / T;
    }
    c.allow_row = (a.allow && c.ok) ? a.allow + (size_t)col * ((a.V + 31) >> 5) : nullptr;
    c.key = c.ok ? row_key(a.noise, col) : RowKey{a.noise.k0, a.noise.k1, a.noise.step};
    return c;
}

// Column contexts of N consecutive columns kept in LDS.  The LDS-tiled
// kernels rebuild a column's context in every tile's epilogue (held in
// registers through the contraction they would spill); reading the
// temperatures, per-row seeds and the device step from global memory there
// would leave loads whose completion the compiler cannot track across the
// contraction loop, and it then drains every load in flight (a full vmcnt
// wait) once per chunk.  Filled once per workgroup before the loop.
template <int N>
struct ColCtxSmem {
    float inv_t[N];
    uint32_t k0[N], k1[N], step[N];
    uint32_t flags[N];   // bit 0: column < B, bit 1: greedy
};

template <int N>
__device__ __forceinline__ void col_ctx_store(ColCtxSmem<N>& s, const Stage1Args& a, int col0) {
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        const ColCtx c = col_ctx(a, col0 + i);
        s.inv_t[i] = c.inv_t;
        s.k0[i] = c.key.k0;
        s.k1[i] = c.key.k1;
        s.step[i] = c.key.step;
        s.flags[i] = (c.ok ? 1u : 0u) | (c.greedy ? 2u : 0u);
    }
}

template <int N>
__device__ __forceinline__ ColCtx col_ctx_load(const ColCtxSmem<N>& s, const Stage1Args& a,
                                               int col0, int i) {
    ColCtx c;
    c.col = col0 + i;
    const uint32_t f = s.flags[i];
    c.ok = (f & 1u) != 0;
    c.greedy = (f & 2u) != 0;
    c.inv_t = s.inv_t[i];
    c.allow_row = (a.allow && c.ok) ? a.allow + (size_t)c.col * ((a.V + 31) >> 5) : nullptr;
    c.key = RowKey{s.k0[i], s.k1[i], s.step[i]};
    return c;
}

// The allow word of column c that holds rows row0..row0+3 (row0 % 4 == 0, so
// one word holds all four): read only for a masked column and rows inside V;
// all ones otherwise.  One read per fold instead of one per row: each wait
// for it also waits for every load issued before it.
__device__ __forceinline__ uint32_t allow_word(const Stage1Args& a, const ColCtx& c, int row0,
                                               bool blk_ok) {
    // (read through a global pointer: the row pointer may be null, and as a
    // generic pointer its read would be a FLAT load, whose wait also drains
    // every load in flight)
    typedef __attribute__((address_space(1))) const uint32_t global_u32;
    return (c.allow_row && blk_ok && row0 < a.V) ? ((const global_u32*)c.allow_row)[row0 >> 5]
                                                 : ~0u;
}

// Tempered, masked logits x of four consecutive rows row0..row0+3 (local W
// rows) of one column: -inf past V, at or past n_valid, where the allow bit
// (of `word`, from allow_word) is clear, and for NaN.
__device__ __forceinline__ void lane_x(const Stage1Args& a, const ColCtx& c, f32x4 v, int row0,
                                       bool blk_ok, uint32_t word, float (&x)[4]) {
    const int gid0 = a.v_offset + row0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = row0 + r;
        bool ok = blk_ok && c.ok && (i < a.V) && (gid0 + r < a.n_valid);
        if (a.allow) ok = ok && ((word >> (i & 31)) & 1u);   // uniform
        const float xv = v[r] * c.inv_t;
        x[r] = (ok && xv == xv) ? xv : -INFINITY;
    }
}

// x as above and the noisy scores s = x + Gumbel (s = x for greedy columns).
// UKEY: calls with one key (no per-row seeds) take the key from the call, so
// that its schedule of round keys stays on the scalar unit (the per-column
// copy would take vector adds); a kernel whose registers are short keeps the
// per-column key.
template <bool UKEY = false>
__device__ __forceinline__ void lane_scores(const Stage1Args& a, const ColCtx& c, f32x4 v,
                                            int row0, bool blk_ok, uint32_t word, float (&x)[4],
                                            float (&s)[4]) {
    const int gid0 = a.v_offset + row0;
    lane_x(a, c, v, row0, blk_ok, word, x);
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = x[r];
    if (!c.greedy && blk_ok && c.ok) {
        const uint4 ctr = make_uint4((uint32_t)gid0 >> 2, (uint32_t)c.col, c.key.step, kStreamToken);
        uint4 rw;
        if (UKEY && a.noise.seeds == nullptr) {   // uniform
            uint32_t k0 = a.noise.k0, k1 = a.noise.k1;
            asm volatile("" : "+s"(k0), "+s"(k1));
            rw = philox4x32_10(ctr, k0, k1);
        } else {
            rw = philox4x32_10(ctr, c.key.k0, c.key.k1);
        }
        s[0] += gumbel_from_word(rw.x);
        s[1] += gumbel_from_word(rw.y);
        s[2] += gumbel_from_word(rw.z);
        s[3] += gumbel_from_word(rw.w);
    }
}

// The same with the allow word read here.
__device__ __forceinline__ void lane_scores(const Stage1Args& a, const ColCtx& c, f32x4 v,
                                            int row0, bool blk_ok, float (&x)[4],
                                            float (&s)[4]) {
    lane_scores(a, c, v, row0, blk_ok, allow_word(a, c, row0, blk_ok), x, s);
}

// Folds four (x, s) pairs into a column's running winner and log-mass.
template <int VAR>
__device__ __forceinline__ void fold(uint64_t& best, Lse& lse, const float (&x)[4],
                                     const float (&s)[4], int gid0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        // (selects, no branch: a masked row offers the empty key, and
        // lse_add leaves the state as it is for x = -inf)
        const uint64_t k = x[r] > -INFINITY ? pack_key(s[r], gid0 + r) : pack_key(-INFINITY, -1);
        best = key_max(best, k);
        if constexpr (VAR == kVarGrouped) lse = lse_add(lse, x[r]);
    }
}

// Combines the four lanes that share a column (lanes l, l^16, l^32, l^48).
template <int VAR>
__device__ __forceinline__ void column_reduce(uint64_t& best, Lse& lse) {
    best = key_max(best, shfl_xor_u64(best, 16));
    best = key_max(best, shfl_xor_u64(best, 32));
    if constexpr (VAR == kVarGrouped) {
#pragma unroll
        for (int m = 16; m <= 32; m <<= 1)
            lse = lse_merge(lse, Lse{__shfl_xor(lse.mx, m, 64), __shfl_xor(lse.sm, m, 64)});
    }
}

// Writes (or, with MERGE, merges into) the record of column c.col at slot p.
template <int VAR, bool MERGE>
__device__ __forceinline__ void put_record(const Stage1Args& a, int p, const ColCtx& c,
                                           uint64_t best, Lse lse) {
    if (!c.ok) return;
    const size_t o = a.rec_cols ? (size_t)p * a.rec_cols + c.col : (size_t)c.col * a.P + p;
    float L = c.greedy ? lse.mx : lse_value(lse);
    if constexpr (MERGE) {
        const int32_t old_id = a.pidx[o];
        if (old_id >= 0) best = key_max(best, pack_key(a.pm[o], old_id));
        if constexpr (VAR == kVarGrouped) {
            const float Lo = a.pL[o];
            if (c.greedy)
                L = fmaxf(L, Lo);
            else
                L = lse_value(lse_merge(Lse{Lo, 1.f}, Lse{L, 1.f}));
        }
    }
    const int32_t id = key_index(best);
    a.pm[o] = id >= 0 ? key_score(best) : -INFINITY;
    a.pidx[o] = id;
    if constexpr (VAR == kVarGrouped) a.pL[o] = L;
}

}  // namespace fs

// Exact top-k selection for the top-k truncation variant ("FlashSampling"
// explainer on aitrends.kr, implementation paragraph: top-k candidates per
// tile, then a global top-k merge).  The candidate set is the k valid ids
// with the largest tempered logit x, ties to the lower id; the sample is the
// largest noisy score s = x + Gumbel among them, so noise is only needed for
// the row's final k candidates.
//
// Selection works on the order-preserving 32-bit image of x (masked ids map
// to 0, below every valid value): the k-th largest value t is found bit by
// bit from the top by counting the values >= a candidate threshold with wave
// ballots; the values > t are taken, and of the values == t the lowest ids
// (a second bitwise search, only when there are more ties than places).
// Every step is a count, so the result does not depend on timing.
#pragma once

#include "fs_device.h"
#include "fs_epilogue.h"
#include "fs_internal.h"

#include <type_traits>

namespace fs {

// Order image of x for the selection: increasing in x, 0 for -inf (no
// candidate).  (x is never -0: the MFMA sums start from +0, and a sum that
// cancels to zero rounds to +0.)
__device__ __forceinline__ uint32_t topk_order(float x) {
    return x > -INFINITY ? float_to_ordered(x) : 0u;
}

// Set lanes of a wave-wide predicate (the same value in every lane).
__device__ __forceinline__ int wave_count(bool p) { return __popcll(__ballot(p)); }

constexpr int bits_for(int m) { return m < 2 ? 1 : 1 + bits_for(m >> 1); }

// Wave-wide sum of per-lane counts 0 <= c <= M, one ballot per bit of c:
// the per-lane sums run on the vector unit, so only a few vector-to-scalar
// hand-offs remain per count.
template <int M>
__device__ __forceinline__ int wave_sum(int c) {
    int n = 0;
#pragma unroll
    for (int b = 0; b < bits_for(M); ++b) n += __popcll(__ballot((c >> b) & 1)) << b;
    return n;
}

// Gumbel noise of global id gid in batch row b (token stream).
__device__ __forceinline__ float token_gumbel(uint32_t k0, uint32_t k1, uint32_t step, int b,
                                              int gid) {
    const uint4 w4 =
        philox4x32_10(make_uint4((uint32_t)gid >> 2, (uint32_t)b, step, kStreamToken), k0, k1);
    const int q = gid & 3;
    const uint32_t word = q == 0 ? w4.x : q == 1 ? w4.y : q == 2 ? w4.z : w4.w;
    return gumbel_from_word(word);
}

// Lanes where pred(i) holds, summed over a lane's M predicates: each
// predicate is one compare straight into a lane mask and a scalar bit count
// (the M compares are issued before the counts are added).
template <int M, typename P>
__device__ __forceinline__ int wave_count_each(P pred) {
    uint64_t m[M];
#pragma unroll
    for (int i = 0; i < M; ++i) m[i] = __builtin_amdgcn_ballot_w64(pred(i));
    int n = 0;
#pragma unroll
    for (int i = 0; i < M; ++i) n += __popcll(m[i]);
    return n;
}

// The k-th largest of the 64 * M values of each of C sets (M per lane), or
// 0 when a set holds fewer than k nonzero values; bit by bit from the top,
// every count a set of wave ballots.  With LOW > 0 the search stops above
// bit LOW: the result is then the k-th largest value with its low LOW bits
// cleared, still a value that at least k entries reach (a lower bound).  The
// C searches are independent chains of compare, bit count and scalar select;
// their compares are issued together.
template <int C, int M, int LOW = 0>
__device__ __forceinline__ void wave_kth(const uint32_t (&v)[C][M], int k, uint32_t (&t)[C]) {
#pragma unroll
    for (int c = 0; c < C; ++c) t[c] = 0;
    for (int bit = 31; bit >= LOW; --bit) {
        uint32_t cand[C];
        uint64_t m[C][M];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            cand[c] = t[c] | (1u << bit);
#pragma unroll
            for (int i = 0; i < M; ++i) m[c][i] = __builtin_amdgcn_ballot_w64(v[c][i] >= cand[c]);
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            int n = 0;
#pragma unroll
            for (int i = 0; i < M; ++i) n += __popcll(m[c][i]);
            if (n >= k) t[c] = cand[c];
        }
    }
}

// Exact top-k among M entries per lane, for C independent sets at once:
// marks the k largest pairs (u, tb) of each set, compared by u and then by
// tb, among its entries with u > 0 (u == 0: no entry; the pairs of real
// entries are distinct), or all its real entries when there are at most k.
// With tb = ~id the lower id wins a tie in u.
template <int C, int M>
__device__ __forceinline__ void wave_select(const uint32_t (&u)[C][M], const uint32_t (&tb)[C][M],
                                            int k, bool (&sel)[C][M]) {
    // per set: take u > t, and u == t with tb >= tt (t, tt wave-uniform)
    uint32_t t[C], tt[C];
    bool big[C];
    int need[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        big[c] = wave_count_each<M>([&](int i) { return u[c][i] >= 1u; }) > k;
        t[c] = 0;
        tt[c] = 0;
    }
    bool any_big = false;
#pragma unroll
    for (int c = 0; c < C; ++c) any_big = any_big || big[c];
    // (with at most k real entries in every set there is nothing to search)
    for (int bit = 31; any_big && bit >= 0; --bit) {
        uint32_t cand[C];
        uint64_t m[C][M];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            cand[c] = t[c] | (1u << bit);
#pragma unroll
            for (int i = 0; i < M; ++i) m[c][i] = __builtin_amdgcn_ballot_w64(u[c][i] >= cand[c]);
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            int n = 0;
#pragma unroll
            for (int i = 0; i < M; ++i) n += __popcll(m[c][i]);
            if (n >= k) t[c] = cand[c];
        }
    }
    bool any_tie = false;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if (!big[c]) t[c] = 0;   // at most k: every real entry
        // t >= 1 for a big set, and t + 1 does not wrap (t is at most the image of +inf)
        need[c] = big[c] ? k - wave_count_each<M>([&](int i) { return u[c][i] > t[c]; }) : 0;
        big[c] = big[c] && wave_count_each<M>([&](int i) { return u[c][i] == t[c]; }) > need[c];
        any_tie = any_tie || big[c];
    }
    if (any_tie) {   // more equal values at t than places: the largest tb among them
        for (int bit = 31; bit >= 0; --bit) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const uint32_t cand = tt[c] | (1u << bit);
                if (big[c] && wave_count_each<M>([&](int i) {
                        return u[c][i] == t[c] && tb[c][i] >= cand;
                    }) >= need[c])
                    tt[c] = cand;
            }
        }
    }
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int i = 0; i < M; ++i)
            sel[c][i] = u[c][i] > t[c] || (t[c] > 0 && u[c][i] == t[c] && tb[c][i] >= tt[c]);
}

// Writes the (x, id) of the marked entries of set c to its candidate list
// (ballot-prefix order, positions 0, 1, ...); returns their number.
// rowx(c, i, row, x) gives an entry; ids are row_id(ids, row).
template <int C, int M, typename RowX>
__device__ __forceinline__ int write_selected(const Stage1Args& a, const bool (&sel)[C][M], int c,
                                              RowX rowx, const RowIds& ids, size_t o) {
    const uint64_t below = (1ull << (threadIdx.x & 63)) - 1ull;
    int nsel = 0;
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const uint64_t sb = __ballot(sel[c][i]);
        if (sel[c][i]) {
            const int pos = nsel + __popcll(sb & below);
            int row;
            float x;
            rowx(c, i, row, x);
            a.cx[o + pos] = x;
            a.cidx[o + pos] = row_id(ids, row);
        }
        nsel += __popcll(sb);
    }
    return nsel;
}

// x of an order image (0: no candidate, -inf).
__device__ __forceinline__ float topk_value(uint32_t u) {
    return u ? ordered_to_float(u) : -INFINITY;
}

// Dense lists (k reaches every row of the fullest workgroup): the x of rows
// [0, nr) of each of the nc columns, in store order, then -inf up to
// a.topk_len; the ids are implied by the position.  The store holds order
// images (topk_order); a.topk_len and nr are multiples of 16 and the list
// offsets o[c] multiples of a.topk_len.
template <int C>
__device__ __forceinline__ void topk_write_dense(const Stage1Args& a, int nc,
                                                 uint32_t* const (&uc)[C], int nr,
                                                 const size_t (&o)[C]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if (c >= nc) break;
        for (int r = 4 * lane; r < a.topk_len; r += 256) {
            const uint4 v = r < nr ? *reinterpret_cast<const uint4*>(uc[c] + r)
                                   : uint4{0u, 0u, 0u, 0u};
            *reinterpret_cast<f32x4*>(a.cx + o[c] + r) =
                f32x4{topk_value(v.x), topk_value(v.y), topk_value(v.z), topk_value(v.w)};
        }
    }
}

// One wave, C columns at once: the top-k candidates of the rows of C
// columns whose order images (topk_order of x) sit in LDS at uc[c][row]:
// rows [0, nr) are the workgroup's, rows [nr, 64 NR) hold 0, and row r is
// global id row_id(ids, r), increasing in r.  Each uc[c] is 16-byte
// aligned, belongs to this wave alone and is overwritten.  Columns c >= nc
// are not real: their candidates are not written.  Writes the
// min(k, valid rows) candidates (x, id) of column c at offset o[c] of a.cx /
// a.cidx and fills the list's other slots, up to a.topk_len >= min(k, nr),
// with (-inf, -1).  The noise is drawn later, for the row's final k only.
//
// A lower bound cuts the work: the k-th largest of the lanes' two largest
// values is at most the column's k-th largest value (k of the column's
// values are at least that large; for k > 128 there is no such bound and
// every valid value is a survivor).  Usually little more than k values reach
// it; those are compacted to one (value, row) pair per lane and the exact
// selection runs on them, all C columns interleaved (other paths take up to
// four per lane, or all entries, one column at a time).
template <int C, int NR>
__device__ __forceinline__ void topk_select_columns(const Stage1Args& a, int nc,
                                                   uint32_t* const (&uc)[C], int nr,
                                                   const RowIds& ids, const size_t (&o)[C]) {
    static_assert(NR % 2 == 0 && NR * 64 >= 640, "row store of at least 640 entries");
    constexpr int kCap = 256;     // compacted pairs per column
    constexpr int kDummy = 300;   // pair slot written by lanes that keep nothing
    constexpr int PK = NR % 4 == 0 ? 4 : 2;   // entries per LDS read
    const int lane = threadIdx.x & 63;
    const int k = a.topk;
    (void)nr;
    // entry i = PK * q + j of this lane is row 64 PK q + PK lane + j
    auto row_of = [&](int i) { return 64 * PK * (i / PK) + PK * lane + (i % PK); };
    uint32_t u[C][NR];
    uint32_t top[C][2];   // the lane's two largest values
#pragma unroll
    for (int c = 0; c < C; ++c) {
        top[c][0] = top[c][1] = 0;
#pragma unroll
        for (int q = 0; q < NR / PK; ++q) {
            if constexpr (PK == 4) {
                const uint4 v4 = *reinterpret_cast<const uint4*>(uc[c] + 256 * q + 4 * lane);
                u[c][4 * q] = v4.x;
                u[c][4 * q + 1] = v4.y;
                u[c][4 * q + 2] = v4.z;
                u[c][4 * q + 3] = v4.w;
            } else {
                const uint2 v2 = *reinterpret_cast<const uint2*>(uc[c] + 128 * q + 2 * lane);
                u[c][2 * q] = v2.x;
                u[c][2 * q + 1] = v2.y;
            }
#pragma unroll
            for (int j = 0; j < PK; ++j) {
                const uint32_t v = u[c][PK * q + j];
                const uint32_t lo2 = v < top[c][0] ? v : top[c][0];
                top[c][0] = v > top[c][0] ? v : top[c][0];
                top[c][1] = lo2 > top[c][1] ? lo2 : top[c][1];
            }
        }
    }
    // bound: the k-th largest of the 2 * 64 lane tops (0 when there are fewer)
    uint32_t lo[C];
    wave_kth<C, 2, 16>(top, k, lo);   // to 16 bits: a bound, slightly below the exact one
    int nmax = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        lo[c] = lo[c] > 1u ? lo[c] : 1u;
        const int n = wave_count_each<NR>([&](int i) { return u[c][i] >= lo[c]; });
        if (c < nc) nmax = n > nmax ? n : nmax;
    }

    int nsel[C];
#pragma unroll
    for (int c = 0; c < C; ++c) nsel[c] = 0;
    if (nmax <= kCap) {
        // compact the values >= lo as (u, row) pairs to uc[c][0, 2 kCap)
        // (every lane has read its entries above)
        int cnt[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            uint2* pair = reinterpret_cast<uint2*>(uc[c]);
            int base = 0;
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const bool keep = u[c][i] >= lo[c];
                const uint64_t kb = __builtin_amdgcn_ballot_w64(keep);
                const int pos = (int)__builtin_amdgcn_mbcnt_hi(
                    (uint32_t)(kb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)kb, (uint32_t)base));
                pair[keep ? pos : kDummy] = uint2{u[c][i], (uint32_t)row_of(i)};
                base += __popcll(kb);
            }
            cnt[c] = base;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        if (nmax <= 64) {
            // the usual case: one survivor per lane, the C columns interleaved
            uint32_t v[C][1], tb[C][1];
            bool sel[C][1];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const uint2 pr = reinterpret_cast<const uint2*>(uc[c])[lane];
                v[c][0] = lane < cnt[c] ? pr.x : 0u;
                tb[c][0] = ~pr.y;
            }
            wave_select<C, 1>(v, tb, k, sel);
#pragma unroll
            for (int c = 0; c < C; ++c)
                if (c < nc)
                    nsel[c] = write_selected<C, 1>(
                        a, sel, c,
                        [&](int cc, int, int& row, float& x) {
                            row = (int)~tb[cc][0];
                            x = topk_value(v[cc][0]);
                        },
                        ids, o[c]);
        } else {
            // one column at a time, up to two or four survivors per lane
            auto run1 = [&](int c, auto m_tag) {
                constexpr int M = decltype(m_tag)::value;
                uint32_t v[1][M], tb[1][M];
                bool sel[1][M];
#pragma unroll
                for (int j = 0; j < M; ++j) {
                    const int q = lane + 64 * j;
                    const uint2 pr = reinterpret_cast<const uint2*>(uc[c])[q];
                    v[0][j] = q < cnt[c] ? pr.x : 0u;
                    tb[0][j] = ~pr.y;
                }
                wave_select<1, M>(v, tb, k, sel);
                return write_selected<1, M>(
                    a, sel, 0,
                    [&](int, int j, int& row, float& x) {
                        row = (int)~tb[0][j];
                        x = topk_value(v[0][j]);
                    },
                    ids, o[c]);
            };
#pragma unroll
            for (int c = 0; c < C; ++c)
                if (c < nc)
                    nsel[c] = cnt[c] <= 128 ? run1(c, std::integral_constant<int, 2>{})
                                            : run1(c, std::integral_constant<int, 4>{});
        }
    } else {
        // more than 256 values reach the bound (many equal values): the
        // exact selection on every entry, one column at a time
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (c >= nc) break;
            uint32_t ucol[1][NR], tb[1][NR];
            bool sel[1][NR];
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                ucol[0][i] = u[c][i];
                tb[0][i] = ~(uint32_t)row_of(i);
            }
            wave_select<1, NR>(ucol, tb, k, sel);
            nsel[c] = write_selected<1, NR>(
                a, sel, 0,
                [&](int, int i, int& row, float& x) {
                    row = row_of(i);
                    x = topk_value(ucol[0][i]);
                },
                ids, o[c]);
        }
    }
    // unused slots of the lists
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if (c >= nc) break;
        for (int q = nsel[c] + lane; q < a.topk_len; q += 64) {
            a.cx[o[c] + q] = -INFINITY;
            a.cidx[o[c] + q] = -1;
        }
    }
}

}  // namespace fs

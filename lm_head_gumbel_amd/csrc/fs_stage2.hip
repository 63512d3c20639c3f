// Stage 2 of fused LM-head sampling and the small kernels around it:
//  * flat reduction: argmax over per-workgroup winners (FlashSampling
//    explainer on aitrends.kr, Stage 2 paragraph);
//  * grouped reduction: per-tile records from the partial records, then the
//    hierarchical resample t* = argmax_t (L_t + G_t) (explainer,
//    tensor-parallel and Group-Gumbel-Max paragraphs);
//  * top-k: global top-k by x over the workgroup candidates, then argmax s;
//  * online binary merge of group summaries (Group-Gumbel-Max paragraph);
//  * unfused baseline: inverse-CDF draw from written logits;
//  * a noise dump used by the tests.
#include "fs_device.h"
#include "fs_internal.h"
#include "fs_topk.h"

#include <algorithm>

namespace fs {

constexpr int kRedThreads = 256;
constexpr int kGrpThreads = 1024;   // grouped stage 2: a thread per tile up to 1024 tiles

// Block-wide maximum of a packed key (NT threads); every thread gets it.
template <int NT = kRedThreads>
__device__ uint64_t block_max_key(uint64_t k) {
    __shared__ uint64_t part[NT / 64];
    for (int m = 32; m >= 1; m >>= 1) k = key_max(k, shfl_xor_u64(k, m));
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) part[wave] = k;
    __syncthreads();
    uint64_t r = part[0];
    for (int i = 1; i < NT / 64; ++i) r = key_max(r, part[i]);
    return r;
}

__global__ __launch_bounds__(kRedThreads) void stage2_flat_kernel(const float* pm,
                                                                  const int32_t* pidx, int P,
                                                                  int B, int32_t* out_idx,
                                                                  float* out_score,
                                                                  SchedState* sched) {
    const int b = blockIdx.x;
    // stage 1 is done: mark the unit scheduler initialised for the next call
    if (sched && b == 0 && threadIdx.x == 0) {
        sched->word = (unsigned long long)kSchedTag32 << 32;
        sched->exits = 0ull;
        sched->tag = kSchedTag;
    }
    uint64_t best = pack_key(-INFINITY, -1);
    for (int p = threadIdx.x; p < P; p += kRedThreads) {
        const int32_t id = pidx[(size_t)b * P + p];
        if (id >= 0) best = key_max(best, pack_key(pm[(size_t)b * P + p], id));
    }
    best = block_max_key(best);
    if (threadIdx.x == 0) {
        const int32_t id = key_index(best);
        out_idx[b] = id;
        if (out_score) out_score[b] = id >= 0 ? key_score(best) : -INFINITY;
    }
}

__device__ __forceinline__ bool row_is_greedy(const float* temp, int b, uint32_t flags) {
    if (flags & kFlagNoNoise) return true;
    const float T = temp ? temp[b] : 1.f;
    return !(T > 0.f);
}

// One tile of a grouped row: merges its record slots s0 .. s1 into the
// tile's winner key k (largest score) and log-mass L (greedy rows: the
// largest tempered logit).
struct TileRec {
    uint64_t k;
    float L;
};
__device__ __forceinline__ TileRec grouped_merge(const float* pm, const int32_t* pidx,
                                                 const float* pL, int P, int b, int s0, int s1,
                                                 bool greedy) {
    uint64_t k = pack_key(-INFINITY, -1);
    Lse l = lse_empty();
    // eight records at a time: their loads go out together
    for (int s8 = s0; s8 <= s1; s8 += 8) {
        float m8[8], L8[8];
        int32_t i8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const size_t o = (size_t)b * P + (s8 + q);
            const bool in = s8 + q <= s1;
            i8[q] = in ? pidx[o] : -1;
            m8[q] = in ? pm[o] : -INFINITY;
            L8[q] = in ? pL[o] : -INFINITY;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (i8[q] >= 0) k = key_max(k, pack_key(m8[q], i8[q]));
            if (greedy)
                l.mx = fmaxf(l.mx, L8[q]);
            else
                l = lse_merge(l, Lse{L8[q], 1.f});
        }
    }
    return TileRec{k, greedy ? l.mx : lse_value(l)};
}

__device__ __forceinline__ void store_tile(const TileRec& r, int b, int T, int t, float* tile_max,
                                           int32_t* tile_idx, float* tile_L) {
    const int32_t id = key_index(r.k);
    const size_t ot = (size_t)b * T + t;
    tile_max[ot] = id >= 0 ? key_score(r.k) : -INFINITY;
    tile_idx[ot] = id;
    tile_L[ot] = r.L;
}

// The tile's noisy group score as a key (the group noise is keyed by the
// tile; -inf for an empty tile).
__device__ __forceinline__ uint64_t group_key(const TileRec& r, int b, int t, bool greedy,
                                              const RowKey& rk) {
    const int32_t id = key_index(r.k);
    const float L = r.L;
    if (id < 0 || !(L > -INFINITY)) return pack_key(-INFINITY, -1);
    float sc = L;
    if (!greedy) {
        const uint4 rw = philox4x32_10(make_uint4((uint32_t)t >> 2, (uint32_t)b, rk.step,
                                                  kStreamGroup),
                                       rk.k0, rk.k1);
        const uint32_t words[4] = {rw.x, rw.y, rw.z, rw.w};
        sc += gumbel_from_word(words[t & 3]);
    }
    // tiles hold ascending id ranges, so the lowest id also means the lowest tile
    return pack_key(sc, id);
}

__device__ __forceinline__ void mark_scheduler(SchedState* sched) {
    // stage 1 is done: mark the unit scheduler initialised for the next call
    sched->word = (unsigned long long)kSchedTag32 << 32;
    sched->exits = 0ull;
    sched->tag = kSchedTag;
}

// Records per (range, tile): one workgroup per row, slots w + t of the G
// ranges w of nmb units that meet tile t.
__global__ __launch_bounds__(kGrpThreads) void stage2_grouped_kernel(
    const float* pm, const int32_t* pidx, const float* pL, int P, int B, int T, int G, int nmb,
    int tile_mb, const float* temp, uint32_t flags, NoiseSrc noise, float* tile_max,
    int32_t* tile_idx, float* tile_L, int32_t* out_idx, SchedState* sched) {
    const int b = blockIdx.x;
    if (sched && b == 0 && threadIdx.x == 0) mark_scheduler(sched);
    const bool greedy = row_is_greedy(temp, b, flags);
    const RowKey rk = row_key(noise, b);
    uint64_t best = pack_key(-INFINITY, -1);
    for (int t = threadIdx.x; t < T; t += kGrpThreads) {
        const int first = t * tile_mb;
        const int last = min(nmb, (t + 1) * tile_mb) - 1;
        const TileRec r = grouped_merge(pm, pidx, pL, P, b, part_owner(first, nmb, G) + t,
                                        part_owner(last, nmb, G) + t, greedy);
        store_tile(r, b, T, t, tile_max, tile_idx, tile_L);
        best = key_max(best, group_key(r, b, t, greedy, rk));
    }
    if (out_idx) {
        best = block_max_key<kGrpThreads>(best);
        if (threadIdx.x == 0) out_idx[b] = key_index(best);
    }
}

// A tile's running winner key and log-sum-exp state (value mx + log sm).
// Both merges are symmetric bit for bit, so the two lanes of a shuffle pair
// hold the same state afterwards.
struct TileAcc {
    uint64_t k;
    Lse l;
};

__device__ __forceinline__ TileAcc tile_acc_merge(TileAcc a, TileAcc b) {
    return TileAcc{key_max(a.k, b.k), lse_merge(a.l, b.l)};
}

__device__ __forceinline__ TileAcc shfl_xor_acc(TileAcc a, int m) {
    return TileAcc{shfl_xor_u64(a.k, m), Lse{__shfl_xor(a.l.mx, m, 64), __shfl_xor(a.l.sm, m, 64)}};
}

// One block record as a tile state (ok: the slot belongs to the tile).  A
// greedy row's log-mass is its maximum (the state's mx), so one merge serves
// both kinds of row.
__device__ __forceinline__ TileAcc block_acc(bool ok, int32_t id, float m, float L) {
    return TileAcc{ok && id >= 0 ? pack_key(m, id) : pack_key(-INFINITY, -1),
                   ok && L > -INFINITY ? Lse{L, 1.f} : lse_empty()};
}

// Block records, block-major (record of row b and block s at s C + b), tiles
// of at most kGrpColBlocks blocks: a thread per (row, tile).  Lanes 0..31 of
// a wave take 32 consecutive rows of one tile and lanes 32..63 the next tile,
// so every record load of a wave reads two whole 128-byte lines, and a
// thread's blocks (at most kGrpColBlocks) are loaded at once and merged in
// block order.  Workgroup (x, y) takes rows 32 y .. 32 y + 31 and tiles
// x tpw .. x tpw + tpw - 1 (eight per round).  The row's sample meets over
// the workgroup's tiles (lanes, then waves through LDS) and then over the
// workgroups of the row in the row's [key, count] pair of gsel, as below.
constexpr int kGrpColBlocks = 8;

__global__ __launch_bounds__(256) void stage2_grouped_cols_kernel(
    const float* pm, const int32_t* pidx, const float* pL, int C, int B, int T, int nmb,
    int tile_mb, int tpw, const float* temp, uint32_t flags, NoiseSrc noise, float* tile_max,
    int32_t* tile_idx, float* tile_L, int32_t* out_idx, unsigned long long* gsel,
    SchedState* sched) {
    __shared__ uint64_t wbest[4][32];
    if (sched && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) mark_scheduler(sched);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int b = blockIdx.y * 32 + (lane & 31);   // < C
    const bool col_ok = b < B;
    const int bq = col_ok ? b : 0;
    const bool greedy = row_is_greedy(temp, bq, flags);
    const RowKey rk = row_key(noise, bq);
    const int tslot = wave * 2 + (lane >> 5);   // 0..7
    const int tend = min(T, ((int)blockIdx.x + 1) * tpw);
    uint64_t best = pack_key(-INFINITY, -1);
    for (int t0 = blockIdx.x * tpw; t0 < tend; t0 += 8) {   // uniform
        const int t = t0 + tslot;
        const bool ok = col_ok && t < tend;
        int32_t id[kGrpColBlocks];
        float m[kGrpColBlocks], L[kGrpColBlocks];
#pragma unroll
        for (int j = 0; j < kGrpColBlocks; ++j) {
            const int s = min(min(t, T - 1) * tile_mb + min(j, tile_mb - 1), nmb - 1);
            const size_t o = (size_t)s * C + b;
            id[j] = pidx[o];
            m[j] = pm[o];
            L[j] = pL[o];
        }
        TileAcc a = block_acc(false, -1, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < kGrpColBlocks; ++j)
            a = tile_acc_merge(a, block_acc(ok && j < tile_mb && t * tile_mb + j < nmb, id[j], m[j],
                                            L[j]));
        if (ok) {
            const TileRec tr{a.k, greedy ? a.l.mx : lse_value(a.l)};
            store_tile(tr, b, T, t, tile_max, tile_idx, tile_L);
            best = key_max(best, group_key(tr, b, t, greedy, rk));
        }
    }
    if (!out_idx) return;   // uniform
    best = key_max(best, shfl_xor_u64(best, 32));
    if (lane < 32) wbest[wave][lane] = best;
    __syncthreads();
    if (wave == 0 && lane < 32 && col_ok) {
        best = key_max(key_max(wbest[0][lane], wbest[1][lane]), key_max(wbest[2][lane], wbest[3][lane]));
        if (gridDim.x == 1) {
            out_idx[b] = key_index(best);
        } else {
            // relaxed device-scope atomics, each waited for before the next
            // (see stage2_grouped_blocks_kernel)
            unsigned long long old = __hip_atomic_fetch_max(
                &gsel[kGselStride * b], (unsigned long long)best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("" : "+v"(old));
            const unsigned long long n = __hip_atomic_fetch_add(
                &gsel[kGselStride * b + 1], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (n == gridDim.x - 1) {
                unsigned long long zero = 0ull;
                asm volatile("" : "+v"(zero));
                const unsigned long long k = __hip_atomic_fetch_max(
                    &gsel[kGselStride * b], zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                out_idx[b] = key_index(key_max(k, old));
            }
        }
    }
}

// Records per 16-row block (slot = block), block-major: the record of
// (row b, block s) at s C + b.  Tiles of more than kGrpColBlocks blocks.
// Tile t goes to rpt = 2^rpt_log2
// consecutive threads (rpt: the power of two at or above tile_mb, at most
// kGrpBlkThreads), thread j of them merging blocks t tile_mb + j len .. + len
// - 1 (len = 1 unless a tile has more blocks than a workgroup has threads);
// a pass covers kGrpBlkThreads / rpt tiles, so consecutive threads read
// consecutive records.  Workgroup (c, b) takes passes c ppw .. c ppw + ppw - 1
// of row b and loads the records of up to kGrpBlkBatch of them together; each
// pass's runs then meet in an xor tree (shuffles inside a wave, the tile's
// waves in order through LDS), the same merge order on every call.
// Afterwards every thread of a tile's group holds the tile, and the passes
// are dealt out so that a thread finishes (log-mass, outputs, group noise) at
// most ceil(kGrpBlkBatch / rpt) tiles.  The row's sample is the largest
// group key over its tiles (Group-Gumbel-Max): with several workgroups per
// row their keys meet in the row's [key, count] pair of gsel (cleared by
// stage 1), an atomic maximum, and the workgroup that counts last writes it.
constexpr int kGrpBlkThreads = 256;
constexpr int kGrpBlkBatch = 8;

template <bool ONE>   // len == 1
__global__ __launch_bounds__(kGrpBlkThreads) void stage2_grouped_blocks_kernel(
    const float* pm, const int32_t* pidx, const float* pL, int P, int B, int T, int nmb,
    int tile_mb, int rpt_log2, int ppw, int C, const float* temp, uint32_t flags, NoiseSrc noise,
    float* tile_max, int32_t* tile_idx, float* tile_L, int32_t* out_idx,
    unsigned long long* gsel, SchedState* sched) {
    __shared__ uint64_t wk[kGrpBlkBatch][kGrpBlkThreads / 64];
    __shared__ Lse wl[kGrpBlkBatch][kGrpBlkThreads / 64];
    const int b = blockIdx.y;
    if (sched && b == 0 && blockIdx.x == 0 && threadIdx.x == 0) mark_scheduler(sched);
    const bool greedy = row_is_greedy(temp, b, flags);
    const RowKey rk = row_key(noise, b);
    const int rpt = 1 << rpt_log2;
    const int run = threadIdx.x & (rpt - 1);
    const int grp = threadIdx.x >> rpt_log2;
    const int len = (tile_mb + rpt - 1) >> rpt_log2;   // blocks per run
    const int tpp = kGrpBlkThreads >> rpt_log2;        // tiles per pass
    const int npass = min((T + tpp - 1) / tpp, ((int)blockIdx.x + 1) * ppw);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    uint64_t best = pack_key(-INFINITY, -1);
    for (int p0 = blockIdx.x * ppw; p0 < npass; p0 += kGrpBlkBatch) {   // uniform
        TileAcc r[kGrpBlkBatch];
        if constexpr (ONE) {
            // one record per pass, loaded unconditionally at a clamped slot:
            // every load of the batch goes out before the first is used
            int32_t id[kGrpBlkBatch];
            float m[kGrpBlkBatch], L[kGrpBlkBatch];
            bool ok[kGrpBlkBatch];
#pragma unroll
            for (int q = 0; q < kGrpBlkBatch; ++q) {
                const int t = (p0 + q) * tpp + grp;
                const int s = t * tile_mb + run;
                ok[q] = p0 + q < npass && t < T && run < tile_mb && s < nmb;
                const size_t o = (size_t)min(s, nmb - 1) * C + b;
                id[q] = pidx[o];
                m[q] = pm[o];
                L[q] = pL[o];
            }
#pragma unroll
            for (int q = 0; q < kGrpBlkBatch; ++q) r[q] = block_acc(ok[q], id[q], m[q], L[q]);
        } else {
            // runs of len blocks, eight records at a time
#pragma unroll
            for (int q = 0; q < kGrpBlkBatch; ++q) {
                const int t = (p0 + q) * tpp + grp;
                const int s0 = t * tile_mb + run * len;
                const int s1 = p0 + q < npass && t < T ? min(min(s0 + len, (t + 1) * tile_mb), nmb)
                                                       : s0;   // end
                TileAcc a = block_acc(false, -1, 0.f, 0.f);
                for (int s8 = s0; s8 < s1; s8 += 8) {
                    int32_t id[8];
                    float m[8], L[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const size_t o = (size_t)min(s8 + j, s1 - 1) * C + b;
                        id[j] = pidx[o];
                        m[j] = pm[o];
                        L[j] = pL[o];
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        a = tile_acc_merge(a, block_acc(s8 + j < s1, id[j], m[j], L[j]));
                }
                r[q] = a;
            }
        }
#pragma unroll
        for (int q = 0; q < kGrpBlkBatch; ++q)
            for (int mm = 1; mm < rpt && mm < 64; mm <<= 1)
                r[q] = tile_acc_merge(r[q], shfl_xor_acc(r[q], mm));
        if (rpt > 64) {   // uniform: a tile spans rpt / 64 waves
            __syncthreads();   // the previous batch is done with wk, wl
            if (lane == 0) {
#pragma unroll
                for (int q = 0; q < kGrpBlkBatch; ++q) {
                    wk[q][wave] = r[q].k;
                    wl[q][wave] = r[q].l;
                }
            }
            __syncthreads();
            const int w0 = wave & ~((rpt >> 6) - 1);
#pragma unroll
            for (int q = 0; q < kGrpBlkBatch; ++q) {
                r[q] = TileAcc{wk[q][w0], wl[q][w0]};
                for (int ww = w0 + 1; ww < w0 + (rpt >> 6); ++ww)
                    r[q] = tile_acc_merge(r[q], TileAcc{wk[q][ww], wl[q][ww]});
            }
        }
        // thread `run` of a group finishes passes q = run, run + rpt, ...
        for (int q0 = 0; q0 < kGrpBlkBatch; q0 += rpt) {   // uniform
            const int qs = q0 + run;
            // a = r[qs], as selects on the bits (an opaque mask per pass keeps
            // the compiler from turning the chain into an indexed array in
            // scratch memory)
            uint64_t ak = 0ull;
            uint32_t amx = 0u, asm_ = 0u;
#pragma unroll
            for (int q = 0; q < kGrpBlkBatch; ++q) {
                uint32_t mk = qs == q ? ~0u : 0u;
                asm volatile("" : "+v"(mk));
                const uint64_t mk64 = ((uint64_t)mk << 32) | mk;
                ak |= r[q].k & mk64;
                amx |= __float_as_uint(r[q].l.mx) & mk;
                asm_ |= __float_as_uint(r[q].l.sm) & mk;
            }
            const TileAcc a{ak, Lse{__uint_as_float(amx), __uint_as_float(asm_)}};
            const int t = (p0 + qs) * tpp + grp;
            if (qs < kGrpBlkBatch && p0 + qs < npass && t < T) {
                const TileRec tr{a.k, greedy ? a.l.mx : lse_value(a.l)};
                store_tile(tr, b, T, t, tile_max, tile_idx, tile_L);
                best = key_max(best, group_key(tr, b, t, greedy, rk));
            }
        }
    }
    if (out_idx) {   // uniform
        best = block_max_key<kGrpBlkThreads>(best);
        if (threadIdx.x == 0) {
            if (gridDim.x == 1) {
                out_idx[b] = key_index(best);
            } else {
                // Relaxed device-scope atomics, each waited for before the
                // next is issued: this workgroup's maximum has been performed
                // before its count, so the workgroup that counts last finds
                // every maximum in.  (Release and acquire at device scope
                // would write back and invalidate the whole L2 of the XCD.)
                unsigned long long old = __hip_atomic_fetch_max(
                    &gsel[kGselStride * b], (unsigned long long)best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                asm volatile("" : "+v"(old));   // the maximum has returned
                const unsigned long long n = __hip_atomic_fetch_add(
                    &gsel[kGselStride * b + 1], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (n == gridDim.x - 1) {   // every workgroup of the row is in
                    // read back as an atomic where the others were performed
                    // (an opaque operand keeps it from becoming a plain load)
                    unsigned long long zero = 0ull;
                    asm volatile("" : "+v"(zero));
                    const unsigned long long k = __hip_atomic_fetch_max(
                        &gsel[kGselStride * b], zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    out_idx[b] = key_index(key_max(k, old));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// top-k: candidates [B][G][L] (x, id) from stage 1, one list per workgroup
// (unused entries have id -1).  The row's k largest (x, -id) over all lists
// are selected exactly; optionally only the top-p prefix of them is kept;
// the noise s = x + Gumbel is drawn for the kept only and the largest s wins.
//
// stage2_topk_kernel (k <= 64): one workgroup of 512 threads per row holds
// the G*L candidates in registers (PER per thread).  A lower bound prunes
// the candidates: in each wave the k-th largest of the 64 lane maxima is at
// most the row's k-th largest x, and so is the largest of these wave bounds.
// The few candidates that reach it are gathered in LDS and one wave selects
// among them (a bound once more, from the lanes' two largest, then an exact
// bitwise search with ties to the lower id).  When too many reach it, the
// whole block runs the exact search on all candidates.  Larger k, or more
// than 512 * 64 candidates, take the sliced selection below.
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 512;
static_assert(kTopkThreads == kTopkStage2Threads, "the host plan picks the one-kernel form");
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkGather = 512;   // gathered candidates, at most 8 per lane of one wave

// Block-wide sum of per-wave counts (each wave passes its uniform count).
// The two halves of red alternate between calls, so one barrier suffices.
__device__ __forceinline__ int block_count(int wave_cnt, int (&red)[2][kTopkWaves], int& parity) {
    if ((threadIdx.x & 63) == 0) red[parity][threadIdx.x >> 6] = wave_cnt;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int i = 0; i < kTopkWaves; ++i) t += red[parity][i];
    parity ^= 1;
    return t;
}

__device__ uint64_t block_max_key_topk(uint64_t k) {
    __shared__ uint64_t part[kTopkWaves];
    for (int m = 32; m >= 1; m >>= 1) k = key_max(k, shfl_xor_u64(k, m));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = k;
    __syncthreads();
    uint64_t r = part[0];
    for (int i = 1; i < kTopkWaves; ++i) r = key_max(r, part[i]);
    return r;
}

__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
    for (int m = 32; m >= 1; m >>= 1) k = key_max(k, shfl_xor_u64(k, m));
    return k;
}

// Key (s, id) of a selected candidate of row b: s = x + Gumbel, or x on a
// greedy row.
__device__ __forceinline__ uint64_t scored_key(uint32_t u, int32_t id, int b, bool greedy,
                                               const RowKey& rk) {
    const float x = ordered_to_float(u);
    const float s = greedy ? x : x + token_gumbel(rk.k0, rk.k1, rk.step, b, id);
    return pack_key(s, id);
}

// Wave-wide bitonic sort of one 64-bit key per lane, largest key in lane 0.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t key) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint64_t o = shfl_xor_u64(key, stride);
            // blocks of `size` lanes alternate direction; the last one is descending
            const bool take_max = ((lane & stride) == 0) == ((lane & size) == 0);
            key = take_max ? (key > o ? key : o) : (key < o ? key : o);
        }
    return key;
}

// One wave: the sample among the row's selected top-k candidates, at most 64
// and one per lane, as the key (order image of x << 32) | ~id (0: none).
// With top_p < 1 the candidates are sorted by key (x descending, ties to
// the lower id) and only those whose exclusive softmax mass (float64) is
// below top_p times the set's mass are kept ("flashinfer.cake_sampling",
// launch forms).  The noise is drawn for the kept candidates only.  Returns
// the winning id in every lane (-1 when there is none).
__device__ int32_t finish_topk(uint64_t key, int b, bool greedy, float top_p,
                               const RowKey& rk) {
    const int lane = threadIdx.x & 63;
    bool keep = key != 0ull;
    if (top_p < 1.f) {
        key = wave_sort_desc(key);
        keep = key != 0ull;
        const double x = ordered_to_float((uint32_t)(key >> 32));
        const double xmax = __shfl(x, 0, 64);   // lane 0 holds the largest
        const double q = keep ? exp(x - xmax) : 0.0;
        double incl = q;   // inclusive prefix sum over the sorted lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        const double total = __shfl(incl, 63, 64);
        keep = keep && (incl - q) < (double)top_p * total;
    }
    uint64_t best = pack_key(-INFINITY, -1);
    if (keep)
        best = scored_key((uint32_t)(key >> 32), (int32_t)~(uint32_t)key, b, greedy, rk);
    return key_index(wave_max_key(best));
}

template <int PER>
__global__ __launch_bounds__(kTopkThreads) void stage2_topk_kernel(
    const float* cx, const int32_t* cidx, int G, int L, int B, int k, float top_p,
    const float* temp, uint32_t flags, NoiseSrc noise, int32_t* out_idx, SchedState* sched) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const bool greedy = row_is_greedy(temp, b, flags);
    // stage 1 is done: mark the unit scheduler initialised for the next call
    if (sched && b == 0 && threadIdx.x == 0) {
        sched->word = (unsigned long long)kSchedTag32 << 32;
        sched->exits = 0ull;
        sched->tag = kSchedTag;
    }
    __shared__ int red[2][kTopkWaves];
    __shared__ uint32_t wbound[kTopkWaves];
    __shared__ uint32_t g_u[kTopkGather];
    __shared__ uint32_t g_tb[kTopkGather];
    __shared__ int g_n;
    int parity = 0;
    // candidate e = threadIdx.x + 512 * i of the row's G * L (its lists are
    // contiguous).  Every candidate is loaded up front, unconditionally
    // (slots past the end re-read candidate 0 and are then ignored), so the
    // loads of a thread are all in flight together.
    const int n = G * L;
    const size_t row = (size_t)b * n;
    uint32_t u[PER];
    int32_t iv[PER];
    uint32_t lmax = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const bool ok = threadIdx.x + kTopkThreads * i < n;
        const size_t o = row + (ok ? threadIdx.x + kTopkThreads * i : 0);
        const int32_t id = cidx[o];
        const float xv = cx[o];
        iv[i] = ok ? id : -1;
        u[i] = iv[i] >= 0 ? topk_order(xv) : 0u;
        lmax = u[i] > lmax ? u[i] : lmax;
    }

    // lower bound and gathering of the candidates that reach it
    uint32_t wb[1];
    const uint32_t lm[1][1] = {{lmax}};
    wave_kth<1, 1, 16>(lm, k, wb);
    if (lane == 0) wbound[wave] = wb[0];
    if (threadIdx.x == 0) g_n = 0;
    __syncthreads();
    uint32_t lo = 1;
#pragma unroll
    for (int i = 0; i < kTopkWaves; ++i) lo = wbound[i] > lo ? wbound[i] : lo;
    // each wave reserves room for all its survivors with one atomic, then
    // writes them at ballot-prefix positions
    {
        int c = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) c += u[i] >= lo ? 1 : 0;
        const int nw = wave_sum<PER>(c);
        int base = 0;
        if (lane == 0 && nw > 0) base = atomicAdd(&g_n, nw);
        base = __shfl(base, 0, 64);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const bool keep = u[i] >= lo;
            const uint64_t kb = __ballot(keep);
            const int pos = base + (int)__builtin_amdgcn_mbcnt_hi(
                                       (uint32_t)(kb >> 32),
                                       __builtin_amdgcn_mbcnt_lo((uint32_t)kb, 0u));
            if (keep && pos < kTopkGather) {
                g_u[pos] = u[i];
                g_tb[pos] = ~(uint32_t)iv[i];
            }
            base += __popcll(kb);
        }
    }
    __syncthreads();
    const int ng = g_n;   // uniform

    if (ng <= kTopkGather) {
        if (wave != 0) return;
        // one wave: eight gathered candidates per lane, the bound once more
        uint32_t v[1][8], tb[1][8];
        uint32_t top[1][2] = {{0u, 0u}};   // the lane's two largest
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int q = lane + 64 * j;
            v[0][j] = q < ng ? g_u[q] : 0u;
            tb[0][j] = g_tb[q];
            const uint32_t lo1 = v[0][j] < top[0][0] ? v[0][j] : top[0][0];
            top[0][0] = v[0][j] > top[0][0] ? v[0][j] : top[0][0];
            top[0][1] = lo1 > top[0][1] ? lo1 : top[0][1];
        }
        uint32_t th[1];
        wave_kth<1, 2, 16>(top, k, th);
        const uint32_t lo2 = th[0] > 1u ? th[0] : 1u;
        int c2 = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) c2 += v[0][j] >= lo2 ? 1 : 0;
        const int n2 = wave_sum<8>(c2);
        uint64_t key = 0ull;   // this lane's selected candidate, if any
        if (n2 <= 64) {
            // compact to one per lane (every lane has read its entries above)
            int base = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool keep = v[0][j] >= lo2;
                const uint64_t kb = __ballot(keep);
                if (keep) {
                    const int pos = base + (int)__builtin_amdgcn_mbcnt_hi(
                                               (uint32_t)(kb >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)kb, 0u));
                    g_u[pos] = v[0][j];
                    g_tb[pos] = tb[0][j];
                }
                base += __popcll(kb);
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            uint32_t w1[1][1], t1[1][1];
            bool sel[1][1];
            w1[0][0] = lane < n2 ? g_u[lane] : 0u;
            t1[0][0] = g_tb[lane];
            wave_select<1, 1>(w1, t1, k, sel);
            if (sel[0][0]) key = ((uint64_t)w1[0][0] << 32) | t1[0][0];
        } else {
            // at most k <= 64 selected: gather them one per lane
            bool sel[1][8];
            wave_select<1, 8>(v, tb, k, sel);
            __builtin_amdgcn_wave_barrier();
            int base = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint64_t sb = __ballot(sel[0][j]);
                if (sel[0][j]) {
                    const int pos = base + (int)__builtin_amdgcn_mbcnt_hi(
                                               (uint32_t)(sb >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)sb, 0u));
                    g_u[pos] = v[0][j];
                    g_tb[pos] = tb[0][j];
                }
                base += __popcll(sb);
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            if (lane < base) key = ((uint64_t)g_u[lane] << 32) | g_tb[lane];
        }
        const int32_t id = finish_topk(key, b, greedy, top_p, row_key(noise, b));
        if (lane == 0) out_idx[b] = id;
        return;
    }

    // many candidates reach the bound: exact search over all of them
    auto count_ge = [&](uint32_t t) {
        int c = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) c += u[i] >= t ? 1 : 0;
        return block_count(wave_sum<PER>(c), red, parity);
    };
    // take u > t and, of u == t, the `need` lowest ids (ids <= id_max); with
    // at most k valid candidates every valid one (t = 1 lies below them all)
    uint32_t t = 1;
    int need = 0;
    int id_max = INT32_MAX;
    if (count_ge(1) > k) {
        t = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = t | (1u << bit);
            if (count_ge(cand) >= k) t = cand;
        }
        const int gt = count_ge(t + 1);   // t <= image of +inf: no wrap
        need = k - gt;
        const int ties = count_ge(t) - gt;
        if (ties > need) {
            // smallest m with #(u == t and id <= m) >= need
            auto count_tie_le = [&](int m) {
                int c = 0;
#pragma unroll
                for (int i = 0; i < PER; ++i) c += (u[i] == t && iv[i] <= m) ? 1 : 0;
                return block_count(wave_sum<PER>(c), red, parity);
            };
            int lo_id = 0;
            for (int bit = 30; bit >= 0; --bit)
                if (count_tie_le(lo_id + (1 << bit) - 1) < need) lo_id += 1 << bit;
            id_max = lo_id;
        }
    }

    // gather the (at most k) selected in LDS, then one wave finishes
    __syncthreads();   // every wave is done reading the gather area
    if (threadIdx.x == 0) g_n = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i)
        if (u[i] > t || (need > 0 && u[i] == t && iv[i] <= id_max)) {
            const int pos = atomicAdd(&g_n, 1);
            if (pos < 64) {
                g_u[pos] = u[i];
                g_tb[pos] = ~(uint32_t)iv[i];
            }
        }
    __syncthreads();
    if (wave == 0) {
        const int nsel = g_n < 64 ? g_n : 64;
        const uint64_t key = lane < nsel ? ((uint64_t)g_u[lane] << 32) | g_tb[lane] : 0ull;
        const int32_t id = finish_topk(key, b, greedy, top_p, row_key(noise, b));
        if (lane == 0) out_idx[b] = id;
    }
}

// ---------------------------------------------------------------------------
// Large-k selection: any k up to kMaxK over any number of candidates.  The
// row's candidates (G lists of L entries) are cut into slices of at most
// kSliceCap; one workgroup of 1024 threads per (slice, row) holds its slice
// in registers and selects the slice's k largest (x, ~id) keys exactly, writing
// them as a new list; the S new lists per row are selected from again until
// one workgroup holds the whole row, which selects, applies the optional
// top-p cut and draws.  (The k largest of a row are among the k largest of
// every part that holds them.)
//
// Selection of one slice: the range [min, max] of its valid x is cut into
// kBins equal-width bins (monotone in x) and counted; the bin where the count
// from the top first reaches k is the tie bin.  Entries of higher bins are
// selected outright; the tie bin's entries are sorted by key in LDS and the
// first (k - above) of them complete the selection.  The top of a logit
// distribution is sparse, so the tie bin usually holds few entries; when it
// holds more than kTieCap (many equal x), an exact radix search over the tie
// bin's keys (eight passes of eight bits) finds the cut instead.  A slice
// with at most k valid entries keeps them all.  With top-p the finishing
// workgroup sorts its selection, keeps the prefix whose exclusive mass
// (float64) is below top_p times the selection's mass, and draws.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kMaxK = kSelThreads;   // the finish holds one selected entry per thread
constexpr int kSelPer = 16;          // candidates per thread, in registers
constexpr int kSliceCap = kSelThreads * kSelPer;   // candidates per workgroup
static_assert(kSliceCap == kTopkSliceCap, "the host plan sizes the selection levels");
constexpr int kBins = 2048;          // two per thread
constexpr int kTieCap = 4096;

// Block-wide bitonic sort of keys[0, N) in LDS, N a power of two, descending.
__device__ __forceinline__ void block_sort_desc(uint64_t* keys, int N) {
    for (int size = 2; size <= N; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int p = threadIdx.x; p < N / 2; p += kSelThreads) {
                const int i = 2 * p - (p & (stride - 1));
                const int j = i + stride;
                const bool desc = (i & size) == 0;
                const uint64_t ki = keys[i], kj = keys[j];
                if ((ki < kj) == desc) {
                    keys[i] = kj;
                    keys[j] = ki;
                }
            }
            __syncthreads();
        }
}

// Pads keys[n, N) with 0 (N the next power of two) and sorts keys[0, N).
__device__ __forceinline__ void block_sort_prefix(uint64_t* keys, int n) {
    int N = 1;
    while (N < n) N <<= 1;
    for (int i = n + threadIdx.x; i < N; i += kSelThreads) keys[i] = 0ull;
    __syncthreads();
    block_sort_desc(keys, N);
}

// Inclusive and exclusive prefix sums of v over the threads of the block, in
// thread order (slot: one entry per wave).  Ends with a barrier.
template <typename T>
__device__ __forceinline__ void block_scan(T v, T* slot, T& incl, T& excl) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T s = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const T o = __shfl_up(s, off, 64);
        if (lane >= off) s += o;
    }
    T e = __shfl_up(s, 1, 64);
    if (lane == 0) e = T(0);
    if (lane == 63) slot[wave] = s;
    __syncthreads();
    T before = T(0);
#pragma unroll
    for (int i = 0; i < kSelWaves - 1; ++i) before += i < wave ? slot[i] : T(0);
    __syncthreads();
    incl = before + s;
    excl = before + e;
}

struct SelSmem {
    uint64_t gk[kMaxK];        // the selection
    uint64_t tk[kTieCap];      // the tie bin's keys
    uint32_t hist[kBins];
    int islot[kSelWaves];
    double dslot[kSelWaves];
    uint64_t kslot[kSelWaves];
    uint32_t mn, mx;
    int cnt, bin, above, need;
    uint64_t prefix;
    double total;
};

// Slice blockIdx.x of row blockIdx.y: candidates e in [e0, e0 + n) of the
// row's G lists of L entries (candidate e is entry e % L of list e / L, at
// offset b * G * L + e: a row's lists are contiguous); thread t holds entries
// t + 1024 j in registers.  DENSE: list w holds every row stage-1
// workgroup w kept, in its store order, and no ids (entry r is id v_offset +
// w u + (r / u) unit_stride + r % u, u = unit_rows, a power of two).
// FINISH == false: writes the slice's selection as list blockIdx.x of
// length k of ox / oidx ([B][S][k], padding (-inf, -1)).  FINISH == true
// (one slice): the draw, to out_idx[b].
template <bool FINISH, bool DENSE>
__global__ __launch_bounds__(kSelThreads) void stage2_topk_select_kernel(
    const float* cx, const int32_t* cidx, int G, int L, int B, int k, int per_slice,
    DenseIds dn, float* ox, int32_t* oidx, float top_p, const float* temp, uint32_t flags,
    NoiseSrc noise, int32_t* out_idx) {
    __shared__ SelSmem sm;
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int e0 = blockIdx.x * per_slice;
    const int n = min(per_slice, G * L - e0);   // 1 .. kSliceCap by the launch
    if (threadIdx.x == 0) {
        sm.mn = 0xFFFFFFFFu;
        sm.mx = 0u;
        sm.cnt = 0;
    }
    for (int i = threadIdx.x; i < kBins; i += kSelThreads) sm.hist[i] = 0u;

    // the slice into registers.  The loads are unconditional (slots past the
    // slice re-read its first entry and are then dropped), so that all of
    // them are in flight together.  x = -inf: no candidate.
    float x[kSelPer];
    int32_t id[DENSE ? 1 : kSelPer];   // dense lists: ids from the position
    {
        const float* xs = cx + (size_t)b * G * L + e0;
        const int32_t* is = cidx + (size_t)b * G * L + e0;
#pragma unroll
        for (int j = 0; j < kSelPer; ++j) {
            const int i = j * kSelThreads + (int)threadIdx.x;
            const bool ok = i < n;
            const float xv = xs[ok ? i : 0];
            x[j] = ok ? xv : -INFINITY;
            if constexpr (!DENSE) {
                const int32_t iv = is[ok ? i : 0];
                id[j] = ok ? iv : -1;
            }
        }
    }
    // (list, entry) of entry j: steps of (1024 / L, 1024 % L) from the first
    const int dq = kSelThreads / L, dr = kSelThreads % L;
    const int ush = __builtin_ctz((unsigned)dn.unit_rows);   // dense: unit_rows = 2^ush
    const int umask = dn.unit_rows - 1;
    const int w_start = (e0 + (int)threadIdx.x) / L;
    const int r_start = e0 + (int)threadIdx.x - w_start * L;
    // Visits this thread's entries in order: fn(j, id_of), id_of() giving
    // the id of entry j (for dense lists computed from (list, entry),
    // stepped along, so that it is only formed where it is used).
    auto walk = [&](auto fn) {
        int w = w_start, r = r_start;
        if constexpr (DENSE) {
            // a fresh copy per walk: the steps are recomputed, not kept live
            // in registers across the kernel
            asm volatile("" : "+v"(w), "+v"(r));
        }
#pragma unroll
        for (int j = 0; j < kSelPer; ++j) {
            auto id_of = [&]() -> int32_t {
                if constexpr (DENSE)
                    return dn.v_offset + (w << ush) + (r >> ush) * dn.unit_stride + (r & umask);
                else
                    return id[j];
            };
            fn(j, id_of);
            w += dq;
            r += dr;
            if (r >= L) {
                r -= L;
                ++w;
            }
        }
    };
    // Writes the keys of the entries where pred(j, id_of) holds to
    // dst[base, ...) in thread order: a block scan of the per-thread counts
    // gives each thread its first position.  Positions >= cap are dropped.
    // The caller synchronises before reading dst.
    auto compact = [&](auto pred, uint64_t* dst, int base, int cap) {
        int c = 0;
        walk([&](int j, auto id_of) { c += pred(j, id_of) ? 1 : 0; });
        int incl, excl;
        block_scan(c, sm.islot, incl, excl);
        int pos = base + excl;
        walk([&](int j, auto id_of) {
            if (pred(j, id_of)) {
                if (pos < cap) dst[pos] = pack_key(x[j], id_of());
                ++pos;
            }
        });
    };

    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
        if (x[j] > -INFINITY) {
            const uint32_t u = float_to_ordered(x[j]);
            mn = u < mn ? u : mn;
            mx = u > mx ? u : mx;
            ++cnt;
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint32_t a1 = __shfl_xor(mn, m, 64), a2 = __shfl_xor(mx, m, 64);
        mn = a1 < mn ? a1 : mn;
        mx = a2 > mx ? a2 : mx;
        cnt += __shfl_xor(cnt, m, 64);
    }
    __syncthreads();   // the counters are set
    if (lane == 0 && cnt > 0) {
        atomicMin(&sm.mn, mn);
        atomicMax(&sm.mx, mx);
        atomicAdd(&sm.cnt, cnt);
    }
    __syncthreads();
    const int total = sm.cnt;
    const int nsel = total < k ? total : k;   // the selection is gk[0, nsel)

    if (total <= k) {
        compact([&](int j, auto) { return x[j] > -INFINITY; }, sm.gk, 0, kMaxK);
        __syncthreads();
    } else {
        const float fmin = ordered_to_float(sm.mn), fmax = ordered_to_float(sm.mx);
        const float scale = fmax > fmin ? (float)kBins / (fmax - fmin) : 0.f;
        // bin of entry j (-1: none); monotone in x, and a NaN (inf * 0 when
        // the range overflows) lands in bin 0
        auto bin_at = [&](int j) {
            const float t = fminf(fmaxf((x[j] - fmin) * scale, 0.f), (float)(kBins - 1));
            return x[j] > -INFINITY ? (int)t : -1;
        };
#pragma unroll
        for (int j = 0; j < kSelPer; ++j) {
            const int bn = bin_at(j);
            if (bn >= 0) atomicAdd(&sm.hist[bn], 1u);
        }
        __syncthreads();
        {
            // counts from the top bin down: thread t owns bins kBins - 1 - 2t
            // and kBins - 2 - 2t; exactly one thread holds the bin where the
            // running count first reaches k
            const int hb = kBins - 1 - 2 * (int)threadIdx.x;
            const int c = (int)sm.hist[hb] + (int)sm.hist[hb - 1];
            int incl, excl;
            block_scan(c, sm.islot, incl, excl);
            if (excl < k && incl >= k) {
                const bool upper = excl + (int)sm.hist[hb] >= k;
                sm.bin = upper ? hb : hb - 1;
                sm.above = upper ? excl : excl + (int)sm.hist[hb];   // in bins above the tie bin
            }
            __syncthreads();
        }
        const int bk = sm.bin, above = sm.above;
        const int need = k - above;   // 1 .. entries of the tie bin
        const int ntie = (int)sm.hist[bk];
        if (ntie <= kTieCap) {
            // entries above the tie bin are selected, the tie bin's gathered:
            // one scan of both counts (16 bits each)
            int ch = 0, ct = 0;
#pragma unroll
            for (int j = 0; j < kSelPer; ++j) {
                const int bn = bin_at(j);
                ch += bn > bk ? 1 : 0;
                ct += bn == bk ? 1 : 0;
            }
            int incl, excl;
            block_scan(ch | (ct << 16), sm.islot, incl, excl);
            int ph = excl & 0xFFFF, pt = excl >> 16;
            walk([&](int j, auto id_of) {
                const int bn = bin_at(j);
                if (bn > bk) sm.gk[ph++] = pack_key(x[j], id_of());
                if (bn == bk) sm.tk[pt++] = pack_key(x[j], id_of());
            });
            __syncthreads();
            if (ntie > need) {
                if (ntie <= 64) {
                    if (threadIdx.x < 64) {   // one wave sorts the few ties
                        const uint64_t key = wave_sort_desc(lane < ntie ? sm.tk[lane] : 0ull);
                        if (lane < need) sm.gk[above + lane] = key;
                    }
                } else {
                    block_sort_prefix(sm.tk, ntie);
                    for (int i = threadIdx.x; i < need; i += kSelThreads)
                        sm.gk[above + i] = sm.tk[i];
                }
            } else {
                for (int i = threadIdx.x; i < need; i += kSelThreads) sm.gk[above + i] = sm.tk[i];
            }
            __syncthreads();
        } else {
            compact([&](int j, auto) { return bin_at(j) > bk; }, sm.gk, 0, kMaxK);
            // exact radix search for the need-th largest (x, ~id) key of the
            // tie bin, eight bits at a time from the top: first the order
            // image u of x, then ~id among the entries at that u; thread
            // t < 256 owns digit 255 - t
            uint32_t ucut = 0u, tcut = 0u;
            int left = need;
            for (int pass = 0; pass < 8; ++pass) {
                const bool on_id = pass >= 4;
                const int shift = 24 - 8 * (pass & 3);
                const uint32_t hi_mask = (pass & 3) == 0 ? 0u : (~0u << (shift + 8));
                const uint32_t cut = on_id ? tcut : ucut;
                __syncthreads();   // every thread is done with hist
                for (int i = threadIdx.x; i < 256; i += kSelThreads) sm.hist[i] = 0u;
                __syncthreads();
                walk([&](int j, auto id_of) {
                    if (bin_at(j) == bk) {
                        const uint32_t u = float_to_ordered(x[j]);
                        if (on_id ? u == ucut : true) {
                            const uint32_t v = on_id ? ~(uint32_t)id_of() : u;
                            if ((v & hi_mask) == cut) atomicAdd(&sm.hist[(v >> shift) & 0xFFu], 1u);
                        }
                    }
                });
                __syncthreads();
                const int c = threadIdx.x < 256 ? (int)sm.hist[255 - threadIdx.x] : 0;
                int incl, excl;
                block_scan(c, sm.islot, incl, excl);
                if (excl < left && incl >= left) {
                    sm.prefix = (uint64_t)(cut | ((255u - threadIdx.x) << shift));
                    sm.need = left - excl;
                }
                __syncthreads();
                if (on_id)
                    tcut = (uint32_t)sm.prefix;
                else
                    ucut = (uint32_t)sm.prefix;
                left = sm.need;
            }
            // the keys are distinct: exactly `need` of the tie bin are >= (ucut, tcut)
            compact(
                [&](int j, auto id_of) {
                    if (bin_at(j) != bk) return false;
                    const uint32_t u = float_to_ordered(x[j]);
                    return u > ucut || (u == ucut && ~(uint32_t)id_of() >= tcut);
                },
                sm.gk, above, kMaxK);
            __syncthreads();
        }
    }

    const int t = threadIdx.x;
    if constexpr (!FINISH) {
        // the slice's list: its selection, then padding
        const size_t o = ((size_t)b * gridDim.x + blockIdx.x) * k;
        for (int i = t; i < k; i += kSelThreads) {
            const uint64_t key = i < nsel ? sm.gk[i] : 0ull;
            ox[o + i] = i < nsel ? key_score(key) : -INFINITY;
            oidx[o + i] = i < nsel ? key_index(key) : -1;
        }
    } else {
        // the optional top-p cut over the sorted selection, then the draw
        const bool greedy = row_is_greedy(temp, b, flags);
        const bool topp = top_p < 1.f && nsel > 0;
        if (topp) block_sort_prefix(sm.gk, nsel);
        const uint64_t mine = t < nsel ? sm.gk[t] : 0ull;
        bool keep = t < nsel;
        if (topp) {
            const double x0 = key_score(sm.gk[0]);   // the largest
            const double q = keep ? exp((double)key_score(mine) - x0) : 0.0;
            double incl, excl;
            block_scan(q, sm.dslot, incl, excl);
            if (t == kSelThreads - 1) sm.total = incl;
            __syncthreads();
            keep = keep && excl < (double)top_p * sm.total;
        }
        uint64_t best = pack_key(-INFINITY, -1);
        if (keep)
            best = scored_key((uint32_t)(mine >> 32), (int32_t)~(uint32_t)mine, b, greedy,
                              row_key(noise, b));
        best = wave_max_key(best);
        if (lane == 0) sm.kslot[t >> 6] = best;
        __syncthreads();
        if (t == 0) {
            uint64_t r = sm.kslot[0];
#pragma unroll
            for (int i = 1; i < kSelWaves; ++i) r = key_max(r, sm.kslot[i]);
            out_idx[b] = key_index(r);
        }
    }
}

// ---------------------------------------------------------------------------
// online binary merge: one thread per row, chunks in order
// ---------------------------------------------------------------------------
__global__ void merge_online_kernel(int B, int C, const int32_t* z, const float* L,
                                    const float* temp, NoiseSrc noise, uint32_t flags,
                                    int32_t* out_idx, float* out_L) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const bool greedy = row_is_greedy(temp, b, flags);
    const RowKey rk = row_key(noise, b);
    int32_t zz = C > 0 ? z[(size_t)b * C] : -1;
    float A = C > 0 ? L[(size_t)b * C] : -INFINITY;
    for (int c = 1; c < C; ++c) {
        const float Lc = L[(size_t)b * C + c];
        const int32_t zc = z[(size_t)b * C + c];
        if (greedy) {
            if (Lc > A) { zz = zc; A = Lc; }
            continue;
        }
        if (!(Lc > -INFINITY)) continue;
        const float hi = fmaxf(A, Lc);
        const float A_new = hi + log1pf(expf(-fabsf(A - Lc)));   // logaddexp(A, L_c)
        const float p = expf(Lc - A_new);
        const uint4 rw = philox4x32_10(
            make_uint4((uint32_t)c >> 2, (uint32_t)b, rk.step, kStreamMerge), rk.k0, rk.k1);
        const uint32_t words[4] = {rw.x, rw.y, rw.z, rw.w};
        const float u = uniform_from_word(words[c & 3]);
        if (u < p) zz = zc;
        A = A_new;
    }
    out_idx[b] = zz;
    if (out_L) out_L[b] = A;
}

// ---------------------------------------------------------------------------
// unfused multinomial baseline
//  pass 1 (grid nchunk x B): per chunk of a row, the max of x, the sum of
//          exp(x - max) and the argmax key (for greedy rows);
//  pass 2 (grid B): total mass Z, target u*Z, the chunk holding it, then an
//          in-chunk inclusive scan to find the first id whose cumulative
//          mass exceeds the target.
// ---------------------------------------------------------------------------
struct XArgs {
    const float* logits;
    const float* temp;
    const uint32_t* allow;
    int B, V, n_valid, v_offset;
    uint32_t flags;
};

__device__ __forceinline__ float x_of(const XArgs& a, int b, int i, float inv_t) {
    if (i >= a.V || a.v_offset + i >= a.n_valid) return -INFINITY;
    if (a.allow) {
        const int words = (a.V + 31) >> 5;
        if (!((a.allow[(size_t)b * words + (i >> 5)] >> (i & 31)) & 1u)) return -INFINITY;
    }
    const float x = a.logits[(size_t)b * a.V + i] * inv_t;
    return x == x ? x : -INFINITY;
}

__device__ __forceinline__ float inv_temp(const XArgs& a, int b, bool& greedy) {
    greedy = row_is_greedy(a.temp, b, a.flags);
    return greedy ? 1.f : 1.f / (a.temp ? a.temp[b] : 1.f);
}

__global__ __launch_bounds__(kRedThreads) void multinomial_pass1(XArgs a, int chunk, int nchunk,
                                                                 float* ws_m, float* ws_s,
                                                                 uint64_t* ws_key) {
    const int c = blockIdx.x, b = blockIdx.y;
    bool greedy;
    const float inv_t = inv_temp(a, b, greedy);
    const int i0 = c * chunk, i1 = min(a.V, i0 + chunk);
    Lse l = lse_empty();
    uint64_t best = pack_key(-INFINITY, -1);
    for (int i = i0 + threadIdx.x; i < i1; i += kRedThreads) {
        const float x = x_of(a, b, i, inv_t);
        l = lse_add(l, x);
        if (x > -INFINITY) best = key_max(best, pack_key(x, a.v_offset + i));
    }
    for (int m = 32; m >= 1; m >>= 1) {
        l = lse_merge(l, Lse{__shfl_xor(l.mx, m, 64), __shfl_xor(l.sm, m, 64)});
        best = key_max(best, shfl_xor_u64(best, m));
    }
    __shared__ float smx[4], ssm[4];
    __shared__ uint64_t skey[4];
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { smx[wave] = l.mx; ssm[wave] = l.sm; skey[wave] = best; }
    __syncthreads();
    if (threadIdx.x == 0) {
        Lse r = Lse{smx[0], ssm[0]};
        uint64_t k = skey[0];
        for (int i = 1; i < 4; ++i) { r = lse_merge(r, Lse{smx[i], ssm[i]}); k = key_max(k, skey[i]); }
        const size_t o = (size_t)b * nchunk + c;
        ws_m[o] = r.mx;
        ws_s[o] = r.sm;
        ws_key[o] = k;
    }
}

// Pass 2 of the multinomial baseline.  The chunk is split into 256
// contiguous runs of `chunk / 256` ids, one per thread; one block scan over
// the run masses finds the run holding the target, whose thread then walks
// its ids in order.
__global__ __launch_bounds__(kRedThreads) void multinomial_pass2(XArgs a, int chunk, int nchunk,
                                                                 const float* ws_m,
                                                                 const float* ws_s,
                                                                 const uint64_t* ws_key,
                                                                 NoiseSrc noise,
                                                                 int32_t* out_idx) {
    const int b = blockIdx.x;
    bool greedy;
    const float inv_t = inv_temp(a, b, greedy);
    __shared__ float s_M, s_base, s_target;
    __shared__ int s_chunk, s_found, s_last;
    __shared__ float scan[kRedThreads];
    if (threadIdx.x == 0) {
        // sequential over the row's chunks: global max, total mass, target chunk
        float M = -INFINITY;
        uint64_t k = pack_key(-INFINITY, -1);
        for (int c = 0; c < nchunk; ++c) {
            M = fmaxf(M, ws_m[(size_t)b * nchunk + c]);
            k = key_max(k, ws_key[(size_t)b * nchunk + c]);
        }
        s_chunk = -1;
        s_found = 0x7FFFFFFF;
        s_last = -1;
        if (greedy || !(M > -INFINITY)) {
            out_idx[b] = key_index(k);
        } else {
            float Z = 0.f;
            for (int c = 0; c < nchunk; ++c) {
                const float m = ws_m[(size_t)b * nchunk + c];
                if (m > -INFINITY) Z += ws_s[(size_t)b * nchunk + c] * __expf(m - M);
            }
            const RowKey rk = row_key(noise, b);
            const uint4 rw =
                philox4x32_10(make_uint4(0u, (uint32_t)b, rk.step, kStreamMultinomial), rk.k0, rk.k1);
            const float target = uniform_from_word(rw.x) * Z;
            float acc = 0.f, acc_last = 0.f;
            int last = -1, sel = -1;
            for (int c = 0; c < nchunk; ++c) {
                const float m = ws_m[(size_t)b * nchunk + c];
                if (!(m > -INFINITY)) continue;
                const float cm = ws_s[(size_t)b * nchunk + c] * __expf(m - M);
                last = c;
                acc_last = acc;
                if (target < acc + cm) { sel = c; break; }
                acc += cm;
            }
            if (sel < 0) { sel = last; acc = acc_last; }   // rounding: the last chunk with mass
            s_chunk = sel;
            s_base = acc;
            s_target = target;
            s_M = M;
        }
    }
    __syncthreads();
    const int c = s_chunk;
    if (c < 0) return;   // greedy or empty row: already written
    const float M = s_M, target = s_target;
    const int per = chunk / kRedThreads;
    const int j0 = c * chunk + threadIdx.x * per;
    const int j1 = min(a.V, j0 + per);
    float mass = 0.f;
    int my_last = -1;
    for (int i = j0; i < j1; ++i) {
        const float x = x_of(a, b, i, inv_t);
        if (x > -INFINITY) { mass += __expf(x - M); my_last = i; }
    }
    scan[threadIdx.x] = mass;
    __syncthreads();
    for (int off = 1; off < kRedThreads; off <<= 1) {   // inclusive scan of run masses
        const float v = threadIdx.x >= off ? scan[threadIdx.x - off] : 0.f;
        __syncthreads();
        scan[threadIdx.x] += v;
        __syncthreads();
    }
    const float incl = s_base + scan[threadIdx.x];
    const float excl = incl - mass;
    if (my_last >= 0) atomicMax(&s_last, my_last);
    if (mass > 0.f && excl <= target && target < incl) {
        float acc = excl;
        int pick = my_last;
        for (int i = j0; i < j1; ++i) {
            const float x = x_of(a, b, i, inv_t);
            if (!(x > -INFINITY)) continue;
            acc += __expf(x - M);
            if (target < acc) { pick = i; break; }
        }
        atomicMin(&s_found, pick);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        // rounding can leave the target past the chunk's scanned mass: the
        // draw then belongs to the chunk's last valid id
        const int i = s_found != 0x7FFFFFFF ? s_found : s_last;
        out_idx[b] = i >= 0 ? a.v_offset + i : -1;
    }
}

__global__ void fill_idx_kernel(int32_t* out, int n, int32_t value, float* score) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        out[i] = value;
        if (score) score[i] = -INFINITY;
    }
}

__global__ void debug_noise_kernel(uint32_t k0, uint32_t k1, uint32_t step, uint32_t stream_id,
                                   int b0, int nb, int64_t i0, int ni, uint32_t* words,
                                   float* gumbel) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    const int r = blockIdx.y;
    if (j >= ni || r >= nb) return;
    const uint64_t i = (uint64_t)i0 + j;
    const uint4 rw = philox4x32_10(
        make_uint4((uint32_t)(i >> 2), (uint32_t)(b0 + r), step, stream_id), k0, k1);
    const uint32_t wv[4] = {rw.x, rw.y, rw.z, rw.w};
    const uint32_t word = wv[i & 3];
    if (words) words[(size_t)r * ni + j] = word;
    if (gumbel) gumbel[(size_t)r * ni + j] = gumbel_from_word(word);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_stage2_flat(const float* pm, const int32_t* pidx, int P, int B,
                              int32_t* out_idx, float* out_score, SchedState* sched,
                              hipStream_t stream) {
    hipLaunchKernelGGL(stage2_flat_kernel, dim3(B), dim3(kRedThreads), 0, stream, pm, pidx, P,
                       B, out_idx, out_score, sched);
    return hipGetLastError();
}

hipError_t launch_stage2_grouped(const float* pm, const int32_t* pidx, const float* pL, int P,
                                 int rec_cols, int B, int T, int G, int nmb, int tile_mb, const float* temp,
                                 uint32_t flags, const NoiseSrc& noise, float* tile_max,
                                 int32_t* tile_idx, float* tile_L, int32_t* out_idx,
                                 unsigned long long* gsel, SchedState* sched, hipStream_t stream) {
    if (gsel && tile_mb <= kGrpColBlocks) {
        // a thread per (row, tile): about two workgroups per compute unit
        const int cgroups = rec_cols / 32;
        const int rounds = (T + 7) / 8;
        const int want = std::max(1, std::min(rounds, (2 * 256 + cgroups - 1) / cgroups));
        const int tpw = 8 * ((rounds + want - 1) / want);
        const int chunks = (T + tpw - 1) / tpw;
        if (chunks > kMaxGridX || cgroups > kMaxGridY || rec_cols % 32 != 0 || rec_cols < B)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(stage2_grouped_cols_kernel, dim3(chunks, cgroups), dim3(256), 0, stream,
                           pm, pidx, pL, rec_cols, B, T, nmb, tile_mb, tpw, temp, flags, noise,
                           tile_max, tile_idx, tile_L, out_idx, gsel, sched);
    } else if (gsel) {
        // rpt: the power of two at or above tile_mb, at most kGrpBlkThreads
        int lg = 0;
        while ((1 << lg) < tile_mb && (2 << lg) <= kGrpBlkThreads) ++lg;
        const int tpp = kGrpBlkThreads >> lg;
        const int passes = (T + tpp - 1) / tpp;
        // workgroups per row: at least two per compute unit over all rows,
        // at most one batch of passes each
        const int want = std::max(1, std::min(passes, (2 * 256 + B - 1) / B));
        int ppw = std::max((passes + want - 1) / want, 1);
        ppw = std::min(ppw, kGrpBlkBatch);
        const int chunks = (passes + ppw - 1) / ppw;
        if (chunks > kMaxGridX || B > kMaxGridY) return hipErrorInvalidValue;
        if ((1 << lg) >= tile_mb)
            hipLaunchKernelGGL(stage2_grouped_blocks_kernel<true>, dim3(chunks, B),
                               dim3(kGrpBlkThreads), 0, stream, pm, pidx, pL, P, B, T, nmb, tile_mb,
                               lg, ppw, rec_cols, temp, flags, noise, tile_max, tile_idx, tile_L,
                               out_idx, gsel, sched);
        else
            hipLaunchKernelGGL(stage2_grouped_blocks_kernel<false>, dim3(chunks, B),
                               dim3(kGrpBlkThreads), 0, stream, pm, pidx, pL, P, B, T, nmb, tile_mb,
                               lg, ppw, rec_cols, temp, flags, noise, tile_max, tile_idx, tile_L,
                               out_idx, gsel, sched);
    } else {
        hipLaunchKernelGGL(stage2_grouped_kernel, dim3(B), dim3(kGrpThreads), 0, stream, pm, pidx,
                           pL, P, B, T, G, nmb, tile_mb, temp, flags, noise, tile_max, tile_idx,
                           tile_L, out_idx, sched);
    }
    return hipGetLastError();
}

hipError_t launch_stage2_topk(const float* cx, const int32_t* cidx, int G, int L, int B, int k,
                              DenseIds dn, float top_p, const float* temp, uint32_t flags,
                              const NoiseSrc& noise, int32_t* out_idx, void* scratch,
                              SchedState* sched, hipStream_t stream) {
    if (k < 1 || k > kMaxK || L < 1 || G < 1) return hipErrorInvalidValue;
    const bool dense = dn.on != 0;
#define FS_TOPK2(PER_)                                                                       \
    if (!dense && k <= 64 && (int64_t)G * L <= (int64_t)kTopkThreads * PER_) {             \
        hipLaunchKernelGGL(stage2_topk_kernel<PER_>, dim3(B), dim3(kTopkThreads), 0, stream, \
                           cx, cidx, G, L, B, k, top_p, temp, flags, noise, out_idx, sched); \
        return hipGetLastError();                                                            \
    }
    FS_TOPK2(4)
    FS_TOPK2(8)
    FS_TOPK2(16)
    FS_TOPK2(32)
    FS_TOPK2(64)
#undef FS_TOPK2
    if ((int64_t)G * L > INT32_MAX / 4) return hipErrorInvalidValue;
    // selection levels over slices until one workgroup holds a row
    const size_t list = stage2_topk_scratch_bytes(G, L, B, k, dense) / 4;
    if (list > 0 && !scratch) return hipErrorInvalidValue;
    char* base = static_cast<char*>(scratch);
    const float* ix = cx;
    const int32_t* ii = cidx;
    int g = G, l = L;
    bool first_dense = dense;   // only the first level reads dense lists
    for (int level = 0; (int64_t)g * l > kSliceCap; ++level) {
        const int n = g * l;
        const int S0 = (n + kSliceCap - 1) / kSliceCap;
        const int per = (n + S0 - 1) / S0;   // balanced slices of at most kSliceCap
        const int S = (n + per - 1) / per;   // every slice non-empty
        char* lv = base + (size_t)(level & 1) * 2 * list;
        float* ox = reinterpret_cast<float*>(lv);
        int32_t* oi = reinterpret_cast<int32_t*>(lv + list);
        if (first_dense)
            hipLaunchKernelGGL((stage2_topk_select_kernel<false, true>), dim3(S, B),
                               dim3(kSelThreads), 0, stream, ix, ii, g, l, B, k, per, dn, ox, oi,
                               top_p, temp, flags, noise, out_idx);
        else
            hipLaunchKernelGGL((stage2_topk_select_kernel<false, false>), dim3(S, B),
                               dim3(kSelThreads), 0, stream, ix, ii, g, l, B, k, per, dn, ox, oi,
                               top_p, temp, flags, noise, out_idx);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        ix = ox;
        ii = oi;
        g = S;
        l = k;
        first_dense = false;
    }
    if (first_dense)
        hipLaunchKernelGGL((stage2_topk_select_kernel<true, true>), dim3(1, B), dim3(kSelThreads),
                           0, stream, ix, ii, g, l, B, k, g * l, dn, nullptr, nullptr, top_p,
                           temp, flags, noise, out_idx);
    else
        hipLaunchKernelGGL((stage2_topk_select_kernel<true, false>), dim3(1, B),
                           dim3(kSelThreads), 0, stream, ix, ii, g, l, B, k, g * l, dn, nullptr,
                           nullptr, top_p, temp, flags, noise, out_idx);
    return hipGetLastError();
}

hipError_t launch_merge_online(int B, int C, const int32_t* z, const float* L, const float* temp,
                               const NoiseSrc& noise, uint32_t flags, int32_t* out_idx,
                               float* out_L, hipStream_t stream) {
    hipLaunchKernelGGL(merge_online_kernel, dim3((B + 63) / 64), dim3(64), 0, stream, B, C, z, L,
                       temp, noise, flags, out_idx, out_L);
    return hipGetLastError();
}

hipError_t launch_multinomial(const float* logits, const float* temp, const uint32_t* allow,
                              int B, int V, int n_valid, int v_offset, const NoiseSrc& noise,
                              uint32_t flags, int nchunk, int chunk,
                              float* ws_m, float* ws_s, uint64_t* ws_key, int32_t* out_idx,
                              hipStream_t stream) {
    XArgs a{logits, temp, allow, B, V, n_valid, v_offset, flags};
    hipLaunchKernelGGL(multinomial_pass1, dim3(nchunk, B), dim3(kRedThreads), 0, stream, a, chunk,
                       nchunk, ws_m, ws_s, ws_key);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(multinomial_pass2, dim3(B), dim3(kRedThreads), 0, stream, a, chunk, nchunk,
                       ws_m, ws_s, ws_key, noise, out_idx);
    return hipGetLastError();
}

hipError_t launch_fill_idx(int32_t* out, int n, int32_t value, float* score, hipStream_t stream) {
    hipLaunchKernelGGL(fill_idx_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, out, n, value,
                       score);
    return hipGetLastError();
}

hipError_t launch_debug_noise(uint32_t k0, uint32_t k1, uint32_t step, uint32_t stream_id,
                              int b0, int nb, int64_t i0, int ni, uint32_t* words, float* gumbel,
                              hipStream_t stream) {
    hipLaunchKernelGGL(debug_noise_kernel, dim3((ni + 255) / 256, nb), dim3(256), 0, stream, k0,
                       k1, step, stream_id, b0, nb, i0, ni, words, gumbel);
    return hipGetLastError();
}

}  // namespace fs

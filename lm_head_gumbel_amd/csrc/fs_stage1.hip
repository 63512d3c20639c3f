// Stage 1 of fused LM-head sampling on gfx950: one workgroup owns a
// contiguous, balanced range of 16-row vocabulary blocks; it computes their
// logits for 16*NB batch rows on chip with bf16 MFMA (FP32 accumulation),
// applies temperature and masks, adds Philox-Gumbel noise, and keeps only
// per-(row, tile) winners ("FlashSampling: Fast and Memory-Efficient Exact
// Sampling", Abstract; FlashSampling explainer on aitrends.kr, Stage 1
// paragraph).  Variants: flat winners, grouped winners with the tile
// log-mass (explainer, tensor-parallel paragraph), per-workgroup top-k
// candidates (explainer, implementation paragraph), and the unfused
// baseline that writes the logits instead.
//
// Work layout
//  * The four waves of a workgroup split the hidden dimension: wave w sums
//    over k-steps [w*nks/4, (w+1)*nks/4) (a k-step is 32 elements).  Their
//    partial 16x16 tiles meet in LDS in a fixed order, so results do not
//    depend on timing.
//  * MFMA v_mfma_f32_16x16x32_bf16: operand A = 16 vocab rows of W, operand
//    B = 16 batch rows of H.  Lane l supplies row (l & 15) and eight
//    consecutive k of group (l >> 4); A and B use the same k assignment, so
//    the contraction is unchanged by it.  Each lane's 16-byte load is a
//    contiguous piece of one W row, four lanes cover 64 contiguous bytes.
//  * Output lane l holds rows 4*(l >> 4) .. +3 of column (l & 15): one Philox
//    block (counter id >> 2) serves exactly one lane's four ids for a row.
#include "fs_device.h"
#include "fs_internal.h"
#include "fs_mfma.h"

#include <type_traits>

namespace fs {

template <int NB, int MPI>
struct Stage1Smem {
    f32x4 red[2][kWaves][MPI][NB][64];  // partial tiles of the four waves, double-buffered
    uint64_t fkey[kWaves][16];          // segment flush: per-wave column winners
    float fmx[kWaves][16];
    float fsm[kWaves][16];
};

// Top-k candidate lists: per column a sorted list of 64 keys (x, id)
// followed by 64 slots for the newest block group.
template <int NB>
struct TopkSmem {
    uint64_t key[16 * NB][128];
};
struct NoTopkSmem {};

// Sort the 128-entry arrays of every column by key, descending (bitonic
// network over all columns at once; 256 threads).
template <int NB>
__device__ void topk_sort(TopkSmem<NB>& t) {
    constexpr int N = 128;
    constexpr int pairs = 16 * NB * N / 2;
    for (int size = 2; size <= N; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int p = threadIdx.x; p < pairs; p += kThreads) {
                const int c = p / (N / 2);
                const int q = p % (N / 2);
                const int i = 2 * q - (q & (stride - 1));   // lower index of the pair
                const int j = i + stride;
                const bool desc = (i & size) == 0;
                const uint64_t ki = t.key[c][i], kj = t.key[c][j];
                if ((ki < kj) == desc) {
                    t.key[c][i] = kj;
                    t.key[c][j] = ki;
                }
            }
            __syncthreads();
        }
    }
}

template <int NB, int MPI, int KS, int VAR>
__global__ __launch_bounds__(kThreads) void stage1_kernel(Stage1Args a) {
    static_assert(4 % NB == 0, "NB must divide the wave count");
    static_assert(VAR != kVarTopk || MPI == 4, "top-k stages 64 new rows per group");
    __shared__ Stage1Smem<NB, MPI> sm;
    using TkSmem = typename std::conditional<VAR == kVarTopk, TopkSmem<NB>, NoTopkSmem>::type;
    __shared__ TkSmem tk;

    const int w = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15;
    const int kg = lane >> 4;
    const int mb0 = part_begin(w, a.nmb, a.G);
    const int mb1 = part_begin(w + 1, a.nmb, a.G);
    const int bbase = blockIdx.y * 16 * NB;

    // hidden-dimension range of this wave, in 32-element k-steps
    const int nks = (a.d + 31) >> 5;
    const int ks0 = wave * nks / kWaves;
    const int ks1 = (wave + 1) * nks / kWaves;

    // H rows this lane feeds to the MFMA B operand (one per N-block); rows
    // past B reuse row B - 1 and their columns are discarded
    const uint16_t* hrow[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        const int b = bbase + n * 16 + r16;
        hrow[n] = a.H + (size_t)(b < a.B ? b : a.B - 1) * a.d;
    }

    // epilogue column of this thread (fixed: N-block wave % NB, column lane & 15)
    const int ncol = wave % NB;
    const int col = bbase + ncol * 16 + r16;
    const bool col_ok = col < a.B;
    bool greedy = true;
    float inv_t = 1.f;
    if (col_ok) {
        const float T = a.temp ? a.temp[col] : 1.f;
        greedy = (a.flags & kFlagNoNoise) || !(T > 0.f);
        inv_t = greedy ? 1.f : 1.f / T;
    }
    const int allow_words = (a.V + 31) >> 5;
    const RowKey rk = col_ok ? row_key(a.noise, col) : RowKey{0u, 0u, 0u};
    const uint32_t* allow_row = (a.allow && col_ok) ? a.allow + (size_t)col * allow_words : nullptr;

    if constexpr (VAR == kVarTopk) {
        for (int e = threadIdx.x; e < 16 * NB * 128; e += kThreads) tk.key[e / 128][e % 128] = 0ull;
        __syncthreads();
    }

    // Software pipeline over the flattened (group, k-stage) stream of this
    // wave: the loads of the next stage (the next group's first stage at the
    // end of a group) are issued before the MFMAs of the current one, so they
    // stay in flight across the LDS reduction and the epilogue.
    const int n_it = ((ks1 - ks0 + KS - 1) / KS + 1) & ~1;   // even: ping-pong A/B
    const bool has_k = ks1 > ks0;
    Operands<NB, MPI, KS> opA, opB;
    const uint16_t* wrow[MPI];
    const uint16_t* wnext[MPI];
    Group cur = group_at<MPI>(mb0, mb1, a.tile_mb);
    group_rows<MPI>(wrow, a.W, cur, r16, a.V, a.d);
    if (has_k) load_operands<NB, MPI, KS>(opA, wrow, hrow, 0, ks0, ks1, kg, a.d);
    const uint16_t* wsel[MPI];

    uint64_t best = pack_key(-INFINITY, -1);
    Lse lse = lse_empty();
    int buf = 0;
    while (true) {
        const int gnext = cur.g + cur.nvm;
        const bool more = gnext < mb1;
        // after the last group the prefetch re-reads this group's first stage
        // (cache hits, never used): keeping every load unconditional keeps the
        // wait counts exact, so no wait drains the pipeline early
        const Group nxt = more ? group_at<MPI>(gnext, mb1, a.tile_mb) : cur;
        group_rows<MPI>(wnext, a.W, nxt, r16, a.V, a.d);

        // ---- contraction of this group over the wave's k-range ----
        f32x4 acc[MPI][NB];
#pragma unroll
        for (int j = 0; j < MPI; ++j)
#pragma unroll
            for (int n = 0; n < NB; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (has_k) {
            // sched_barrier keeps the compiler from sinking the prefetch below
            // the MFMAs, which would let the in-flight loads drain every stage
            for (int it = 0; it < n_it; it += 2) {
                load_operands<NB, MPI, KS>(opB, wrow, hrow, it + 1, ks0, ks1, kg, a.d);
                __builtin_amdgcn_sched_barrier(0);
                mfma_operands<NB, MPI, KS>(acc, opA);
                __builtin_amdgcn_sched_barrier(0);
                const bool same = it + 2 < n_it;
#pragma unroll
                for (int j = 0; j < MPI; ++j) wsel[j] = same ? wrow[j] : wnext[j];
                load_operands<NB, MPI, KS>(opA, wsel, hrow, same ? it + 2 : 0, ks0, ks1, kg, a.d);
                __builtin_amdgcn_sched_barrier(0);
                mfma_operands<NB, MPI, KS>(acc, opB);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- the four waves' partial tiles meet in LDS (fixed order) ----
#pragma unroll
        for (int j = 0; j < MPI; ++j)
#pragma unroll
            for (int n = 0; n < NB; ++n) sm.red[buf][wave][j][n][lane] = acc[j][n];
        __syncthreads();

        // ---- epilogue: a unit is four rows of one column (one MFMA lane's share) ----
#pragma unroll
        for (int q = 0; q < (MPI * NB + kWaves - 1) / kWaves; ++q) {
            const int jn = wave + kWaves * q;      // uniform across the wave
            if (jn >= MPI * NB) break;
            const int n = jn % NB;                 // == ncol
            const int j = jn / NB;
            const bool blk_ok = j < cur.nvm;
            f32x4 v = sm.red[buf][0][j][n][lane];
#pragma unroll
            for (int ww = 1; ww < kWaves; ++ww) v += sm.red[buf][ww][j][n][lane];
            const int row0 = (cur.g + j) * kMBlock + 4 * kg;   // local W row of v[0]

            if constexpr (VAR == kVarLogits) {
                if (blk_ok && col_ok) {
                    float* dst = a.logits + (size_t)col * a.V;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (row0 + r < a.V) dst[row0 + r] = v[r];
                }
            } else {
                float x[4];
                const int gid0 = a.v_offset + row0;
                // one allow word holds the lane's four rows (row0 % 4 == 0)
                const uint32_t word =
                    (allow_row && blk_ok && row0 < a.V) ? allow_row[row0 >> 5] : ~0u;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = row0 + r;
                    bool ok = blk_ok && col_ok && (i < a.V) && (gid0 + r < a.n_valid);
                    if (a.allow) ok = ok && ((word >> (i & 31)) & 1u);   // uniform
                    const float xv = v[r] * inv_t;
                    x[r] = (ok && xv == xv) ? xv : -INFINITY;
                }
                float s[4] = {x[0], x[1], x[2], x[3]};
                if (VAR != kVarTopk && !greedy && blk_ok && col_ok) {
                    const uint4 rw = philox4x32_10(
                        make_uint4((uint32_t)gid0 >> 2, (uint32_t)col, rk.step, kStreamToken),
                        rk.k0, rk.k1);
                    s[0] += gumbel_from_word(rw.x);
                    s[1] += gumbel_from_word(rw.y);
                    s[2] += gumbel_from_word(rw.z);
                    s[3] += gumbel_from_word(rw.w);
                }
                if constexpr (VAR == kVarTopk) {
                    // stage this group's values in the new half of the column list
                    const int slot = 64 + (j * 16 + 4 * kg) % 64;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool live = x[r] > -INFINITY;
                        tk.key[ncol * 16 + r16][slot + r] = live ? pack_key(x[r], gid0 + r) : 0ull;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (x[r] > -INFINITY) {
                            best = key_max(best, pack_key(s[r], gid0 + r));
                            if constexpr (VAR == kVarGrouped) lse = lse_add(lse, x[r]);
                        }
                    }
                }
            }
        }
        // The next group writes the other reduction buffer; this one is
        // rewritten two groups later, after every wave has passed the next
        // group's barrier and so has finished reading it.
        buf ^= 1;

        if constexpr (VAR == kVarTopk) {
            __syncthreads();     // every slot of the new half is written (empty ones as key 0)
            topk_sort<NB>(tk);   // ends with a barrier
        }

        // ---- segment end: combine the column winners and write a partial record ----
        if constexpr (VAR == kVarFlat || VAR == kVarGrouped) {
            if (cur.g + cur.nvm == cur.seg_end) {
                best = key_max(best, shfl_xor_u64(best, 16));
                best = key_max(best, shfl_xor_u64(best, 32));
                if constexpr (VAR == kVarGrouped) {
#pragma unroll
                    for (int m = 16; m <= 32; m <<= 1) {
                        Lse o{__shfl_xor(lse.mx, m, 64), __shfl_xor(lse.sm, m, 64)};
                        lse = lse_merge(lse, o);
                    }
                }
                if (lane < 16) {
                    sm.fkey[wave][lane] = best;
                    sm.fmx[wave][lane] = lse.mx;
                    sm.fsm[wave][lane] = lse.sm;
                }
                __syncthreads();
                if (threadIdx.x < 16 * NB) {
                    const int n = threadIdx.x >> 4;
                    const int c = threadIdx.x & 15;
                    const int b = bbase + n * 16 + c;
                    uint64_t k = pack_key(-INFINITY, -1);
                    Lse l = lse_empty();
                    for (int ww = n; ww < kWaves; ww += NB) {
                        k = key_max(k, sm.fkey[ww][c]);
                        l = lse_merge(l, Lse{sm.fmx[ww][c], sm.fsm[ww][c]});
                    }
                    if (b < a.B) {
                        const int p = (VAR == kVarGrouped) ? w + cur.t : w;
                        const size_t o = (size_t)b * a.P + p;
                        const int32_t id = key_index(k);
                        a.pm[o] = id >= 0 ? key_score(k) : -INFINITY;
                        a.pidx[o] = id;
                        if constexpr (VAR == kVarGrouped) {
                            const float T = a.temp ? a.temp[b] : 1.f;
                            const bool g_row = (a.flags & kFlagNoNoise) || !(T > 0.f);
                            a.pL[o] = g_row ? l.mx : lse_value(l);
                        }
                    }
                }
                __syncthreads();
                best = pack_key(-INFINITY, -1);
                lse = lse_empty();
            }
        }

        if (!more) break;
        cur = nxt;
#pragma unroll
        for (int j = 0; j < MPI; ++j) wrow[j] = wnext[j];
    }

    if constexpr (VAR == kVarTopk) {
        // the first k entries of each column list are this workgroup's candidates
        for (int e = threadIdx.x; e < 16 * NB * a.topk; e += kThreads) {
            const int c = e / a.topk;
            const int r = e % a.topk;
            const int b = bbase + c;
            if (b >= a.B) continue;
            const uint64_t k = tk.key[c][r];
            const size_t o = ((size_t)b * a.G + w) * a.topk_len + r;   // topk_len == topk here
            const bool live = k != 0ull;
            a.cx[o] = live ? key_score(k) : -INFINITY;
            a.cidx[o] = live ? key_index(k) : -1;
        }
    }
}

template <int NB, int MPI, int KS, int VAR>
static hipError_t launch_one(const Stage1Args& a, int grid_y, hipStream_t stream) {
    hipLaunchKernelGGL((stage1_kernel<NB, MPI, KS, VAR>), dim3(a.G, grid_y), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

// Instantiated (NB, MPI, KS) shapes.  MPI*KS sets the W bytes in flight per
// wave and stage; NB*KS the H loads; the register budget bounds both.
template <int VAR>
static hipError_t launch_var(const Stage1Args& a, int grid_y, const Stage1Config& c,
                             hipStream_t stream) {
#define FS_SHAPE(N_, M_, K_) \
    if (c.nb == N_ && c.mpi == M_ && c.ks == K_) return launch_one<N_, M_, K_, VAR>(a, grid_y, stream);
    FS_SHAPE(1, 4, 2)
    FS_SHAPE(2, 4, 1)
    if constexpr (VAR != kVarTopk) {
        FS_SHAPE(1, 4, 4)
        FS_SHAPE(1, 8, 1)
        FS_SHAPE(1, 8, 2)
        FS_SHAPE(1, 2, 4)
        FS_SHAPE(2, 4, 2)
        FS_SHAPE(2, 2, 2)
        FS_SHAPE(2, 8, 1)
        FS_SHAPE(4, 2, 1)
        FS_SHAPE(4, 4, 1)
    }
#undef FS_SHAPE
    return hipErrorInvalidValue;
}

hipError_t launch_stage1(int variant, const Stage1Args& a, int grid_y, const Stage1Config& cfg,
                         hipStream_t stream) {
    switch (variant) {
        case kVarFlat: return launch_var<kVarFlat>(a, grid_y, cfg, stream);
        case kVarGrouped: return launch_var<kVarGrouped>(a, grid_y, cfg, stream);
        case kVarLogits: return launch_var<kVarLogits>(a, grid_y, cfg, stream);
        case kVarTopk: return launch_var<kVarTopk>(a, grid_y, cfg, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fs

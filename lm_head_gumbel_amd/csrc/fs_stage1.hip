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

#include <type_traits>

namespace fs {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

template <int NB, int MPI>
struct Stage1Smem {
    f32x4 red[kWaves][MPI][NB][64];     // partial tiles of the four waves
    uint64_t fkey[kWaves][16];          // segment flush: per-wave column winners
    float fmx[kWaves][16];
    float fsm[kWaves][16];
};

// Top-k candidate lists: per column a sorted list of 64 (key, s) entries
// followed by 64 slots for the newest block group.
template <int NB>
struct TopkSmem {
    uint64_t key[16 * NB][128];
    float s[16 * NB][128];
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
                    const float si = t.s[c][i];
                    t.s[c][i] = t.s[c][j];
                    t.s[c][j] = si;
                }
            }
            __syncthreads();
        }
    }
}

template <int NB, int MPI, int VAR>
__global__ __launch_bounds__(kThreads) void stage1_kernel(Stage1Args a) {
    static_assert(4 % NB == 0, "NB must divide the wave count");
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

    // H rows this lane feeds to the MFMA B operand (one per N-block)
    const uint16_t* hrow[NB];
    bool hok[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        const int b = bbase + n * 16 + r16;
        hok[n] = b < a.B;
        hrow[n] = a.H + (size_t)(hok[n] ? b : 0) * a.d;
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
    const uint32_t* allow_row = (a.allow && col_ok) ? a.allow + (size_t)col * allow_words : nullptr;

    if constexpr (VAR == kVarTopk) {
        for (int e = threadIdx.x; e < 16 * NB * 128; e += kThreads) {
            tk.key[e / 128][e % 128] = 0ull;
            tk.s[e / 128][e % 128] = -INFINITY;
        }
        __syncthreads();
    }

    int mb = mb0;
    while (mb < mb1) {
        const int t = mb / a.tile_mb;
        const int64_t tile_end = (int64_t)(t + 1) * a.tile_mb;
        const int seg_end = tile_end < mb1 ? (int)tile_end : mb1;

        uint64_t best = pack_key(-INFINITY, -1);
        Lse lse = lse_empty();

        for (int g = mb; g < seg_end; g += MPI) {
            const int nvm = min(MPI, seg_end - g);   // valid blocks in this group
            f32x4 acc[MPI][NB];
            const uint16_t* wrow[MPI];
            bool wok[MPI];
#pragma unroll
            for (int j = 0; j < MPI; ++j) {
                const int row = (g + j) * kMBlock + r16;
                wok[j] = (j < nvm) && (row < a.V);
                wrow[j] = a.W + (size_t)(wok[j] ? row : 0) * a.d;
#pragma unroll
                for (int n = 0; n < NB; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};
            }

            constexpr int KS = 4;
            for (int ks = ks0; ks < ks1; ks += KS) {
                bf16x8 wf[MPI][KS];
                bf16x8 hf[NB][KS];
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    const int k = (ks + kk) * 32 + kg * 8;
                    const bool kok = (ks + kk < ks1) && (k < a.d);
#pragma unroll
                    for (int j = 0; j < MPI; ++j)
                        wf[j][kk] = (kok && wok[j]) ? load_bf16x8(wrow[j] + k) : zero_bf16x8();
#pragma unroll
                    for (int n = 0; n < NB; ++n)
                        hf[n][kk] = (kok && hok[n]) ? load_bf16x8(hrow[n] + k) : zero_bf16x8();
                }
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                    for (int j = 0; j < MPI; ++j)
#pragma unroll
                        for (int n = 0; n < NB; ++n)
                            acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                wf[j][kk], hf[n][kk], acc[j][n], 0, 0, 0);
            }

#pragma unroll
            for (int j = 0; j < MPI; ++j)
#pragma unroll
                for (int n = 0; n < NB; ++n) sm.red[wave][j][n][lane] = acc[j][n];
            __syncthreads();

            // epilogue: unit u covers four rows of one column (an MFMA lane's share)
#pragma unroll
            for (int q = 0; q < (MPI * NB + kWaves - 1) / kWaves; ++q) {
                const int jn = wave + kWaves * q;      // uniform across the wave
                if (jn >= MPI * NB) break;
                const int n = jn % NB;                 // == ncol
                const int j = jn / NB;
                const bool blk_ok = j < nvm;
                f32x4 v = sm.red[0][j][n][lane];
#pragma unroll
                for (int ww = 1; ww < kWaves; ++ww) v += sm.red[ww][j][n][lane];
                const int row0 = (g + j) * kMBlock + 4 * kg;   // local W row of v[0]

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
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = row0 + r;
                        bool ok = blk_ok && col_ok && (i < a.V) && (gid0 + r < a.n_valid);
                        if (ok && allow_row) ok = (allow_row[i >> 5] >> (i & 31)) & 1u;
                        float xv = v[r] * inv_t;
                        x[r] = (ok && xv == xv) ? xv : -INFINITY;
                    }
                    float s[4] = {x[0], x[1], x[2], x[3]};
                    if (!greedy && blk_ok && col_ok) {
                        const uint4 rw = philox4x32_10(
                            make_uint4((uint32_t)gid0 >> 2, (uint32_t)col, a.step, kStreamToken),
                            a.k0, a.k1);
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
                            tk.s[ncol * 16 + r16][slot + r] = live ? s[r] : -INFINITY;
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
            if constexpr (VAR == kVarTopk) {
                // every slot of the new half was written above (empty blocks as key 0)
                __syncthreads();
                topk_sort<NB>(tk);   // ends with a barrier
            } else {
                __syncthreads();     // sm.red is rewritten by the next group
            }
        }

        if constexpr (VAR == kVarFlat || VAR == kVarGrouped) {
            // combine the four lanes sharing a column, then the waves sharing it
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
                    const int p = (VAR == kVarGrouped) ? w + t : w;
                    const size_t o = (size_t)p * a.B + b;
                    const int32_t id = key_index(k);
                    a.pm[o] = id >= 0 ? key_score(k) : -INFINITY;
                    a.pidx[o] = id;
                    if constexpr (VAR == kVarGrouped) {
                        bool g_row = true;
                        const float T = a.temp ? a.temp[b] : 1.f;
                        g_row = (a.flags & kFlagNoNoise) || !(T > 0.f);
                        a.pL[o] = g_row ? l.mx : lse_value(l);
                    }
                }
            }
            __syncthreads();
        }
        mb = seg_end;
    }

    if constexpr (VAR == kVarTopk) {
        // the first k entries of each column list are this workgroup's candidates
        for (int e = threadIdx.x; e < 16 * NB * a.topk; e += kThreads) {
            const int c = e / a.topk;
            const int r = e % a.topk;
            const int b = bbase + c;
            if (b >= a.B) continue;
            const uint64_t k = tk.key[c][r];
            const size_t o = ((size_t)w * a.B + b) * a.topk + r;
            const bool live = k != 0ull;
            a.cx[o] = live ? key_score(k) : -INFINITY;
            a.cs[o] = live ? tk.s[c][r] : -INFINITY;
            a.cidx[o] = live ? key_index(k) : -1;
        }
    }
}

template <int NB, int MPI, int VAR>
static hipError_t launch_one(const Stage1Args& a, int grid_y, hipStream_t stream) {
    hipLaunchKernelGGL((stage1_kernel<NB, MPI, VAR>), dim3(a.G, grid_y), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

template <int VAR>
static hipError_t launch_var(const Stage1Args& a, int grid_y, const Stage1Config& c,
                             hipStream_t stream) {
    if (c.nb == 1 && c.mpi == 4) return launch_one<1, 4, VAR>(a, grid_y, stream);
    if (c.nb == 2 && c.mpi == 4) return launch_one<2, 4, VAR>(a, grid_y, stream);
    if constexpr (VAR != kVarTopk) {
        if (c.nb == 4 && c.mpi == 2) return launch_one<4, 2, VAR>(a, grid_y, stream);
    }
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

// Stage 1 of fused LM-head sampling with the hidden states resident in
// registers (gfx950).  A workgroup of NW waves owns a balanced, contiguous
// range of 16-row vocabulary blocks; the waves split the hidden dimension, and
// each wave loads its slice of H (HK k-steps of 32 elements, all 16*NB batch
// rows) into registers once.  The only loads left in the contraction loop are
// the W stream, which leaves the vector-memory pipeline to W alone.  Logits of
// MPI blocks at a time meet in LDS in a fixed wave order, and the epilogue
// (temperature, masks, Philox-Gumbel noise, per-tile winners and log-mass)
// follows ("FlashSampling: Fast and Memory-Efficient Exact Sampling",
// Abstract; FlashSampling explainer on aitrends.kr, Stage 1 and
// tensor-parallel paragraphs).  The top-k variant keeps the tempered logits
// of its whole row range in LDS (the range is at most TopkRows<NB, HL>::kRows
// rows, the host sizes the grid for it) and selects each column's k best at
// the end (implementation paragraph of the explainer).
//
// The per-group loop is unrolled at compile time (HK k-steps per wave, HK/KS
// stages), so register indices into the resident H are static and every load
// is unconditional; the next group's first stage is prefetched before the
// last MFMAs of the current group and stays in flight through the reduction
// and the epilogue.  Requires nks == NW * HK (the host checks).
#include "fs_device.h"
#include "fs_epilogue.h"
#include "fs_internal.h"
#include "fs_mfma.h"
#include "fs_topk.h"

#include <type_traits>

namespace fs {

template <int MPI, int KS>
struct WStage {
    bf16x8 w[MPI][KS];
};

// W fragments of stage `it` (k-steps ks0 + it*KS ..) of the rows in wrow.
template <int MPI, int KS>
__device__ __forceinline__ void load_w(WStage<MPI, KS>& s, const uint16_t* (&wrow)[MPI], int it,
                                       int ks0, int kg, int d) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const int k = (ks0 + it * KS + kk) * 32 + kg * 8;
        const int kc = k < d ? k : d - 8;   // the matching H fragment is zero
#pragma unroll
        for (int j = 0; j < MPI; ++j) s.w[j][kk] = load_bf16x8(wrow[j] + kc);
    }
}

// MFMAs of stage `it` with the H fragments in registers (k-steps it * KS ..
// + KS - 1 < HK; the index is clamped so that the call compiles for every
// unrolled stage).
template <int NB, int MPI, int KS, int HK>
__device__ __forceinline__ void mfma_w(f32x4 (&acc)[MPI][NB], const WStage<MPI, KS>& s,
                                       const bf16x8 (&h)[NB][HK], int it) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const int ks = it * KS + kk < HK ? it * KS + kk : HK - 1;
#pragma unroll
        for (int j = 0; j < MPI; ++j)
#pragma unroll
            for (int n = 0; n < NB; ++n)
                acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s.w[j][kk], h[n][ks], acc[j][n],
                                                                    0, 0, 0);
    }
}

// Whole-line W loads (stages of an even number KS of k-steps).  The k-steps
// of a stage come in pairs, and one instruction reads the pair's 128-byte
// line of 8 rows of a block: lane l reads row 8 h + (l & 7) of the block (h,
// the instruction's half of the block), bytes 16 (l >> 3) .. of the line.  As
// an MFMA A operand that lane is row (l & 7) + 8 ((l >> 3) & 1), k-slots
// 8 (l >> 4) ..: rows 0-7 hold the line's even 16-byte pieces of the half's
// eight rows, rows 8-15 their odd pieces.  Two MFMAs take them apart: the
// operand with the odd pieces zeroed against H's even pieces, and with the
// even pieces zeroed against its odd pieces (H slot group g of a pair holds
// pieces 2 g and 2 g + 1: h_pair_k), both into the half's accumulator, whose
// rows r and r + 8 then hold the two partial sums of the half's row r
// (combine_halves).  A 16-byte piece per lane of a whole line per instruction
// streams HBM faster than a 64-byte piece of each of 16 rows, and the
// streaming cache policy helps it further (it slows the 64-byte pieces).
template <int MPI, int KS>
__device__ __forceinline__ void load_w_lines(WStage<MPI, KS>& s, const uint16_t* (&wrow)[MPI][2],
                                             int it, int ks0, int lane, int d) {
#pragma unroll
    for (int p = 0; p < KS / 2; ++p) {
        const int k = (ks0 + it * KS + 2 * p) * 32 + (lane >> 3) * 8;
        const int kc = k < d ? k : d - 8;   // the matching H fragment is zero
#pragma unroll
        for (int j = 0; j < MPI; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) s.w[j][2 * p + h] = load_bf16x8_nt(wrow[j][h] + kc);
    }
}

// Element offset (from k-step 0 of the wave's slice) of this lane's H piece
// for k-slot group `kg` in k-step ks of the whole-line layout: k-steps 2 q and
// 2 q + 1 hold the even and odd 16-byte pieces of the pair's 64 k.
__device__ __forceinline__ int h_pair_k(int ks, int kg) {
    return (ks & ~1) * 32 + kg * 16 + (ks & 1) * 8;
}

// The A operand of one whole-line load split by piece parity.
__device__ __forceinline__ void split_pieces(bf16x8 a, uint32_t even, bf16x8& ae, bf16x8& ao) {
    const u32x4 v = __builtin_bit_cast(u32x4, a);
    ae = __builtin_bit_cast(bf16x8, v & even);
    ao = __builtin_bit_cast(bf16x8, v & ~even);
}

template <int NB, int MPI, int KS, int HK>
__device__ __forceinline__ void mfma_w_lines(f32x4 (&acc)[MPI][2][NB], const WStage<MPI, KS>& s,
                                             const bf16x8 (&h)[NB][HK], int it, uint32_t even) {
#pragma unroll
    for (int p = 0; p < KS / 2; ++p) {
        const int ks = it * KS + 2 * p + 1 < HK ? it * KS + 2 * p : HK - 2;
#pragma unroll
        for (int j = 0; j < MPI; ++j)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                bf16x8 ae, ao;
                split_pieces(s.w[j][2 * p + hh], even, ae, ao);
#pragma unroll
                for (int n = 0; n < NB; ++n) {
                    acc[j][hh][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ae, h[n][ks],
                                                                            acc[j][hh][n], 0, 0, 0);
                    acc[j][hh][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, h[n][ks + 1],
                                                                            acc[j][hh][n], 0, 0, 0);
                }
            }
    }
}

template <int NB, int MPI, int KS, int HK>
__device__ __forceinline__ void mfma_w_lines_lds(f32x4 (&acc)[MPI][2][NB],
                                                 const WStage<MPI, KS>& s, const bf16x8* hl,
                                                 int it, uint32_t even) {
#pragma unroll
    for (int p = 0; p < KS / 2; ++p) {
        const int q = it * KS + 2 * p - HK;
        bf16x8 he[NB], ho[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            he[n] = hl[(q * NB + n) * 64];
            ho[n] = hl[((q + 1) * NB + n) * 64];
        }
#pragma unroll
        for (int j = 0; j < MPI; ++j)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                bf16x8 ae, ao;
                split_pieces(s.w[j][2 * p + hh], even, ae, ao);
#pragma unroll
                for (int n = 0; n < NB; ++n) {
                    acc[j][hh][n] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(ae, he[n], acc[j][hh][n], 0, 0, 0);
                    acc[j][hh][n] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, ho[n], acc[j][hh][n], 0, 0, 0);
                }
            }
    }
}

// The block's tile in the usual MFMA output layout from the two halves'
// accumulators: lanes 0-31 of half h hold its rows' even-piece sums and lanes
// 32-63 their odd-piece sums, so one swap of lanes 32-63 of half 0 with lanes
// 0-31 of half 1 and an add leave rows 0-7 of the block (half 0) in lanes
// 0-31 and rows 8-15 (half 1) in lanes 32-63.
__device__ __forceinline__ f32x4 combine_halves(f32x4 a0, f32x4 a1) {
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // (the elements are copied out first: a bit cast of a vector element
        // in place read element 0 for every i)
        const float x0 = a0[i], x1 = a1[i];
        const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x0),
                                                         __builtin_bit_cast(uint32_t, x1), false,
                                                         false);
        r[i] = __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
    }
    return r;
}

// MFMAs of stage `it` with the H fragments in LDS: k-step it * KS + kk - HK of
// hl ([HL][NB] fragments, 64 lanes each, this lane's entry).
template <int NB, int MPI, int KS, int HK>
__device__ __forceinline__ void mfma_w_lds(f32x4 (&acc)[MPI][NB], const WStage<MPI, KS>& s,
                                           const bf16x8* hl, int it) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        bf16x8 hb[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n) hb[n] = hl[((it * KS + kk - HK) * NB + n) * 64];
#pragma unroll
        for (int j = 0; j < MPI; ++j)
#pragma unroll
            for (int n = 0; n < NB; ++n)
                acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s.w[j][kk], hb[n], acc[j][n],
                                                                    0, 0, 0);
    }
}

template <int NB, int MPI, int NW>
struct ResidentSmem {
    f32x4 red[2][NW][MPI][NB][64];   // partial tiles of the waves, double-buffered
    uint64_t fkey[NW][16];
    float fmx[NW][16];
    float fsm[NW][16];
    int dyn;            // flat and top-k: units from the ticket counter
    int next_unit[2];   // ticket order: a unit taken by ticket (-1: none)
};

// Top-k: order images of the x of the workgroup's rows, one padded row of
// LDS per column (also the scratch area of the column's selection).
template <int NB, int NW, int HL>
struct TopkRowsSmem {
    alignas(16) uint32_t u[16 * NB][TopkRows<NB, HL>::kStride];
    int unit[TopkRows<NB, HL>::kRows / 16];   // vocabulary unit of each store unit
};
struct NoTopkRows {};

// Grouped: the records (winner key and log-mass per column) of the 16-row
// blocks the workgroup has walked, kept here and written out when the store
// is full and after the walk.  A record store inside the walk would hold back
// the loads issued after it (its wait is counted with theirs): 15 us of 240
// at B = 32.
template <int NB>
struct BlockRecSmem {
    static constexpr int kSlots = 64;
    uint64_t key[kSlots][16 * NB];
    float mx[kSlots][16 * NB];
    float sm[kSlots][16 * NB];
    int blk[kSlots];   // block of each slot
};
struct NoRec {};

// The last HL k-steps of each wave's H slice, when the registers cannot hold
// the whole slice: per wave [HL][NB] fragments of 64 lanes (each lane reads
// back only what it wrote).
template <int NB, int NW, int HL>
struct HlSmem {
    bf16x8 h[NW][HL][NB][64];
};
struct NoHl {};

template <int NB, int MPI, int NW, int HL>
constexpr bool topk_fits() {
    return sizeof(ResidentSmem<NB, MPI, NW>) + sizeof(TopkRowsSmem<NB, NW, HL>) +
               (HL > 0 ? sizeof(HlSmem<NB, NW, (HL > 0 ? HL : 1)>) : 0) <=
           160 * 1024;
}

template <int NB, int MPI, int KS, int NW, int HK, int HL, int VAR>
__global__ __launch_bounds__(64 * NW) void resident_kernel(Stage1Args a) {
    static_assert(NW % NB == 0, "NB must divide the wave count");
    static_assert(HK % KS == 0 && HL % KS == 0 && (HK + HL) % (2 * KS) == 0,
                  "stages are processed in pairs");
    constexpr int HT = HK + HL;   // k-steps per wave
    constexpr int NIT = HT / KS;
    // whole-line W loads (load_w_lines) where the stages hold pairs of k-steps
    constexpr bool FL = KS % 2 == 0;
    __shared__ ResidentSmem<NB, MPI, NW> sm;
    using HlPart = typename std::conditional<(HL > 0), HlSmem<NB, NW, (HL > 0 ? HL : 1)>, NoHl>::type;
    __shared__ HlPart hls;
    using TkSmem =
        typename std::conditional<VAR == kVarTopk, TopkRowsSmem<NB, NW, HL>, NoTopkRows>::type;
    __shared__ TkSmem tk;
    static_assert(MPI * NB <= NW, "every (block, N-block) pair of a group has a wave");
    using RecPart = typename std::conditional<VAR == kVarGrouped, BlockRecSmem<NB>, NoRec>::type;
    __shared__ RecPart rec;

    // Row range w and batch group y of this workgroup.  With xcd_pair the grid
    // is 1-D and the ny groups of a range get ids L, L + 8, L + 16, ...:
    // workgroups are dealt to the eight XCDs round-robin, so the groups that
    // read the same W rows run at the same time on one XCD and share its L2.
    int w, y;
    if (a.xcd_pair) {
        const int L = blockIdx.x;
        const int per = 8 * a.ny;
        y = (L % per) / 8;
        w = (L / per) * 8 + (L % 8);
    } else {
        w = blockIdx.x;
        y = blockIdx.y;
    }
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15;
    const int kg = lane >> 4;
    // Every variant walks units of MPI blocks strided by G (unit w, w + G,
    // w + 2G, ...): at any moment the workgroups read neighbouring parts of W,
    // which streams HBM better than one contiguous range per workgroup (6.10
    // against 5.78 TB/s at B = 32, d = 4096, V = 151936).  Any partition gives
    // the same flat sample (the noise is keyed by the global id), the same
    // top-k set (the row store maps back to global ids) and the same grouped
    // records (one per 16-row block, its slot the block).  mb0 is the first
    // block, mb1 one past the last unit's blocks.
    //
    // Flat, grouped and top-k with a scheduler block (one batch group; top-k with lists
    // that carry ids, its store unit table giving the ids): the first a.dyn_k0 >= 3
    // units of a workgroup are w, w + G, w + 2G, ... as in the strided order,
    // every later one comes from a ticket t (unit k0 G + t), so that the
    // workgroups that run faster take more of the last units and all finish
    // close together.  The ticket taken at the start of group i (before the
    // group's own loads: the previous group's prefetch, which the group waits
    // for first, does not wait for it) is read at the end of group i and
    // names the unit of group i + 2, whose rows group i + 1 prefetches: a
    // workgroup is committed at most two units ahead when the tickets run
    // out.  Tickets are handed out in order, so a workgroup that has one past
    // the end takes no more; the last workgroup to finish resets the counts.
    const int nunits = (a.nmb + MPI - 1) / MPI;   // strided: the host keeps G <= nunits
    bool dyn = false;
    if constexpr (VAR == kVarFlat || VAR == kVarTopk || VAR == kVarGrouped) {
        if (a.sched != nullptr) {   // uniform
            if (threadIdx.x == 0) {
                const unsigned long long tag =
                    __hip_atomic_load(&a.sched->tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const unsigned long long word =
                    __hip_atomic_load(&a.sched->word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                sm.dyn = tag == kSchedTag && (unsigned int)(word >> 32) == kSchedTag32;
            }
            __syncthreads();
            dyn = sm.dyn != 0;
        }
    }
    int mb0, mb1;
    {
        const int last = w + a.G * ((nunits - 1 - w) / a.G);
        mb0 = w * MPI;
        mb1 = dyn ? a.nmb : min(last * MPI + MPI, a.nmb);
    }
    const int bbase = y * 16 * NB;
    const int ks0 = wave * HT;
    constexpr int kTopkRows = TopkRows<NB, HL>::kRows;   // top-k: rows the store holds

    // this wave's slice of H, resident for the whole kernel (rows past B reuse
    // row B - 1, their columns are discarded; k past d reads zeros): the first
    // HK k-steps in registers, the last HL in LDS
    bf16x8 hres[NB][HK];
    const bf16x8* hl = nullptr;
    if constexpr (HL > 0) hl = &hls.h[wave][0][0][lane];
    {
        const uint16_t* zero = reinterpret_cast<const uint16_t*>(g_zero16);
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const int b = bbase + n * 16 + r16;
            const uint16_t* hrow = a.H + (size_t)(b < a.B ? b : a.B - 1) * a.d;
#pragma unroll
            for (int s = 0; s < HK; ++s) {
                const int k = FL ? ks0 * 32 + h_pair_k(s, kg) : (ks0 + s) * 32 + kg * 8;
                hres[n][s] = load_bf16x8(k < a.d ? hrow + k : zero);
            }
            if constexpr (HL > 0) {
#pragma unroll
                for (int s = 0; s < HL; ++s) {
                    const int k =
                        FL ? ks0 * 32 + h_pair_k(HK + s, kg) : (ks0 + HK + s) * 32 + kg * 8;
                    hls.h[wave][s][n][lane] = load_bf16x8(k < a.d ? hrow + k : zero);
                }
            }
        }
    }

    // epilogue column of this thread: N-block wave % NB, column lane & 15
    const int ncol = wave % NB;
    const ColCtx cc = col_ctx(a, bbase + ncol * 16 + r16);
    WStage<MPI, KS> sa, sb;
    // rows of this lane's loads: row r16 of each block, or (whole lines)
    // rows lane & 7 and 8 + (lane & 7)
    const uint16_t* wrow[MPI][FL ? 2 : 1];
    const uint16_t* wnext[MPI][FL ? 2 : 1];
    auto rows_of = [&](const uint16_t* (&dst)[MPI][FL ? 2 : 1], const Group& gr)
                       __attribute__((always_inline)) {
        const uint16_t* t[MPI];
#pragma unroll
        for (int h = 0; h < (FL ? 2 : 1); ++h) {
            group_rows<MPI>(t, a.W, gr, FL ? 8 * h + (lane & 7) : r16, a.V, a.d);
#pragma unroll
            for (int j = 0; j < MPI; ++j) dst[j][h] = t[j];
        }
    };
    auto load_stage = [&](WStage<MPI, KS>& st, const uint16_t* (&rows)[MPI][FL ? 2 : 1], int it)
                          __attribute__((always_inline)) {
        if constexpr (FL) {
            load_w_lines<MPI, KS>(st, rows, it, ks0, lane, a.d);
        } else {
            const uint16_t* t[MPI];
#pragma unroll
            for (int j = 0; j < MPI; ++j) t[j] = rows[j][0];
            load_w<MPI, KS>(st, t, it, ks0, kg, a.d);
        }
    };
    const uint32_t even = ((lane >> 3) & 1) ? 0u : ~0u;   // whole lines: even pieces
    // (groups never end at a tile: records are per block)
    constexpr int kNoSeg = INT32_MAX / 2;
    Group cur = group_at<MPI>(mb0, mb1, kNoSeg);
    rows_of(wrow, cur);
    load_stage(sa, wrow, 0);

    uint64_t best = pack_key(-INFINITY, -1);
    Lse lse = lse_empty();
    int buf = 0;
    int stored = 0;   // top-k: blocks in the row store (the workgroup's blocks in walk order)
    int nrec = 0;     // grouped: block records in the store
    // ticket order: first block of the next group's unit (mb1: none)
    int gi = 0;                 // group index
    int dyn_next = (w + a.G) * MPI;
    bool grabbing = dyn;        // no ticket past the end seen yet (uniform)
    unsigned int ticket = 0;    // (thread 0)
    while (true) {
        // (only a workgroup's last unit can be short)
        const int gnext = dyn ? dyn_next : cur.g + a.G * MPI;
        const bool more = gnext < mb1;
        // after the last group the prefetch re-reads this group's first stage
        // (cache hits, never used), keeping every load unconditional
        const Group nxt = more ? group_at<MPI>(gnext, mb1, kNoSeg) : cur;
        rows_of(wnext, nxt);
        // the ticket for the unit of group i + 2 (top-k: only while the row
        // store has room for it)
        const bool take = grabbing && more && gi + 2 >= a.dyn_k0 &&
                          (VAR != kVarTopk || (gi + 3) * MPI * kMBlock <= kTopkRows);   // uniform
        if (take && threadIdx.x == 0)
            ticket = (unsigned int)__hip_atomic_fetch_add(&a.sched->word, 1ull, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);

        // (whole lines: an accumulator per half block)
        f32x4 acc[MPI][FL ? 2 : 1][NB];
#pragma unroll
        for (int j = 0; j < MPI; ++j)
#pragma unroll
            for (int h = 0; h < (FL ? 2 : 1); ++h)
#pragma unroll
                for (int n = 0; n < NB; ++n) acc[j][h][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto mfma_stage = [&](const WStage<MPI, KS>& st, int it) __attribute__((always_inline)) {
            if constexpr (FL) {
                if (HL == 0 || it * KS < HK)
                    mfma_w_lines<NB, MPI, KS, HK>(acc, st, hres, it, even);
                else
                    mfma_w_lines_lds<NB, MPI, KS, HK>(acc, st, hl, it, even);
            } else {
                f32x4 (&a1)[MPI][NB] = *reinterpret_cast<f32x4 (*)[MPI][NB]>(&acc[0][0][0]);
                if (HL == 0 || it * KS < HK)
                    mfma_w<NB, MPI, KS, HK>(a1, st, hres, it);
                else
                    mfma_w_lds<NB, MPI, KS, HK>(a1, st, hl, it);
            }
        };
        // sched_barrier keeps the prefetch ahead of the MFMAs it overlaps
#pragma unroll
        for (int it = 0; it < NIT; it += 2) {
            load_stage(sb, wrow, it + 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_stage(sa, it);
            __builtin_amdgcn_sched_barrier(0);
            if (it + 2 < NIT)
                load_stage(sa, wrow, it + 2);
            else
                load_stage(sa, wnext, 0);
            __builtin_amdgcn_sched_barrier(0);
            mfma_stage(sb, it + 1);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- the waves' partial tiles meet in LDS, summed in wave order ----
#pragma unroll
        for (int j = 0; j < MPI; ++j)
#pragma unroll
            for (int n = 0; n < NB; ++n)
                sm.red[buf][wave][j][n][lane] =
                    FL ? combine_halves(acc[j][0][n], acc[j][FL ? 1 : 0][n]) : acc[j][0][n];
        if (take && threadIdx.x == 0) {   // this group's ticket, back by now
            const int u = a.dyn_k0 * a.G + (int)ticket;
            sm.next_unit[buf] = u < nunits ? u : -1;
        }
        __syncthreads();
        if (dyn) {   // the unit of group i + 2
            if (gi + 2 < a.dyn_k0) {
                dyn_next = (w + (gi + 2) * a.G) * MPI;
            } else if (take) {
                const int u = sm.next_unit[buf];
                if (u < 0) grabbing = false;
                dyn_next = u >= 0 ? u * MPI : mb1;
            } else {
                dyn_next = mb1;
            }
        }
        ++gi;

#pragma unroll
        for (int q = 0; q < (MPI * NB + NW - 1) / NW; ++q) {
            const int jn = wave + NW * q;      // uniform across the wave
            if (jn >= MPI * NB) break;
            const int n = jn % NB;             // == ncol
            const int j = jn / NB;
            if (j >= cur.nvm) continue;        // uniform
            f32x4 v = sm.red[buf][0][j][n][lane];
#pragma unroll
            for (int ww = 1; ww < NW; ++ww) v += sm.red[buf][ww][j][n][lane];
            const int row0 = (cur.g + j) * kMBlock + 4 * kg;
            if constexpr (VAR == kVarLogits) {
                if (cc.ok) {
                    float* dst = a.logits + (size_t)cc.col * a.V;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (row0 + r < a.V) dst[row0 + r] = v[r];
                }
            } else {
                // The allow word is read only when a mask is given, in a copy
                // of the epilogue of its own: where both cases shared one
                // copy, the wait for that read was on the common path, and a
                // wait for one load waits for every load issued before it,
                // the next group's prefetch included.
                auto scores = [&](auto masked, float (&x)[4], float (&s)[4])
                                  __attribute__((always_inline)) {
                    const uint32_t word =
                        decltype(masked)::value ? allow_word(a, cc, row0, true) : ~0u;
                    if constexpr (VAR == kVarTopk)
                        lane_x(a, cc, v, row0, true, word, x);
                    else
                        lane_scores<true>(a, cc, v, row0, true, word, x, s);
                };
                float x[4], s[4];
                if (a.allow)   // uniform
                    scores(std::true_type{}, x, s);
                else
                    scores(std::false_type{}, x, s);
                if constexpr (VAR == kVarTopk) {
                    *reinterpret_cast<uint4*>(
                        &tk.u[ncol * 16 + r16][(stored + j) * kMBlock + 4 * kg]) =
                        uint4{topk_order(x[0]), topk_order(x[1]), topk_order(x[2]),
                              topk_order(x[3])};
                } else if constexpr (VAR == kVarGrouped) {
                    // the block's record for these 16 columns: this wave alone
                    // holds them (no barrier), into the store's next slot
                    uint64_t kb = pack_key(-INFINITY, -1);
                    Lse lb = lse_empty();
                    fold<VAR>(kb, lb, x, s, a.v_offset + row0);
                    column_reduce<VAR>(kb, lb);
                    if (lane < 16) {
                        rec.key[nrec + j][n * 16 + lane] = kb;
                        rec.mx[nrec + j][n * 16 + lane] = lb.mx;
                        rec.sm[nrec + j][n * 16 + lane] = lb.sm;
                    }
                    if (n == 0 && lane == 0) rec.blk[nrec + j] = cur.g + j;
                } else {
                    fold<VAR>(best, lse, x, s, a.v_offset + row0);
                }
            }
        }
        // the next group writes the other buffer; this one is rewritten two
        // groups on, after every wave has passed the next group's barrier
        buf ^= 1;
        if constexpr (VAR == kVarTopk)
            if (threadIdx.x == 0) tk.unit[stored / MPI] = cur.g / MPI;
        stored += cur.nvm;

        if constexpr (VAR == kVarFlat) {
            // flat: one record, after the workgroup's last group
            if (!more) {
                column_reduce<VAR>(best, lse);
                if (lane < 16) {
                    sm.fkey[wave][lane] = best;
                    sm.fmx[wave][lane] = lse.mx;
                    sm.fsm[wave][lane] = lse.sm;
                }
                __syncthreads();
                if (threadIdx.x < 16 * NB) {
                    const int n = threadIdx.x >> 4;
                    const ColCtx c = col_ctx(a, bbase + n * 16 + (threadIdx.x & 15));
                    uint64_t k = pack_key(-INFINITY, -1);
                    Lse l = lse_empty();
                    for (int ww = n; ww < NW; ww += NB) {
                        k = key_max(k, sm.fkey[ww][threadIdx.x & 15]);
                        l = lse_merge(l, Lse{sm.fmx[ww][threadIdx.x & 15],
                                             sm.fsm[ww][threadIdx.x & 15]});
                    }
                    put_record<VAR, false>(a, w, c, k, l);
                }
                __syncthreads();
            }
        }
        if constexpr (VAR == kVarGrouped) {
            // the block records go out when the store is full and after the
            // walk (every wave is past its slot writes at the first barrier)
            nrec += cur.nvm;
            if (!more || nrec + MPI > BlockRecSmem<NB>::kSlots) {   // uniform
                __syncthreads();
                for (int e = threadIdx.x; e < nrec * 16 * NB; e += 64 * NW) {
                    const int sl = e / (16 * NB);
                    const int c = e % (16 * NB);
                    const ColCtx cx = col_ctx(a, bbase + c);
                    put_record<VAR, false>(a, rec.blk[sl], cx, rec.key[sl][c],
                                           Lse{rec.mx[sl][c], rec.sm[sl][c]});
                }
                __syncthreads();
                nrec = 0;
            }
        }

        if (!more) break;
        cur = nxt;
#pragma unroll
        for (int j = 0; j < MPI; ++j)
#pragma unroll
            for (int h = 0; h < (FL ? 2 : 1); ++h) wrow[j][h] = wnext[j][h];
    }
    if constexpr (VAR == kVarGrouped) {
        // stage 2's per-row [key, count] pairs start cleared (after the walk:
        // no store is pending during it)
        if (a.gsel && blockIdx.x == 0 && blockIdx.y == 0)
            for (int b = threadIdx.x; b < 2 * a.B; b += blockDim.x)
                a.gsel[kGselStride * (b >> 1) + (b & 1)] = 0ull;
    }
    if (dyn && threadIdx.x == 0) {
        // every ticket of this workgroup has returned (each was read back);
        // the last workgroup out resets the counts for the next call
        const unsigned long long e = __hip_atomic_fetch_add(&a.sched->exits, 1ull, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
        if (e == (unsigned long long)(a.G - 1)) {
            __hip_atomic_store(&a.sched->word, (unsigned long long)kSchedTag32 << 32,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.sched->exits, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    if constexpr (VAR == kVarTopk) {
        // every row of the workgroup's units is in LDS, store row r being
        // global id row_id(ids, r): each wave selects for its columns wave,
        // wave + NW, ... all at once
        static_assert((16 * NB) % NW == 0, "every wave selects for the same number of columns");
        constexpr int C = 16 * NB / NW;
        constexpr int kRows = TopkRows<NB, HL>::kRows;
        // rows past the workgroup's hold no candidate
        const int nr = stored * kMBlock;
        for (int e = threadIdx.x; e < 16 * NB * (kRows - nr); e += 64 * NW)
            tk.u[e % (16 * NB)][nr + e / (16 * NB)] = 0u;
        __syncthreads();
        uint32_t* uc[C];
        size_t o[C];
        int nc = 0;
#pragma unroll
        for (int q = 0; q < C; ++q) {
            const int cl = wave + NW * q;
            const bool ok = bbase + cl < a.B;
            nc += ok ? 1 : 0;   // valid columns come first
            uc[q] = tk.u[cl];
            o[q] = ((size_t)(bbase + (ok ? cl : 0)) * a.G + w) * a.topk_len;
        }
        const RowIds ids{a.v_offset, MPI * kMBlock, tk.unit};
        if (nc > 0) {
            if (a.topk_dense)
                topk_write_dense<C>(a, nc, uc, nr, o);
            else
                topk_select_columns<C, kRows / 64>(a, nc, uc, nr, ids, o);
        }
    }
}

template <int NB, int MPI, int KS, int NW, int HK, int HL, int VAR>
static hipError_t launch_res(const Stage1Args& a, int grid_y, hipStream_t stream) {
    if constexpr (VAR == kVarTopk && !topk_fits<NB, MPI, NW, HL>()) {
        return hipErrorInvalidValue;   // the row store does not fit next to this shape's LDS
    } else {
        const dim3 grid = a.xcd_pair ? dim3(a.G * grid_y) : dim3(a.G, grid_y);
        hipLaunchKernelGGL((resident_kernel<NB, MPI, KS, NW, HK, HL, VAR>), grid, dim3(64 * NW), 0,
                           stream, a);
        return hipGetLastError();
    }
}

// The shapes of FS_RESIDENT_SHAPES (fs_plan.h): their top-k column must say
// whether the row store fits in LDS beside the shape's own areas.
#define FS_RES_CHECK(NB_, MPI_, KS_, NW_, HK_, HL_, TK_)          \
    static_assert(topk_fits<NB_, MPI_, NW_, HL_>() == (TK_ != 0), \
                  "top-k column of FS_RESIDENT_SHAPES");
FS_RESIDENT_SHAPES(FS_RES_CHECK)
#undef FS_RES_CHECK

#define FS_RES_MATCH(NB_, MPI_, KS_, NW_, HK_, HL_) \
    (c.nb == NB_ && c.mpi == MPI_ && c.ks == KS_ && c.nw == NW_ && c.hk == HK_ && c.hl == HL_)

template <int VAR>
static hipError_t launch_res_var(const Stage1Args& a, int grid_y, const ResidentConfig& c,
                                 hipStream_t stream) {
#define FS_RES(NB_, MPI_, KS_, NW_, HK_, HL_, TK_)    \
    if (FS_RES_MATCH(NB_, MPI_, KS_, NW_, HK_, HL_)) \
        return launch_res<NB_, MPI_, KS_, NW_, HK_, HL_, VAR>(a, grid_y, stream);
    FS_RESIDENT_SHAPES(FS_RES)
#undef FS_RES
    return hipErrorInvalidValue;
}

hipError_t launch_resident(int variant, const Stage1Args& a, int grid_y, const ResidentConfig& c,
                           hipStream_t stream) {
    switch (variant) {
        case kVarFlat: return launch_res_var<kVarFlat>(a, grid_y, c, stream);
        case kVarGrouped: return launch_res_var<kVarGrouped>(a, grid_y, c, stream);
        case kVarLogits: return launch_res_var<kVarLogits>(a, grid_y, c, stream);
        case kVarTopk: return launch_res_var<kVarTopk>(a, grid_y, c, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fs

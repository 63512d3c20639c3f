// Stage 1 for large batches (32 < B <= 256 columns per workgroup) with the W
// rows streamed straight into registers and the sampling epilogue fused in
// ("FlashSampling: Fast and Memory-Efficient Exact Sampling", Abstract;
// FlashSampling explainer on aitrends.kr, Stage 1).
//
// A workgroup of 8 waves owns a balanced, contiguous range of 16-row
// vocabulary blocks and walks it in tiles of 256 rows.  Each wave owns 32 rows
// of a tile against all NT = 16 RB batch columns: its W fragments go from
// global memory straight into a ring of PF k-steps of registers (the W stream
// never touches LDS, and its loads keep PF k-steps in flight across tile
// boundaries), while H goes in chunks of KCS k-steps through registers into
// two LDS stages shared by the waves.  Only the H chunks need the waves in
// step (one barrier per chunk); v_mfma_f32_16x16x32_bf16 with W as the A
// operand (16 rows) and H as B (16 columns).
//
// Every global load of the loop is issued so that the compiler does not track
// it (load_untracked), and the loop waits for exactly the loads it needs with
// counted s_waitcnt vmcnt: the compiler's own bookkeeping loses count across
// the loop's back edge and would otherwise drain every load in flight, W
// prefetch included, at the start of each chunk.
//
// The rows of a tile are dealt to the waves in groups of four consecutive rows
// (tile row ((4 j + g) 8 + wave) 4 + r for block j, group g, row r), so that
// a range's last, partial tile still spreads its rows over every wave (one
// wave streaming a partial tile alone would be slow), while each lane's four
// output rows stay consecutive ids: one Philox block serves them.
//
// After each tile the waves fold its logits into per-column winners
// (temperature, masks, Philox-Gumbel noise) and merge them into a per-wave LDS
// row; the waves' rows meet at the end and become the workgroup's record.
#include "fs_device.h"
#include "fs_epilogue.h"
#include "fs_internal.h"
#include "fs_mfma.h"

#include <type_traits>
#include <utility>

namespace fs {

namespace {

constexpr int kRWaves = 8;

template <int N>
__device__ __forceinline__ void rows_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// tile row of A-operand row `ar` (0..15) of block j of wave `wave`: block j
// covers tile rows 128 j .. 128 j + 127 across the waves
__device__ __forceinline__ int rows_tile_row(int wave, int j, int ar) {
    return ((j * 4 + (ar >> 2)) * kRWaves + wave) * 4 + (ar & 3);
}

// The grouped variant keeps a record per 16-row vocabulary block, so each
// block of a tile lies in one wave: block j of wave `wave` is the tile's
// block j kRWaves + wave (tile rows 16 (j kRWaves + wave) ..), and the
// block's record is one column reduction of that wave's MFMA tile.  Block
// j = 0 still covers tile rows 0 .. 127.
template <int VAR>
__device__ __forceinline__ int rows_row(int wave, int j, int ar) {
    if constexpr (VAR == kVarGrouped)
        return (j * kRWaves + wave) * 16 + ar;
    else
        return rows_tile_row(wave, j, ar);
}

// The W ring is refilled in groups of GQ k-steps: after k-step kk with
// kk % GQ == GQ - 1, the loads of k-steps kk + PF - GQ + 1 .. kk + PF go out
// back to back, so that each row is read in runs of 64 GQ bytes (whole
// 128-byte lines leave the L1 cache as one request, and DRAM pages see runs
// instead of single lines).  The load of k-step kk thus went out at the end of
// k-step e = (kk | (GQ - 1)) - PF, and the wait before k-step kk lets these
// loads stay in flight: the later members of its group and the later groups
// ((PF - 1 - kk % GQ) JN loads), and the H part loads issued since, at the
// k-steps of this chunk from e + 1 on that are multiples of KP (parts of the
// previous chunk are not counted: a wait for fewer younger loads than there
// are waits longer, never shorter).
constexpr int rows_h_issues(int kk, int PF, int KP, int GQ) {
    int n = 0;
    for (int q = (kk | (GQ - 1)) - PF + 1 < 0 ? 0 : (kk | (GQ - 1)) - PF + 1; q <= kk; ++q)
        n += q % KP == 0;
    return n;
}
constexpr int rows_w_younger(int kk, int PF, int JN, int GQ) { return (PF - 1 - kk % GQ) * JN; }

template <typename F, int... I>
__device__ __forceinline__ void rows_static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void rows_static_for(F&& f) {
    rows_static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int RB, int KCS>
struct RowsGeom {
    static constexpr int kNT = RB * 16;
    static constexpr int kStage = KCS * kNT * 64;               // bytes of one H stage
    static constexpr int kHL = kStage / 1024 / kRWaves;         // direct loads per wave per chunk
    static_assert(kHL >= 1 && kStage % (1024 * kRWaves) == 0, "H stage");
};

// Block records held in LDS until the kernel ends (grouped variant): the
// first NREC blocks of the row range; the later ones are stored as their
// tiles end.  A record store inside the loop has to complete before the next
// counted wait, which drains the W loads in flight with it.
template <int NT, int NREC>
struct RowsRecs {
    float m[NREC][NT];
    int32_t idx[NREC][NT];
    float L[NREC][NT];
};
struct RowsNoRecs {};

// LDS-held block records: 64 blocks at 64 columns (48 KiB beside the 64 KiB
// of H stages); none at more columns, whose H stages leave too little room.
template <int RB, int VAR>
constexpr int rows_nrec() { return VAR == kVarGrouped && RB == 4 ? 64 : 0; }

template <int RB, int KCS, int NREC>
struct RowsSmem {
    alignas(1024) char hs0[RowsGeom<RB, KCS>::kStage];   // H stages (two arrays: each
    alignas(1024) char hs1[RowsGeom<RB, KCS>::kStage];   // chunk names its own)
    uint64_t key[kRWaves][RB * 16];   // per-wave column winners
    ColCtxSmem<RB * 16> cols;
    std::conditional_t<(NREC > 0), RowsRecs<RB * 16, NREC>, RowsNoRecs> recs;
};

// A 16-byte global load the compiler does not track: the caller waits for it
// with s_waitcnt vmcnt before the first use of the result, counting every
// load issued after it, and neither copies nor spills the result before then
// (the loop keeps each one in a fixed register of its ring).
__device__ __forceinline__ bf16x8 load_untracked(const uint16_t* p) {
    u32x4 r;
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p) : "memory");
    return __builtin_bit_cast(bf16x8, r);
}

}  // namespace

// RB 16-column blocks per workgroup, KRA 16-row blocks per wave and tile,
// chunks of KCS k-steps, a W ring of PF k-steps refilled GQ at a time.  LEAN: the flat epilogue for
// calls with one Philox key and no allow mask (a kernel of its own: beside
// the general epilogue it would not fit in registers).
template <int RB, int KRA, int KCS, int PF, int GQ, int VAR, bool LEAN>
__global__ __launch_bounds__(64 * kRWaves, 1) void rows_kernel(Stage1Args a) {
    static_assert(VAR == kVarFlat || VAR == kVarLogits || VAR == kVarGrouped, "variant");
    static_assert(!LEAN || VAR == kVarFlat, "lean epilogue: flat only");
    static_assert(KRA >= 1 && KRA <= 4 && KCS % PF == 0 && (GQ & (GQ - 1)) == 0 && PF % GQ == 0 &&
                      PF >= 2 * GQ,
                  "shape");
    using Geo = RowsGeom<RB, KCS>;
    constexpr int NT = Geo::kNT;
    constexpr int HL = Geo::kHL;
    constexpr int kRMT = kRWaves * KRA * 16;   // rows per tile
    constexpr int NREC = rows_nrec<RB, VAR>();
    __shared__ RowsSmem<RB, KCS, NREC> sm;

    // row range w and column group y (see resident_kernel for the XCD pairing)
    int w, y;
    if (a.xcd_pair) {
        const int Lg = blockIdx.x;
        const int per = 8 * a.ny;
        y = (Lg % per) / 8;
        w = (Lg / per) * 8 + (Lg % 8);
    } else {
        w = blockIdx.x;
        y = blockIdx.y;
    }
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int r16 = lane & 15;
    const int kg = lane >> 4;
    const int bbase = y * NT;
    const int row0 = part_begin(w, a.nmb, a.G) * kMBlock;
    const int row_end = min(part_begin(w + 1, a.nmb, a.G) * kMBlock, a.V);
    const int nks = a.d / 32;
    const int nch = nks / KCS;                                   // chunks per tile
    // Each row range walks d from its own starting chunk (and wraps): rows of
    // W lie d elements apart, a power of two at the usual sizes, so ranges
    // that all read the same offset at once would load a few HBM channels
    // and leave the rest idle.  The sum over d does not depend on the order.
    const int rot = w % nch;
    const int ntiles = (row_end - row0 + kRMT - 1) / kRMT;       // >= 1 (G <= nmb)
    const int nsteps = ntiles * nks;

    // the call's own key and step (uniform): the lean epilogue's noise when
    // no per-row seeds are given
    const uint32_t ukey0 = a.noise.k0, ukey1 = a.noise.k1;
    const uint32_t ustep = a.noise.step_ptr ? *a.noise.step_ptr : a.noise.step;
    // rows at or past `lim` are out: past the range, past V or at or past n_valid
    const int lim = min(row_end, a.n_valid - a.v_offset);

    col_ctx_store(sm.cols, a, bbase);
    for (int e = tid; e < kRWaves * NT; e += 64 * kRWaves)
        (&sm.key[0][0])[e] = pack_key(-INFINITY, -1);
    __syncthreads();

    // H chunks: piece i of this lane goes to LDS row 16 q + (lane >> 2), slot
    // lane & 3 of a stage (q = wave HL + i; row kk NT + col holds 64 bytes of
    // column col at k-step kk, its 16-byte pieces swizzled: piece p at slot
    // p ^ ((col >> 2) & 3), so that the fragment reads of 16 columns are
    // conflict-free); the lanes of a wave write 1 KiB contiguously.  A wave's
    // HL pieces share the k-step kk and the slot, their columns step by 16.
    static_assert(NT % (16 * HL) == 0, "a wave's H pieces lie in one k-step");
    const int hr = 16 * wave * HL + (lane >> 2);
    const int hcol = hr % NT;
    const int hk = (hr / NT) * 32 + (((lane & 3) ^ ((hcol >> 2) & 3)) << 3);
    // A chunk's H goes through registers in HP parts of HLP loads: part p is
    // loaded at k-step p KP of the previous chunk and written to LDS KP
    // k-steps later (two parts where a whole chunk in registers would not
    // fit beside the accumulators and the W ring).
    constexpr int HP = RB * KRA >= 32 ? 2 : 1;
    constexpr int HLP = HL / HP;
    constexpr int KP = KCS / HP;
    static_assert(HL % HP == 0 && KCS % HP == 0 && (KCS / HP) % GQ == 0, "H parts");
    bf16x8 hreg[HLP];
    auto load_h = [&](int cg, int part) __attribute__((always_inline)) {   // chunk cg % nch of its tile
        // (the addresses are formed here, per part, from an opaque column:
        // hoisted out of the loop they would take 2 HL registers)
        int c0 = bbase + hcol;
        asm volatile("" : "+v"(c0));
        const int k = hk + ((cg + rot) % nch) * KCS * 32;
#pragma unroll
        for (int ii = 0; ii < HLP; ++ii) {
            const int i = part * HLP + ii;
            const int b = min(c0 + 16 * i, a.B - 1);   // padding columns, discarded
            hreg[ii] = load_untracked(a.H + (size_t)b * a.d + k);
        }
    };
    auto store_h = [&](char* st, int part) __attribute__((always_inline)) {
#pragma unroll
        for (int ii = 0; ii < HLP; ++ii)
            *reinterpret_cast<bf16x8*>(st + (wave * HL + part * HLP + ii) * 1024 + lane * 16) =
                hreg[ii];
    };
    // W fragments of global k-step g (tile g / nks): rows past the range re-read
    // its last row (their results are discarded)
    int ld_tile = 0, ld_ks = 0;   // the k-step the next W load is for (advanced by one per load)
    bf16x8 wr[PF][KRA];
    // (jn: blocks loaded, KRA, or 1 in a short last tile whose other blocks
    // hold no rows: a load whose result is never read must not be issued,
    // the compiler would reuse its registers while it is in flight)
    auto load_w = [&](bf16x8 (&dst)[KRA], auto jn) __attribute__((always_inline)) {
        const int base = row0 + ld_tile * kRMT;
        const int ks = ld_ks + rot * KCS;
        const int k = (ks < nks ? ks : ks - nks) * 32 + kg * 8;
#pragma unroll
        for (int j = 0; j < decltype(jn)::value; ++j) {
            const int r = min(base + rows_row<VAR>(wave, j, r16), row_end - 1);
            dst[j] = load_untracked(a.W + (size_t)r * a.d + k);
        }
        if (ld_tile * nks + ld_ks + 1 < nsteps) {   // clamp at the last k-step
            if (++ld_ks == nks) {
                ld_ks = 0;
                ++ld_tile;
            }
        }
    };

    f32x4 acc[KRA][RB];
#pragma unroll
    for (int j = 0; j < KRA; ++j)
#pragma unroll
        for (int n = 0; n < RB; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // prologue: H chunk 0 into stage 0, W k-steps 0 .. PF-1 in flight
#pragma unroll
    for (int part = 0; part < HP; ++part) {
        load_h(0, part);
        rows_wait_vmcnt<0>();
        __builtin_amdgcn_sched_barrier(0);
        store_h(sm.hs0, part);
    }
#pragma unroll
    for (int p = 0; p < PF; ++p) load_w(wr[p], std::integral_constant<int, KRA>{});

    const int nchunks = ntiles * nch;   // even: the host requires nch even
    // one chunk: read from stage `st`, the next chunk goes to `other`
    // (the chunk that ends a tile is always the second of a pair: nch is
    // even).  A tile with at most 128 rows left in the range (`half`) has
    // rows in block j = 0 only (rows_row): the other blocks' loads,
    // MFMAs and noise are skipped.  Such a tile comes last and runs in a loop
    // of its own, entered with no load in flight, where every k-step issues
    // one W load per wave: the waits count JN loads per k-step.
    auto chunk = [&](int cg, const char* st, char* other, auto second, auto half)
                     __attribute__((always_inline)) {
        constexpr int JN = decltype(half)::value ? 1 : KRA;   // blocks with rows
        const auto jn = std::integral_constant<int, JN>{};
        // every wave's part of chunk cg is in `st` (written at the end of the
        // previous chunk), and every wave is past its reads of `other`
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes done
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const int cnext = cg + 1 < nchunks ? cg + 1 : cg;   // the last chunk loads itself again
        rows_static_for<KCS>([&](auto kc) __attribute__((always_inline)) {
            constexpr int kk = decltype(kc)::value;
            if constexpr (kk % KP == 0) {
                if constexpr (kk > 0) {
                    // H part kk / KP - 1 has landed once only the KP JN W
                    // refills since are younger
                    rows_wait_vmcnt<KP * JN>();
                    __builtin_amdgcn_sched_barrier(0);
                    store_h(other, kk / KP - 1);
                }
                load_h(cnext, kk / KP);
            }
            // W k-step cg KCS + kk has landed once only the ring's other
            // (PF - 1) JN loads and the H parts issued since are younger
            rows_wait_vmcnt<rows_w_younger(kk, PF, JN, GQ) + rows_h_issues(kk, PF, KP, GQ) * HLP>();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int n = 0; n < RB; ++n) {
                const int col = n * 16 + r16;
                const bf16x8 bf = *reinterpret_cast<const bf16x8*>(
                    st + (kk * NT + col) * 64 + ((kg ^ ((col >> 2) & 3)) << 4));
#pragma unroll
                for (int j = 0; j < JN; ++j)
                    acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wr[kk % PF][j], bf,
                                                                        acc[j][n], 0, 0, 0);
            }
            // issue order: each fragment's read two fragments ahead of its
            // MFMAs (the compiler would read all RB fragments first, 4 RB
            // registers, which RB = 16 cannot afford)
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int n = 0; n < RB - 2; ++n) {
                __builtin_amdgcn_sched_group_barrier(0x008, JN, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * JN, 0);
            if constexpr (kk % GQ == GQ - 1) {   // k-steps kk + PF - GQ + 1 .. kk + PF
                rows_static_for<GQ>([&](auto qc) __attribute__((always_inline)) {
                    load_w(wr[(kk - GQ + 1 + decltype(qc)::value) % PF], jn);
                });
            }
        });
        // the last H part of chunk cg + 1 into `other`
        rows_wait_vmcnt<KP * JN>();
        __builtin_amdgcn_sched_barrier(0);
        store_h(other, HP - 1);

        if (decltype(second)::value && (cg + 1) % nch == 0) {
            // the tile is complete: fold its logits into this wave's column
            // winners (the column contexts come from LDS; the refills of the
            // next tile's first k-steps stay in flight meanwhile)
            const int tbase = row0 + (cg / nch) * kRMT;
            // the column contexts are read again for every tile: an index the
            // compiler cannot see through keeps it from hoisting the reads out
            // of the loop, where 16 RB column contexts would not fit in registers
            int fresh = 0;
            asm volatile("" : "+v"(fresh));
            auto fold_tile = [&](auto masked) __attribute__((always_inline)) {
                rows_static_for<RB>([&](auto nc) {
                    constexpr int n = decltype(nc)::value;
                    const ColCtx cx = col_ctx_load(sm.cols, a, bbase, n * 16 + r16 + fresh);
                    uint64_t best = pack_key(-INFINITY, -1);
                    Lse unused = lse_empty();
                    rows_static_for<JN>([&](auto jc) {
                        constexpr int j = decltype(jc)::value;
                        const int rowg = tbase + rows_row<VAR>(wave, j, 4 * kg);   // 4 consecutive rows
                        const bool ok = rowg < row_end;
                        if constexpr (VAR == kVarLogits) {
                            if (cx.ok && ok) {
                                float* dst = a.logits + (size_t)cx.col * a.V;
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    if (rowg + r < a.V) dst[rowg + r] = acc[j][n][r];
                            }
                        } else if constexpr (VAR == kVarGrouped) {
                            // the record of block j kRWaves + wave for these
                            // 16 columns (block-major, slot = the block)
                            const uint32_t word =
                                decltype(masked)::value ? allow_word(a, cx, rowg, ok) : ~0u;
                            float x[4], sc[4];
                            lane_scores(a, cx, acc[j][n], rowg, ok, word, x, sc);
                            uint64_t kb = pack_key(-INFINITY, -1);
                            Lse lb = lse_empty();
                            fold<kVarGrouped>(kb, lb, x, sc, a.v_offset + rowg);
                            column_reduce<kVarGrouped>(kb, lb);
                            const int blk_row = tbase + (j * kRWaves + wave) * 16;
                            const int slot = (blk_row - row0) / kMBlock;   // uniform
                            if (lane < 16 && blk_row < row_end) {
                                bool held = false;
                                if constexpr (NREC > 0) {
                                    if (slot < NREC) {
                                        // the values put_record would write,
                                        // stored at the end of the kernel
                                        const int32_t id = key_index(kb);
                                        const int c = n * 16 + lane;
                                        sm.recs.m[slot][c] = id >= 0 ? key_score(kb) : -INFINITY;
                                        sm.recs.idx[slot][c] = id;
                                        sm.recs.L[slot][c] = cx.greedy ? lb.mx : lse_value(lb);
                                        held = true;
                                    }
                                }
                                if (!held)
                                    put_record<kVarGrouped, false>(a, blk_row / kMBlock, cx, kb,
                                                                   lb);
                            }
                        } else {
                            const uint32_t word =
                                decltype(masked)::value ? allow_word(a, cx, rowg, ok) : ~0u;
                            float x[4], sc[4];
                            lane_scores(a, cx, acc[j][n], rowg, ok, word, x, sc);
                            fold<kVarFlat>(best, unused, x, sc, a.v_offset + rowg);
                        }
                    });
                    if constexpr (VAR == kVarFlat) {
                        column_reduce<kVarFlat>(best, unused);
                        if (lane < 16) {
                            uint64_t& slot = sm.key[wave][n * 16 + lane];
                            slot = key_max(slot, best);
                        }
                    }
                });
            };
            // The lean epilogue, for calls with one key and no allow mask:
            // the Philox key schedule stays scalar, each lane keeps its best
            // score and row as floats (a NaN score never compares greater;
            // rows come in increasing order, so a tie keeps the lowest id),
            // and rows at or past `lim` never take.  Temperature and noise as
            // in lane_scores; greedy columns take no noise.
            auto fold_lean = [&]() __attribute__((always_inline)) {
                // the key and step, opaque per tile: the twenty round keys are
                // then formed on the scalar unit here instead of being kept
                // through the loop
                uint32_t k0 = ukey0, k1 = ukey1, st = ustep;
                asm volatile("" : "+s"(k0), "+s"(k1), "+s"(st));
                rows_static_for<RB>([&](auto nc) {
                    constexpr int n = decltype(nc)::value;
                    const int c = n * 16 + r16 + fresh;
                    const float inv_t = sm.cols.inv_t[c];
                    const bool noisy = (sm.cols.flags[c] & 3u) == 1u;   // inside B, not greedy
                    float bs = -INFINITY;
                    int bi = -1;
                    rows_static_for<JN>([&](auto jc) {
                        constexpr int j = decltype(jc)::value;
                        const int rowg = tbase + rows_row<VAR>(wave, j, 4 * kg);
                        const int gid0 = a.v_offset + rowg;
                        float g[4] = {0.f, 0.f, 0.f, 0.f};
                        if (noisy) {
                            const uint4 rw = philox4x32_10(
                                make_uint4((uint32_t)gid0 >> 2, (uint32_t)(bbase + c), st,
                                           kStreamToken),
                                k0, k1);
                            g[0] = gumbel_from_word(rw.x);
                            g[1] = gumbel_from_word(rw.y);
                            g[2] = gumbel_from_word(rw.z);
                            g[3] = gumbel_from_word(rw.w);
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float sv = acc[j][n][r] * inv_t + g[r];
                            const bool take = sv > bs && rowg + r < lim;
                            bs = take ? sv : bs;
                            bi = take ? gid0 + r : bi;
                        }
                    });
                    uint64_t best = pack_key(bi >= 0 ? bs : -INFINITY, bi);
                    Lse unused = lse_empty();
                    column_reduce<kVarFlat>(best, unused);
                    if (lane < 16) {
                        uint64_t& slot = sm.key[wave][n * 16 + lane];
                        slot = key_max(slot, best);
                    }
                    // one column block at a time: interleaved, their noise
                    // chains would not fit beside the accumulators
                    __builtin_amdgcn_sched_barrier(0);
                });
            };
            if constexpr (VAR == kVarLogits || VAR == kVarGrouped) {
                fold_tile(std::integral_constant<bool, VAR == kVarGrouped>{});
                // the loop's counted waits assume loads only: stores may
                // complete out of order with them, so none stays in flight
                // (a tile whose block records all stay in LDS stored nothing)
                if (VAR == kVarLogits || (tbase - row0) / kMBlock + kRMT / kMBlock > NREC)
                    rows_wait_vmcnt<0>();
            } else if constexpr (LEAN) {
                fold_lean();
            } else {
                fold_tile(std::true_type{});   // the general epilogue (tests allow only if given)
            }
#pragma unroll
            for (int j = 0; j < JN; ++j)
#pragma unroll
                for (int n = 0; n < RB; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    // only a range's last tile can be short: the full tiles first, then a
    // half tile in a loop of its own
    const bool tail_half = KRA > 1 && row_end - (row0 + (ntiles - 1) * kRMT) <= 128;
    const int nfull = (tail_half ? ntiles - 1 : ntiles) * nch;
    int cg = 0;
    for (; cg < nfull; cg += 2) {
        chunk(cg, sm.hs0, sm.hs1, std::false_type{}, std::false_type{});
        chunk(cg + 1, sm.hs1, sm.hs0, std::true_type{}, std::false_type{});
    }
    // nothing stays in flight from one loop into the other: the compiler
    // may place the ring in other registers there
    rows_wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    for (; cg < nchunks; cg += 2) {
        chunk(cg, sm.hs0, sm.hs1, std::false_type{}, std::true_type{});
        chunk(cg + 1, sm.hs1, sm.hs0, std::true_type{}, std::true_type{});
    }
    // the trailing loads (refills past the end) land before the wave goes on
    rows_wait_vmcnt<0>();

    if constexpr (VAR == kVarGrouped) {
        // stage 2's per-row [key, count] pairs start cleared
        if (a.gsel && blockIdx.x == 0 && blockIdx.y == 0)
            for (int b = tid; b < 2 * a.B; b += 64 * kRWaves)
                a.gsel[kGselStride * (b >> 1) + (b & 1)] = 0ull;
        if constexpr (NREC > 0) {
            // the block records held in LDS (block-major, as put_record)
            __syncthreads();
            const int nheld = min((row_end - row0 + kMBlock - 1) / kMBlock, NREC);
            for (int e = tid; e < nheld * NT; e += 64 * kRWaves) {
                const int slot = e / NT, c = e % NT;
                if (bbase + c < a.B) {
                    const size_t o = (size_t)(row0 / kMBlock + slot) * a.rec_cols + bbase + c;
                    a.pm[o] = sm.recs.m[slot][c];
                    a.pidx[o] = sm.recs.idx[slot][c];
                    a.pL[o] = sm.recs.L[slot][c];
                }
            }
        }
    }
    if constexpr (VAR == kVarFlat) {
        __syncthreads();
        for (int c = tid; c < NT; c += 64 * kRWaves) {
            uint64_t k = sm.key[0][c];
#pragma unroll
            for (int ww = 1; ww < kRWaves; ++ww) k = key_max(k, sm.key[ww][c]);
            const ColCtx cc = col_ctx_load(sm.cols, a, bbase, c);
            put_record<kVarFlat, false>(a, w, cc, k, lse_empty());
        }
    }
}

template <int RB, const RowsShape& S, int VAR>
static hipError_t launch_rows_shape(const Stage1Args& a, int grid_y, hipStream_t stream) {
    static_assert(S.nt == 16 * RB, "shape");
    const dim3 grid = a.xcd_pair ? dim3(a.G * grid_y) : dim3(a.G, grid_y);
    const dim3 block(64 * kRWaves);
    if (VAR == kVarFlat && a.allow == nullptr && a.noise.seeds == nullptr)
        hipLaunchKernelGGL((rows_kernel<RB, S.kra, S.kcs, S.pf, S.gq, VAR, VAR == kVarFlat>), grid,
                           block, 0, stream, a);
    else
        hipLaunchKernelGGL((rows_kernel<RB, S.kra, S.kcs, S.pf, S.gq, VAR, false>), grid, block, 0,
                           stream, a);
    return hipGetLastError();
}

template <int VAR>
static hipError_t launch_rows_var(const Stage1Args& a, int nt, int grid_y, hipStream_t stream) {
    if (nt == kRows64.nt) return launch_rows_shape<4, kRows64, VAR>(a, grid_y, stream);
    if (nt == kRows128.nt) return launch_rows_shape<8, kRows128, VAR>(a, grid_y, stream);
    if (nt == kRows256.nt) return launch_rows_shape<16, kRows256, VAR>(a, grid_y, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_rows(int variant, const Stage1Args& a, int nt, int grid_y, hipStream_t stream) {
    if (variant == kVarFlat) return launch_rows_var<kVarFlat>(a, nt, grid_y, stream);
    if (variant == kVarGrouped) {
        // (at 256 columns the grouped epilogue would spill inside the loop:
        // larger batches take several 128-column groups)
        if (nt == kRows64.nt) return launch_rows_shape<4, kRows64, kVarGrouped>(a, grid_y, stream);
        if (nt == kRows128.nt) return launch_rows_shape<8, kRows128, kVarGrouped>(a, grid_y, stream);
        return hipErrorInvalidValue;
    }
    if (variant == kVarLogits) return launch_rows_var<kVarLogits>(a, nt, grid_y, stream);
    return hipErrorInvalidValue;
}

}  // namespace fs

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
constexpr int kRA = 2;                       // 16-row blocks per wave and tile
constexpr int kRMT = kRWaves * kRA * 16;     // 256 rows per tile

template <int N>
__device__ __forceinline__ void rows_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// tile row of A-operand row `ar` (0..15) of block j of wave `wave`
__device__ __forceinline__ int rows_tile_row(int wave, int j, int ar) {
    return ((j * 4 + (ar >> 2)) * kRWaves + wave) * 4 + (ar & 3);
}

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

template <int RB, int KCS>
struct RowsSmem {
    alignas(1024) char hs0[RowsGeom<RB, KCS>::kStage];   // H stages (two arrays: each
    alignas(1024) char hs1[RowsGeom<RB, KCS>::kStage];   // chunk names its own)
    uint64_t key[kRWaves][RB * 16];   // per-wave column winners
    ColCtxSmem<RB * 16> cols;
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

template <int RB, int KCS, int VAR>
__global__ __launch_bounds__(64 * kRWaves, 1) void rows_kernel(Stage1Args a) {
    static_assert(VAR == kVarFlat || VAR == kVarLogits, "variant");
    using Geo = RowsGeom<RB, KCS>;
    constexpr int NT = Geo::kNT;
    constexpr int HL = Geo::kHL;
    constexpr int PF = KCS;   // W ring depth: one chunk of k-steps
    __shared__ RowsSmem<RB, KCS> sm;

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
    // k-steps later (RB = 16 takes two parts: a whole chunk in registers
    // would not fit beside its accumulators and the W ring).
    constexpr int HP = RB == 16 ? 2 : 1;
    constexpr int HLP = HL / HP;
    constexpr int KP = KCS / HP;
    static_assert(HL % HP == 0 && KCS % HP == 0, "H parts");
    bf16x8 hreg[HLP];
    auto load_h = [&](int cg, int part) __attribute__((always_inline)) {   // chunk cg % nch of its tile
        // (the addresses are formed here, per part, from an opaque column:
        // hoisted out of the loop they would take 2 HL registers)
        int c0 = bbase + hcol;
        asm volatile("" : "+v"(c0));
        const int k = hk + (cg % nch) * KCS * 32;
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
    const int trow0 = rows_tile_row(wave, 0, r16);
    const int trow1 = rows_tile_row(wave, 1, r16);
    int ld_tile = 0, ld_ks = 0;   // the k-step the next W load is for (advanced by one per load)
    bf16x8 wr[PF][kRA];
    auto load_w = [&](bf16x8 (&dst)[kRA]) __attribute__((always_inline)) {
        const int base = row0 + ld_tile * kRMT;
        const int rA = min(base + trow0, row_end - 1);
        const int rB = min(base + trow1, row_end - 1);
        const int k = ld_ks * 32 + kg * 8;
        dst[0] = load_untracked(a.W + (size_t)rA * a.d + k);
        dst[1] = load_untracked(a.W + (size_t)rB * a.d + k);
        if (ld_tile * nks + ld_ks + 1 < nsteps) {   // clamp at the last k-step
            if (++ld_ks == nks) {
                ld_ks = 0;
                ++ld_tile;
            }
        }
    };

    f32x4 acc[kRA][RB];
#pragma unroll
    for (int j = 0; j < kRA; ++j)
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
    for (int p = 0; p < PF; ++p) load_w(wr[p]);

    const int nchunks = ntiles * nch;   // even: the host requires nch even
    // one chunk: read from stage `st`, the next chunk goes to `other`
    // (the chunk that ends a tile is always the second of a pair: nch is even)
    auto chunk = [&](int cg, const char* st, char* other, auto second) __attribute__((always_inline)) {
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
                    // H part kk / KP - 1 has landed once only the KP kRA W
                    // refills since are younger
                    rows_wait_vmcnt<KP * kRA>();
                    __builtin_amdgcn_sched_barrier(0);
                    store_h(other, kk / KP - 1);
                }
                load_h(cnext, kk / KP);
            }
            // W k-step cg KCS + kk has landed once only the ring's other
            // (PF - 1) kRA loads and the H parts loaded so far are younger
            rows_wait_vmcnt<(PF - 1) * kRA + (kk / KP + 1) * HLP>();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int n = 0; n < RB; ++n) {
                const int col = n * 16 + r16;
                const bf16x8 bf = *reinterpret_cast<const bf16x8*>(
                    st + (kk * NT + col) * 64 + ((kg ^ ((col >> 2) & 3)) << 4));
#pragma unroll
                for (int j = 0; j < kRA; ++j)
                    acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wr[kk][j], bf, acc[j][n], 0,
                                                                        0, 0);
            }
            // issue order: each fragment's read two fragments ahead of its
            // MFMAs (the compiler would read all RB fragments first, 4 RB
            // registers, which RB = 16 cannot afford)
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int n = 0; n < RB - 2; ++n) {
                __builtin_amdgcn_sched_group_barrier(0x008, kRA, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * kRA, 0);
            load_w(wr[kk]);   // the k-step PF ahead
        });
        // the last H part of chunk cg + 1 into `other`
        rows_wait_vmcnt<KP * kRA>();
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
                    rows_static_for<kRA>([&](auto jc) {
                        constexpr int j = decltype(jc)::value;
                        const int rowg = tbase + rows_tile_row(wave, j, 4 * kg);   // 4 consecutive rows
                        const bool ok = rowg < row_end;
                        if constexpr (VAR == kVarLogits) {
                            if (cx.ok && ok) {
                                float* dst = a.logits + (size_t)cx.col * a.V;
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    if (rowg + r < a.V) dst[rowg + r] = acc[j][n][r];
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
                rows_static_for<RB>([&](auto nc) {
                    constexpr int n = decltype(nc)::value;
                    const int c = n * 16 + r16 + fresh;
                    const float inv_t = sm.cols.inv_t[c];
                    const bool noisy = (sm.cols.flags[c] & 3u) == 1u;   // inside B, not greedy
                    float bs = -INFINITY;
                    int bi = -1;
                    rows_static_for<kRA>([&](auto jc) {
                        constexpr int j = decltype(jc)::value;
                        const int rowg = tbase + rows_tile_row(wave, j, 4 * kg);
                        const int gid0 = a.v_offset + rowg;
                        float g[4] = {0.f, 0.f, 0.f, 0.f};
                        if (noisy) {
                            const uint4 rw = philox4x32_10(
                                make_uint4((uint32_t)gid0 >> 2, (uint32_t)(bbase + c), ustep,
                                           kStreamToken),
                                ukey0, ukey1);
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
                });
            };
            if constexpr (VAR == kVarLogits) {
                fold_tile(std::false_type{});
                // the loop's counted waits assume loads only: stores may
                // complete out of order with them, so none stays in flight
                rows_wait_vmcnt<0>();
            } else if (a.allow != nullptr || a.noise.seeds != nullptr) {
                fold_tile(std::true_type{});   // the general epilogue (tests allow only if given)
            } else {
                fold_lean();
            }
#pragma unroll
            for (int j = 0; j < kRA; ++j)
#pragma unroll
                for (int n = 0; n < RB; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    for (int cg = 0; cg < nchunks; cg += 2) {
        chunk(cg, sm.hs0, sm.hs1, std::false_type{});
        chunk(cg + 1, sm.hs1, sm.hs0, std::true_type{});
    }
    // the trailing loads (refills past the end) land before the wave goes on
    rows_wait_vmcnt<0>();

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

template <int RB, int KCS, int VAR>
static hipError_t launch_rows_shape(const Stage1Args& a, int grid_y, hipStream_t stream) {
    const dim3 grid = a.xcd_pair ? dim3(a.G * grid_y) : dim3(a.G, grid_y);
    hipLaunchKernelGGL((rows_kernel<RB, KCS, VAR>), grid, dim3(64 * kRWaves), 0, stream, a);
    return hipGetLastError();
}

template <int VAR>
static hipError_t launch_rows_var(const Stage1Args& a, int nt, int grid_y, hipStream_t stream) {
    if (nt == 64) return launch_rows_shape<4, kRowsKcs64, VAR>(a, grid_y, stream);
    if (nt == 128) return launch_rows_shape<8, kRowsKcs128, VAR>(a, grid_y, stream);
    if (nt == 256) return launch_rows_shape<16, kRowsKcs256, VAR>(a, grid_y, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_rows(int variant, const Stage1Args& a, int nt, int grid_y, hipStream_t stream) {
    if (variant == kVarFlat) return launch_rows_var<kVarFlat>(a, nt, grid_y, stream);
    if (variant == kVarLogits) return launch_rows_var<kVarLogits>(a, nt, grid_y, stream);
    return hipErrorInvalidValue;
}

}  // namespace fs

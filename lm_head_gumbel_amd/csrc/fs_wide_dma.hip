// Stage 1 for large batches with the tiles fed by direct-to-LDS loads
// (gfx950 global_load_lds_dwordx4), with the sampling epilogue fused in
// ("FlashSampling: Fast and Memory-Efficient Exact Sampling", Abstract;
// FlashSampling explainer on aitrends.kr, Stage 1).
//
// A workgroup of 8 waves owns a balanced range of 16-row vocabulary blocks and
// walks it in tiles of 256 rows against NT = 256 batch columns (the largest
// batches: each W tile is then read once for all of them).  The
// hidden dimension is consumed in chunks of 32 (one MFMA k-step): per chunk the
// W tile (256 rows x 64 bytes) and the H tile (NT rows x 64 bytes) go from
// global memory straight into one of NS LDS stages, without passing through
// registers, so NS - 1 chunks of loads are in flight while one is computed.
// Each wave computes a 128 x NT/4 sub-tile with v_mfma_f32_16x16x32_bf16.
//
// LDS layout: a row is 64 bytes (four 16-byte pieces, eight k each); piece p of
// row r is stored at slot p ^ ((r >> 2) & 3), which makes the fragment reads of
// 16 consecutive rows (one MFMA operand) conflict-free.  The direct loads write
// 64 lanes x 16 bytes = 1 KiB contiguously, 16 rows per instruction; each lane
// therefore fetches the global piece that belongs in its slot.
//
// After the last chunk of a tile the waves fold its logits into per-column
// winners (temperature, masks, Philox-Gumbel noise) exactly as the other
// stage-1 kernels do; the two row-halves' winners meet in LDS at the end.
#include "fs_device.h"
#include "fs_epilogue.h"
#include "fs_internal.h"
#include "fs_mfma.h"

#include <type_traits>
#include <utility>

namespace fs {

namespace {

constexpr int kDThreads = 512;
constexpr int kDMT = 256;   // rows per tile
constexpr int kDKC = 32;    // k per chunk

template <int NT>
struct WideDmaGeom {
    static constexpr int kRows = kDMT + NT;                  // LDS rows per stage
    static constexpr int kStageBytes = kRows * 64;
    static constexpr int kStages = NT == 256 ? 4 : 6;        // 128 or 144 KiB
    static constexpr int kLoads = kRows / 16 / (kDThreads / 64);   // direct loads per thread per chunk
};

template <int NT>
struct WideDmaSmem {
    alignas(1024) char buf[WideDmaGeom<NT>::kStages][WideDmaGeom<NT>::kStageBytes];
    uint64_t fkey[2][NT];
    ColCtxSmem<NT> cols;
};

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// f(std::integral_constant<int, i>{}) for i = 0 .. N-1: indices that are
// constants from the start, so the accumulator array stays in registers
// through the large unrolled epilogue
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace

template <int NT, int VAR>
__global__ __launch_bounds__(kDThreads) void wide_dma_kernel(Stage1Args a) {
    static_assert(NT == 128 || NT == 256, "column tile");
    static_assert(VAR == kVarFlat || VAR == kVarLogits, "variant");
    using Geo = WideDmaGeom<NT>;
    constexpr int NS = Geo::kStages;
    constexpr int L = Geo::kLoads;
    constexpr int WM = 2, WN = 4;
    constexpr int MF = kDMT / WM / 16;   // 8 A fragments per wave
    constexpr int NF = NT / WN / 16;     // 2 or 4 B fragments per wave
    __shared__ WideDmaSmem<NT> sm;

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
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int mb0 = part_begin(w, a.nmb, a.G);
    const int mb1 = part_begin(w + 1, a.nmb, a.G);
    const int row_end = min(mb1 * kMBlock, a.V);   // one past this range's last row
    const int bbase = y * NT;
    const int nchunks = a.d / kDKC;
    const int ntiles = (mb1 - mb0 + 15) / 16;
    const int total = ntiles * nchunks;

    // Direct loads: instruction i of wave `wave` fills LDS rows 16 rb .. 16 rb + 15
    // of a stage, rb = wave * L + i; lane l writes row 16 rb + (l >> 2), slot l & 3,
    // which holds global piece (l & 3) ^ ((row >> 2) & 3).  Element offsets below
    // are relative to the chunk's k = 0 (W: from the range's first row).
    const uint16_t* wbase = a.W + (size_t)mb0 * kMBlock * a.d;
    const int first_row = mb0 * kMBlock;
    int gofs[L];        // element offset of this lane's piece (W rows: for tile 0)
    bool is_w[L];
    int wrow_of[L];     // tile-relative W row (W pieces only)
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int row = 16 * (wave * L + i) + (lane >> 2);
        const int piece = (lane & 3) ^ ((row >> 2) & 3);
        is_w[i] = row < kDMT;
        wrow_of[i] = row;
        if (!is_w[i]) {
            int b = bbase + (row - kDMT);
            b = b < a.B ? b : a.B - 1;   // padding columns reuse row B - 1, discarded later
            gofs[i] = b * a.d + piece * 8;
        } else {
            gofs[i] = piece * 8;
        }
    }
    // W element offsets of this lane's pieces for a tile (rows past the range
    // re-read its last row)
    int wofs[L];
    auto set_tile = [&](int tile) {
#pragma unroll
        for (int i = 0; i < L; ++i) {
            int row = (mb0 + tile * 16) * kMBlock + wrow_of[i];
            row = row < row_end ? row : row_end - 1;
            wofs[i] = (row - first_row) * a.d + gofs[i];
        }
    };
    // issue the direct loads of chunk q (clamped to the last chunk: past the end
    // they refill a stage that is never read) into stage q % NS
    int cur_tile = -1;
    auto issue = [&](int q) {
        q = q < total ? q : total - 1;
        const int t = q / nchunks;
        const int k = (q - t * nchunks) * kDKC;
        if (t != cur_tile) {
            set_tile(t);
            cur_tile = t;
        }
        char* stage = sm.buf[q % NS];
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const uint16_t* src = is_w[i] ? wbase + wofs[i] + k : a.H + gofs[i] + k;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)src,
                (void __attribute__((address_space(3)))*)(stage + (wave * L + i) * 1024), 16, 0, 0);
        }
    };

    // the contexts of the workgroup's columns, read back in every epilogue
    col_ctx_store(sm.cols, a, bbase);
    __syncthreads();

    // per-lane column winners of this wave (one per B fragment)
    uint64_t best[NF];
#pragma unroll
    for (int n = 0; n < NF; ++n) best[n] = pack_key(-INFINITY, -1);
    Lse unused = lse_empty();

    f32x4 acc[MF][NF];
#pragma unroll
    for (int j = 0; j < MF; ++j)
#pragma unroll
        for (int n = 0; n < NF; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LDS byte offset of (row, piece kg) with the swizzle
    auto frag_off = [&](int row) { return row * 64 + ((kg ^ ((row >> 2) & 3)) << 4); };

    // (every range holds at least one block: the host keeps G <= nmb)
#pragma unroll 1
    for (int q = 0; q < NS - 1 && total > 0; ++q) issue(q);

#pragma unroll 1
    for (int s = 0; s < total; ++s) {
        // chunk s has landed once only the NS - 2 younger chunks are pending;
        // the barrier also tells that every wave is done with chunk s - 1
        // (a plain s_barrier: a workgroup fence here would wait for every
        // pending load, the younger chunks included)
        wait_vmcnt<L * (NS - 2)>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(s + NS - 1);   // into the stage of chunk s - 1
        __builtin_amdgcn_sched_barrier(0);

        const int tile = s / nchunks;
        const int c = s - tile * nchunks;
        const int blk0 = mb0 + tile * 16 + wm * MF;
        const int nvalid = min(MF, mb1 - blk0);   // blocks of this wave inside the range
        const char* base = sm.buf[s % NS];
        if (nvalid > 0) {
            bf16x8 bf[NF];
#pragma unroll
            for (int n = 0; n < NF; ++n)
                bf[n] = *reinterpret_cast<const bf16x8*>(
                    base + frag_off(kDMT + wn * (NT / WN) + n * 16 + r16));
#pragma unroll
            for (int j = 0; j < MF; ++j) {
                const bf16x8 af =
                    *reinterpret_cast<const bf16x8*>(base + frag_off(wm * (kDMT / WM) + j * 16 + r16));
#pragma unroll
                for (int n = 0; n < NF; ++n)
                    acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[n], acc[j][n], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);

        if (c + 1 == nchunks) {
            // the tile is complete: fold its logits into the column winners
            // (the column contexts are rebuilt per tile from LDS: registers
            // held through the contraction would spill)
            ColCtx cxs[NF];
            static_for<NF>([&](auto nc) {
                constexpr int n = decltype(nc)::value;
                cxs[n] = col_ctx_load(sm.cols, a, bbase, wn * (NT / WN) + n * 16 + r16);
            });
            // MASKED: the allow words are read here.  Without a mask (a
            // uniform branch) the epilogue issues no memory load at all, so
            // nothing makes the loads of the next chunks wait.
            auto fold_tile = [&](auto masked) {
                static_for<MF>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    if (j < nvalid) {   // uniform
                        const int row0 = (blk0 + j) * kMBlock + 4 * kg;
                        static_for<NF>([&](auto nc) {
                            constexpr int n = decltype(nc)::value;
                            const ColCtx& cx = cxs[n];
                            if constexpr (VAR == kVarLogits) {
                                if (cx.ok) {
                                    float* dst = a.logits + (size_t)cx.col * a.V;
#pragma unroll
                                    for (int r = 0; r < 4; ++r)
                                        if (row0 + r < a.V) dst[row0 + r] = acc[j][n][r];
                                }
                            } else {
                                const uint32_t word =
                                    decltype(masked)::value ? allow_word(a, cx, row0, true) : ~0u;
                                float x[4], sc[4];
                                lane_scores(a, cx, acc[j][n], row0, true, word, x, sc);
                                fold<kVarFlat>(best[n], unused, x, sc, a.v_offset + row0);
                            }
                        });
                    }
                });
            };
            if (a.allow != nullptr)
                fold_tile(std::true_type{});
            else
                fold_tile(std::false_type{});
#pragma unroll
            for (int j = 0; j < MF; ++j)
#pragma unroll
                for (int n = 0; n < NF; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // the trailing loads (refills past the end) must land before the LDS is released
    wait_vmcnt<0>();

    if constexpr (VAR == kVarFlat) {
        // the two row-halves' column winners meet in LDS
#pragma unroll
        for (int n = 0; n < NF; ++n) {
            column_reduce<kVarFlat>(best[n], unused);
            if (lane < 16) sm.fkey[wm][wn * (NT / WN) + n * 16 + lane] = best[n];
        }
        __syncthreads();
        if (tid < NT) {
            const ColCtx cc = col_ctx(a, bbase + tid);
            const uint64_t k = key_max(sm.fkey[0][tid], sm.fkey[1][tid]);
            put_record<kVarFlat, false>(a, w, cc, k, lse_empty());
        }
    }
}

template <int NT, int VAR>
static hipError_t launch_wide_dma_nt(const Stage1Args& a, int grid_y, hipStream_t stream) {
    const dim3 grid = a.xcd_pair ? dim3(a.G * grid_y) : dim3(a.G, grid_y);
    hipLaunchKernelGGL((wide_dma_kernel<NT, VAR>), grid, dim3(kDThreads), 0, stream, a);
    return hipGetLastError();
}

// nt == 256 only: at 128 columns the register-staged kernel of fs_wide.hip is
// faster (measured 4.01 against 3.84 TB/s at B = 128)
hipError_t launch_wide_dma(int variant, const Stage1Args& a, int nt, int grid_y,
                           hipStream_t stream) {
    if (nt != 256) return hipErrorInvalidValue;
    if (variant == kVarFlat) return launch_wide_dma_nt<256, kVarFlat>(a, grid_y, stream);
    if (variant == kVarLogits) return launch_wide_dma_nt<256, kVarLogits>(a, grid_y, stream);
    return hipErrorInvalidValue;
}

}  // namespace fs

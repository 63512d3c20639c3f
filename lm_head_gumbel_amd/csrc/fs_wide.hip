// Grouped stage 1 for 32 < B <= 64 (gfx950): an LDS-tiled bf16 GEMM with the
// sampling epilogue fused in ("FlashSampling: Fast and Memory-Efficient Exact
// Sampling", Abstract; FlashSampling explainer on aitrends.kr, Stage 1 and the
// Group-Gumbel-Max paragraph).  Flat and logits calls at these batch sizes
// take the row-streaming kernel (fs_rows.hip); the kernel below keeps its
// general shape (NT = 64 or 128) but only the grouped 64-column variant is
// built.
//
// A workgroup (8 waves) owns a balanced range of 16-row vocabulary blocks and
// walks it in tiles of MT rows (128 for NT = 64 batch columns, 256 for 128).
// For each tile it contracts over the hidden dimension in chunks of KC (128 or
// 64): the W tile (MT rows x 2 KC bytes) and the H tile (NT batch rows x 2 KC
// bytes) are loaded cooperatively, one row run per group of lanes, written to
// a double-buffered LDS area with 16 bytes of padding per row (conflict-free
// fragment reads), and each wave computes an MT/2 x NT/4 sub-tile with
// v_mfma_f32_16x16x32_bf16.  W is read from HBM once; H (at most 256 x d bf16)
// stays in L2.  After the last chunk of a tile the waves fold their logits into
// per-column winners (temperature, masks, Philox-Gumbel noise); the column
// winners of the two row-halves meet in LDS at the end and become the
// workgroup's record.
//
// Global loads run two chunks ahead: the loads of chunk s+2 are issued before
// the MFMAs of chunk s into one of two register stages, and chunk s+1 (in the
// other stage) is written to LDS after them, so two chunks of loads are in
// flight while a chunk is computed.
#include "fs_device.h"
#include "fs_epilogue.h"
#include "fs_internal.h"
#include "fs_mfma.h"

#include <type_traits>

namespace fs {

// Tile geometry per column count: rows per tile and k per chunk.  NT = 64
// takes 128 x 128 (256-byte runs per W row); NT = 128 keeps 256 x 64, where
// the taller tile's reuse of each H chunk matters more (measured: B = 64
// 5.09 against 4.96 TB/s, B = 128 4.21 against 3.88).
template <int NT>
struct WideGeom {
    static constexpr int kMT = NT == 64 ? 128 : 256;   // rows per tile
    static constexpr int kKC = NT == 64 ? 128 : 64;    // k per chunk
    static constexpr int kTB = kMT / 16;               // 16-row blocks per tile
    static constexpr int kKS = kKC / 32;               // MFMA k-steps per chunk
    static constexpr int kPR = kKC * 2 / 16;           // 16-byte pieces per row and chunk
    static constexpr int kRowBytes = kKC * 2 + 16;     // LDS row stride (16 bytes of pad)
};

template <int NT>
struct WideSmem {
    char buf[2][(WideGeom<NT>::kMT + NT) * WideGeom<NT>::kRowBytes];
    uint64_t fkey[2][NT];
};

// Grouped variant: per (row-half, vocabulary tile of the range, column) the
// winner and log-mass gathered so far; a range meets at most kWideMaxTiles
// tiles (the host checks).
template <int NT>
struct WideTileSmem {
    uint64_t key[2][kWideMaxTiles][NT];
    float mx[2][kWideMaxTiles][NT];
    float sm[2][kWideMaxTiles][NT];
};
struct NoWideTiles {};

template <int NT, int NTHR, int VAR>
__global__ __launch_bounds__(NTHR, 1) void wide_kernel(Stage1Args a) {
    static_assert((NT == 64 || NT == 128) && NTHR == 512, "column tile and workgroup size");
    static_assert(VAR == kVarFlat || VAR == kVarLogits || (VAR == kVarGrouped && NT == 64),
                  "variant");
    using Geo = WideGeom<NT>;
    constexpr int kMT = Geo::kMT, kKC = Geo::kKC, kTB = Geo::kTB, kKS = Geo::kKS;
    constexpr int kPR = Geo::kPR, kRowBytes = Geo::kRowBytes;
    constexpr int WM = 2, WN = NTHR / 64 / WM;   // wave grid: 2 x 4
    constexpr int RW = kMT / WM;          // rows per wave
    constexpr int MF = RW / 16;           // A fragments
    constexpr int NF = NT / WN / 16;      // 1 or 2 B fragments
    constexpr int WP = kMT * kPR / NTHR;  // W pieces of 16 B per thread per chunk
    constexpr int HP = NT * kPR / NTHR;   // H pieces
    __shared__ WideSmem<NT> sm;
    using TileSmem =
        typename std::conditional<VAR == kVarGrouped, WideTileSmem<NT>, NoWideTiles>::type;
    __shared__ TileSmem tsm;

    // row range w and column group y (see resident_kernel for the XCD pairing)
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
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int r16 = lane & 15;
    const int kg = lane >> 4;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int mb0 = part_begin(w, a.nmb, a.G);
    const int mb1 = part_begin(w + 1, a.nmb, a.G);
    const int row_end = min(mb1 * kMBlock, a.V);          // one past this range's last row
    const int bbase = y * NT;
    const int nchunks = a.d / kKC;
    const int ntiles = (mb1 - mb0 + kTB - 1) / kTB;
    const int total = ntiles * nchunks;

    // cooperative loader: piece q = tid + 512 i covers 16 bytes of row q / kPR
    // at byte (q % kPR) * 16 of the chunk; kPR lanes read a row's whole run
    // (longer runs per row stream HBM better: a probe of this pattern reads
    // 5.99 TB/s with 256-byte runs, 5.59 with 128-byte runs).
    // Offsets are 32-bit element offsets from the range's first W row and
    // from H (a range spans a few hundred rows, H at most 256 rows).
    const uint16_t* wbase = a.W + (size_t)mb0 * kMBlock * a.d;
    const int first_row = mb0 * kMBlock;
    int wofs[WP];
    int hofs[HP];
#pragma unroll
    for (int i = 0; i < HP; ++i) {
        const int q = tid + NTHR * i;
        int b = bbase + q / kPR;
        b = b < a.B ? b : a.B - 1;   // padding columns reuse row B - 1, discarded later
        hofs[i] = b * a.d + (q % kPR) * 8;
    }
    auto set_tile_rows = [&](int tile) {
#pragma unroll
        for (int i = 0; i < WP; ++i) {
            const int q = tid + NTHR * i;
            int row = (mb0 + tile * kTB) * kMBlock + q / kPR;
            row = row < row_end ? row : row_end - 1;   // never read another range's rows
            wofs[i] = (row - first_row) * a.d + (q % kPR) * 8;
        }
    };
    // LDS byte offset of piece i of this thread (W rows first, then H rows)
    auto lds_off = [&](int i, int row_base) {
        const int q = tid + NTHR * i;
        return (row_base + q / kPR) * kRowBytes + (q % kPR) * 16;
    };

    // two register stages: chunk s+1 waits in one while chunk s+2 is fetched
    // into the other
    u32x4 wst[2][WP], hst[2][HP];
    auto load_chunk = [&](int r, int c) {
        const int k = c * kKC;
#pragma unroll
        for (int i = 0; i < WP; ++i) wst[r][i] = *(const global_u32x4*)(wbase + wofs[i] + k);
#pragma unroll
        for (int i = 0; i < HP; ++i) hst[r][i] = *(const global_u32x4*)(a.H + hofs[i] + k);
    };
    auto store_chunk = [&](int r, int b) {
        char* base = sm.buf[b];
#pragma unroll
        for (int i = 0; i < WP; ++i) *reinterpret_cast<u32x4*>(base + lds_off(i, 0)) = wst[r][i];
#pragma unroll
        for (int i = 0; i < HP; ++i) *reinterpret_cast<u32x4*>(base + lds_off(i, kMT)) = hst[r][i];
    };

    // per-lane column winners of this wave (one per B fragment); only the
    // reciprocal temperature is kept per column, the rest of the column
    // context is rebuilt in the epilogue without memory reads
    float inv_t[NF];
    uint64_t best[NF];
    RowKey key[NF];
#pragma unroll
    for (int n = 0; n < NF; ++n) {
        const ColCtx c = col_ctx(a, bbase + wn * (NT / WN) + n * 16 + r16);
        inv_t[n] = c.greedy ? 0.f : c.inv_t;   // 0 marks a greedy column
        key[n] = c.key;
        best[n] = pack_key(-INFINITY, -1);
    }
    Lse unused = lse_empty();

    f32x4 acc[MF][NF];
#pragma unroll
    for (int j = 0; j < MF; ++j)
#pragma unroll
        for (int n = 0; n < NF; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // chunk sequence q = tile * nchunks + c.  Loads run two chunks ahead of
    // the MFMAs and are issued unconditionally (past the end they re-read the
    // last chunk, never stored), so the loop is straight-line code and every
    // wait can leave the younger chunk's loads in flight.
    auto load_seq = [&](int r, int q) {
        q = q < total ? q : total - 1;
        const int t = q / nchunks;
        const int c = q - t * nchunks;
        set_tile_rows(t);
        load_chunk(r, c);
    };
    // grouped: vocabulary tiles t_first .. t_last meet this range
    const int t_first = VAR == kVarGrouped ? mb0 / a.tile_mb : 0;
    const int ntl = VAR == kVarGrouped ? (mb1 - 1) / a.tile_mb - t_first + 1 : 0;
    if constexpr (VAR == kVarGrouped) {
        for (int e = tid; e < 2 * kWideMaxTiles * NT; e += NTHR) {
            const int h = e / (kWideMaxTiles * NT), tl = (e / NT) % kWideMaxTiles, col = e % NT;
            tsm.key[h][tl][col] = pack_key(-INFINITY, -1);
            tsm.mx[h][tl][col] = -INFINITY;
            tsm.sm[h][tl][col] = 0.f;
        }
    }

    load_seq(0, 0);
    load_seq(1, 1);
    store_chunk(0, 0);
    __syncthreads();

    // one step: chunk s (LDS buffer s & 1) through the MFMAs while chunk s+2
    // is fetched into register stage R2 = s & 1; then chunk s+1 (stage R1)
    // goes to the other LDS buffer
    auto step = [&](int s, auto R1, auto R2) {
        const int tile = s / nchunks;
        const int c = s - tile * nchunks;
        load_seq(R2, s + 2);
        __builtin_amdgcn_sched_barrier(0);

        // blocks of this wave that hold rows of the range (the last tile may be short)
        const int blk0 = mb0 + tile * kTB + wm * MF;
        const int nvalid = min(MF, mb1 - blk0);
        if (nvalid > 0) {
            const char* base = sm.buf[s & 1];
#pragma unroll
            for (int kk = 0; kk < kKS; ++kk) {
                bf16x8 bf[NF];
#pragma unroll
                for (int n = 0; n < NF; ++n) {
                    const int col = wn * (NT / WN) + n * 16 + r16;
                    bf[n] = *reinterpret_cast<const bf16x8*>(base + (kMT + col) * kRowBytes +
                                                             kk * 64 + kg * 16);
                }
#pragma unroll
                for (int j = 0; j < MF; ++j) {
                    const int row = wm * RW + j * 16 + r16;
                    const bf16x8 af =
                        *reinterpret_cast<const bf16x8*>(base + row * kRowBytes + kk * 64 + kg * 16);
#pragma unroll
                    for (int n = 0; n < NF; ++n)
                        acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[n], acc[j][n],
                                                                            0, 0, 0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);

        if constexpr (VAR == kVarGrouped) {
          if (c + 1 == nchunks) {
            // the tile is complete: this wave's 16-row blocks in order; a
            // record segment (vocabulary tile) ends where the tile index
            // changes, and its column winners and log-mass are merged into
            // the range's per-tile slots of this row-half
            int t_cur = -1;
            uint64_t gbest = pack_key(-INFINITY, -1);
            Lse glse = lse_empty();
            const int col = wn * (NT / WN) + r16;   // one B fragment per wave
            auto flush = [&]() {
                column_reduce<kVarGrouped>(gbest, glse);
                if (lane < 16) {
                    const int tl = t_cur - t_first;
                    tsm.key[wm][tl][col] = key_max(tsm.key[wm][tl][col], gbest);
                    const Lse o = lse_merge(Lse{tsm.mx[wm][tl][col], tsm.sm[wm][tl][col]}, glse);
                    tsm.mx[wm][tl][col] = o.mx;
                    tsm.sm[wm][tl][col] = o.sm;
                }
            };
            ColCtx cx;
            cx.col = bbase + col;
            cx.ok = cx.col < a.B;
            cx.greedy = !(inv_t[0] > 0.f);
            cx.inv_t = cx.greedy ? 1.f : inv_t[0];
            cx.allow_row =
                (a.allow && cx.ok) ? a.allow + (size_t)cx.col * ((a.V + 31) >> 5) : nullptr;
            cx.key = key[0];
#pragma unroll
            for (int j = 0; j < MF; ++j) {
                if (j >= nvalid) continue;   // uniform
                const int t = (blk0 + j) / a.tile_mb;
                if (t != t_cur) {   // uniform
                    if (t_cur >= 0) flush();
                    t_cur = t;
                    gbest = pack_key(-INFINITY, -1);
                    glse = lse_empty();
                }
                const int row0 = (blk0 + j) * kMBlock + 4 * kg;
                float x[4], sc[4];
                lane_scores(a, cx, acc[j][0], row0, true, x, sc);
                fold<kVarGrouped>(gbest, glse, x, sc, a.v_offset + row0);
            }
            if (t_cur >= 0) flush();
#pragma unroll
            for (int j = 0; j < MF; ++j) acc[j][0] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        } else if (c + 1 == nchunks) {
            // the tile is complete: fold its logits into the column winners
#pragma unroll
            for (int j = 0; j < MF; ++j) {
                if (j >= nvalid) continue;   // uniform
                const int row0 = (blk0 + j) * kMBlock + 4 * kg;
#pragma unroll
                for (int n = 0; n < NF; ++n) {
                    ColCtx cx;
                    cx.col = bbase + wn * (NT / WN) + n * 16 + r16;
                    cx.ok = cx.col < a.B;
                    cx.greedy = !(inv_t[n] > 0.f);
                    cx.inv_t = cx.greedy ? 1.f : inv_t[n];
                    cx.allow_row = (a.allow && cx.ok)
                                       ? a.allow + (size_t)cx.col * ((a.V + 31) >> 5) : nullptr;
                    cx.key = key[n];
                    if constexpr (VAR == kVarLogits) {
                        if (cx.ok) {
                            float* dst = a.logits + (size_t)cx.col * a.V;
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (row0 + r < a.V) dst[row0 + r] = acc[j][n][r];
                        }
                    } else {
                        float x[4], sc[4];
                        lane_scores(a, cx, acc[j][n], row0, true, x, sc);
                        fold<kVarFlat>(best[n], unused, x, sc, a.v_offset + row0);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < MF; ++j)
#pragma unroll
                for (int n = 0; n < NF; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        if (s + 1 < total) store_chunk(R1, (s + 1) & 1);
        __syncthreads();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    for (int s = 0; s < total; s += 2) {
        step(s, I1{}, I0{});                   // chunk s+1 sits in stage 1, s+2 goes to stage 0
        if (s + 1 < total) step(s + 1, I0{}, I1{});
    }
    // the last prefetches re-read chunks that are never stored: wait for them
    // before the registers go away
    __builtin_amdgcn_s_waitcnt(0);

    if constexpr (VAR == kVarGrouped) {
        // one record per (column, vocabulary tile of the range): the two
        // row-halves' slots merged, at record slot w + t
        __syncthreads();
        for (int e = tid; e < ntl * NT; e += NTHR) {
            const int tl = e / NT, col = e % NT;
            const ColCtx c = col_ctx(a, bbase + col);
            const uint64_t k = key_max(tsm.key[0][tl][col], tsm.key[1][tl][col]);
            const Lse l = lse_merge(Lse{tsm.mx[0][tl][col], tsm.sm[0][tl][col]},
                                    Lse{tsm.mx[1][tl][col], tsm.sm[1][tl][col]});
            put_record<kVarGrouped, false>(a, w + t_first + tl, c, k, l);
        }
    }

    if constexpr (VAR == kVarFlat) {
        // the two row-halves' column winners meet in LDS
#pragma unroll
        for (int n = 0; n < NF; ++n) {
            column_reduce<kVarFlat>(best[n], unused);
            if (lane < 16) sm.fkey[wm][wn * (NT / WN) + n * 16 + lane] = best[n];
        }
        __syncthreads();
        if (tid < NT) {
            const ColCtx c = col_ctx(a, bbase + tid);
            const uint64_t k = key_max(sm.fkey[0][tid], sm.fkey[1][tid]);
            put_record<kVarFlat, false>(a, w, c, k, lse_empty());
        }
    }
}

template <int NT, int VAR>
static hipError_t launch_wide_nt(const Stage1Args& a, int grid_y, hipStream_t stream) {
    constexpr int NTHR = 512;
    const dim3 grid = a.xcd_pair ? dim3(a.G * grid_y) : dim3(a.G, grid_y);
    hipLaunchKernelGGL((wide_kernel<NT, NTHR, VAR>), grid, dim3(NTHR), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_wide(int variant, const Stage1Args& a, int nt, int grid_y, hipStream_t stream) {
    if (variant == kVarGrouped && nt == 64) return launch_wide_nt<64, kVarGrouped>(a, grid_y, stream);
    return hipErrorInvalidValue;
}

}  // namespace fs

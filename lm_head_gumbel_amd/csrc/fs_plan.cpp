// Launch planning and workspace layout of libfs (host C++, no HIP): which
// stage-1 kernel runs a call, its grid, the record slots, and where each array
// sits in the caller's workspace.  Every decision depends only on fs_params,
// the variant and the device's compute-unit count.
#include "fs_plan.h"

#include <algorithm>
#include <climits>

namespace fs {

namespace {

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Stage-1 shape of the streaming and cooperative kernels per batch size.
Stage1Config pick_config(bool stream, int B) {
    if (stream) {
        if (B <= 16) return Stage1Config{1, 4, 2};
        if (B <= 32) return Stage1Config{2, 4, 1};
        return Stage1Config{4, 2, 2};
    }
    return B <= 16 ? Stage1Config{1, 4, 2} : Stage1Config{2, 4, 1};
}

// Resident-H shape for a batch, hidden size and variant (nw == 0: none
// instantiated).  Two batch blocks per workgroup are preferred, also for 16
// rows or fewer (the second block is padding: its MFMAs are free in this
// HBM-bound loop, and the two-block shapes stream W faster, 198 against
// 230 us at B = 8, d = 4096, V = 151936); where no such shape holds the
// hidden size, one block per workgroup is used with more batch groups.
ResidentConfig pick_resident(int nks, int variant) {
    ResidentConfig c = resident_default(2, nks, variant);
    if (c.nw == 0) c = resident_default(1, nks, variant);
    return c;
}

// The LDS-tiled kernels address W and H with 32-bit element offsets from the
// range's first row and from H: both spans must stay below 2^31 elements.
bool wide_offsets_fit(const Plan& pl, int G) {
    const int64_t range_rows = (int64_t)ceil_div(pl.nmb, G) * kMBlock + 256;
    return (int64_t)pl.B * pl.d < INT32_MAX && range_rows * pl.d < INT32_MAX;
}

// Rows a resident top-k workgroup keeps at most: ceil(units / G) units of
// mpi blocks.
int64_t resident_topk_wg_rows(const Plan& pl) {
    const int mpi = pl.rcfg.mpi;
    const int nunits = ceil_div(pl.nmb, mpi);
    return (int64_t)ceil_div(nunits, pl.G) * mpi * kMBlock;
}

}  // namespace

bool resident_supported(const ResidentConfig& c, int variant) {
#define FS_RES(NB_, MPI_, KS_, NW_, HK_, HL_, TK_)                                        \
    if (c.nb == NB_ && c.mpi == MPI_ && c.ks == KS_ && c.nw == NW_ && c.hk == HK_ && \
        c.hl == HL_)                                                                   \
        return variant != kVarTopk || TK_;
    FS_RESIDENT_SHAPES(FS_RES)
#undef FS_RES
    return false;
}

ResidentConfig resident_default(int nb, int nks, int variant) {
#define FS_RES(NB_, MPI_, KS_, NW_, HK_, HL_, TK_)                          \
    if (nb == NB_ && nks == NW_ * (HK_ + HL_) && (variant != kVarTopk || TK_)) \
        return ResidentConfig{NB_, MPI_, KS_, NW_, HK_, HL_};
    FS_RESIDENT_SHAPES(FS_RES)
#undef FS_RES
    return ResidentConfig{0, 0, 0, 0, 0, 0};
}

int resident_topk_rows(const ResidentConfig& c) { return topk_store_rows(c.nb, c.hl); }

fs_status check_params(const fs_params* p) {
    if (!p) return FS_ERR_INVALID_ARG;
    if (p->B < 0 || p->d < 0 || p->V < 0 || p->v_offset < 0 || p->tile_v < 0)
        return FS_ERR_INVALID_ARG;
    if (p->B > kMaxB) return FS_ERR_UNSUPPORTED;
    if ((int64_t)p->v_offset + p->V > INT32_MAX) return FS_ERR_INVALID_ARG;
    if (p->d % 8 != 0) return FS_ERR_UNSUPPORTED;
    if (p->v_offset % kMBlock != 0) return FS_ERR_UNSUPPORTED;
    if (p->tile_v % kMBlock != 0) return FS_ERR_UNSUPPORTED;
    if (p->flags & ~kFlagNoNoise) return FS_ERR_INVALID_ARG;
    return FS_OK;
}

void make_plan(const fs_params* p, int variant, int cus, Plan& pl) {
    cus = std::max(1, cus);
    pl.variant = variant;
    pl.B = p->B;
    pl.d = p->d;
    pl.V = p->V;
    pl.n_valid = p->n_valid;
    pl.v_offset = p->v_offset;
    pl.tile_v = p->tile_v ? p->tile_v : kDefaultTileV;
    pl.T = ceil_div(p->V, pl.tile_v);
    pl.nmb = ceil_div(p->V, kMBlock);
    pl.tile_mb = (variant == kVarGrouped) ? pl.tile_v / kMBlock : INT32_MAX / 2;
    const int nks = ceil_div(p->d, 32);

    // 1. kernel family
    pl.kind = kCoop;
    pl.nt = 0;
    pl.rcfg = pick_resident(nks, variant);
    const bool resident_ok = pl.rcfg.nw > 0 && resident_supported(pl.rcfg, variant);
    if (variant == kVarTopk) {
        if (resident_ok) pl.kind = kResident;
    } else {
        if (resident_ok)
            pl.kind = kResident;
        else if (pl.nmb >= 4)
            pl.kind = kStream;
        // large batches: W rows streamed into registers against all the
        // workgroup's columns (up to 256), H in chunks through LDS; also
        // where no resident shape holds the hidden size, or only a one-block
        // shape that would need several batch groups (each reading W again)
        // (grouped: at most 128 columns per workgroup, more in column groups)
        const int nt = p->B <= kRows64.nt                                 ? kRows64.nt
                       : p->B <= kRows128.nt || variant == kVarGrouped ? kRows128.nt
                                                                         : kRows256.nt;
        const bool rows_better =
            p->B > 32 || !resident_ok || (pl.rcfg.nb == 1 && p->B > 16);
        // (grouped too: a record per 16-row block, as the resident kernel
        // writes them)
        if (variant != kVarTopk && rows_better && p->d > 0 && p->d % (64 * rows_kcs(nt)) == 0 &&
            pl.nmb >= 4) {
            pl.kind = kRows;
            pl.nt = nt;
        }
        // grouped records up to 64 columns: one workgroup per CU, each range
        // meeting at most kWideMaxTiles vocabulary tiles (its slots live in LDS)
        if (variant == kVarGrouped && pl.kind != kRows && p->B > 32 && p->B <= 64 && p->d > 0 &&
            p->d % 128 == 0) {
            const int g = std::max(1, std::min(pl.nmb, cus));
            const int blocks = ceil_div(pl.nmb, g);   // longest range
            if ((blocks - 1 + pl.tile_mb - 1) / pl.tile_mb + 1 <= kWideMaxTiles &&
                wide_offsets_fit(pl, g)) {
                pl.kind = kWide;
                pl.nt = 64;
            }
        }
    }
    pl.stream = pl.kind == kStream;
    pl.cfg = pick_config(pl.stream, p->B);
    // grouped on the resident kernel: a record per 16-row block, so that its
    // walk takes the strided (and ticket) order like flat
    pl.unit_rec = variant == kVarGrouped && (pl.kind == kResident || pl.kind == kRows);
    pl.rec_cols = pl.unit_rec ? (pl.B + 31) / 32 * 32 : 0;

    // 2. batch groups
    const int cols = (pl.kind == kWide || pl.kind == kRows) ? pl.nt
                     : pl.kind == kResident ? 16 * pl.rcfg.nb
                                            : 16 * pl.cfg.nb;
    pl.grid_y = ceil_div(p->B, cols);

    // 3. workgroups along the vocabulary and record slots
    int workers;
    if (pl.kind == kStream) {
        // four worker waves per workgroup, at most one worker per block
        pl.G = std::max(1, std::min(pl.nmb / 4, cus));
        workers = 4 * pl.G;
    } else {
        pl.G = std::max(1, std::min(pl.nmb, cus));
        workers = pl.G;
    }
    // resident flat, logits and top-k stride units of mpi blocks over the
    // workgroups: at most one workgroup per unit
    const bool strided = pl.kind == kResident;   // (grouped too: block records)
    const int nunits = strided ? ceil_div(pl.nmb, pl.rcfg.mpi) : pl.nmb;
    const int max_g = nunits;
    if (pl.G > max_g) {
        pl.G = max_g;
        workers = max_g;
    }
    // resident top-k keeps the x of all its units in LDS: enough workgroups
    // that none holds more units than that store
    int min_g = 1;
    if (variant == kVarTopk && pl.kind == kResident) {
        const int cap_units = resident_topk_rows(pl.rcfg) / (kMBlock * pl.rcfg.mpi);
        min_g = ceil_div(nunits, cap_units);
        if (pl.G < min_g) {
            pl.G = min_g;
            workers = min_g;
        }
    }
    pl.xcd_pair = 0;
    if ((pl.kind == kResident || pl.kind == kWide || pl.kind == kRows) && pl.grid_y > 1) {
        // all batch groups of a row range resident at once, on one XCD
        int g = (cus / pl.grid_y) / 8 * 8;
        if (g < min_g) g = (min_g + 7) / 8 * 8;
        if (g >= 8 && g <= max_g && (pl.kind != kWide || wide_offsets_fit(pl, g))) {
            pl.G = g;
            workers = g;
            pl.xcd_pair = 1;
        }
    }
    pl.P = pl.unit_rec ? pl.nmb : workers + (variant == kVarGrouped ? pl.T - 1 : 0);
    pl.k0 = (uint32_t)(p->seed & 0xFFFFFFFFu);
    pl.k1 = (uint32_t)(p->seed >> 32);

    // stage 1: (G, grid_y), or G grid_y along x with the XCD pairing; the
    // stage-2 kernels of grouped and flat take one workgroup per batch row
    // along x, top-k's selection levels (slices, B)
    const int64_t gx = pl.xcd_pair ? (int64_t)pl.G * pl.grid_y : pl.G;
    // (top-k and grouped block records: stage 2 takes the rows along y)
    pl.launchable = gx <= kMaxGridX && (pl.xcd_pair || pl.grid_y <= kMaxGridY) &&
                    ((variant != kVarTopk && !pl.unit_rec) || pl.B <= kMaxGridY);
}

size_t part_bytes(const Plan& pl) {
    return (size_t)pl.grid_y * (4 * (size_t)pl.G) * 2 * pl.cfg.nb * 1024;
}

int dynamic_k0(const Plan& pl) {
    // Each ticket costs its workgroup a wait behind the ticket's round trip,
    // so only about the last kDepth units per workgroup come by ticket:
    // enough to even out the workgroups' finishing times (measured at
    // B = 32, d = 4096: depth 1-4 within 0.7 us of each other, all units by
    // ticket 11 us slower).  One batch group and at least three units per
    // workgroup.
    constexpr int kDepth = 2;
    if (pl.variant != kVarFlat && pl.variant != kVarTopk && !pl.unit_rec) return 0;
    if (pl.kind != kResident || pl.grid_y != 1 || pl.xcd_pair) return 0;
    const int nunits = ceil_div(pl.nmb, std::max(1, pl.rcfg.mpi));
    const int per = nunits / pl.G;   // units every workgroup has in the strided order
    const int k0 = std::max(3, per - kDepth);
    return per >= 3 ? k0 : 0;
}

int topk_len(const Plan& pl, int k) {
    if (pl.kind != kResident) return k;
    return (int)std::min<int64_t>(k, resident_topk_wg_rows(pl));
}

bool topk_dense(const Plan& pl, int k) {
    return pl.kind == kResident && k > kMaxTopKCoop && (int64_t)k >= resident_topk_wg_rows(pl);
}

bool topk_launchable(const Plan& pl, int k) {
    return pl.launchable && (int64_t)pl.G * topk_len(pl, k) <= INT32_MAX / 4;
}

bool topk_small_path(int G, int L, int k) {   // the dense form never takes it
    return k <= 64 && (int64_t)G * L <= (int64_t)kTopkStage2Threads * 64;
}

size_t stage2_topk_scratch_bytes(int G, int L, int B, int k, bool dense) {
    const int64_t n = (int64_t)G * L;
    if ((topk_small_path(G, L, k) && !dense) || n <= kTopkSliceCap) return 0;
    const int64_t S = (n + kTopkSliceCap - 1) / kTopkSliceCap;
    return 4 * align_up((size_t)S * B * k * 4);   // lists of two levels: x and ids
}

WsLayout layout(int ws_variant, const Plan& pl, int k) {
    WsLayout w;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t r = off;
        off = align_up(off + bytes);
        return r;
    };
    const size_t B = (size_t)pl.B;
    if (ws_variant == FS_VARIANT_FLAT || ws_variant == FS_VARIANT_GROUPED) {
        const size_t P = (size_t)pl.P;
        // block records: block-major with rec_cols columns per block
        const size_t cols = ws_variant == FS_VARIANT_GROUPED && pl.rec_cols ? pl.rec_cols : B;
        w.pm = take(P * cols * 4);
        w.pidx = take(P * cols * 4);
        if (ws_variant == FS_VARIANT_GROUPED) w.pL = take(P * cols * 4);
        if (pl.stream) w.part = take(part_bytes(pl));
        if (ws_variant == FS_VARIANT_GROUPED && pl.unit_rec) w.gsel = take(B * 8 * kGselStride);
        w.sched = take(kSchedBytes);
    } else if (ws_variant == FS_VARIANT_TOPK) {
        const int L = topk_len(pl, k);
        const bool dense = topk_dense(pl, k);
        const size_t n = (size_t)pl.G * B * (size_t)L;
        w.cx = take(n * 4);
        if (!dense) w.cidx = take(n * 4);
        const size_t sb = stage2_topk_scratch_bytes(pl.G, L, pl.B, k, dense);
        if (sb) w.sel = take(sb);
        w.sched = take(kSchedBytes);
    } else if (ws_variant == FS_VARIANT_LOGITS) {
        if (pl.stream) w.part = take(part_bytes(pl));
    } else if (ws_variant == FS_VARIANT_MULTINOMIAL) {
        const size_t nchunk = (size_t)ceil_div(pl.V, kMultinomialChunk);
        w.mm = take(nchunk * B * 4);
        w.ms = take(nchunk * B * 4);
        w.mkey = take(nchunk * B * 8);
    }
    w.total = off;
    return w;
}

}  // namespace fs

// Host side of libfs: argument validation, launch planning, workspace layout
// and the extern "C" entry points declared in include/fs.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "fs.h"
#include "fs_internal.h"

namespace {

using namespace fs;

constexpr int kDefaultTileV = 128;
constexpr int kMaxTopK = 1024;
constexpr int kMaxTopKCoop = 64;   // the cooperative kernel keeps sorted lists of at most 64
constexpr int kMultinomialChunk = 2048;
constexpr int kMaxB = 1 << 20;
constexpr size_t kAlign = 256;

struct DeviceInfo {
    bool ok = false;      // a gfx950 device
    int cus = 0;
};

std::mutex g_mu;
DeviceInfo g_dev[64];
bool g_dev_init[64];

// Workgroups per compute unit along the vocabulary; FS_WG_PER_CU overrides
// the default for tuning experiments.
int wg_per_cu() {
    static int v = [] {
        const char* e = std::getenv("FS_WG_PER_CU");
        int x = e ? std::atoi(e) : 0;
        return (x >= 1 && x <= 16) ? x : 1;
    }();
    return v;
}

bool current_device(DeviceInfo& out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return false;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_dev_init[dev]) {
        DeviceInfo info;
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
            info.ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
            info.cus = prop.multiProcessorCount;
        } else {
            (void)hipGetLastError();
        }
        g_dev[dev] = info;
        g_dev_init[dev] = true;
    }
    out = g_dev[dev];
    return out.ok && out.cus > 0;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Stage-1 kernels: resident (H slice in registers; the default for the
// common shapes), stream (independent worker waves, H reloaded per stage) and
// coop (workgroup-cooperative, H reloaded per stage; top-k and the shapes the
// others do not cover).
enum Stage1Kind { kCoop = 0, kStream = 1, kResident = 2, kWide = 3 };

// Validated shape of one call and its launch plan.
struct Plan {
    int B, d, V, n_valid, v_offset, tile_v, tile_mb, T, nmb, G;
    int kind;      // Stage1Kind
    bool stream;   // kind == kStream
    int P;         // record slots per row
    Stage1Config cfg;
    ResidentConfig rcfg;
    int nt;        // kWide: batch columns per workgroup
    int grid_y;
    int xcd_pair;
    uint32_t k0, k1;
};

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

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

// Stage-1 shape per batch size; FS_STAGE1_CFG="nb,mpi,ks" overrides it for
// tuning experiments (an unknown shape makes the launch fail with FS_ERR_HIP).
Stage1Config pick_config(bool stream, int B) {
    static const char* env = std::getenv("FS_STAGE1_CFG");
    if (env && stream) {
        Stage1Config c{0, 0, 0};
        if (std::sscanf(env, "%d,%d,%d", &c.nb, &c.mpi, &c.ks) == 3) return c;
    }
    if (stream) {
        if (B <= 16) return Stage1Config{1, 4, 2};
        if (B <= 32) return Stage1Config{2, 4, 1};
        return Stage1Config{4, 2, 2};
    }
    return B <= 16 ? Stage1Config{1, 4, 2} : Stage1Config{2, 4, 1};
}

// FS_SMALL_NB1=1: one batch block per workgroup for B <= 16 (tuning
// experiments; by default two, the second one padding).
bool small_nb1() {
    static const bool on = [] {
        const char* e = std::getenv("FS_SMALL_NB1");
        return e && e[0] == '1';
    }();
    return on;
}

// Resident-H shape for a batch, hidden size and variant (nw == 0: none
// instantiated).  Two batch blocks per workgroup are preferred, also for 16
// rows or fewer (the second block is padding: its MFMAs are free in this
// HBM-bound loop, and the two-block shapes stream W faster, 198 against
// 230 us at B = 8, d = 4096, V = 151936); where no such shape holds the
// hidden size, one block per workgroup is used with more batch groups.
// FS_RES_CFG="nb,mpi,ks,nw" overrides the choice for tuning experiments.
ResidentConfig pick_resident(int B, int nks, int variant) {
    static const char* env = std::getenv("FS_RES_CFG");
    if (env) {
        ResidentConfig c{0, 0, 0, 0, 0, 0};
        const int n = std::sscanf(env, "%d,%d,%d,%d,%d", &c.nb, &c.mpi, &c.ks, &c.nw, &c.hl);
        if ((n == 4 || n == 5) && c.nw > 0 && nks % c.nw == 0 && nks / c.nw > c.hl) {
            c.hk = nks / c.nw - c.hl;
            return c;
        }
        return ResidentConfig{0, 0, 0, 0, 0, 0};
    }
    const int first = B <= 16 && small_nb1() ? 1 : 2;
    ResidentConfig c = resident_default(first, nks, variant);
    if (c.nw == 0) c = resident_default(3 - first, nks, variant);
    return c;
}

// FS_WIDE=0 disables the LDS-tiled large-batch kernel (tuning experiments).
bool wide_enabled() {
    static const bool on = [] {
        const char* e = std::getenv("FS_WIDE");
        return !(e && e[0] == '0');
    }();
    return on;
}

// FS_XCD_PAIR=0 disables the XCD pairing of batch groups (tuning experiments).
bool xcd_pairing() {
    static const bool on = [] {
        const char* e = std::getenv("FS_XCD_PAIR");
        return !(e && e[0] == '0');
    }();
    return on;
}

// FS_STAGE1_KIND=coop|stream forces a kernel family for tuning experiments.
int forced_kind() {
    static const int k = [] {
        const char* e = std::getenv("FS_STAGE1_KIND");
        if (!e) return -1;
        if (!std::strcmp(e, "coop")) return (int)kCoop;
        if (!std::strcmp(e, "stream")) return (int)kStream;
        return -1;
    }();
    return k;
}

void make_plan(const fs_params* p, int variant, int cus, Plan& pl) {
    pl.B = p->B;
    pl.d = p->d;
    pl.V = p->V;
    pl.n_valid = p->n_valid;
    pl.v_offset = p->v_offset;
    pl.tile_v = p->tile_v ? p->tile_v : kDefaultTileV;
    pl.T = (p->V + pl.tile_v - 1) / pl.tile_v;
    pl.nmb = (p->V + kMBlock - 1) / kMBlock;
    pl.tile_mb = (variant == kVarGrouped) ? pl.tile_v / kMBlock : INT32_MAX / 2;
    const int nks = (p->d + 31) / 32;

    // 1. kernel family
    pl.kind = kCoop;
    pl.nt = 0;
    const int forced = forced_kind();
    pl.rcfg = pick_resident(p->B, nks, variant);
    const bool resident_ok = pl.rcfg.nw > 0 && resident_supported(pl.rcfg, variant);
    if (variant == kVarTopk) {
        if (resident_ok && forced < 0) pl.kind = kResident;
    } else {
        if (resident_ok)
            pl.kind = kResident;
        else if (pl.nmb >= 4)
            pl.kind = kStream;
        if (forced == kCoop || (forced == kStream && pl.nmb >= 4)) pl.kind = forced;
        // large batches: the LDS-tiled kernel shares each W tile among all columns
        // (chunks of d: 128 deep for 64 columns, 64 deep for 128)
        if ((variant == kVarFlat || variant == kVarLogits) && p->B > 32 && p->d > 0 &&
            p->d % (p->B <= 64 ? 128 : 64) == 0 && forced < 0 && wide_enabled()) {
            pl.kind = kWide;
            pl.nt = p->B <= 64 ? 64 : p->B <= 128 ? 128 : 256;
        }
        // grouped records up to 64 columns: one workgroup per CU, each range
        // meeting at most 16 vocabulary tiles (its per-tile slots live in LDS)
        if (variant == kVarGrouped && p->B > 32 && p->B <= 64 && p->d > 0 && p->d % 128 == 0 &&
            forced < 0 && wide_enabled()) {
            const int g = std::max(1, std::min(pl.nmb, cus));
            const int blocks = (pl.nmb + g - 1) / g;   // longest range
            if ((blocks - 1 + pl.tile_mb - 1) / pl.tile_mb + 1 <= kWideMaxTiles) {
                pl.kind = kWide;
                pl.nt = 64;
            }
        }
    }
    pl.stream = pl.kind == kStream;
    pl.cfg = pick_config(pl.stream, p->B);

    // 2. batch groups
    const int cols = pl.kind == kWide       ? pl.nt
                     : pl.kind == kResident ? 16 * pl.rcfg.nb
                                            : 16 * pl.cfg.nb;
    pl.grid_y = (p->B + cols - 1) / cols;

    // 3. workgroups along the vocabulary and record slots
    int workers;
    if (pl.kind == kStream) {
        // four worker waves per workgroup, at most one worker per block
        pl.G = std::max(1, std::min(pl.nmb / 4, cus * wg_per_cu()));
        workers = 4 * pl.G;
    } else {
        const int per_cu = pl.kind == kWide ? 1 : wg_per_cu();   // the wide kernel fills LDS
        pl.G = std::max(1, std::min(pl.nmb, cus * per_cu));
        workers = pl.G;
    }
    // resident flat, logits and top-k stride units of mpi blocks over the
    // workgroups: at most one workgroup per unit
    const bool strided = pl.kind == kResident && variant != kVarGrouped;
    const int nunits = strided ? (pl.nmb + pl.rcfg.mpi - 1) / pl.rcfg.mpi : pl.nmb;
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
        min_g = (nunits + cap_units - 1) / cap_units;
        if (pl.G < min_g) {
            pl.G = min_g;
            workers = min_g;
        }
    }
    pl.xcd_pair = 0;
    if ((pl.kind == kResident || pl.kind == kWide) && pl.grid_y > 1 && xcd_pairing()) {
        // all batch groups of a row range resident at once, on one XCD
        const int per_cu = pl.kind == kWide ? 1 : wg_per_cu();
        int g = (cus * per_cu / pl.grid_y) / 8 * 8;
        if (g < min_g) g = (min_g + 7) / 8 * 8;
        if (g >= 8 && g <= max_g) {
            pl.G = g;
            workers = g;
            pl.xcd_pair = 1;
        }
    }
    pl.P = workers + (variant == kVarGrouped ? pl.T - 1 : 0);
    pl.k0 = (uint32_t)(p->seed & 0xFFFFFFFFu);
    pl.k1 = (uint32_t)(p->seed >> 32);
}

// Workspace layout per variant (each array 256-byte aligned).
struct Workspace {
    float* pm = nullptr;
    int32_t* pidx = nullptr;
    float* pL = nullptr;
    float* cx = nullptr;
    int32_t* cidx = nullptr;
    float* mm = nullptr;
    float* ms = nullptr;
    uint64_t* mkey = nullptr;
    void* part = nullptr;   // streaming stage 1: parked partial sums of split blocks
    SchedState* sched = nullptr;   // flat: unit scheduler block (kept from call to call)
    void* sel = nullptr;    // top-k: lists of the intermediate selection levels
};

// Partial sums parked by the streaming kernel: per y-block, worker and side
// (head, tail), nb 16x16 FP32 tiles.
size_t part_bytes(const Plan& pl) {
    return (size_t)pl.grid_y * (4 * pl.G) * 2 * pl.cfg.nb * 1024;
}

// Rows a resident top-k workgroup keeps at most: ceil(units / G) units of
// mpi blocks.
int64_t resident_topk_wg_rows(const Plan& pl) {
    const int mpi = pl.rcfg.mpi;
    const int nunits = (pl.nmb + mpi - 1) / mpi;
    return (int64_t)((nunits + pl.G - 1) / pl.G) * mpi * kMBlock;
}

// Units each workgroup of the resident flat stage 1 takes in the strided
// order before it turns to the ticket counter (0: strided order only).  Each
// ticket costs its workgroup a wait behind the ticket's round trip, so only
// about the last kDynDepth units per workgroup come by ticket: enough to
// even out the workgroups' finishing times.  One batch group and at least
// three units per workgroup; FS_DYN=<depth> overrides the depth and FS_DYN=0
// switches the tickets off (tuning experiments).
int dynamic_k0(const Plan& pl) {
    static const int depth = [] {
        const char* e = std::getenv("FS_DYN");
        return e ? std::atoi(e) : 2;
    }();
    if (depth <= 0 || pl.kind != kResident || pl.grid_y != 1 || pl.xcd_pair) return 0;
    const int nunits = (pl.nmb + pl.rcfg.mpi - 1) / std::max(1, pl.rcfg.mpi);
    const int per = nunits / pl.G;   // units every workgroup has in the strided order
    const int k0 = std::max(3, per - depth);
    return per >= 3 ? k0 : 0;
}

// Entries per top-k candidate list: a list never needs more than the rows of
// its workgroup.
int topk_len(const Plan& pl, int k) {
    if (pl.kind != kResident) return k;
    return (int)std::min<int64_t>(k, resident_topk_wg_rows(pl));
}

// Dense lists: for k above 64 that reaches every row of the fullest
// workgroup, stage 1 writes the x of all its rows in store order and no ids
// (the selection happens in stage 2 alone).
bool topk_dense(const Plan& pl, int k) {
    return pl.kind == kResident && k > kMaxTopKCoop && (int64_t)k >= resident_topk_wg_rows(pl);
}

size_t layout(int variant, const Plan& pl, int k, char* base, Workspace* w) {
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* r = base ? base + off : nullptr;
        off = align_up(off + bytes);
        return r;
    };
    const size_t B = (size_t)pl.B;
    if (variant == FS_VARIANT_FLAT || variant == FS_VARIANT_GROUPED) {
        const size_t P = (size_t)pl.P;
        char* a = take(P * B * 4);
        char* b = take(P * B * 4);
        char* c = variant == FS_VARIANT_GROUPED ? take(P * B * 4) : nullptr;
        char* d = pl.stream ? take(part_bytes(pl)) : nullptr;
        char* e = variant == FS_VARIANT_FLAT ? take(sizeof(SchedState)) : nullptr;
        if (w) {
            w->pm = (float*)a;
            w->pidx = (int32_t*)b;
            w->pL = (float*)c;
            w->part = d;
            w->sched = (SchedState*)e;
        }
    } else if (variant == FS_VARIANT_TOPK) {
        const int L = topk_len(pl, k);
        const bool dense = topk_dense(pl, k);
        const size_t n = (size_t)pl.G * B * (size_t)L;
        char* a = take(n * 4);
        char* c = dense ? nullptr : take(n * 4);
        const size_t sb = stage2_topk_scratch_bytes(pl.G, L, pl.B, k, dense);
        char* d = sb ? take(sb) : nullptr;
        char* e = take(sizeof(SchedState));
        if (w) {
            w->cx = (float*)a;
            w->cidx = (int32_t*)c;
            w->sel = d;
            w->sched = (SchedState*)e;
        }
    } else if (variant == FS_VARIANT_LOGITS) {
        char* a = pl.stream ? take(part_bytes(pl)) : nullptr;
        if (w) w->part = a;
    } else if (variant == FS_VARIANT_MULTINOMIAL) {
        const size_t nchunk = (size_t)(pl.V + kMultinomialChunk - 1) / kMultinomialChunk;
        char* a = take(nchunk * B * 4);
        char* b = take(nchunk * B * 4);
        char* c = take(nchunk * B * 8);
        if (w) { w->mm = (float*)a; w->ms = (float*)b; w->mkey = (uint64_t*)c; }
    }
    return off;
}

fs_status from_hip(hipError_t e) { return e == hipSuccess ? FS_OK : FS_ERR_HIP; }

NoiseSrc noise_src(const Plan& pl, const fs_params* p) {
    return NoiseSrc{pl.k0, pl.k1, p->step, p->seeds, p->step_ptr};
}

Stage1Args stage1_args(const Plan& pl, const fs_params* p, const void* H, const void* W,
                       const float* temp, const uint32_t* allow) {
    Stage1Args a{};
    a.H = static_cast<const uint16_t*>(H);
    a.W = static_cast<const uint16_t*>(W);
    a.temp = temp;
    a.allow = allow;
    a.B = pl.B;
    a.d = pl.d;
    a.V = pl.V;
    a.n_valid = pl.n_valid;
    a.v_offset = pl.v_offset;
    a.nmb = pl.nmb;
    a.G = pl.G;
    a.tile_mb = pl.tile_mb;
    a.ny = pl.grid_y;
    a.xcd_pair = pl.xcd_pair;
    a.P = pl.P;
    a.noise = noise_src(pl, p);
    a.flags = p->flags;
    return a;
}

// Checks shared by the fused entry points once B > 0 and V > 0.
fs_status check_operands(const fs_params* p, const void* H, const void* W) {
    if (p->d > 0 && (!H || !W)) return FS_ERR_INVALID_ARG;
    if (p->d > 0 && (!aligned16(H) || !aligned16(W))) return FS_ERR_UNSUPPORTED;
    return FS_OK;
}

// Top-k (top_p >= 1) or top-p after top-k (0 < top_p < 1): shared body.
fs_status sample_topk(const fs_params* p, const void* H, const void* W, const float* temp,
                      const uint32_t* allow, int32_t k, float top_p, int32_t* out_idx, void* ws,
                      size_t ws_bytes, void* stream) {
    fs_status st = check_params(p);
    if (st != FS_OK) return st;
    if (k < 1) return FS_ERR_INVALID_ARG;
    if (!(top_p > 0.f && top_p <= 1.f)) return FS_ERR_INVALID_ARG;   // NaN included
    if (k > kMaxTopK) return FS_ERR_UNSUPPORTED;
    if (p->B == 0) return FS_OK;
    if (!out_idx) return FS_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p->V > 0 && (st = check_operands(p, H, W)) != FS_OK) return st;
    DeviceInfo dev;
    if (!current_device(dev)) return FS_ERR_UNSUPPORTED;
    if (p->V == 0) return from_hip(launch_fill_idx(out_idx, p->B, -1, nullptr, s));
    Plan pl;
    make_plan(p, kVarTopk, dev.cus, pl);
    if (pl.kind != kResident && k > kMaxTopKCoop) return FS_ERR_UNSUPPORTED;
    Workspace w;
    const size_t need = layout(FS_VARIANT_TOPK, pl, k, nullptr, nullptr);
    if (!ws || ws_bytes < need) return FS_ERR_WORKSPACE;
    layout(FS_VARIANT_TOPK, pl, k, static_cast<char*>(ws), &w);
    Stage1Args a = stage1_args(pl, p, H, W, temp, allow);
    a.topk = k;
    a.topk_len = topk_len(pl, k);
    a.topk_dense = topk_dense(pl, k) ? 1 : 0;
    a.cx = w.cx;
    a.cidx = w.cidx;
    // ticket order where the one-kernel stage 2 follows (it sets the block up);
    // dense lists imply their ids by the strided order
    const bool tickets = pl.kind == kResident && !a.topk_dense &&
                         topk_small_path(pl.G, a.topk_len, k);
    a.dyn_k0 = tickets ? dynamic_k0(pl) : 0;
    a.sched = a.dyn_k0 > 0 ? w.sched : nullptr;
    hipError_t e = pl.kind == kResident ? launch_resident(kVarTopk, a, pl.grid_y, pl.rcfg, s)
                                        : launch_stage1(kVarTopk, a, pl.grid_y, pl.cfg, s);
    if (e != hipSuccess) return FS_ERR_HIP;
    const int unit_rows = pl.kind == kResident ? pl.rcfg.mpi * kMBlock : kMBlock;
    const DenseIds dn{a.topk_dense, pl.v_offset, unit_rows, pl.G * unit_rows};
    return from_hip(launch_stage2_topk(w.cx, w.cidx, pl.G, a.topk_len, pl.B, k, dn, top_p, temp,
                                       p->flags, noise_src(pl, p), out_idx, w.sel,
                                       tickets ? w.sched : nullptr, s));
}

}  // namespace

extern "C" {

const char* fs_status_string(fs_status s) {
    switch (s) {
        case FS_OK: return "FS_OK";
        case FS_ERR_INVALID_ARG: return "FS_ERR_INVALID_ARG";
        case FS_ERR_UNSUPPORTED: return "FS_ERR_UNSUPPORTED";
        case FS_ERR_WORKSPACE: return "FS_ERR_WORKSPACE";
        case FS_ERR_HIP: return "FS_ERR_HIP";
    }
    return "FS_ERR_UNKNOWN";
}

const char* fs_version(void) { return "libfs 0.1 (gfx950)"; }

int32_t fs_num_tiles(const fs_params* p) {
    if (check_params(p) != FS_OK) return -1;
    const int tv = p->tile_v ? p->tile_v : kDefaultTileV;
    return (p->V + tv - 1) / tv;
}

size_t fs_workspace_bytes(const fs_params* p, int variant, int32_t k) {
    if (check_params(p) != FS_OK) return 0;
    if (variant < FS_VARIANT_FLAT || variant > FS_VARIANT_LOGITS) return 0;
    if (variant == FS_VARIANT_TOPK && (k < 1 || k > kMaxTopK)) return 0;
    DeviceInfo dev;
    if (!current_device(dev)) return 0;
    Plan pl;
    make_plan(p, variant == FS_VARIANT_GROUPED  ? kVarGrouped
                 : variant == FS_VARIANT_TOPK   ? kVarTopk
                 : variant == FS_VARIANT_LOGITS ? kVarLogits
                                                : kVarFlat,
              dev.cus, pl);
    if (variant == FS_VARIANT_TOPK && pl.kind != kResident && k > kMaxTopKCoop) return 0;
    return std::max(kAlign, layout(variant, pl, k, nullptr, nullptr));
}

// Shared front half of fs_sample and fs_sample_stage1: validation, plan,
// workspace carve-up and the stage-1 launch.  `done` is set when nothing is
// left to do (B == 0, or V == 0 after filling the outputs).
static fs_status flat_stage1(const fs_params* p, const void* H, const void* W, const float* temp,
                             const uint32_t* allow, int32_t* out_idx, float* out_score,
                             void* ws, size_t ws_bytes, hipStream_t s, bool need_out,
                             Plan& pl, Workspace& w, bool& done) {
    done = true;
    fs_status st = check_params(p);
    if (st != FS_OK) return st;
    if (p->B == 0) return FS_OK;
    if (need_out && !out_idx) return FS_ERR_INVALID_ARG;
    if (p->V > 0 && (st = check_operands(p, H, W)) != FS_OK) return st;
    DeviceInfo dev;
    if (!current_device(dev)) return FS_ERR_UNSUPPORTED;
    if (p->V == 0)
        return need_out ? from_hip(launch_fill_idx(out_idx, p->B, -1, out_score, s)) : FS_OK;
    make_plan(p, kVarFlat, dev.cus, pl);
    const size_t need = layout(FS_VARIANT_FLAT, pl, 0, nullptr, nullptr);
    if (!ws || ws_bytes < need) return FS_ERR_WORKSPACE;
    layout(FS_VARIANT_FLAT, pl, 0, static_cast<char*>(ws), &w);
    Stage1Args a = stage1_args(pl, p, H, W, temp, allow);
    a.pm = w.pm;
    a.pidx = w.pidx;
    a.dyn_k0 = dynamic_k0(pl);
    a.sched = a.dyn_k0 > 0 ? w.sched : nullptr;
    const hipError_t e =
        pl.kind == kWide       ? launch_wide(kVarFlat, a, pl.nt, pl.grid_y, s)
        : pl.kind == kResident ? launch_resident(kVarFlat, a, pl.grid_y, pl.rcfg, s)
        : pl.stream          ? launch_stream(kVarFlat, a, pl.grid_y, pl.cfg, w.part, need_out, s)
                             : launch_stage1(kVarFlat, a, pl.grid_y, pl.cfg, s);
    if (e != hipSuccess) return FS_ERR_HIP;
    done = false;
    return FS_OK;
}

fs_status fs_sample(const fs_params* p, const void* H, const void* W, const float* temp,
                    const uint32_t* allow, int32_t* out_idx, float* out_score, void* ws,
                    size_t ws_bytes, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    Plan pl;
    Workspace w;
    bool done;
    fs_status st = flat_stage1(p, H, W, temp, allow, out_idx, out_score, ws, ws_bytes, s, true,
                               pl, w, done);
    if (st != FS_OK || done) return st;
    return from_hip(launch_stage2_flat(w.pm, w.pidx, pl.P, pl.B, out_idx, out_score, w.sched, s));
}

fs_status fs_sample_stage1(const fs_params* p, const void* H, const void* W, const float* temp,
                           const uint32_t* allow, void* ws, size_t ws_bytes, void* stream) {
    Plan pl;
    Workspace w;
    bool done;
    return flat_stage1(p, H, W, temp, allow, nullptr, nullptr, ws, ws_bytes,
                       static_cast<hipStream_t>(stream), false, pl, w, done);
}

fs_status fs_sample_grouped(const fs_params* p, const void* H, const void* W,
                            const float* temp, const uint32_t* allow, float* tile_max,
                            int32_t* tile_idx, float* tile_logmass, int32_t* out_idx, void* ws,
                            size_t ws_bytes, void* stream) {
    fs_status st = check_params(p);
    if (st != FS_OK) return st;
    if (p->B == 0) return FS_OK;
    if (p->V > 0 && (!tile_max || !tile_idx || !tile_logmass)) return FS_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p->V > 0 && (st = check_operands(p, H, W)) != FS_OK) return st;
    DeviceInfo dev;
    if (!current_device(dev)) return FS_ERR_UNSUPPORTED;
    if (p->V == 0) return out_idx ? from_hip(launch_fill_idx(out_idx, p->B, -1, nullptr, s)) : FS_OK;
    Plan pl;
    make_plan(p, kVarGrouped, dev.cus, pl);
    Workspace w;
    const size_t need = layout(FS_VARIANT_GROUPED, pl, 0, nullptr, nullptr);
    if (!ws || ws_bytes < need) return FS_ERR_WORKSPACE;
    layout(FS_VARIANT_GROUPED, pl, 0, static_cast<char*>(ws), &w);
    Stage1Args a = stage1_args(pl, p, H, W, temp, allow);
    a.pm = w.pm;
    a.pidx = w.pidx;
    a.pL = w.pL;
    hipError_t e =
        pl.kind == kWide       ? launch_wide(kVarGrouped, a, pl.nt, pl.grid_y, s)
        : pl.kind == kResident ? launch_resident(kVarGrouped, a, pl.grid_y, pl.rcfg, s)
        : pl.stream            ? launch_stream(kVarGrouped, a, pl.grid_y, pl.cfg, w.part, true, s)
                               : launch_stage1(kVarGrouped, a, pl.grid_y, pl.cfg, s);
    if (e != hipSuccess) return FS_ERR_HIP;
    // record slot (worker w, tile t) is w + t; the streaming kernel's workers
    // own ranges of (block, quarter) units, the cooperative kernel's of blocks
    const int workers = pl.stream ? 4 * pl.G : pl.G;
    const int units = pl.stream ? 4 * pl.nmb : pl.nmb;
    const int tile_units = pl.stream ? 4 * pl.tile_mb : pl.tile_mb;
    return from_hip(launch_stage2_grouped(w.pm, w.pidx, w.pL, pl.P, pl.B, pl.T, workers, units,
                                          tile_units, temp, p->flags, noise_src(pl, p), tile_max,
                                          tile_idx, tile_logmass, out_idx, s));
}


fs_status fs_sample_topk(const fs_params* p, const void* H, const void* W, const float* temp,
                         const uint32_t* allow, int32_t k, int32_t* out_idx, void* ws,
                         size_t ws_bytes, void* stream) {
    return sample_topk(p, H, W, temp, allow, k, 1.f, out_idx, ws, ws_bytes, stream);
}

fs_status fs_sample_topk_topp(const fs_params* p, const void* H, const void* W, const float* temp,
                              const uint32_t* allow, int32_t k, float top_p, int32_t* out_idx,
                              void* ws, size_t ws_bytes, void* stream) {
    return sample_topk(p, H, W, temp, allow, k, top_p, out_idx, ws, ws_bytes, stream);
}

fs_status fs_merge_online_dev(int32_t B, int32_t C, const int32_t* z, const float* L,
                              const float* temp, uint64_t seed, const uint64_t* seeds,
                              uint32_t step, const uint32_t* step_ptr, uint32_t flags,
                              int32_t* out_idx, float* out_L, void* stream) {
    if (B < 0 || C < 0) return FS_ERR_INVALID_ARG;
    if (flags & ~kFlagNoNoise) return FS_ERR_INVALID_ARG;
    if (B == 0) return FS_OK;
    if (!out_idx || (C > 0 && (!z || !L))) return FS_ERR_INVALID_ARG;
    DeviceInfo dev;
    if (!current_device(dev)) return FS_ERR_UNSUPPORTED;
    const NoiseSrc noise{(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32), step, seeds,
                         step_ptr};
    return from_hip(launch_merge_online(B, C, z, L, temp, noise, flags, out_idx, out_L,
                                        static_cast<hipStream_t>(stream)));
}

fs_status fs_merge_online(int32_t B, int32_t C, const int32_t* z, const float* L,
                          const float* temp, uint64_t seed, uint32_t step, uint32_t flags,
                          int32_t* out_idx, float* out_L, void* stream) {
    return fs_merge_online_dev(B, C, z, L, temp, seed, nullptr, step, nullptr, flags, out_idx,
                               out_L, stream);
}

fs_status fs_logits(const fs_params* p, const void* H, const void* W, float* logits,
                    void* ws, size_t ws_bytes, void* stream) {
    fs_status st = check_params(p);
    if (st != FS_OK) return st;
    if (p->B == 0 || p->V == 0) return FS_OK;
    if (!logits) return FS_ERR_INVALID_ARG;
    if ((st = check_operands(p, H, W)) != FS_OK) return st;
    DeviceInfo dev;
    if (!current_device(dev)) return FS_ERR_UNSUPPORTED;
    Plan pl;
    make_plan(p, kVarLogits, dev.cus, pl);
    Stage1Args a = stage1_args(pl, p, H, W, nullptr, nullptr);
    a.logits = logits;
    if (pl.kind == kWide)
        return from_hip(launch_wide(kVarLogits, a, pl.nt, pl.grid_y,
                                    static_cast<hipStream_t>(stream)));
    if (pl.kind == kResident)
        return from_hip(launch_resident(kVarLogits, a, pl.grid_y, pl.rcfg,
                                        static_cast<hipStream_t>(stream)));
    if (!pl.stream)
        return from_hip(launch_stage1(kVarLogits, a, pl.grid_y, pl.cfg,
                                      static_cast<hipStream_t>(stream)));
    // the split blocks' partial sums travel through the caller's workspace
    Workspace w;
    if (!ws || ws_bytes < layout(FS_VARIANT_LOGITS, pl, 0, nullptr, nullptr))
        return FS_ERR_WORKSPACE;
    layout(FS_VARIANT_LOGITS, pl, 0, static_cast<char*>(ws), &w);
    return from_hip(launch_stream(kVarLogits, a, pl.grid_y, pl.cfg, w.part, true,
                                  static_cast<hipStream_t>(stream)));
}

fs_status fs_multinomial(const fs_params* p, const float* logits, const float* temp,
                         const uint32_t* allow, int32_t* out_idx, void* ws, size_t ws_bytes,
                         void* stream) {
    fs_status st = check_params(p);
    if (st != FS_OK) return st;
    if (p->B == 0) return FS_OK;
    if (!out_idx || (p->V > 0 && !logits)) return FS_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceInfo dev;
    if (!current_device(dev)) return FS_ERR_UNSUPPORTED;
    if (p->V == 0) return from_hip(launch_fill_idx(out_idx, p->B, -1, nullptr, s));
    Plan pl;
    make_plan(p, kVarFlat, dev.cus, pl);
    Workspace w;
    const size_t need = layout(FS_VARIANT_MULTINOMIAL, pl, 0, nullptr, nullptr);
    if (!ws || ws_bytes < need) return FS_ERR_WORKSPACE;
    layout(FS_VARIANT_MULTINOMIAL, pl, 0, static_cast<char*>(ws), &w);
    const int nchunk = (p->V + kMultinomialChunk - 1) / kMultinomialChunk;
    return from_hip(launch_multinomial(logits, temp, allow, p->B, p->V, p->n_valid, p->v_offset,
                                       noise_src(pl, p), p->flags, nchunk,
                                       kMultinomialChunk, w.mm, w.ms, w.mkey, out_idx, s));
}

fs_status fs_debug_noise(uint64_t seed, uint32_t step, uint32_t stream_id, int32_t b0,
                         int32_t nb, int64_t i0, int32_t ni, uint32_t* words, float* gumbel,
                         void* stream) {
    if (nb < 0 || ni < 0 || i0 < 0 || b0 < 0) return FS_ERR_INVALID_ARG;
    if (nb == 0 || ni == 0 || (!words && !gumbel)) return FS_OK;
    if (nb > 65535) return FS_ERR_UNSUPPORTED;
    DeviceInfo dev;
    if (!current_device(dev)) return FS_ERR_UNSUPPORTED;
    return from_hip(launch_debug_noise((uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32),
                                       step, stream_id, b0, nb, i0, ni, words, gumbel,
                                       static_cast<hipStream_t>(stream)));
}

fs_status fs_debug_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t grid,
                              void* stream) {
    if (!src || !sink || grid < 1 || bytes % 16 != 0) return FS_ERR_INVALID_ARG;
    if (!aligned16(src)) return FS_ERR_UNSUPPORTED;
    DeviceInfo dev;
    if (!current_device(dev)) return FS_ERR_UNSUPPORTED;
    return from_hip(launch_read_probe(src, bytes, sink, grid, static_cast<hipStream_t>(stream)));
}

fs_status fs_debug_copy(void* dst, const void* src, size_t bytes, int32_t grid, void* stream) {
    if (!src || !dst || grid < 1 || bytes % 16 != 0) return FS_ERR_INVALID_ARG;
    if (!aligned16(src) || !aligned16(dst)) return FS_ERR_UNSUPPORTED;
    DeviceInfo dev;
    if (!current_device(dev)) return FS_ERR_UNSUPPORTED;
    return from_hip(launch_copy(dst, src, bytes, grid, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

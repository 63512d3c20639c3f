// Host side of libfs: argument validation, launch planning, workspace layout
// and the extern "C" entry points declared in include/fs.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "fs.h"
#include "fs_internal.h"

namespace {

using namespace fs;

// Scratch memory of fs_sample_noalloc: one array per device, held for the
// life of the process.  In host code this name is a host-side stand-in, not
// a device address: the address each device's copy has is taken once per
// device with hipGetSymbolAddress (DeviceInfo::scratch) and only that is
// used.  The first kSchedBytes hold the unit scheduler block at a fixed
// place; the call's records follow.
constexpr size_t kScratchBytes = (size_t)FS_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceInfo {
    bool ok = false;      // a gfx950 device
    int cus = 0;
    void* scratch = nullptr;   // this device's copy of `scratch` (null: not found)
};

std::mutex g_mu;
DeviceInfo g_dev[64];
bool g_dev_init[64];

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
        if (info.ok) {   // with device `dev` current
            void* ptr = nullptr;
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess && ptr)
                info.scratch = ptr;
            else
                (void)hipGetLastError();
        }
        g_dev[dev] = info;
        g_dev_init[dev] = true;
    }
    out = g_dev[dev];
    return out.ok && out.cus > 0;
}

// Device pointers of the workspace arrays of one call.
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
    unsigned long long* gsel = nullptr;   // grouped block records: stage 2's sample pairs
    SchedState* sched = nullptr;   // flat: unit scheduler block (kept from call to call)
    void* sel = nullptr;    // top-k: lists of the intermediate selection levels
};

Workspace carve(char* base, const WsLayout& l) {
    auto at = [&](size_t off) -> void* { return off == kAbsent ? nullptr : base + off; };
    Workspace w;
    w.pm = static_cast<float*>(at(l.pm));
    w.pidx = static_cast<int32_t*>(at(l.pidx));
    w.pL = static_cast<float*>(at(l.pL));
    w.cx = static_cast<float*>(at(l.cx));
    w.cidx = static_cast<int32_t*>(at(l.cidx));
    w.sel = at(l.sel);
    w.mm = static_cast<float*>(at(l.mm));
    w.ms = static_cast<float*>(at(l.ms));
    w.mkey = static_cast<uint64_t*>(at(l.mkey));
    w.part = at(l.part);
    w.gsel = static_cast<unsigned long long*>(at(l.gsel));
    w.sched = static_cast<SchedState*>(at(l.sched));
    return w;
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

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
    a.rec_cols = 0;
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
    if (!topk_launchable(pl, k)) return FS_ERR_UNSUPPORTED;
    const WsLayout lay = layout(FS_VARIANT_TOPK, pl, k);
    if (!ws || ws_bytes < lay.total) return FS_ERR_WORKSPACE;
    const Workspace w = carve(static_cast<char*>(ws), lay);
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
    const int64_t tv = p->tile_v ? p->tile_v : kDefaultTileV;
    return (int32_t)(((int64_t)p->V + tv - 1) / tv);
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
    if (!pl.launchable) return 0;
    if (variant == FS_VARIANT_TOPK && pl.kind != kResident && k > kMaxTopKCoop) return 0;
    if (variant == FS_VARIANT_TOPK && !topk_launchable(pl, k)) return 0;
    if (variant == FS_VARIANT_MULTINOMIAL && p->B > kMaxGridY) return 0;
    return std::max(kAlign, layout(variant, pl, k).total);
}

// Shared front half of fs_sample and fs_sample_stage1: validation, plan,
// workspace carve-up and the stage-1 launch.  `done` is set when nothing is
// left to do (B == 0, or V == 0 after filling the outputs).
// own_scratch: the workspace is the device's scratch array of
// fs_sample_noalloc (ws and ws_bytes are ignored): its scheduler block sits
// at a fixed place, the first kSchedBytes, and the records follow.
static fs_status flat_stage1(const fs_params* p, const void* H, const void* W, const float* temp,
                             const uint32_t* allow, int32_t* out_idx, float* out_score,
                             void* ws, size_t ws_bytes, hipStream_t s, bool need_out,
                             bool own_scratch, Plan& pl, Workspace& w, bool& done) {
    done = true;
    fs_status st = check_params(p);
    if (st != FS_OK) return st;
    if (p->B == 0) return FS_OK;
    if (need_out && !out_idx) return FS_ERR_INVALID_ARG;
    if (p->V > 0 && (st = check_operands(p, H, W)) != FS_OK) return st;
    DeviceInfo dev;
    if (!current_device(dev)) return FS_ERR_UNSUPPORTED;
    if (own_scratch) {
        if (!dev.scratch) return FS_ERR_HIP;
        ws = dev.scratch;
        ws_bytes = kScratchBytes;
    }
    if (p->V == 0)
        return need_out ? from_hip(launch_fill_idx(out_idx, p->B, -1, out_score, s)) : FS_OK;
    make_plan(p, kVarFlat, dev.cus, pl);
    if (!pl.launchable) return FS_ERR_UNSUPPORTED;
    const WsLayout lay = layout(FS_VARIANT_FLAT, pl, 0);
    const size_t head = own_scratch ? kSchedBytes : 0;
    if (!ws || ws_bytes < head + lay.total) return FS_ERR_WORKSPACE;
    w = carve(static_cast<char*>(ws) + head, lay);
    if (own_scratch) w.sched = static_cast<SchedState*>(ws);
    Stage1Args a = stage1_args(pl, p, H, W, temp, allow);
    a.pm = w.pm;
    a.pidx = w.pidx;
    a.dyn_k0 = dynamic_k0(pl);
    a.sched = a.dyn_k0 > 0 ? w.sched : nullptr;
    const hipError_t e =
        pl.kind == kRows       ? launch_rows(kVarFlat, a, pl.nt, pl.grid_y, s)
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
                               false, pl, w, done);
    if (st != FS_OK || done) return st;
    return from_hip(launch_stage2_flat(w.pm, w.pidx, pl.P, pl.B, out_idx, out_score, w.sched, s));
}

fs_status fs_sample_noalloc(const fs_params* p, const void* H, const void* W, const float* temp,
                            const uint32_t* allow, int32_t* out_idx, float* out_score,
                            void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    Plan pl;
    Workspace w;
    bool done;
    fs_status st = flat_stage1(p, H, W, temp, allow, out_idx, out_score, nullptr, 0, s, true,
                               true, pl, w, done);
    if (st != FS_OK || done) return st;
    return from_hip(launch_stage2_flat(w.pm, w.pidx, pl.P, pl.B, out_idx, out_score, w.sched, s));
}

fs_status fs_sample_stage1(const fs_params* p, const void* H, const void* W, const float* temp,
                           const uint32_t* allow, void* ws, size_t ws_bytes, void* stream) {
    Plan pl;
    Workspace w;
    bool done;
    return flat_stage1(p, H, W, temp, allow, nullptr, nullptr, ws, ws_bytes,
                       static_cast<hipStream_t>(stream), false, false, pl, w, done);
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
    if (!pl.launchable) return FS_ERR_UNSUPPORTED;
    const WsLayout lay = layout(FS_VARIANT_GROUPED, pl, 0);
    if (!ws || ws_bytes < lay.total) return FS_ERR_WORKSPACE;
    const Workspace w = carve(static_cast<char*>(ws), lay);
    Stage1Args a = stage1_args(pl, p, H, W, temp, allow);
    a.pm = w.pm;
    a.pidx = w.pidx;
    a.pL = w.pL;
    a.rec_cols = pl.rec_cols;
    // unit records: the ticket order like flat once stage 2 has set up the
    // scheduler block
    a.dyn_k0 = dynamic_k0(pl);
    a.sched = a.dyn_k0 > 0 ? w.sched : nullptr;
    a.gsel = w.gsel;
    hipError_t e =
        pl.kind == kRows       ? launch_rows(kVarGrouped, a, pl.nt, pl.grid_y, s)
        : pl.kind == kWide     ? launch_wide(kVarGrouped, a, pl.nt, pl.grid_y, s)
        : pl.kind == kResident ? launch_resident(kVarGrouped, a, pl.grid_y, pl.rcfg, s)
        : pl.stream            ? launch_stream(kVarGrouped, a, pl.grid_y, pl.cfg, w.part, true, s)
                               : launch_stage1(kVarGrouped, a, pl.grid_y, pl.cfg, s);
    if (e != hipSuccess) return FS_ERR_HIP;
    // record slot (worker w, tile t) is w + t; the streaming kernel's workers
    // own ranges of (block, quarter) units, the cooperative kernel's of blocks;
    // with unit records the slot is the block
    const int workers = pl.stream ? 4 * pl.G : pl.G;
    const int units = pl.stream ? 4 * pl.nmb : pl.nmb;
    const int tile_units = pl.stream ? 4 * pl.tile_mb : pl.tile_mb;
    return from_hip(launch_stage2_grouped(w.pm, w.pidx, w.pL, pl.P, pl.rec_cols, pl.B, pl.T, workers, units,
                                          tile_units, temp, p->flags, noise_src(pl, p), tile_max,
                                          tile_idx, tile_logmass, out_idx, w.gsel,
                                          a.dyn_k0 > 0 ? w.sched : nullptr, s));
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
    if (!pl.launchable) return FS_ERR_UNSUPPORTED;
    Stage1Args a = stage1_args(pl, p, H, W, nullptr, nullptr);
    a.logits = logits;
    if (pl.kind == kRows)
        return from_hip(launch_rows(kVarLogits, a, pl.nt, pl.grid_y,
                                    static_cast<hipStream_t>(stream)));
    if (pl.kind == kResident)
        return from_hip(launch_resident(kVarLogits, a, pl.grid_y, pl.rcfg,
                                        static_cast<hipStream_t>(stream)));
    if (!pl.stream)
        return from_hip(launch_stage1(kVarLogits, a, pl.grid_y, pl.cfg,
                                      static_cast<hipStream_t>(stream)));
    // the split blocks' partial sums travel through the caller's workspace
    const WsLayout lay = layout(FS_VARIANT_LOGITS, pl, 0);
    if (!ws || ws_bytes < lay.total) return FS_ERR_WORKSPACE;
    const Workspace w = carve(static_cast<char*>(ws), lay);
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
    if (p->B > kMaxGridY) return FS_ERR_UNSUPPORTED;   // one row per workgroup along y
    Plan pl;
    make_plan(p, kVarFlat, dev.cus, pl);
    const WsLayout lay = layout(FS_VARIANT_MULTINOMIAL, pl, 0);
    if (!ws || ws_bytes < lay.total) return FS_ERR_WORKSPACE;
    const Workspace w = carve(static_cast<char*>(ws), lay);
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
    return from_hip(
        launch_read_probe(src, bytes, sink, grid, false, static_cast<hipStream_t>(stream)));
}

fs_status fs_debug_read_probe_nt(const void* src, size_t bytes, uint32_t* sink, int32_t grid,
                                 void* stream) {
    if (!src || !sink || grid < 1 || bytes % 16 != 0) return FS_ERR_INVALID_ARG;
    if (!aligned16(src)) return FS_ERR_UNSUPPORTED;
    DeviceInfo dev;
    if (!current_device(dev)) return FS_ERR_UNSUPPORTED;
    return from_hip(
        launch_read_probe(src, bytes, sink, grid, true, static_cast<hipStream_t>(stream)));
}

fs_status fs_debug_shared_read_probe(const void* src, size_t bytes, int32_t reps, uint32_t* sink,
                                     int32_t grid, void* stream) {
    if (!src || !sink || grid < 1 || reps < 1 || bytes == 0 || bytes % 32768 != 0)
        return FS_ERR_INVALID_ARG;
    if (!aligned16(src)) return FS_ERR_UNSUPPORTED;
    DeviceInfo dev;
    if (!current_device(dev)) return FS_ERR_UNSUPPORTED;
    return from_hip(launch_shared_read_probe(src, bytes, reps, sink, grid,
                                             static_cast<hipStream_t>(stream)));
}

fs_status fs_debug_copy(void* dst, const void* src, size_t bytes, int32_t grid, void* stream) {
    if (!src || !dst || grid < 1 || bytes % 16 != 0) return FS_ERR_INVALID_ARG;
    if (!aligned16(src) || !aligned16(dst)) return FS_ERR_UNSUPPORTED;
    DeviceInfo dev;
    if (!current_device(dev)) return FS_ERR_UNSUPPORTED;
    return from_hip(launch_copy(dst, src, bytes, grid, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// Launch planning and workspace layout of libfs: plain host C++ (no HIP), so
// that the size arithmetic can be built and checked on a CPU alone, under
// address and undefined-behaviour sanitizers.  The plan depends only on the
// call's fs_params, the variant and the device's compute-unit count.
#pragma once

#include <cstddef>
#include <cstdint>

#include "fs.h"

namespace fs {

constexpr int kMBlock = 16;           // vocab rows per MFMA block (M of 16x16x32)
constexpr uint32_t kFlagNoNoise = 1u;
constexpr int kDefaultTileV = 128;
constexpr int kMaxTopK = 1024;
constexpr int kMaxTopKCoop = 64;      // the cooperative kernel keeps sorted lists of at most 64
constexpr int kMultinomialChunk = 2048;
constexpr int kMaxB = 1 << 20;
constexpr size_t kAlign = 256;
constexpr size_t kSchedBytes = 256;   // unit scheduler block of a flat workspace
// Top-k stage 2: threads of the one-kernel form, candidates one selection
// workgroup holds (checked against the kernels in fs_stage2.hip).
constexpr int kTopkStage2Threads = 512;
constexpr int kTopkSliceCap = 1024 * 16;
// Grouped records from the LDS-tiled kernel: a range meets at most this many
// vocabulary tiles (their slots live in LDS).
constexpr int kWideMaxTiles = 16;

enum Stage1Variant { kVarFlat = 0, kVarGrouped = 1, kVarLogits = 2, kVarTopk = 3 };

// Stage-1 kernel families: resident (H slice in registers; the default for
// the common shapes), stream (independent worker waves, H reloaded per stage),
// coop (workgroup-cooperative, H reloaded per stage; top-k and the shapes the
// others do not cover), rows (large batches: W rows streamed into registers,
// H chunks through LDS; flat and logits) and wide (LDS-tiled; grouped records
// for 32 < B <= 64).
enum Stage1Kind { kCoop = 0, kStream = 1, kResident = 2, kWide = 3, kRows = 4 };

// Grouped block records: stage 2's per-row [key, count] sample pairs, one
// pair per 128-byte line (row b's at element kGselStride b of the array), so
// that the atomics of different rows go to different lines.
constexpr int kGselStride = 16;

// The row-streaming large-batch kernel (fs_rows.hip): workgroups of 64, 128
// or 256 batch columns (more columns: several column groups), H chunks of KCS
// k-steps taken in pairs (d a multiple of 64 KCS).
struct RowsShape {
    int nt;    // batch columns per workgroup
    int kra;   // 16-row blocks per wave and tile (tiles of 128 kra rows)
    int kcs;   // k-steps of 32 per H chunk
    int pf;    // k-steps of W in flight per wave (at most)
    int gq;    // k-steps of W loaded at a time (runs of 64 gq bytes per row)
};
constexpr RowsShape kRows64 = {64, 2, 8, 8, 4};
constexpr RowsShape kRows128 = {128, 2, 8, 8, 4};
constexpr RowsShape kRows256 = {256, 2, 4, 4, 2};
constexpr int rows_kcs(int nt) {
    return nt == kRows64.nt ? kRows64.kcs : nt == kRows128.nt ? kRows128.kcs : kRows256.kcs;
}

struct Stage1Config {
    int nb;   // 16-wide batch blocks per workgroup
    int mpi;  // vocab blocks per group
    int ks;   // 32-element k-steps per pipeline stage
};

// Resident-H stage 1: nw waves split the hidden dimension, hk + hl k-steps
// each (nks == nw * (hk + hl); hk of them held in registers, hl in LDS), mpi
// blocks per group, ks k-steps per pipeline stage.
struct ResidentConfig {
    int nb, mpi, ks, nw, hk, hl;
};

// Top-k row store of one resident workgroup: the most vocabulary rows it may
// own (the x of all its columns in LDS): 96 KiB of x, or 640 rows when part
// of the H slice also lives in LDS (hl > 0).  A multiple of 128.
constexpr int topk_store_rows(int nb, int hl) { return hl > 0 ? 640 : 96 * 1024 / (16 * nb * 4); }

// Instantiated resident shapes (nb, mpi, ks, nw, hk, hl, topk), in order of
// preference for a given nb and k-step count nw * (hk + hl); topk = 1 where
// the top-k row store fits in LDS beside the shape's own areas (the kernel
// source checks this column against its LDS structures).  hl > 0 keeps the
// last hl k-steps of each wave's H slice in LDS (d = 5120 with two batch
// blocks; the 18 + 2 split leaves room in LDS for the top-k row store).  Hidden
// sizes and their shapes: 512, 1024, 2048, 3072 (12 k-steps per wave), 4096,
// 5120, and with one batch block and four waves of up to 512 registers (H in
// VGPRs and AGPRs) 6144 and 7168 (48 and 56 k-steps per wave; 8 waves would
// spill there).
#define FS_RESIDENT_SHAPES(X) \
    X(1, 2, 4, 8, 16, 0, 1)   \
    X(1, 4, 2, 8, 16, 0, 0)   \
    X(1, 2, 4, 4, 32, 0, 1)   \
    X(1, 2, 4, 8, 8, 0, 1)    \
    X(1, 2, 2, 8, 20, 0, 1)   \
    X(1, 2, 2, 8, 4, 0, 1)    \
    X(1, 2, 1, 8, 2, 0, 1)    \
    X(2, 1, 4, 8, 16, 0, 1)   \
    X(2, 1, 2, 8, 16, 0, 1)   \
    X(2, 2, 2, 8, 16, 0, 0)   \
    X(2, 1, 2, 8, 16, 4, 0)   \
    X(2, 1, 2, 8, 18, 2, 1)   \
    X(2, 2, 4, 8, 8, 0, 0)    \
    X(2, 2, 2, 8, 4, 0, 0)    \
    X(2, 2, 1, 8, 2, 0, 0)    \
    X(2, 1, 2, 8, 12, 0, 1)   \
    X(1, 2, 2, 8, 12, 0, 1)   \
    X(1, 2, 4, 4, 48, 0, 1)   \
    X(1, 2, 4, 4, 56, 0, 1)

bool resident_supported(const ResidentConfig& c, int variant);
// Preferred instantiated shape for nb batch blocks, nks k-steps and a variant
// (nw == 0: none).
ResidentConfig resident_default(int nb, int nks, int variant);
// Top-k: the most vocabulary rows one resident workgroup of shape c may own.
int resident_topk_rows(const ResidentConfig& c);

// Validated shape of one call and its launch plan.
struct Plan {
    int variant;   // Stage1Variant
    int B, d, V, n_valid, v_offset, tile_v, tile_mb, T, nmb, G;
    int kind;      // Stage1Kind
    bool stream;   // kind == kStream
    int P;         // record slots per row
    Stage1Config cfg;
    ResidentConfig rcfg;
    int nt;        // kWide, kRows: batch columns per workgroup
    int grid_y;
    int xcd_pair;
    // resident grouped: one record per 16-row block (slot = block index, the
    // blocks of a tile merged in stage 2) instead of one per (range, tile):
    // the walk then takes the strided and ticket order of flat; the records
    // are block-major, rec_cols (B rounded up to 32) per block
    bool unit_rec;
    int rec_cols;   // 0: records [B][P]
    uint32_t k0, k1;
    bool launchable;   // the grids fit HIP's limits (else FS_ERR_UNSUPPORTED)
};

// HIP grid limits the plans keep to: at most 65535 workgroups along y, and
// along x at most 2^32 work-items (4M workgroups of up to 1024 threads).
constexpr int kMaxGridY = 65535;
constexpr int64_t kMaxGridX = (int64_t)1 << 22;

// Byte offsets of the workspace arrays of one call (kAbsent: not used) and the
// total size.  Every array starts on a 256-byte boundary.
constexpr size_t kAbsent = ~(size_t)0;
struct WsLayout {
    size_t pm = kAbsent, pidx = kAbsent, pL = kAbsent;   // partial records [B][P]
    size_t cx = kAbsent, cidx = kAbsent;               // top-k candidates [B][G][L]
    size_t sel = kAbsent;                            // top-k selection levels
    size_t mm = kAbsent, ms = kAbsent, mkey = kAbsent;   // multinomial chunk sums
    size_t part = kAbsent;                           // streaming partial sums
    size_t gsel = kAbsent;                           // grouped block records: [B][kGselStride] (a sample pair per line)
    size_t sched = kAbsent;                          // flat/grouped/top-k unit scheduler (last)
    size_t total = 0;
};

// FS_OK, or the status a call with these parameters returns before any work.
fs_status check_params(const fs_params* p);
// Plan of a call that passed check_params with B > 0 and V > 0, on a device
// with `cus` compute units.  variant: Stage1Variant.
void make_plan(const fs_params* p, int variant, int cus, Plan& pl);
// Workspace layout for a workspace variant (FS_VARIANT_*) of a plan.
WsLayout layout(int ws_variant, const Plan& pl, int k);
// Bytes of parked partial sums of the streaming kernel.
size_t part_bytes(const Plan& pl);
// Units each workgroup of the resident flat / top-k stage 1 takes in the
// strided order before it turns to the ticket counter (0: strided order only,
// and for every other variant).
int dynamic_k0(const Plan& pl);
// Entries per top-k candidate list, and whether the lists are dense.
int topk_len(const Plan& pl, int k);
bool topk_dense(const Plan& pl, int k);
// The top-k stages of a plan for k fit their grids and 32-bit candidate counts.
bool topk_launchable(const Plan& pl, int k);
// Stage 2 of top-k in one kernel (k <= 64, lists with ids, at most 512 * 64
// candidates per row).
bool topk_small_path(int G, int L, int k);
// Scratch bytes of the top-k selection levels (0 when one level suffices).
size_t stage2_topk_scratch_bytes(int G, int L, int B, int k, bool dense);

}  // namespace fs

// Internal interfaces between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fs_device.h"
#include "fs_plan.h"

namespace fs {

constexpr int kThreads = 256;      // threads per stage-1 workgroup (4 waves)
constexpr int kWaves = kThreads / 64;

// Balanced split of `nmb` vocab blocks over `G` workgroups: workgroup w owns
// blocks [begin(w), begin(w+1)).  Every workgroup owns at least one block
// when G <= nmb.
__host__ __device__ inline int part_begin(int w, int nmb, int G) {
    return (int)(((int64_t)w * nmb) / G);
}
// The workgroup owning block m.
__host__ __device__ inline int part_owner(int m, int nmb, int G) {
    return (int)((((int64_t)m + 1) * G - 1) / nmb);
}

// Streaming stage 1: a unit is (16-row block, hidden-dimension quarter); worker
// wk of W owns units [wk*U/W, (wk+1)*U/W) of U = 4*nmb.  With W <= nmb every
// range holds >= 4 units, so a block is split between at most two workers.
struct WorkerRange {
    int u0, u1;    // unit range
    int hb, hq;    // head partial block and its first quarter (hq == 0: none)
    int fb0, fb1;  // whole blocks [fb0, fb1)
    int tb, tq;    // tail partial block and its quarter count (tq == 0: none)
};
__host__ __device__ inline WorkerRange worker_range(int wk, int W, int nmb) {
    const int64_t U = 4ll * nmb;
    WorkerRange r;
    r.u0 = (int)(wk * U / W);
    r.u1 = (int)((wk + 1) * U / W);
    r.hb = r.u0 / 4;
    r.hq = r.u0 % 4;
    r.fb0 = (r.u0 + 3) / 4;
    r.fb1 = r.u1 / 4;
    r.tb = r.u1 / 4;
    r.tq = r.u1 % 4;
    return r;
}

// Unit scheduler of the resident flat stage 1, kept in the workspace from
// call to call.  Workgroups take their first units in the strided order and
// the last ones from a ticket counter, so that workgroups that run faster
// take more units.  tag == kSchedTag and the high half of word ==
// kSchedTag32 mark an initialised block (the low half of word counts the
// tickets, exits the workgroups done); any other content (a fresh or foreign
// buffer) makes stage 1 keep the strided order for that call.  The flat
// stage 2 writes (kSchedTag, kSchedTag32 << 32, 0) after every call, and the
// last workgroup to finish a call's stage 1 sets both counts back to 0.
struct SchedState {
    unsigned long long tag;
    unsigned long long word;
    unsigned long long exits;
};
constexpr unsigned long long kSchedTag = 0x4c4d4847554d4231ull;
constexpr unsigned int kSchedTag32 = 0x53434844u;
static_assert(sizeof(SchedState) <= kSchedBytes, "scheduler block");

struct Stage1Args {
    const uint16_t* H;      // [B, d] bf16
    const uint16_t* W;      // [V, d] bf16
    const float* temp;      // [B] or null
    const uint32_t* allow;  // [B, ceil(V/32)] or null
    int B, d, V, n_valid, v_offset;
    int nmb;                // ceil(V / 16)
    int G;                  // workgroups along the vocabulary (gridDim.x)
    int tile_mb;            // blocks per record tile (flat: one segment)
    NoiseSrc noise;         // Philox key and step (per row when given)
    uint32_t flags;
    int topk;               // k of the top-k variant
    int topk_len;           // entries per candidate list: min(k, rows of the longest range)
    int topk_dense;         // lists are whole ranges: every row's x in row order, no ids
    int ny;                 // resident kernel: batch groups sharing one row range
    int xcd_pair;           // resident kernel: 1-D grid, groups of a range on one XCD
    // partial records [B][P] (P slots per row: the workers for flat, workers
    // + T - 1 for grouped, where (worker w, tile t) is slot w + t; the
    // resident kernel's grouped records: one per 16-row block, slot = block)
    int P;
    // 0: records row-major [B][P]; else block-major [P][rec_cols] (the
    // resident kernel's block records: rec_cols = B rounded up to 32, so the
    // records of a block's 32 columns fill whole 128-byte lines written by
    // one workgroup)
    int rec_cols;
    float* pm;
    int32_t* pidx;
    float* pL;
    // resident grouped: stage 2's per-row [key, count] pairs, cleared here
    unsigned long long* gsel;
    // top-k candidates [B][G][topk_len] (row-major: a row's lists are one
    // contiguous run): tempered logit and id
    float* cx;
    int32_t* cidx;
    // unfused baseline output [B, V]
    float* logits;
    // resident flat: unit scheduler (null: strided order) and the units each
    // workgroup takes in the strided order first (3 <= dyn_k0, dyn_k0 G <= nunits)
    SchedState* sched;
    int dyn_k0;
};

hipError_t launch_stage1(int variant, const Stage1Args& a, int grid_y, const Stage1Config& cfg,
                         hipStream_t stream);

// Top-k row store of one resident workgroup: the most vocabulary rows it
// may own (x of all its columns in LDS): 96 KiB of x, or 640 rows when part
// of the H slice also lives in LDS (hl > 0).
template <int NB, int HL>
struct TopkRows {
    static constexpr int kRows = topk_store_rows(NB, HL);   // multiple of 128
    static constexpr int kStride = kRows + 4;   // padded row of one column
};
hipError_t launch_resident(int variant, const Stage1Args& a, int grid_y, const ResidentConfig& c,
                           hipStream_t stream);

// LDS-tiled grouped stage 1 (fs_wide.hip): nt = 64, when every workgroup
// range meets at most kWideMaxTiles vocabulary tiles.
hipError_t launch_wide(int variant, const Stage1Args& a, int nt, int grid_y, hipStream_t stream);

// Row-streaming stage 1 for large batches (fs_rows.hip): flat and logits,
// nt = 64, 128 or 256 batch columns per workgroup, d % (64 rows_kcs(nt)) == 0.
hipError_t launch_rows(int variant, const Stage1Args& a, int nt, int grid_y, hipStream_t stream);

// Streaming stage 1 (flat, grouped or logits) over a.G workgroups of four
// worker waves; `part` holds grid_y * 4 * a.G * 2 * nb KiB of partial sums.
// with_fixup also launches the kernel finishing the split blocks.
hipError_t launch_stream(int variant, const Stage1Args& a, int grid_y, const Stage1Config& cfg,
                         void* part, bool with_fixup, hipStream_t stream);

// sched (may be null): the unit scheduler block, initialised by the kernel.
hipError_t launch_stage2_flat(const float* pm, const int32_t* pidx, int P, int B,
                              int32_t* out_idx, float* out_score, SchedState* sched,
                              hipStream_t stream);

// Grouped records: tile t's are the slots w + t of the G ranges of nmb units
// that meet it (records [B][P]), or with gsel (block records, block-major
// [nmb][rec_cols], slot = block: nmb blocks, tiles of tile_mb) its blocks;
// gsel is the per-row [key, count] pair of the sample, cleared by stage 1,
// at gsel[kGselStride b].  sched as for flat.
hipError_t launch_stage2_grouped(const float* pm, const int32_t* pidx, const float* pL, int P,
                                 int rec_cols, int B, int T, int G, int nmb, int tile_mb, const float* temp,
                                 uint32_t flags, const NoiseSrc& noise, float* tile_max,
                                 int32_t* tile_idx, float* tile_L, int32_t* out_idx,
                                 unsigned long long* gsel, SchedState* sched, hipStream_t stream);

// Candidates [B][G][L] (L entries per list); 1 <= k <= 1024.  With dn.on
// the lists are dense: list w holds the x of every row workgroup w kept, in
// its store order (padded with -inf), and cidx is not read (ids as DenseIds
// says).  top_p >= 1:
// plain top-k; 0 < top_p < 1: top-p after top-k.  scratch: device memory of
// stage2_topk_scratch_bytes(G, L, B, k, dense) bytes (256-byte aligned; may be null
// when that is 0) for the lists of the intermediate selection levels.
// Global ids of the rows a top-k workgroup keeps, in its store order: store
// unit i (unit_rows rows, a power of two) is vocabulary unit tab[i], whose
// rows are ids v_offset + tab[i] unit_rows + 0, 1, ...
struct RowIds {
    int v_offset, unit_rows;
    const int* tab;
};
__device__ inline int row_id(const RowIds& m, int r) {
    return m.v_offset + m.tab[r / m.unit_rows] * m.unit_rows + r % m.unit_rows;
}

// Dense top-k lists (on != 0): entry r of list w has id row_id({v_offset +
// w unit_rows, unit_rows, unit_stride}, r).
struct DenseIds {
    int on, v_offset, unit_rows, unit_stride;
};
// Stage 2 of top-k runs in one kernel (stage2_topk_kernel) when
// topk_small_path holds: sched (may be null; that kernel only) is the unit
// scheduler block of the resident stage 1, initialised by the kernel.
hipError_t launch_stage2_topk(const float* cx, const int32_t* cidx, int G, int L, int B, int k,
                              DenseIds dn, float top_p, const float* temp, uint32_t flags,
                              const NoiseSrc& noise, int32_t* out_idx, void* scratch,
                              SchedState* sched, hipStream_t stream);

hipError_t launch_merge_online(int B, int C, const int32_t* z, const float* L, const float* temp,
                               const NoiseSrc& noise, uint32_t flags,
                               int32_t* out_idx, float* out_L, hipStream_t stream);

hipError_t launch_multinomial(const float* logits, const float* temp, const uint32_t* allow,
                              int B, int V, int n_valid, int v_offset, const NoiseSrc& noise,
                              uint32_t flags, int nchunk, int chunk,
                              float* ws_m, float* ws_s, uint64_t* ws_key, int32_t* out_idx,
                              hipStream_t stream);

hipError_t launch_fill_idx(int32_t* out, int n, int32_t value, float* score, hipStream_t stream);

hipError_t launch_debug_noise(uint32_t k0, uint32_t k1, uint32_t step, uint32_t stream_id,
                              int b0, int nb, int64_t i0, int ni, uint32_t* words, float* gumbel,
                              hipStream_t stream);

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int grid, bool nt,
                             hipStream_t stream);
hipError_t launch_copy(void* dst, const void* src, size_t bytes, int grid, hipStream_t stream);
// bytes a multiple of 32 KiB
hipError_t launch_shared_read_probe(const void* src, size_t bytes, int reps, uint32_t* sink,
                                   int grid, hipStream_t stream);

}  // namespace fs

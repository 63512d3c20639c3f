// Streaming stage 1 of fused LM-head sampling (gfx950): every wave is an
// independent worker that streams its own contiguous share of W once, forms
// the logits of whole 16-row vocabulary blocks in registers with bf16 MFMA
// (FP32 accumulation), and applies temperature, masks, Philox-Gumbel noise
// and the per-tile reductions in its own lanes ("FlashSampling: Fast and
// Memory-Efficient Exact Sampling", Abstract; FlashSampling explainer on
// aitrends.kr, Stage 1 and tensor-parallel paragraphs).
//
// Work split.  The vocabulary is cut into 16-row blocks and the hidden
// dimension into quarters; a unit is (block, quarter), so a call has 4*nmb
// units.  Worker wk of W owns units [wk*U/W, (wk+1)*U/W): a balanced,
// contiguous range.  Inside it the worker meets at most three kinds of items:
//   head  the last quarters of a block that starts in the previous worker,
//   full  whole blocks (processed MPI at a time, never across a tile edge),
//   tail  the first quarters of a block that ends in the next worker.
// Full blocks are finished in the worker.  Head and tail partial sums go to
// the workspace; fixup_kernel adds the two halves of each split block (lower
// quarters first) and finishes it, merging into the record of the worker that
// holds its first quarters.  With W <= nmb a block spans at most two workers.
//
// There is no communication between the waves of a workgroup, so no barrier
// ever stalls the load stream: the loads of the next stage (the next item's
// first stage at the end of an item) are issued before the MFMAs of the
// current one and stay in flight through the epilogue.
#include "fs_device.h"
#include "fs_internal.h"
#include "fs_mfma.h"
#include "fs_epilogue.h"

namespace fs {

enum ItemKind { kHead = 0, kFull = 1, kTail = 2, kNone = 3 };

struct Item {
    int kind;
    int g, nvm;        // first block, blocks in the item
    int ks_lo, ks_hi;  // k-step range
    int t, seg_end;    // tile and segment end (full items)
};

__device__ __forceinline__ int quarter_kstep(int q, int nks) { return q * nks / 4; }

template <int MPI>
__device__ __forceinline__ Item full_item(int g, const WorkerRange& r, int tile_mb, int nks) {
    Item it;
    it.kind = kFull;
    it.g = g;
    it.t = g / tile_mb;
    const int64_t te = (int64_t)(it.t + 1) * tile_mb;
    it.seg_end = te < r.fb1 ? (int)te : r.fb1;
    it.nvm = min(MPI, it.seg_end - g);
    it.ks_lo = 0;
    it.ks_hi = nks;
    return it;
}

__device__ __forceinline__ Item tail_item(const WorkerRange& r, int nks) {
    Item it;
    it.kind = r.tq ? kTail : kNone;
    it.g = r.tb;
    it.nvm = 1;
    it.ks_lo = 0;
    it.ks_hi = quarter_kstep(r.tq, nks);
    it.t = 0;
    it.seg_end = 0;
    return it;
}

template <int MPI>
__device__ __forceinline__ Item first_item(const WorkerRange& r, int tile_mb, int nks) {
    if (r.hq) {
        Item it;
        it.kind = kHead;
        it.g = r.hb;
        it.nvm = 1;
        it.ks_lo = quarter_kstep(r.hq, nks);
        it.ks_hi = nks;
        it.t = 0;
        it.seg_end = 0;
        return it;
    }
    if (r.fb0 < r.fb1) return full_item<MPI>(r.fb0, r, tile_mb, nks);
    return tail_item(r, nks);
}

template <int MPI>
__device__ __forceinline__ Item next_item(const Item& c, const WorkerRange& r, int tile_mb,
                                          int nks) {
    if (c.kind == kHead) {
        if (r.fb0 < r.fb1) return full_item<MPI>(r.fb0, r, tile_mb, nks);
        return tail_item(r, nks);
    }
    if (c.kind == kFull) {
        if (c.g + c.nvm < r.fb1) return full_item<MPI>(c.g + c.nvm, r, tile_mb, nks);
        return tail_item(r, nks);
    }
    Item none = c;
    none.kind = kNone;
    return none;
}

template <int NB, int MPI, int KS, int VAR>
__global__ __launch_bounds__(kThreads) void stream_kernel(Stage1Args a, f32x4* part) {
    static_assert(VAR == kVarFlat || VAR == kVarGrouped || VAR == kVarLogits, "variant");
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15;
    const int kg = lane >> 4;
    const int W = gridDim.x * kWaves;           // workers
    const int wk = blockIdx.x * kWaves + wave;  // this worker
    const int bbase = blockIdx.y * 16 * NB;
    const int nks = (a.d + 31) >> 5;
    const WorkerRange rg = worker_range(wk, W, a.nmb);

    const uint16_t* hrow[NB];
    ColCtx cc[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        const int b = bbase + n * 16 + r16;
        hrow[n] = a.H + (size_t)(b < a.B ? b : a.B - 1) * a.d;
        cc[n] = col_ctx(a, b);
    }

    uint64_t best[NB];
    Lse lse[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        best[n] = pack_key(-INFINITY, -1);
        lse[n] = lse_empty();
    }
    // tiles this worker's unit range touches; each gets a record (empty if
    // the worker holds only a partial block there)
    const int t_last = ((rg.u1 - 1) / 4) / a.tile_mb;
    int t_next = (rg.u0 / 4) / a.tile_mb;
    auto empty_records = [&](int t_end) {
        if constexpr (VAR != kVarLogits) {
            for (; t_next < t_end; ++t_next) {
                if (lane < 16) {
#pragma unroll
                    for (int n = 0; n < NB; ++n)
                        put_record<VAR, false>(a, VAR == kVarGrouped ? wk + t_next : wk, cc[n],
                                               pack_key(-INFINITY, -1), lse_empty());
                }
            }
        }
    };

    Operands<NB, MPI, KS> opA, opB;
    const uint16_t* wrow[MPI];
    const uint16_t* wnext[MPI];
    const uint16_t* wsel[MPI];
    bool pre = false;   // opA already holds the first stage of `cur`
    Item cur = first_item<MPI>(rg, a.tile_mb, nks);
    while (cur.kind != kNone) {
        const Item nxt = next_item<MPI>(cur, rg, a.tile_mb, nks);
        Group gc{cur.g, cur.nvm, 0, 0};
        group_rows<MPI>(wrow, a.W, gc, r16, a.V, a.d);
        const bool nxt_live = nxt.kind != kNone;
        Group gn{nxt_live ? nxt.g : cur.g, nxt_live ? nxt.nvm : cur.nvm, 0, 0};
        group_rows<MPI>(wnext, a.W, gn, r16, a.V, a.d);
        const int nlo = nxt_live ? nxt.ks_lo : cur.ks_lo;
        const int nhi = nxt_live ? nxt.ks_hi : cur.ks_hi;

        // ---- contraction over the item's k-steps ----
        f32x4 acc[MPI][NB];
#pragma unroll
        for (int j = 0; j < MPI; ++j)
#pragma unroll
            for (int n = 0; n < NB; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int n_it = ((cur.ks_hi - cur.ks_lo + KS - 1) / KS + 1) & ~1;
        if (cur.ks_hi > cur.ks_lo) {
            if (!pre)
                load_operands<NB, MPI, KS>(opA, wrow, hrow, 0, cur.ks_lo, cur.ks_hi, kg, a.d);
            // sched_barrier keeps the compiler from sinking the prefetch below
            // the MFMAs, which would let the in-flight loads drain every stage
            for (int it = 0; it < n_it; it += 2) {
                load_operands<NB, MPI, KS>(opB, wrow, hrow, it + 1, cur.ks_lo, cur.ks_hi, kg,
                                           a.d);
                __builtin_amdgcn_sched_barrier(0);
                mfma_operands<NB, MPI, KS>(acc, opA);
                __builtin_amdgcn_sched_barrier(0);
                const bool same = it + 2 < n_it;
#pragma unroll
                for (int j = 0; j < MPI; ++j) wsel[j] = same ? wrow[j] : wnext[j];
                load_operands<NB, MPI, KS>(opA, wsel, hrow, same ? it + 2 : 0,
                                           same ? cur.ks_lo : nlo, same ? cur.ks_hi : nhi, kg,
                                           a.d);
                __builtin_amdgcn_sched_barrier(0);
                mfma_operands<NB, MPI, KS>(acc, opB);
                __builtin_amdgcn_sched_barrier(0);
            }
            pre = nxt_live && nxt.ks_hi > nxt.ks_lo;
        } else {
            pre = false;
        }

        // ---- epilogue ----
        if (cur.kind != kFull) {
            // partial block: park the partial sums for fixup_kernel
            const int side = cur.kind == kHead ? 0 : 1;
            const size_t slot = (((size_t)blockIdx.y * W + wk) * 2 + side) * NB;
#pragma unroll
            for (int n = 0; n < NB; ++n) part[(slot + n) * 64 + lane] = acc[0][n];
        } else {
#pragma unroll
            for (int j = 0; j < MPI; ++j) {
                if (j >= cur.nvm) break;               // uniform
                const int row0 = (cur.g + j) * kMBlock + 4 * kg;
#pragma unroll
                for (int n = 0; n < NB; ++n) {
                    if constexpr (VAR == kVarLogits) {
                        if (cc[n].ok) {
                            float* dst = a.logits + (size_t)cc[n].col * a.V;
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (row0 + r < a.V) dst[row0 + r] = acc[j][n][r];
                        }
                    } else {
                        float x[4], s[4];
                        lane_scores(a, cc[n], acc[j][n], row0, true, x, s);
                        fold<VAR>(best[n], lse[n], x, s, a.v_offset + row0);
                    }
                }
            }
            if constexpr (VAR != kVarLogits) {
                if (cur.g + cur.nvm == cur.seg_end) {   // the tile segment ends here
                    empty_records(cur.t);
#pragma unroll
                    for (int n = 0; n < NB; ++n) {
                        column_reduce<VAR>(best[n], lse[n]);
                        if (lane < 16)
                            put_record<VAR, false>(a, VAR == kVarGrouped ? wk + cur.t : wk,
                                                   cc[n], best[n], lse[n]);
                        best[n] = pack_key(-INFINITY, -1);
                        lse[n] = lse_empty();
                    }
                    t_next = cur.t + 1;
                }
            }
        }
        cur = nxt;
    }
    empty_records(t_last + 1);
}

// Finishes the block split between worker w (its tail: the lower quarters)
// and worker w + 1 (its head), one wave per boundary.
template <int NB, int VAR>
__global__ __launch_bounds__(64) void fixup_kernel(Stage1Args a, int W, const f32x4* part) {
    const int w = blockIdx.x;
    const int lane = threadIdx.x;
    const int kg = lane >> 4;
    const WorkerRange rg = worker_range(w, W, a.nmb);
    if (rg.tq == 0) return;                     // no block ends inside this boundary
    const int b = rg.tb;
    const int bbase = blockIdx.y * 16 * NB;
    const size_t tail = (((size_t)blockIdx.y * W + w) * 2 + 1) * NB;
    const size_t head = (((size_t)blockIdx.y * W + w + 1) * 2 + 0) * NB;
    const int row0 = b * kMBlock + 4 * kg;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        const f32x4 v = part[(tail + n) * 64 + lane] + part[(head + n) * 64 + lane];
        const ColCtx c = col_ctx(a, bbase + n * 16 + (lane & 15));
        if constexpr (VAR == kVarLogits) {
            if (c.ok) {
                float* dst = a.logits + (size_t)c.col * a.V;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (row0 + r < a.V) dst[row0 + r] = v[r];
            }
        } else {
            float x[4], s[4];
            lane_scores(a, c, v, row0, true, x, s);
            uint64_t best = pack_key(-INFINITY, -1);
            Lse lse = lse_empty();
            fold<VAR>(best, lse, x, s, a.v_offset + row0);
            column_reduce<VAR>(best, lse);
            const int t = b / a.tile_mb;
            if (lane < 16) put_record<VAR, true>(a, VAR == kVarGrouped ? w + t : w, c, best, lse);
        }
    }
}

template <int NB, int MPI, int KS, int VAR>
static hipError_t launch_stream_one(const Stage1Args& a, int grid_y, f32x4* part,
                                    bool with_fixup, hipStream_t stream) {
    hipLaunchKernelGGL((stream_kernel<NB, MPI, KS, VAR>), dim3(a.G, grid_y), dim3(kThreads), 0,
                       stream, a, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !with_fixup) return e;
    const int W = a.G * kWaves;
    if (W > 1) {
        hipLaunchKernelGGL((fixup_kernel<NB, VAR>), dim3(W - 1, grid_y), dim3(64), 0, stream, a,
                           W, part);
        e = hipGetLastError();
    }
    return e;
}

template <int VAR>
static hipError_t launch_stream_var(const Stage1Args& a, int grid_y, const Stage1Config& c,
                                    f32x4* part, bool with_fixup, hipStream_t stream) {
#define FS_SHAPE(N_, M_, K_)                          \
    if (c.nb == N_ && c.mpi == M_ && c.ks == K_)      \
        return launch_stream_one<N_, M_, K_, VAR>(a, grid_y, part, with_fixup, stream);
    FS_SHAPE(1, 4, 2)
    FS_SHAPE(1, 2, 4)
    FS_SHAPE(1, 4, 4)
    FS_SHAPE(2, 4, 2)
    FS_SHAPE(2, 2, 4)
    FS_SHAPE(2, 4, 1)
    FS_SHAPE(4, 2, 2)
    FS_SHAPE(4, 4, 1)
#undef FS_SHAPE
    return hipErrorInvalidValue;
}

hipError_t launch_stream(int variant, const Stage1Args& a, int grid_y, const Stage1Config& cfg,
                         void* part, bool with_fixup, hipStream_t stream) {
    f32x4* p = static_cast<f32x4*>(part);
    switch (variant) {
        case kVarFlat: return launch_stream_var<kVarFlat>(a, grid_y, cfg, p, with_fixup, stream);
        case kVarGrouped:
            return launch_stream_var<kVarGrouped>(a, grid_y, cfg, p, with_fixup, stream);
        case kVarLogits:
            return launch_stream_var<kVarLogits>(a, grid_y, cfg, p, with_fixup, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fs

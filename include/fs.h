/*
 * fs.h -- C ABI of libfs: exact categorical sampling fused into the LM-head
 * matmul (FlashSampling-style) for AMD Instinct MI355X (gfx950).
 *
 * Method (pages cited by title and passage):
 *  - "FlashSampling: Fast and Memory-Efficient Exact Sampling"
 *    (tomesphere.com/paper/2603.15854), Abstract: compute logits tile by tile
 *    on chip, add Gumbel noise, keep one maximiser per row and vocabulary
 *    tile, finish with a small reduction over tiles; the logits never reach
 *    HBM.  Exact because argmax decomposes over partitions; grouped variants
 *    are exact by hierarchical factorisation of the categorical law.
 *  - "FlashSampling: 빠르고 메모리 효율적인 정확한 샘플링 기법"
 *    (aitrends.kr/articles/26667): Stage 1 paragraph (per-tile logits,
 *    temperature and masking, g = -log(-log u), s = l + g, write m and idx),
 *    Stage 2 paragraph (argmax over tile maxima), tensor-parallel paragraph
 *    (per-group log-mass L = log sum exp l), Group-Gumbel-Max paragraph
 *    (hierarchical and online binary-merge sampling), implementation
 *    paragraph (FP32 noise and accumulation; top-k extension).
 *  - "flashinfer.cake_sampling" (docs.flashinfer.ai), "Correctness contract":
 *    lower index wins ties; explicit seed/offset so graph replays never read a
 *    generator; requests a kernel cannot serve are reported, not failed.
 *  - "On-Chip LLM: Sampling Without Asking" (mikeayles.com): argmax(l + T g)
 *    samples softmax(l / T); zero noise is greedy decoding.
 *
 * Definitions shared by every entry point
 *  - Operands: H is [B, d] bfloat16, row-major (row stride d).  W is [V, d]
 *    bfloat16, row-major: row j holds the weights of global id v_offset + j.
 *    d must be a multiple of 8; H and W must be 16-byte aligned.
 *  - Logit l[b, j] = sum_k H[b, k] W[j, k], accumulated in FP32 (bf16 MFMA
 *    products, FP32 sums; never rounded to bf16).
 *  - Temperature: temp[b] > 0 gives x = l / temp[b].  temp[b] <= 0 or NaN
 *    makes row b greedy (no noise, x = l).  temp == NULL means 1 for every
 *    row.  The FS_NO_NOISE flag makes every row greedy.
 *  - Mask: id i is masked (x = -inf) when i >= n_valid, or when allow is not
 *    NULL and bit (j & 31) of allow[b * ceil(V/32) + (j >> 5)] is 0 (j = i -
 *    v_offset).  A NaN logit counts as masked.
 *  - Noise: r = word (i & 3) of Philox-4x32-10 with key (seed low 32 bits,
 *    seed high 32 bits) and counter (i >> 2, b, step, 0), i the global id
 *    (Salmon et al., SC'11, section 3).  v = (r + 1/2) 2^-32, u = 1 - v,
 *    g = -log(-log u) in FP32.  s = x + g.  Greedy rows: g = 0.
 *  - Ties: lowest global id (and lowest tile) wins.  A row with no valid id
 *    returns index -1.
 *
 * Conventions
 *  - Ownership: the caller allocates every device buffer, including the
 *    workspace sized by fs_workspace_bytes.  The library allocates no device
 *    memory and keeps no state besides a per-device property cache.  A
 *    workspace needs no initialisation.  A flat workspace (FS_VARIANT_FLAT)
 *    carries a small work-scheduling block from one fs_sample /
 *    fs_sample_stage1 call to the next (its last 256 bytes): any content
 *    there, a fresh buffer's included, gives correct results (an
 *    unrecognised block makes that call schedule its work statically and
 *    fs_sample then sets it up), but code other than these calls should not
 *    write into a flat workspace between them, unless it zeroes it whole.
 *  - Asynchrony: every call enqueues work on `stream` (a hipStream_t; NULL is
 *    the default stream) and returns; outputs are valid once the stream has
 *    executed the work.  The host never reads device memory.
 *  - Errors: arguments are validated on the host before anything is
 *    enqueued; a failing call enqueues nothing.  FS_ERR_HIP reports a launch
 *    error from the HIP runtime.  Data conditions (all ids masked, NaN
 *    logits, non-positive temperatures) are results, not errors.
 *  - Reentrancy: calls on different streams with separate workspaces may run
 *    concurrently; two calls sharing one workspace must be ordered.
 */
#ifndef FS_H_
#define FS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FS_OK = 0,
    FS_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad k, ...          */
    FS_ERR_UNSUPPORTED = 2,  /* valid request this build cannot serve (alignment,
                                tile size, d % 8, k range, no gfx950 device,
                                launch grids beyond HIP's limits)                */
    FS_ERR_WORKSPACE = 3,    /* workspace pointer null or smaller than required */
    FS_ERR_HIP = 4           /* the HIP runtime reported an error               */
} fs_status;

/* flag bits of fs_params.flags */
enum { FS_NO_NOISE = 1u << 0 };  /* seed-less: every row greedy (argmax x) */

/* workspace variants for fs_workspace_bytes */
enum {
    FS_VARIANT_FLAT = 0,
    FS_VARIANT_GROUPED = 1,
    FS_VARIANT_TOPK = 2,
    FS_VARIANT_MULTINOMIAL = 3,
    FS_VARIANT_LOGITS = 4
};

typedef struct {
    int32_t B;        /* rows of H (decode batch); 0 is a no-op                 */
    int32_t d;        /* hidden size; multiple of 8                             */
    int32_t V;        /* rows of W in this call (vocabulary or its shard)       */
    int32_t n_valid;  /* global ids >= n_valid are masked; >= v_offset+V: none  */
    int32_t v_offset; /* global id of W row 0; multiple of 16                   */
    int32_t tile_v;   /* ids per tile of the grouped records; multiple of 16,
                         0 selects 128                                          */
    uint64_t seed;    /* Philox key                                             */
    uint32_t step;    /* decode step: Philox counter word 2                     */
    uint32_t flags;   /* FS_NO_NOISE                                            */
    /* Calls a HIP graph can replay with fresh noise (graph-friendly decode
     * loops; the cake_sampling page's correctness contract keeps the generator
     * out of a captured region and takes explicit seed and offset instead):
     * seeds: NULL, or device [B] uint64: row b's Philox key is seeds[b]
     *        (per-request seeds), replacing `seed`;
     * step_ptr: NULL, or a device uint32 read when the kernels run, replacing
     *        `step` (the caller advances it on the device between replays).
     * Both are read, never written; they must stay valid until the call's
     * work on the stream completes. */
    const uint64_t* seeds;
    const uint32_t* step_ptr;
} fs_params;

/* Human-readable name of a status code (static storage). */
const char* fs_status_string(fs_status s);

/* Library version string (static storage). */
const char* fs_version(void);

/* Number of record tiles T = ceil(V / tile_v) (tile_v 0 read as 128); -1 on
 * invalid parameters. */
int32_t fs_num_tiles(const fs_params* p);

/* Bytes of device workspace the entry point `variant` needs for `p` on the
 * current device (k: the top-k size for FS_VARIANT_TOPK, ignored otherwise).
 * Returns 0 on invalid parameters.  The size depends on the device's compute
 * unit count, so query it on the device that will run the call. */
size_t fs_workspace_bytes(const fs_params* p, int variant, int32_t k);

/* fs_sample -- flat fused sample (Stage 1 + Stage 2 of the FlashSampling
 * explainer; the Abstract's "one maximiser per row and tile, then a small
 * reduction").  Streams W once; logits stay on chip.
 *   H, W      device, as defined above
 *   temp      device float [B] or NULL
 *   allow     device uint32 [B, ceil(V/32)] or NULL
 *   out_idx   device int32 [B]: argmax_i s (global id), -1 if nothing valid
 *   out_score device float [B] or NULL: the winning s (-inf if nothing valid)
 *   ws        device workspace of fs_workspace_bytes(p, FS_VARIANT_FLAT, 0)
 */
fs_status fs_sample(const fs_params* p, const void* H, const void* W, const float* temp,
                    const uint32_t* allow, int32_t* out_idx, float* out_score,
                    void* ws, size_t ws_bytes, void* stream);

/* fs_sample_noalloc -- fs_sample for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc.  It calls no allocator: its workspace is a scratch
 * array the library holds in device memory for the life of the process, one
 * of FS_NOALLOC_SCRATCH_BYTES per device (reserved when the library is
 * loaded), so the caller passes only inputs and outputs.  Arguments and
 * results are those of fs_sample without the workspace.  A call whose
 * workspace would exceed the array (fs_workspace_bytes(p, FS_VARIANT_FLAT,
 * 0) + 256 > FS_NOALLOC_SCRATCH_BYTES; e.g. B > 32 with a hidden size that
 * only the streaming kernel serves) returns FS_ERR_WORKSPACE and enqueues
 * nothing.  Every call on a device shares that device's array and it keeps
 * the last call's contents (no call needs it cleared): calls that overlap on
 * one device -- on two streams, or from two host threads without ordering
 * -- race and give wrong results; the caller must order them. */
#define FS_NOALLOC_SCRATCH_BYTES (8u << 20)
fs_status fs_sample_noalloc(const fs_params* p, const void* H, const void* W, const float* temp,
                            const uint32_t* allow, int32_t* out_idx, float* out_score,
                            void* stream);

/* fs_sample_stage1 -- the fused Stage-1 kernel of fs_sample alone: streams W,
 * computes the logits on chip and leaves the per-workgroup winners in `ws`
 * (layout internal to the library) without the Stage-2 reduction.  For timing
 * the dominant kernel in isolation; arguments as for fs_sample. */
fs_status fs_sample_stage1(const fs_params* p, const void* H, const void* W, const float* temp,
                           const uint32_t* allow, void* ws, size_t ws_bytes, void* stream);

/* fs_sample_grouped -- per-tile records plus a hierarchical resample
 * (FlashSampling explainer, tensor-parallel and Group-Gumbel-Max paragraphs).
 * Tile t covers W rows [t*tile_v, min((t+1)*tile_v, V)).  Outputs, each
 * device [B, T] row-major (T = fs_num_tiles(p)):
 *   tile_max      m_t = max s over the tile (-inf if all masked)
 *   tile_idx      idx_t = lowest global id attaining m_t (-1 if all masked)
 *   tile_logmass  L_t = log sum exp x over the tile (greedy rows: max x)
 * out_idx (device int32 [B], or NULL to skip): idx_{t*} with
 * t* = argmax_t (L_t + G_t), G_t a standard Gumbel from word (t & 3) of the
 * Philox block (t >> 2, b, step, 1); greedy rows take G = 0.
 * ws: fs_workspace_bytes(p, FS_VARIANT_GROUPED, 0) bytes. */
fs_status fs_sample_grouped(const fs_params* p, const void* H, const void* W,
                            const float* temp, const uint32_t* allow, float* tile_max,
                            int32_t* tile_idx, float* tile_logmass, int32_t* out_idx,
                            void* ws, size_t ws_bytes, void* stream);

/* fs_sample_topk -- top-k restricted sample (FlashSampling explainer,
 * implementation paragraph: the tile scheme extends to top-k).  S_b = the k
 * valid ids with the largest x (lowest id on ties; every valid id when fewer
 * than k); out_idx[b] = argmax over S_b of s.  1 <= k <= 1024 (else
 * FS_ERR_INVALID_ARG below 1, FS_ERR_UNSUPPORTED above).  k > 64 needs the
 * register-resident stage-1 kernel: ceil(d / 32) * 32 one of 512, 1024, 2048,
 * 4096 or 5120; other hidden sizes return FS_ERR_UNSUPPORTED for such k, and
 * fs_workspace_bytes returns 0 for them.
 * ws: fs_workspace_bytes(p, FS_VARIANT_TOPK, k) bytes. */
fs_status fs_sample_topk(const fs_params* p, const void* H, const void* W, const float* temp,
                         const uint32_t* allow, int32_t k, int32_t* out_idx,
                         void* ws, size_t ws_bytes, void* stream);

/* fs_sample_topk_topp -- top-p after top-k (FlashSampling explainer, top-p
 * paragraph: compress the candidates with top-k first, then apply top-p to
 * the few left; the cut follows the rule of the "flashinfer.cake_sampling"
 * page, launch forms).  S_b as for fs_sample_topk, ordered by x descending
 * (ties to the lower id); with q = softmax of x over S_b, element j of that
 * order is kept when the mass of the elements before it is below top_p
 * (computed in float64 from the FP32 x); out_idx[b] = argmax over the kept
 * elements of s.  0 < top_p <= 1 (else FS_ERR_INVALID_ARG); top_p = 1 gives
 * fs_sample_topk's result.  k as for fs_sample_topk.  Same workspace as
 * fs_sample_topk. */
fs_status fs_sample_topk_topp(const fs_params* p, const void* H, const void* W, const float* temp,
                              const uint32_t* allow, int32_t k, float top_p, int32_t* out_idx,
                              void* ws, size_t ws_bytes, void* stream);

/* fs_merge_online -- online binary merge of C group summaries (FlashSampling
 * explainer, Group-Gumbel-Max paragraph).  z and L are device [B, C]
 * row-major (e.g. tile_idx and tile_logmass of fs_sample_grouped with one
 * tile per chunk).  Starting from (z_0, A = L_0), chunk c replaces the sample
 * when u_c < exp(L_c - logaddexp(A, L_c)), u_c = (r + 1/2) 2^-32 with r word
 * (c & 3) of the Philox block (c >> 2, b, step, 2); then A = logaddexp(A, L_c).
 * Greedy rows (temp[b] <= 0, or FS_NO_NOISE in flags) replace when L_c > A
 * and keep A = max.  out_idx device int32 [B]; out_L device float [B] or NULL
 * (the final A). */
fs_status fs_merge_online(int32_t B, int32_t C, const int32_t* z, const float* L,
                          const float* temp, uint64_t seed, uint32_t step, uint32_t flags,
                          int32_t* out_idx, float* out_L, void* stream);

/* fs_merge_online_dev -- fs_merge_online with its noise key and step taken
 * as fs_params takes them for graph replay: seeds NULL (then `seed` for
 * every row) or device [B] uint64 per-row keys; step_ptr NULL (then `step`)
 * or a device uint32 read when the kernel runs. */
fs_status fs_merge_online_dev(int32_t B, int32_t C, const int32_t* z, const float* L,
                              const float* temp, uint64_t seed, const uint64_t* seeds,
                              uint32_t step, const uint32_t* step_ptr, uint32_t flags,
                              int32_t* out_idx, float* out_L, void* stream);

/* fs_logits -- unfused baseline, step 1: writes l[b, j] (FP32, no
 * temperature, no mask) to device logits [B, V] row-major.  This is the
 * tensor the fused path never materialises (FlashSampling explainer,
 * problem statement).  ws: fs_workspace_bytes(p, FS_VARIANT_LOGITS, 0) bytes
 * (partial sums of the vocabulary blocks split between workers). */
fs_status fs_logits(const fs_params* p, const void* H, const void* W, float* logits,
                    void* ws, size_t ws_bytes, void* stream);

/* fs_multinomial -- unfused baseline, step 2: reads device logits [B, V]
 * (row-major FP32, as written by fs_logits), applies temperature and masks as
 * above, and draws by inverse CDF: out_idx[b] = the smallest id whose
 * cumulative softmax probability exceeds u, u = (r + 1/2) 2^-32 with r word 0
 * of the Philox block (0, b, step, 3).  Greedy rows return argmax x.
 * ws: fs_workspace_bytes(p, FS_VARIANT_MULTINOMIAL, 0) bytes. */
fs_status fs_multinomial(const fs_params* p, const float* logits, const float* temp,
                         const uint32_t* allow, int32_t* out_idx, void* ws, size_t ws_bytes,
                         void* stream);

/* fs_debug_noise -- test export: for rows b0..b0+nb-1 and global ids
 * i0..i0+ni-1 writes the raw Philox words (device uint32 [nb, ni], may be
 * NULL) and the FP32 Gumbel values the kernels use (device float [nb, ni],
 * may be NULL) of noise stream `stream_id`.  i0 must be >= 0. */
fs_status fs_debug_noise(uint64_t seed, uint32_t step, uint32_t stream_id, int32_t b0,
                         int32_t nb, int64_t i0, int32_t ni, uint32_t* words, float* gumbel,
                         void* stream);

/* fs_debug_read_probe -- reads `bytes` (a multiple of 16) of device memory at
 * `src` (16-byte aligned) once with 16-byte loads from `grid` workgroups of
 * 256 threads, folding the data into sink (device uint32 [grid * 256]).  The
 * practical HBM read ceiling that stage 1 is compared with. */
fs_status fs_debug_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t grid,
                              void* stream);

/* fs_debug_read_probe_nt -- the same read with nontemporal loads (the
 * streaming cache policy, `nt` on the global loads): each instruction reads
 * whole 128-byte lines, and this variant reaches a higher HBM read rate than
 * the plain one.  Same arguments and errors as fs_debug_read_probe. */
fs_status fs_debug_read_probe_nt(const void* src, size_t bytes, uint32_t* sink, int32_t grid,
                                 void* stream);

/* fs_debug_shared_read_probe -- every one of `grid` workgroups of 256
 * threads reads all `bytes` (a positive multiple of 32768) at `src` (16-byte
 * aligned) `reps` (>= 1) times with 16-byte loads, each workgroup starting at
 * its own offset, folding the data into sink (device uint32 [grid * 256]).
 * With a buffer that fits one XCD's L2 cache this measures the rate at which
 * the compute units take data from L2 (grid * reps * bytes bytes in all): the
 * ceiling of a stage 1 that re-reads its H tiles from L2. */
fs_status fs_debug_shared_read_probe(const void* src, size_t bytes, int32_t reps, uint32_t* sink,
                                     int32_t grid, void* stream);

/* fs_debug_copy -- plain device copy of `bytes` (a multiple of 16; both
 * pointers 16-byte aligned, no overlap) from `grid` workgroups of 256 threads:
 * a kernel of known traffic for calibrating hardware byte counters. */
fs_status fs_debug_copy(void* dst, const void* src, size_t bytes, int32_t grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FS_H_ */

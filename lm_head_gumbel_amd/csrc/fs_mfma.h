// MFMA operand streaming shared by the stage-1 kernels (gfx950,
// v_mfma_f32_16x16x32_bf16): 16-byte global loads of W and H fragments in a
// software-pipelined stage structure, and the MFMA sweep over a stage.
#pragma once

#include "fs_device.h"
#include "fs_internal.h"

namespace fs {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(1))) const u32x4 global_u32x4;

// 16-byte load through a global-address-space pointer, so it is issued as a
// global_load (FLAT loads would also count against the LDS wait counter and
// force full waits).
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *(const global_u32x4*)(p));
}

// The same with the streaming (nontemporal) cache policy: for a stream read
// once in whole 128-byte lines per instruction.
__device__ __forceinline__ bf16x8 load_bf16x8_nt(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const global_u32x4*)(p)));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// One pipeline stage of MFMA operands: KS k-steps for MPI vocab blocks (A)
// and NB batch blocks (B).
template <int NB, int MPI, int KS>
struct Operands {
    bf16x8 w[MPI][KS];
    bf16x8 h[NB][KS];
};

// Group of up to MPI consecutive vocab blocks inside one record segment.
struct Group {
    int g;        // first block
    int nvm;      // blocks in the group
    int seg_end;  // end block of the segment (tile or workgroup range)
    int t;        // tile index of the segment
};

template <int MPI>
__device__ __forceinline__ Group group_at(int g, int mb1, int tile_mb) {
    Group r;
    r.g = g;
    r.t = g / tile_mb;
    const int64_t te = (int64_t)(r.t + 1) * tile_mb;
    r.seg_end = te < mb1 ? (int)te : mb1;
    r.nvm = min(MPI, r.seg_end - g);
    return r;
}

// Sixteen zero bytes: k-steps that must add nothing read their H operand here.
static __device__ const uint32_t g_zero16[4] = {0u, 0u, 0u, 0u};

// Loads stage `it` of a wave's k-range.  Every load is unconditional and in
// bounds: k-steps past the wave's range are clamped to its last k-step and a
// lane's k past d to d - 8, with their H operand read from g_zero16 so they
// add nothing; no instruction touches the loaded registers before the MFMAs,
// so the loads of a stage stay in flight until their data is needed.  Rows
// past V and blocks past the group are clamped by the row pointers; their
// outputs are discarded by the epilogue.
template <int NB, int MPI, int KS>
__device__ __forceinline__ void load_operands(Operands<NB, MPI, KS>& o,
                                              const uint16_t* (&wrow)[MPI],
                                              const uint16_t* (&hrow)[NB], int it, int ks0,
                                              int ks1, int kg, int d) {
    const uint16_t* zero = reinterpret_cast<const uint16_t*>(g_zero16);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        int kstep = ks0 + it * KS + kk;
        const bool kin = kstep < ks1;
        kstep = kin ? kstep : (ks1 > 0 ? ks1 - 1 : 0);
        const int k = kstep * 32 + kg * 8;
        const bool klane = k < d;
        const int kc = klane ? k : d - 8;
#pragma unroll
        for (int j = 0; j < MPI; ++j) o.w[j][kk] = load_bf16x8(wrow[j] + kc);
#pragma unroll
        for (int n = 0; n < NB; ++n)
            o.h[n][kk] = load_bf16x8((kin && klane) ? hrow[n] + kc : zero);
    }
}

template <int NB, int MPI, int KS>
__device__ __forceinline__ void mfma_operands(f32x4 (&acc)[MPI][NB],
                                              const Operands<NB, MPI, KS>& o) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int j = 0; j < MPI; ++j)
#pragma unroll
            for (int n = 0; n < NB; ++n)
                acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.w[j][kk], o.h[n][kk],
                                                                    acc[j][n], 0, 0, 0);
}

// Row pointers of a group: block j past the group reuses block 0's rows and
// rows past V reuse row V - 1 (cache hits; their results are discarded).
template <int MPI>
__device__ __forceinline__ void group_rows(const uint16_t* (&wrow)[MPI], const uint16_t* W,
                                           const Group& gr, int r16, int V, int d) {
#pragma unroll
    for (int j = 0; j < MPI; ++j) {
        int row = ((j < gr.nvm) ? gr.g + j : gr.g) * kMBlock + r16;
        row = row < V ? row : V - 1;
        wrow[j] = W + (size_t)row * d;
    }
}

}  // namespace fs

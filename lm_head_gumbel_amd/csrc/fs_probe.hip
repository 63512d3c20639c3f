// Memory probes: a streaming read (the practical HBM read ceiling that the
// sampler's stage 1 is compared with) and a plain copy (a kernel of known
// traffic, used to calibrate hardware byte counters).
#include "fs_internal.h"

namespace fs {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 global_u32x4;

// Each thread reads `unroll` 16-byte words per trip of a grid-stride loop and
// folds them into one word, written once per thread so nothing is elided.  NT:
// nontemporal loads (the streaming cache policy).
template <bool NT>
__device__ __forceinline__ u32x4 probe_load(const u32x4* p) {
    if constexpr (NT)
        return __builtin_nontemporal_load((const global_u32x4*)p);
    else
        return *(const global_u32x4*)p;
}

template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* src, size_t n16,
                                                         uint32_t* sink) {
    const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    size_t i = tid;
    for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = probe_load<NT>(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = probe_load<NT>(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[tid] = acc;
}

// Every workgroup reads all n16 words `reps` times, each starting at its own
// offset (n16 a multiple of 256 UNROLL): with a buffer that fits one XCD's
// L2 this is the rate at which the compute units take data from L2.
template <int UNROLL>
__global__ __launch_bounds__(256) void shared_read_kernel(const u32x4* src, size_t n16, int reps,
                                                          uint32_t* sink) {
    constexpr size_t kStep = 256 * UNROLL;
    const size_t start = ((size_t)blockIdx.x * kStep) % n16;
    uint32_t acc = 0;
    for (int r = 0; r < reps; ++r) {
        for (size_t i = 0; i < n16; i += kStep) {
            size_t base = i + start;
            base = base >= n16 ? base - n16 : base;
            u32x4 v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                v[u] = *(const global_u32x4*)(src + base + u * 256 + threadIdx.x);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void copy_kernel(u32x4* dst, const u32x4* src, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = *(const global_u32x4*)(src + i);
}

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int grid, bool nt,
                             hipStream_t stream) {
    if (nt)
        hipLaunchKernelGGL((read_probe_kernel<8, true>), dim3(grid), dim3(256), 0, stream,
                           static_cast<const u32x4*>(src), bytes / 16, sink);
    else
        hipLaunchKernelGGL((read_probe_kernel<8, false>), dim3(grid), dim3(256), 0, stream,
                           static_cast<const u32x4*>(src), bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_shared_read_probe(const void* src, size_t bytes, int reps, uint32_t* sink,
                                   int grid, hipStream_t stream) {
    hipLaunchKernelGGL(shared_read_kernel<8>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const u32x4*>(src), bytes / 16, reps, sink);
    return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, stream, static_cast<u32x4*>(dst),
                       static_cast<const u32x4*>(src), bytes / 16);
    return hipGetLastError();
}

}  // namespace fs

// Expert pruning by slicing: dst slab j = src slab keep_idx[j]
// (RAZOR cards: surviving expert weights and router rows are slices of the
// base checkpoint, in the keep-set's order).  A plain gather copy; an id
// outside [0, src_n) is clamped into it, so every read stays inside the
// source bank.
#include "common.h"
#include "kernels.h"

namespace moe {

__device__ __forceinline__ size_t clamp_id(int id, int n) { return (size_t)(id < 0 ? 0 : id >= n ? n - 1 : id); }

__global__ __launch_bounds__(256) void gather_slabs16_kernel(const int32_t* __restrict__ keep, int src_n,
                                                            const uint4* __restrict__ src,
                                                            uint4* __restrict__ dst, size_t nvec) {
    const size_t j = blockIdx.y;
    const uint4* s = src + clamp_id(keep[j], src_n) * nvec;
    uint4* d = dst + j * nvec;
    for (size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec;
         v += (size_t)gridDim.x * blockDim.x)
        d[v] = s[v];
}

__global__ __launch_bounds__(256) void gather_slabs1_kernel(const int32_t* __restrict__ keep, int src_n,
                                                           const uint8_t* __restrict__ src,
                                                           uint8_t* __restrict__ dst, size_t n) {
    const size_t j = blockIdx.y;
    const uint8_t* s = src + clamp_id(keep[j], src_n) * n;
    uint8_t* d = dst + j * n;
    for (size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x; v < n;
         v += (size_t)gridDim.x * blockDim.x)
        d[v] = s[v];
}

hipError_t launch_gather_slabs(const int32_t* keep_idx, int n_keep, int src_n, const void* src, void* dst,
                               size_t slab_bytes, hipStream_t s) {
    if (n_keep == 0 || slab_bytes == 0) return hipSuccess;
    const bool vec = slab_bytes % 16 == 0 && ((uintptr_t)src % 16) == 0 && ((uintptr_t)dst % 16) == 0;
    const size_t units = vec ? slab_bytes / 16 : slab_bytes;
    size_t bx = (units + 255) / 256;
    if (bx > 1024) bx = 1024;
    dim3 grid((unsigned)bx, (unsigned)n_keep);
    if (vec)
        hipLaunchKernelGGL(gather_slabs16_kernel, grid, dim3(256), 0, s, keep_idx, src_n,
                           static_cast<const uint4*>(src), static_cast<uint4*>(dst), units);
    else
        hipLaunchKernelGGL(gather_slabs1_kernel, grid, dim3(256), 0, s, keep_idx, src_n,
                           static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), units);
    return hipGetLastError();
}

}  // namespace moe

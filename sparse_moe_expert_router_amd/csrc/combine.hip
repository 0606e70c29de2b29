// Weighted combine: y[t] = sum_j gate[t][j] * rows[pair_to_row[t*k+j]] + scale_t * shared[t]
// (Qwen3.8-Flash-Next architecture sheet, MoE entries: routed outputs weighted
// by the renormalised gates plus the always-on shared expert).  fp32
// accumulation in slot order, one bf16 rounding.  HBM-bound streaming: each
// thread owns 8 consecutive hidden columns (one 16-byte bf16 vector).
#include "common.h"
#include "kernels.h"

namespace moe {

template <bool kF32Rows>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ rows,
                                                     const int32_t* __restrict__ pair_to_row,
                                                     const float* __restrict__ gate, int T, int k,
                                                     int H, const uint16_t* __restrict__ shared,
                                                     const float* __restrict__ shared_scale,
                                                     uint16_t* __restrict__ y) {
    const int t = blockIdx.x;
    const int nv = H / 8;
    for (int v = threadIdx.x; v < nv; v += blockDim.x) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        for (int j = 0; j < k; ++j) {
            const float g = gate[(size_t)t * k + j];
            const size_t r = (size_t)pair_to_row[(size_t)t * k + j];
            if (kF32Rows) {
                const float4* src = reinterpret_cast<const float4*>(
                    static_cast<const float*>(rows) + r * H + v * 8);
                const float4 a = src[0], b = src[1];
                acc[0] = fmaf(g, a.x, acc[0]); acc[1] = fmaf(g, a.y, acc[1]);
                acc[2] = fmaf(g, a.z, acc[2]); acc[3] = fmaf(g, a.w, acc[3]);
                acc[4] = fmaf(g, b.x, acc[4]); acc[5] = fmaf(g, b.y, acc[5]);
                acc[6] = fmaf(g, b.z, acc[6]); acc[7] = fmaf(g, b.w, acc[7]);
            } else {
                const uint4 w = *reinterpret_cast<const uint4*>(
                    static_cast<const uint16_t*>(rows) + r * H + v * 8);
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = fmaf(g, bf16_to_f32(ww[i] & 0xFFFFu), acc[2 * i]);
                    acc[2 * i + 1] = fmaf(g, bf16_to_f32(ww[i] >> 16), acc[2 * i + 1]);
                }
            }
        }
        if (shared) {
            const float sc = shared_scale ? shared_scale[t] : 1.0f;
            const uint4 w = *reinterpret_cast<const uint4*>(shared + (size_t)t * H + v * 8);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = fmaf(sc, bf16_to_f32(ww[i] & 0xFFFFu), acc[2 * i]);
                acc[2 * i + 1] = fmaf(sc, bf16_to_f32(ww[i] >> 16), acc[2 * i + 1]);
            }
        }
        uint4 out;
        out.x = pack_bf16x2(acc[0], acc[1]);
        out.y = pack_bf16x2(acc[2], acc[3]);
        out.z = pack_bf16x2(acc[4], acc[5]);
        out.w = pack_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<uint4*>(y + (size_t)t * H + v * 8) = out;
    }
}

hipError_t launch_combine(const void* rows, int rows_f32, const int32_t* pair_to_row,
                          const float* gate, int T, int k, int H, const uint16_t* shared,
                          const float* shared_scale, uint16_t* y, hipStream_t s) {
    const int threads = H / 8 >= 256 ? 256 : ((H / 8 + 63) / 64) * 64;
    if (rows_f32)
        hipLaunchKernelGGL(combine_kernel<true>, dim3(T), dim3(threads), 0, s, rows, pair_to_row,
                           gate, T, k, H, shared, shared_scale, y);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3(T), dim3(threads), 0, s, rows, pair_to_row,
                           gate, T, k, H, shared, shared_scale, y);
    return hipGetLastError();
}

}  // namespace moe

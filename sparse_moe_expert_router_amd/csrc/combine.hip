// Weighted combine: y[t] = sum_j gate[t][j] * rows[pair_to_row[t*k+j]] + scale_t * shared[t]
// (Qwen3.8-Flash-Next architecture sheet, MoE entries: routed outputs weighted
// by the renormalised gates plus the always-on shared expert).  fp32
// accumulation in slot order, one bf16 rounding.  HBM-bound streaming: each
// thread owns 8 consecutive hidden columns (one 16-byte bf16 vector).  bf16
// rows are read and y is written with the non-temporal hint (each is touched
// once; 32768-token pruned layer 4.29 -> 4.26 ms a step).
#include "common.h"
#include "kernels.h"

namespace moe {

// Rows of a token are summed in slot order, loaded in batches whose loads all
// go out before any is used (unconditional loads: lanes past the row's end
// read its last vector and discard it): bf16 rows of 9 to 16 slots in one
// batch of exactly that many loads, otherwise batches of 8, 4, 2 and 1 rows.  Each wave
// first reads the token's gates and row indices one per lane and takes them
// as scalars (readlane).  grid = (T, chunks of blockDim 16-byte vectors); a
// wave walks the vectors in steps of the whole grid's width, every lane
// taking part in every step.
// Rows j .. j+N-1 of the current chunk (N a compile-time count): every
// load first, then the weighted sums.
template <int N, bool kF32Rows>
__device__ __forceinline__ void combine_batch(const void* rows, int H, int v, int j, int rl, int gl,
                                              float (&acc)[8]) {
    if constexpr (kF32Rows) {
        float4 a[N], b[N];
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const size_t r = (size_t)__builtin_amdgcn_readlane(rl, j + u);
            const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(rows) + r * H + v * 8);
            a[u] = src[0];
            b[u] = src[1];
        }
        __builtin_amdgcn_sched_barrier(0);  // keeps the scheduler from sinking the loads to their uses
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const float g = __int_as_float(__builtin_amdgcn_readlane(gl, j + u));
            acc[0] = fmaf(g, a[u].x, acc[0]); acc[1] = fmaf(g, a[u].y, acc[1]);
            acc[2] = fmaf(g, a[u].z, acc[2]); acc[3] = fmaf(g, a[u].w, acc[3]);
            acc[4] = fmaf(g, b[u].x, acc[4]); acc[5] = fmaf(g, b[u].y, acc[5]);
            acc[6] = fmaf(g, b[u].z, acc[6]); acc[7] = fmaf(g, b[u].w, acc[7]);
        }
    } else {
        uint4 w[N];
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const size_t r = (size_t)__builtin_amdgcn_readlane(rl, j + u);
            w[u] = ld_stream(reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(rows) + r * H + v * 8));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const float g = __int_as_float(__builtin_amdgcn_readlane(gl, j + u));
            const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = fmaf(g, bf16_to_f32(ww[i] & 0xFFFFu), acc[2 * i]);
                acc[2 * i + 1] = fmaf(g, bf16_to_f32(ww[i] >> 16), acc[2 * i + 1]);
            }
        }
    }
}

template <bool kF32Rows>
__global__ __launch_bounds__(512) void combine_kernel(const void* __restrict__ rows,
                                                     const int32_t* __restrict__ pair_to_row,
                                                     const float* __restrict__ gate, int T, int k,
                                                     int H, const uint16_t* __restrict__ shared,
                                                     const float* __restrict__ shared_scale,
                                                     uint16_t* __restrict__ y) {
    const int t = blockIdx.x;
    const int nv = H / 8;
    const int lane = threadIdx.x % kWave;
    const int stride = gridDim.y * blockDim.x;
    const size_t pbase = (size_t)t * k;
    int gl = 0, rl = 0;  // gate bits and row index of slot j0 + lane
    if (k <= kWave) {
        const int j = min(lane, k - 1);
        gl = __float_as_int(gate[pbase + j]);
        rl = pair_to_row ? pair_to_row[pbase + j] : (int)(pbase + j);
    }
    for (int v0 = blockIdx.y * blockDim.x + (threadIdx.x - lane); v0 < nv; v0 += stride) {
        const bool act = v0 + lane < nv;
        const int v = act ? v0 + lane : nv - 1;
        uint4 sh = make_uint4(0, 0, 0, 0);
        if (shared) sh = *reinterpret_cast<const uint4*>(shared + (size_t)t * H + v * 8);
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += kWave) {
            const int nj = min(kWave, k - j0);
            if (k > kWave) {
                const int j = j0 + min(lane, nj - 1);
                gl = __float_as_int(gate[pbase + j]);
                rl = pair_to_row ? pair_to_row[pbase + j] : (int)(pbase + j);
            }
            int j = 0;
            if constexpr (!kF32Rows) {
                // 9 to 16 bf16 rows in one batch of exactly that many loads
                switch (nj) {
                    case 9: combine_batch<9, false>(rows, H, v, 0, rl, gl, acc); j = nj; break;
                    case 10: combine_batch<10, false>(rows, H, v, 0, rl, gl, acc); j = nj; break;
                    case 11: combine_batch<11, false>(rows, H, v, 0, rl, gl, acc); j = nj; break;
                    case 12: combine_batch<12, false>(rows, H, v, 0, rl, gl, acc); j = nj; break;
                    case 13: combine_batch<13, false>(rows, H, v, 0, rl, gl, acc); j = nj; break;
                    case 14: combine_batch<14, false>(rows, H, v, 0, rl, gl, acc); j = nj; break;
                    case 15: combine_batch<15, false>(rows, H, v, 0, rl, gl, acc); j = nj; break;
                    case 16: combine_batch<16, false>(rows, H, v, 0, rl, gl, acc); j = nj; break;
                    default: break;
                }
            }
            for (; j + 8 <= nj; j += 8) combine_batch<8, kF32Rows>(rows, H, v, j, rl, gl, acc);
            if (j + 4 <= nj) { combine_batch<4, kF32Rows>(rows, H, v, j, rl, gl, acc); j += 4; }
            if (j + 2 <= nj) { combine_batch<2, kF32Rows>(rows, H, v, j, rl, gl, acc); j += 2; }
            if (j < nj) combine_batch<1, kF32Rows>(rows, H, v, j, rl, gl, acc);
        }
        if (shared) {
            const float sc = shared_scale ? shared_scale[t] : 1.0f;
            const uint32_t ww[4] = {sh.x, sh.y, sh.z, sh.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = fmaf(sc, bf16_to_f32(ww[i] & 0xFFFFu), acc[2 * i]);
                acc[2 * i + 1] = fmaf(sc, bf16_to_f32(ww[i] >> 16), acc[2 * i + 1]);
            }
        }
        if (act) {
            uint4 out;
            out.x = pack_bf16x2(acc[0], acc[1]);
            out.y = pack_bf16x2(acc[2], acc[3]);
            out.z = pack_bf16x2(acc[4], acc[5]);
            out.w = pack_bf16x2(acc[6], acc[7]);
            st_stream(y + (size_t)t * H + v * 8, u32x4_t{out.x, out.y, out.z, out.w});
        }
    }
}

hipError_t launch_combine(const void* rows, int rows_f32, const int32_t* pair_to_row,
                          const float* gate, int T, int k, int H, const uint16_t* shared,
                          const float* shared_scale, uint16_t* y, hipStream_t s) {
    const int nv = H / 8;
    // one workgroup per token when there are many tokens (a wave per 64
    // vectors, so that every wave makes one pass at H <= 4096); otherwise
    // one wave per 64 vectors of a token
    int threads = 64, chunks = (nv + 63) / 64;
    if ((long)T * chunks >= 4096) {
        threads = min(((nv + 63) / 64) * 64, 512);
        chunks = 1;
    }
    const dim3 grid(T, chunks);
    if (rows_f32)
        hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(threads), 0, s, rows, pair_to_row, gate, T, k, H,
                           shared, shared_scale, y);
    else
        hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(threads), 0, s, rows, pair_to_row, gate, T, k, H,
                           shared, shared_scale, y);
    return hipGetLastError();
}

}  // namespace moe

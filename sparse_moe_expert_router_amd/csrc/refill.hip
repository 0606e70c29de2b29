// Refill-RMS expert saliency, keep-set selection and the router-norm policy.
//
// RAZOR E256of512 card, "Selection and calibration": for each selected expert
// j of a token, remove j and promote the highest-ranked unselected expert r;
// the saliency of j is the RMS of the resulting change of the layer output,
// conditional on the tokens routed to j; statistics are additive; the
// highest-scoring experts are kept.  The layer for which calibration text is
// never executed is kept by the L2 norm of its router rows instead.
//
// With p_i = exp(l_i - l_0) over the listed experts, A = sum_{i<k} p_i o_i,
// Z = sum_{i<k} p_i and Z' = Z - p_j + p_r, the change of the routed output is
//   delta_j = (A - p_j o_j + p_r o_r) / Z' - A / Z
//           = A (p_j - p_r) / (Z Z') + (p_r o_r - p_j o_j) / Z'
// (the second form avoids subtracting two nearly equal vectors).  The shared
// expert is the same in both outputs and cancels.
#include "common.h"
#include "kernels.h"

namespace moe {

// One workgroup per token: dsq[t][j] = ||delta_j||^2.  KMAX >= k + 1 bounds the
// fully unrolled per-slot arrays so that they stay in registers.
template <int KMAX>
__global__ __launch_bounds__(256) void refill_delta_kernel(const float* __restrict__ rows,
                                                          const int32_t* __restrict__ pair_to_row,
                                                          const float* __restrict__ tl, int k,
                                                          int H, float* __restrict__ dsq) {
    __shared__ float red[4][KMAX];
    const int t = blockIdx.x;
    const int K1 = k + 1;
    float p[KMAX];
    int row[KMAX];
    const float l0 = tl[(size_t)t * K1];
    float Z = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        p[j] = 0.0f;
        row[j] = 0;
        if (j < K1) {
            p[j] = expf(tl[(size_t)t * K1 + j] - l0);
            row[j] = pair_to_row[(size_t)t * K1 + j];
        }
        if (j < k) Z += p[j];
    }
    float pr = 0.0f;
    int rr = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        if (j == k) { pr = p[j]; rr = row[j]; }
    float ca[KMAX], co[KMAX], acc[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const float Zp = Z - p[j] + pr;
        ca[j] = j < k ? (p[j] - pr) / (Z * Zp) : 0.0f;
        co[j] = j < k ? 1.0f / Zp : 0.0f;
        acc[j] = 0.0f;
    }
    const float* orr = rows + (size_t)rr * H;
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
        float o[KMAX];
        float A = 0.0f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            o[j] = j < k ? rows[(size_t)row[j] * H + h] : 0.0f;
            A = fmaf(p[j] * (j < k ? 1.0f : 0.0f), o[j], A);
        }
        const float prk = pr * orr[h];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const float d = fmaf(A, ca[j], (prk - p[j] * o[j]) * co[j]);
            acc[j] = fmaf(d, d, acc[j]);
        }
    }
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        float v = acc[j];
#pragma unroll
        for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
        if (lane == 0) red[wave][j] = v;
    }
    __syncthreads();
    if (threadIdx.x < k) {
        const int j = threadIdx.x;
        dsq[(size_t)t * k + j] = ((red[0][j] + red[1][j]) + red[2][j]) + red[3][j];
    }
}

// One wave per expert: add the expert's selected-slot deltas (fixed order).
__global__ __launch_bounds__(64) void refill_reduce_kernel(const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ sorted_pair,
                                                          const float* __restrict__ dsq,
                                                          const uint8_t* __restrict__ valid, int k,
                                                          float* __restrict__ stat_sum,
                                                          uint32_t* __restrict__ stat_count) {
    const int e = blockIdx.x, lane = threadIdx.x;
    const int K1 = k + 1;
    float s = 0.0f;
    uint32_t c = 0;
    for (int r = offsets[e] + lane; r < offsets[e + 1]; r += kWave) {
        const int pid = sorted_pair[r];
        const int t = pid / K1, slot = pid % K1;
        if (slot < k && (!valid || valid[t])) {
            s += dsq[(size_t)t * k + slot];
            c += 1;
        }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        s += __shfl_xor(s, m, kWave);
        c += __shfl_xor(c, m, kWave);
    }
    if (lane == 0) {
        stat_sum[e] += s;
        stat_count[e] += c;
    }
}

size_t refill_ws_bytes(int T, int k) { return (size_t)T * k * sizeof(float); }

hipError_t launch_refill_score(const float* rows, const int32_t* offsets, const int32_t* sorted_pair,
                               const int32_t* pair_to_row, const float* tl,
                               const uint8_t* valid, int T, int k, int H, int E, float* stat_sum,
                               uint32_t* stat_count, void* ws, hipStream_t s) {
    float* dsq = static_cast<float*>(ws);
    const int K1 = k + 1;
    if (K1 <= 4)
        hipLaunchKernelGGL(refill_delta_kernel<4>, dim3(T), dim3(256), 0, s, rows, pair_to_row, tl, k, H, dsq);
    else if (K1 <= 8)
        hipLaunchKernelGGL(refill_delta_kernel<8>, dim3(T), dim3(256), 0, s, rows, pair_to_row, tl, k, H, dsq);
    else if (K1 <= 12)
        hipLaunchKernelGGL(refill_delta_kernel<12>, dim3(T), dim3(256), 0, s, rows, pair_to_row, tl, k, H, dsq);
    else if (K1 <= 16)
        hipLaunchKernelGGL(refill_delta_kernel<16>, dim3(T), dim3(256), 0, s, rows, pair_to_row, tl, k, H, dsq);
    else
        hipLaunchKernelGGL(refill_delta_kernel<32>, dim3(T), dim3(256), 0, s, rows, pair_to_row, tl, k, H, dsq);
    hipLaunchKernelGGL(refill_reduce_kernel, dim3(E), dim3(64), 0, s, offsets, sorted_pair, dsq,
                       valid, k, stat_sum, stat_count);
    return hipGetLastError();
}

// Rank values (descending, ties to the lower index) and emit the first `keep`
// as a mask and an ascending index list.  block = 1024, E <= 1024.
__device__ void rank_and_keep(const double* val, int E, int keep, uint8_t* mask, int32_t* keep_idx,
                              int* scan) {
    const int e = threadIdx.x;
    int kept = 0;
    if (e < E) {
        const double v = val[e];
        int rank = 0;
        for (int o = 0; o < E; ++o) {
            const double w = val[o];
            rank += (w > v) || (w == v && o < e);
        }
        kept = rank < keep;
        if (mask) mask[e] = (uint8_t)kept;
    }
    scan[e] = kept;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int add = e >= off ? scan[e - off] : 0;
        __syncthreads();
        scan[e] += add;
        __syncthreads();
    }
    if (kept) keep_idx[scan[e] - 1] = e;
}

__global__ __launch_bounds__(1024) void refill_finalize_kernel(const float* __restrict__ stat_sum,
                                                              const uint32_t* __restrict__ stat_count,
                                                              int E, int H, int keep,
                                                              float* __restrict__ score,
                                                              uint8_t* __restrict__ mask,
                                                              int32_t* __restrict__ keep_idx) {
    __shared__ double val[1024];
    __shared__ int scan[1024];
    const int e = threadIdx.x;
    if (e < E) {
        const uint32_t c = stat_count[e];
        const float sc = c ? (float)sqrt((double)stat_sum[e] / ((double)c * (double)H)) : 0.0f;
        score[e] = sc;
        val[e] = (double)sc;  // rank the scores as emitted
    }
    __syncthreads();
    rank_and_keep(val, E, keep, mask, keep_idx, scan);
}

__global__ __launch_bounds__(1024) void router_norm_keep_kernel(const uint16_t* __restrict__ wr, int E,
                                                               int H, int keep,
                                                               float* __restrict__ norm,
                                                               int32_t* __restrict__ keep_idx) {
    __shared__ double val[1024];
    __shared__ int scan[1024];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    for (int e = wave; e < E; e += 1024 / kWave) {
        double s = 0.0;
        for (int h = lane; h < H; h += kWave) {
            const double w = (double)bf16_to_f32(wr[(size_t)e * H + h]);
            s = fma(w, w, s);
        }
#pragma unroll
        for (int m = 1; m < kWave; m <<= 1) s += shfl_xor_f64(s, m);
        if (lane == 0) {
            val[e] = sqrt(s);
            norm[e] = (float)val[e];
        }
    }
    __syncthreads();
    rank_and_keep(val, E, keep, nullptr, keep_idx, scan);
}

hipError_t launch_refill_finalize(const float* stat_sum, const uint32_t* stat_count, int E, int H,
                                  int keep, float* score, uint8_t* mask, int32_t* keep_idx,
                                  hipStream_t s) {
    hipLaunchKernelGGL(refill_finalize_kernel, dim3(1), dim3(1024), 0, s, stat_sum, stat_count, E,
                       H, keep, score, mask, keep_idx);
    return hipGetLastError();
}

hipError_t launch_router_norm_keep(const uint16_t* wr, int E, int H, int keep, float* norm,
                                   int32_t* keep_idx, hipStream_t s) {
    hipLaunchKernelGGL(router_norm_keep_kernel, dim3(1), dim3(1024), 0, s, wr, E, H, keep, norm,
                       keep_idx);
    return hipGetLastError();
}

}  // namespace moe

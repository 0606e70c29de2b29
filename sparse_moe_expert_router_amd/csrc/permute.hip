// Permutation of (token, slot) pairs by expert: a stable counting sort.
//
// The pages route each token to its top-k experts (Qwen3.8-Flash-Next
// architecture sheet, MoE entries) without spelling out how the pairs are
// grouped; this is the plain grouping: rows of expert e are
// [offsets[e], offsets[e+1]), holding its pair ids in ascending order.
//
// Stability inside a chunk of 64 pairs comes from a wave-wide "match":
// ballots over the bits of the expert id give each lane the mask of lanes
// with the same expert; a lane's rank is the count of such lanes below it.
// Chunks are processed in order by one wave, so the order is deterministic.
#include "common.h"
#include "kernels.h"
#include "select.h"

namespace moe {

constexpr int kPermChunk = 512;      // pairs per block in the multi-block path
// Single workgroup: histogram (the clamped expert ids stay in LDS for the
// scatter), exclusive scan (a wave scan per 64 threads, then the waves'
// totals), scatter by wave 0.  block = 256, P <= kSmallPairs.
__global__ __launch_bounds__(256) void permute_small_kernel(const int32_t* __restrict__ idx, int P,
                                                            int E, int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_pair,
                                                            int32_t* __restrict__ pair_to_row) {
    constexpr int kBatch = 4;  // id loads in flight per thread
    __shared__ int cnt[1024];
    __shared__ int ids[kSmallPairs];
    __shared__ int wtot[4];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    for (int p0 = 0; p0 < P; p0 += kBatch * 256) {
        int ev[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) ev[u] = idx[min(p0 + u * 256 + tid, P - 1)];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int p = p0 + u * 256 + tid;
            if (p < P) {
                const int e = clamp_expert(ev[u], E);
                ids[p] = e;
                atomicAdd(&cnt[e], 1);
            }
        }
    }
    __syncthreads();
    // each thread owns experts 4 tid .. 4 tid + 3 (E <= 1024)
    int local[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid * 4 + j;
        local[j] = e < E ? cnt[e] : 0;
        sum += local[j];
    }
    int inc = sum;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        const int o = __shfl_up(inc, m, kWave);
        if (lane >= m) inc += o;
    }
    if (lane == kWave - 1) wtot[wave] = inc;
    __syncthreads();
    int run = inc - sum;
    for (int w = 0; w < wave; ++w) run += wtot[w];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid * 4 + j;
        if (e < E) {
            cnt[e] = run;  // becomes the cursor
            offsets[e] = run;
        }
        run += local[j];
    }
    if (tid == 0) offsets[E] = P;
    __syncthreads();
    if (wave == 0) wave_scatter<true>(ids, 0, P, E, bits_for(E), cnt, sorted_pair, pair_to_row);
}

// Multi-block path, pass 1: per-block histograms counts[b][e].
__global__ __launch_bounds__(256) void permute_hist_kernel(const int32_t* __restrict__ idx, int P,
                                                           int E, int32_t* __restrict__ counts) {
    __shared__ int cnt[1024];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int p0 = blockIdx.x * kPermChunk, p1 = min(P, p0 + kPermChunk);
    for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) atomicAdd(&cnt[clamp_expert(idx[p], E)], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) counts[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Pass 2 (one block of 1024): counts[b][e] becomes the first row of block b's
// pairs of expert e; offsets[] gets the expert boundaries.  Thread (s, e)
// covers a contiguous segment s of the blocks for expert e (S = 1024 / E
// segments), reading eight counts at a time so that their loads overlap.
constexpr int kScanUnroll = 8;

__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t* __restrict__ counts, int nb,
                                                            int E, int P,
                                                            int32_t* __restrict__ offsets) {
    __shared__ int seg_tot[1024];  // [s][e]
    __shared__ int tot[1024];      // expert totals, then their exclusive scan
    const int S = 1024 / E;        // E <= 1024
    const int s = threadIdx.x / E, e = threadIdx.x % E;
    const bool on = s < S;
    const int b0 = on ? (int)((long)nb * s / S) : 0, b1 = on ? (int)((long)nb * (s + 1) / S) : 0;
    // 1. this segment's total
    int sum = 0;
    for (int b = b0; b < b1; b += kScanUnroll) {
        int c[kScanUnroll];
#pragma unroll
        for (int u = 0; u < kScanUnroll; ++u) c[u] = b + u < b1 ? counts[(size_t)(b + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < kScanUnroll; ++u) sum += c[u];
    }
    seg_tot[threadIdx.x] = on ? sum : 0;
    __syncthreads();
    // 2. expert totals and their exclusive scan (ascending expert)
    const int t = threadIdx.x;
    int run = 0;
    if (t < E)
        for (int q = 0; q < S; ++q) run += seg_tot[q * E + t];
    tot[t] = t < E ? run : 0;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int v = t >= off ? tot[t - off] : 0;
        __syncthreads();
        tot[t] += v;
        __syncthreads();
    }
    if (t < E) offsets[t] = tot[t] - run;
    if (t == 0) offsets[E] = P;
    // 3. first row of each block's pairs: expert base + earlier segments + earlier blocks
    if (on) {
        int r = tot[e];  // inclusive: minus expert e's own total gives its base
        for (int q = 0; q < S; ++q) r -= seg_tot[q * E + e] * (q >= s);
        for (int b = b0; b < b1; b += kScanUnroll) {
            int c[kScanUnroll];
#pragma unroll
            for (int u = 0; u < kScanUnroll; ++u) c[u] = b + u < b1 ? counts[(size_t)(b + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < kScanUnroll; ++u) {
                if (b + u < b1) counts[(size_t)(b + u) * E + e] = r;
                r += c[u];
            }
        }
    }
}

// Pass 3: one wave per block scatters its chunk in order.
__global__ __launch_bounds__(64) void permute_scatter_kernel(const int32_t* __restrict__ idx, int P,
                                                             int E,
                                                             const int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ sorted_pair,
                                                             int32_t* __restrict__ pair_to_row) {
    __shared__ int cursor[1024];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cursor[e] = counts[(size_t)blockIdx.x * E + e];
    __syncthreads();
    const int p0 = blockIdx.x * kPermChunk, p1 = min(P, p0 + kPermChunk);
    wave_scatter<false>(idx, p0, p1, E, bits_for(E), cursor, sorted_pair, pair_to_row);
}

size_t permute_ws_bytes(int T, int k, int E) {
    const long P = (long)T * k;
    if (P <= kSmallPairs) return 0;
    const long nb = (P + kPermChunk - 1) / kPermChunk;
    return (size_t)nb * E * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_to_row, void* ws, hipStream_t s) {
    const int P = T * k;
    if (P <= kSmallPairs) {
        hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(256), 0, s, idx, P, E, offsets,
                           sorted_pair, pair_to_row);
        return hipGetLastError();
    }
    const int nb = (P + kPermChunk - 1) / kPermChunk;
    int32_t* counts = static_cast<int32_t*>(ws);
    hipLaunchKernelGGL(permute_hist_kernel, dim3(nb), dim3(256), 0, s, idx, P, E, counts);
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, counts, nb, E, P, offsets);
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(nb), dim3(64), 0, s, idx, P, E, counts,
                       sorted_pair, pair_to_row);
    return hipGetLastError();
}

}  // namespace moe

// Router: exact fp32 logits, wave-level top-k and renormalised gates.
//
// Qwen3.8-Flash-Next architecture sheet, FFN / MoE entries: softmax gating
// over the expert logits, top-k routed experts per token, selected weights
// renormalised to sum to 1.  The logits are defined as the correctly rounded
// fp32 value of the exact dot product x . w_router[e]; here every bf16 x bf16
// product is exact in fp64 and the sum is accumulated with fp64 FMAs, so the
// final fp64 -> fp32 rounding reproduces that value unless an fp64 addition
// rounded AND the sum lies within an fp64 rounding error of an fp32 tie point.
#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Exact logits.  One wave per expert row; lanes split the hidden dimension;
// a tile of up to 16 tokens is staged in LDS in chunks of kChunk columns.
// grid = (ceil(E / kWavesPerWg), ceil(T / 16)), block = 64 * kWavesPerWg.
// ---------------------------------------------------------------------------
constexpr int kLogitTok = 16;
constexpr int kLogitChunk = 1024;
constexpr int kLogitWaves = 8;

__global__ __launch_bounds__(kLogitWaves * kWave) void exact_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int H, int E,
    float* __restrict__ logits) {
    __shared__ uint4 xs[kLogitTok * kLogitChunk / 8];
    const int lane = threadIdx.x % kWave;
    const int e = blockIdx.x * kLogitWaves + threadIdx.x / kWave;
    const int t0 = blockIdx.y * kLogitTok;
    double acc[kLogitTok];
#pragma unroll
    for (int t = 0; t < kLogitTok; ++t) acc[t] = 0.0;

    for (int h0 = 0; h0 < H; h0 += kLogitChunk) {
        const int len = min(kLogitChunk, H - h0);  // multiple of 8
        const int vecs = len / 8;
        __syncthreads();
        for (int v = threadIdx.x; v < kLogitTok * (kLogitChunk / 8); v += blockDim.x) {
            const int t = v / (kLogitChunk / 8), c = v % (kLogitChunk / 8);
            uint4 val = make_uint4(0, 0, 0, 0);
            if (c < vecs && t0 + t < T)
                val = *reinterpret_cast<const uint4*>(x + (size_t)(t0 + t) * H + h0 + c * 8);
            xs[v] = val;
        }
        __syncthreads();
        if (e < E) {
            for (int c = lane; c < vecs; c += kWave) {
                const uint4 w4 = *reinterpret_cast<const uint4*>(wr + (size_t)e * H + h0 + c * 8);
                const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
                double wd[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    wd[2 * i] = (double)bf16_to_f32(ww[i] & 0xFFFFu);
                    wd[2 * i + 1] = (double)bf16_to_f32(ww[i] >> 16);
                }
#pragma unroll
                for (int t = 0; t < kLogitTok; ++t) {
                    const uint4 x4 = xs[t * (kLogitChunk / 8) + c];
                    const uint32_t xx[4] = {x4.x, x4.y, x4.z, x4.w};
                    double a = acc[t];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        a = fma(wd[2 * i], (double)bf16_to_f32(xx[i] & 0xFFFFu), a);
                        a = fma(wd[2 * i + 1], (double)bf16_to_f32(xx[i] >> 16), a);
                    }
                    acc[t] = a;
                }
            }
        }
    }
    if (e >= E) return;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
#pragma unroll
        for (int t = 0; t < kLogitTok; ++t) acc[t] += shfl_xor_f64(acc[t], m);
    }
#pragma unroll
    for (int t = 0; t < kLogitTok; ++t)
        if (lane == t && t0 + t < T) logits[(size_t)(t0 + t) * E + e] = (float)acc[t];
}

hipError_t launch_exact_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E,
                               float* logits, hipStream_t s) {
    dim3 grid((E + kLogitWaves - 1) / kLogitWaves, (T + kLogitTok - 1) / kLogitTok);
    hipLaunchKernelGGL(exact_logits_kernel, grid, dim3(kLogitWaves * kWave), 0, s, x, wr, T, H, E,
                       logits);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k.  One wave per token.  Each expert becomes a 64-bit key whose order
// is (logit descending, index ascending): high word = order-preserving
// encoding of the fp32 logit (-0 canonicalised to +0), low word = ~index.
// k+extra rounds of a wave-wide max pick the winners in rank order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t float_order_key(float l) {
    uint32_t u = __float_as_uint(l + 0.0f);  // -0 + 0 = +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float float_from_order_key(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        uint64_t o = __shfl_xor(v, m, kWave);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                  int K, int k, int32_t* __restrict__ idx,
                                                  float* __restrict__ topk_logit,
                                                  float* __restrict__ gate) {
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;  // whole wave leaves together; no block barrier below
    uint64_t key[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int e = v * kWave + lane;
        key[v] = 0;
        if (e < E)
            key[v] = ((uint64_t)float_order_key(logits[(size_t)t * E + e]) << 32) | (uint32_t)(~e);
    }
    int my_e = 0;
    float my_l = 0.0f;
    for (int r = 0; r < K; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int v = 0; v < VPL; ++v) best = key[v] > best ? key[v] : best;
        best = wave_max_u64(best);
        const int e = (int)(~(uint32_t)best);
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            if (v * kWave + lane == e) key[v] = 0;
        if (lane == r) {
            my_e = e;
            my_l = float_from_order_key((uint32_t)(best >> 32));
        }
    }
    if (lane < K) {
        idx[(size_t)t * K + lane] = my_e;
        if (topk_logit) topk_logit[(size_t)t * K + lane] = my_l;
    }
    if (gate) {
        const float l0 = __shfl(my_l, 0, kWave);
        const float p = lane < k ? expf(my_l - l0) : 0.0f;
        const float z = wave_sum_f32(p);
        if (lane < k) gate[(size_t)t * k + lane] = p / z;
    }
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int extra, int32_t* idx,
                       float* topk_logit, float* gate, hipStream_t s) {
    const int K = k + extra;
    dim3 grid((T + 3) / 4), block(256);
    const int vpl = (E + kWave - 1) / kWave;
    if (vpl <= 1)
        hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, s, logits, T, E, K, k, idx, topk_logit, gate);
    else if (vpl <= 2)
        hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, s, logits, T, E, K, k, idx, topk_logit, gate);
    else if (vpl <= 4)
        hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, logits, T, E, K, k, idx, topk_logit, gate);
    else if (vpl <= 8)
        hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, logits, T, E, K, k, idx, topk_logit, gate);
    else
        hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, logits, T, E, K, k, idx, topk_logit, gate);
    return hipGetLastError();
}

}  // namespace moe

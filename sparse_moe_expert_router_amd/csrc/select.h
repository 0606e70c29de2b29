// Selection helpers shared by the routing and permutation kernels (internal):
// the wave-level top-k over fp32 logits and the stable wave scatter of
// (token, slot) pairs by expert.
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ uint32_t float_order_key(float l) {
    uint32_t u = __float_as_uint(l + 0.0f);  // -0 + 0 = +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float float_from_order_key(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Key of a present expert: never 0 (only a NaN with every bit set encodes to 0).
__device__ __forceinline__ uint32_t expert_key(float l) { return max(float_order_key(l), 1u); }

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// K rounds over key[VPL] (consumed); lane r receives rank r's expert and
// logit.  Every lane of the wave must be active.  Per round: the wave-wide
// maximum key, then the lowest expert holding it: each lane finds its first
// slot v with that key (vector selects); when one lane holds it (the usual
// case) a ballot names the lane, otherwise a wave minimum over the holders'
// expert ids decides.  Scalar work stays small, so that many waves of one
// workgroup do not queue on their compute unit's scalar unit.
template <int VPL>
__device__ __forceinline__ void wave_topk(uint32_t (&key)[VPL], int K, int lane, int& my_e, float& my_l) {
    for (int r = 0; r < K; ++r) {
        uint32_t best = 0;
#pragma unroll
        for (int v = 0; v < VPL; ++v) best = max(best, key[v]);
        best = wave_max_u32(best);
        int vf = VPL;
#pragma unroll
        for (int v = VPL - 1; v >= 0; --v) vf = key[v] == best ? v : vf;
        const uint64_t hit = __ballot(vf < VPL);
        int e;
        if ((hit & (hit - 1)) == 0) {
            const int L = __ffsll((long long)hit) - 1;
            e = __builtin_amdgcn_readlane(vf, L) * kWave + L;
        } else {
            const uint32_t cand = vf < VPL ? (uint32_t)(vf * kWave + lane) : 0xFFFFFFFFu;
            e = (int)~wave_max_u32(~cand);
        }
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            if (v * kWave + lane == e) key[v] = 0;
        if (lane == r) {
            my_e = e;
            my_l = float_from_order_key(best);
        }
    }
}

// Top K of token t's E logits (one wave, every lane active): writes the
// experts and (optionally) the logits of ranks < K and, with gate, the
// renormalised gates of ranks < k.  Returns rank `lane`'s expert in lanes < K.
template <int VPL>
__device__ __forceinline__ int select_token(const float* __restrict__ logits, size_t t, int E, int K, int k,
                                            int lane, int32_t* __restrict__ idx, float* __restrict__ topk_logit,
                                            float* __restrict__ gate) {
    // unconditional loads (clamped index), so that all of them are in flight at once
    float l[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) l[v] = logits[t * E + min(v * kWave + lane, E - 1)];
    uint32_t key[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) key[v] = v * kWave + lane < E ? expert_key(l[v]) : 0u;
    int my_e = 0;
    float my_l = 0.0f;
    wave_topk<VPL>(key, K, lane, my_e, my_l);
    if (lane < K) {
        idx[t * K + lane] = my_e;
        if (topk_logit) topk_logit[t * K + lane] = my_l;
    }
    if (gate) {
        const float l0 = __shfl(my_l, 0, kWave);
        const float p = lane < k ? expf(my_l - l0) : 0.0f;
        const float z = wave_sum_f32(p);
        if (lane < k) gate[t * k + lane] = p / z;
    }
    return my_e;
}

constexpr int kSmallPairs = 4096;    // single-workgroup path up to this many pairs

// Expert ids outside [0, E) are clamped so that every row stays inside the buffers.
__device__ __forceinline__ int clamp_expert(int e, int E) { return min(max(e, 0), E - 1); }

__device__ __forceinline__ int bits_for(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

// One wave scatters pairs [p0, p1) in order; cursor[e] (LDS) is the next row
// of e.  ids: the pairs' expert ids, in global memory (clamped here) or, with
// kClamped, already clamped (the single-workgroup path keeps them in LDS).
template <bool kClamped>
__device__ __forceinline__ void wave_scatter(const int32_t* __restrict__ ids, int p0, int p1, int E, int nbits,
                             int* cursor, int32_t* __restrict__ sorted_pair,
                             int32_t* __restrict__ pair_to_row) {
    const int lane = threadIdx.x % kWave;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    for (int c = p0; c < p1; c += kWave) {
        const int p = c + lane;
        const bool active = p < p1;
        const int e = !active ? 0 : kClamped ? ids[p] : clamp_expert(ids[p], E);
        uint64_t peers = __ballot(active);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t m = __ballot(active && bit);
            peers &= bit ? m : ~m;
        }
        const int rank = __popcll(peers & below);
        const int cnt = __popcll(peers);
        const int base = active ? cursor[e] : 0;
        __builtin_amdgcn_wave_barrier();
        if (active) {
            const int row = base + rank;
            sorted_pair[row] = p;
            pair_to_row[p] = row;
        }
        if (active && rank == 0) cursor[e] = base + cnt;
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace moe

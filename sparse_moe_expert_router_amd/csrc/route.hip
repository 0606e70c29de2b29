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
#include "ffn_internal.h"
#include "kernels.h"
#include "select.h"

namespace moe {

// ---------------------------------------------------------------------------
// Exact logits.  One wave per expert row; lanes split the hidden dimension;
// a tile of TOK tokens (8 or 16) is staged in LDS in chunks of kLogitChunk
// columns (one chunk at H = 2560).  Each thread issues all of its loads for
// a chunk (its share of the router row, then its share of the activation
// tile) before it waits for any, so a chunk costs one memory round trip.
// Small batches take 8-token tiles: twice the workgroups, half the fp64 work
// per wave.
// grid = (ceil(E / kLogitWaves), ceil(T / TOK)), block = 64 * kLogitWaves.
// ---------------------------------------------------------------------------
constexpr int kLogitChunk = 2560;
constexpr int kLogitRowVecs = kLogitChunk / 8;         // 16-byte vectors per token row per chunk
constexpr int kLogitVecs = kLogitRowVecs / kWave;      // 16-byte vectors per lane per chunk
constexpr int kLogitWaves = 4;
constexpr int kLogitThreads = kLogitWaves * kWave;

// One halving step of wave_reduce_tokens: lanes with bit MASK set keep the
// upper half of the N values and receive their partner's upper half.
template <int N, int MASK>
__device__ __forceinline__ void halve_tokens(const double (&a)[N], double (&b)[N / 2], int lane) {
    const bool up = lane & MASK;
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
        const double send = up ? a[j] : a[j + N / 2];
        const double keep = up ? a[j + N / 2] : a[j];
        b[j] = keep + shfl_xor_f64(send, MASK);
    }
}

// Sum a[0..N-1] (N a power of two) over the 64 lanes of a wave: log2(N)
// halving steps with partner masks 32, 16, ..., then single-value steps for
// the remaining masks.  Afterwards lane L holds the total of token
// tok_of_lane<N>(L).
template <int N, int MASK = kWave / 2>
__device__ __forceinline__ double wave_reduce_tokens(const double (&a)[N], int lane) {
    if constexpr (N == 1) {
        double e = a[0];
#pragma unroll
        for (int m = MASK; m >= 1; m >>= 1) e += shfl_xor_f64(e, m);
        return e;
    } else {
        static_assert((N & (N - 1)) == 0 && N <= kWave / 2, "N must be a power of two <= 32");
        double b[N / 2];
        halve_tokens<N, MASK>(a, b, lane);
        return wave_reduce_tokens<N / 2, MASK / 2>(b, lane);
    }
}

// Token held by lane L after wave_reduce_tokens<N>: the halving step with
// mask m sent the upper half of the remaining tokens to lanes with bit m set.
template <int N>
__device__ __forceinline__ int tok_of_lane(int lane) {
    int t = 0;
#pragma unroll
    for (int n = N, m = kWave / 2; n > 1; n >>= 1, m >>= 1) t += (lane & m) ? n / 2 : 0;
    return t;
}

template <int TOK>
__global__ __launch_bounds__(kLogitThreads) void exact_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int H, int E,
    float* __restrict__ logits) {
    constexpr int kStage = TOK * kLogitRowVecs / kLogitThreads;  // tile vectors per thread
    static_assert(TOK * kLogitRowVecs % kLogitThreads == 0, "tile must split evenly");
    __shared__ uint4 xs[TOK * kLogitRowVecs];
    const int lane = threadIdx.x % kWave;
    const int e = blockIdx.x * kLogitWaves + threadIdx.x / kWave;
    const int t0 = blockIdx.y * TOK;
    double acc[TOK];
#pragma unroll
    for (int t = 0; t < TOK; ++t) acc[t] = 0.0;

    for (int h0 = 0; h0 < H; h0 += kLogitChunk) {
        const int len = min(kLogitChunk, H - h0);  // multiple of 8
        const int vecs = len / 8;
        uint4 w4[kLogitVecs];
#pragma unroll
        for (int j = 0; j < kLogitVecs; ++j) {
            const int c = lane + j * kWave;
            w4[j] = (e < E && c < vecs)
                        ? *reinterpret_cast<const uint4*>(wr + (size_t)e * H + h0 + c * 8)
                        : make_uint4(0, 0, 0, 0);
        }
        uint4 st[kStage];
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int v = threadIdx.x + i * kLogitThreads;
            const int t = v / kLogitRowVecs, c = v % kLogitRowVecs;
            st[i] = (c < vecs && t0 + t < T)
                        ? *reinterpret_cast<const uint4*>(x + (size_t)(t0 + t) * H + h0 + c * 8)
                        : make_uint4(0, 0, 0, 0);
        }
        __syncthreads();  // the previous chunk's tile has been read
#pragma unroll
        for (int i = 0; i < kStage; ++i) xs[threadIdx.x + i * kLogitThreads] = st[i];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kLogitVecs; ++j) {
            const int c = lane + j * kWave;
            if (c >= vecs) break;
            const uint32_t ww[4] = {w4[j].x, w4[j].y, w4[j].z, w4[j].w};
            double wd[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wd[2 * i] = (double)bf16_to_f32(ww[i] & 0xFFFFu);
                wd[2 * i + 1] = (double)bf16_to_f32(ww[i] >> 16);
            }
#pragma unroll
            for (int t = 0; t < TOK; ++t) {
                const uint4 x4 = xs[t * kLogitRowVecs + c];
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
    const double tot = wave_reduce_tokens<TOK>(acc, lane);
    const int t = t0 + tok_of_lane<TOK>(lane);
    if (e < E && lane % (kWave / TOK) == 0 && t < T) logits[(size_t)t * E + e] = (float)tot;
}

hipError_t launch_exact_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E,
                               float* logits, hipStream_t s) {
    const unsigned ex = (E + kLogitWaves - 1) / kLogitWaves;
    // 8-token tiles while 16-token tiles would leave the grid under two
    // workgroups per compute unit
    if ((long)ex * ((T + 15) / 16) < 512)
        hipLaunchKernelGGL(exact_logits_kernel<8>, dim3(ex, (T + 7) / 8), dim3(kLogitThreads), 0, s, x, wr,
                           T, H, E, logits);
    else
        hipLaunchKernelGGL(exact_logits_kernel<16>, dim3(ex, (T + 15) / 16), dim3(kLogitThreads), 0, s, x,
                           wr, T, H, E, logits);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k.  One wave per token.  Expert e = v * 64 + lane sits in key[v] of its
// lane as the order-preserving 32-bit encoding of its fp32 logit (-0
// canonicalised to +0; 0 marks "none", real keys are at least 1).  Each of
// the k+extra rounds takes the wave-wide maximum key (DPP inside rows of 16
// lanes, then scalar reads of the four rows); among experts holding that key
// the lowest index wins: ballots in expert order, first hit.  So the ranks
// order (logit descending, index ascending).
// ---------------------------------------------------------------------------
template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                  int K, int k, int32_t* __restrict__ idx,
                                                  float* __restrict__ topk_logit,
                                                  float* __restrict__ gate) {
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;  // whole wave leaves together; no block barrier below
    select_token<VPL>(logits, (size_t)t, E, K, k, lane, idx, topk_logit, gate);
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

// ---------------------------------------------------------------------------
// Top-k and permutation in one workgroup, for decode-sized batches
// (T * k <= kSmallPairs, E <= 1024): 16 waves select the tokens' experts as
// topk_kernel does, keeping the ids in LDS and counting them per expert;
// then an exclusive scan (one expert per thread) gives the offsets, and wave
// 0 scatters the pairs in pair order exactly as the permutation kernels do.
// The results equal those of launch_topk followed by launch_permute.  With
// `slots` it also writes the grouped GEMV's slot table (slot i = the i-th
// non-empty expert in index order with its row range, expert -1 past the
// last), which otherwise takes a launch of its own.
// ---------------------------------------------------------------------------
constexpr int kSelWaves = 16;

template <int VPL>
__global__ __launch_bounds__(kSelWaves * kWave) void topk_permute_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ idx,
    float* __restrict__ topk_logit, float* __restrict__ gate, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_to_row, int4* __restrict__ slots,
    int nslots) {
    __shared__ int cnt[1024];
    __shared__ int ids[kSmallPairs];
    __shared__ int wtot[kSelWaves];
    __shared__ int wne[kSelWaves];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    for (int t = wave; t < T; t += kSelWaves) {
        const int e = select_token<VPL>(logits, (size_t)t, E, k, k, lane, idx, topk_logit, gate);
        if (lane < k) {
            ids[t * k + lane] = e;
            atomicAdd(&cnt[e], 1);
        }
    }
    __syncthreads();
    const int c = tid < E ? cnt[tid] : 0;
    int inc = c;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        const int o = __shfl_up(inc, m, kWave);
        if (lane >= m) inc += o;
    }
    if (lane == kWave - 1) wtot[wave] = inc;
    // non-empty experts of this wave, for the slot table
    const uint64_t ne = __ballot(tid < E && c > 0);
    if (lane == 0) wne[wave] = __popcll(ne);
    __syncthreads();
    int run = inc - c;
    for (int w = 0; w < wave; ++w) run += wtot[w];
    if (tid < E) {
        cnt[tid] = run;  // becomes the cursor
        offsets[tid] = run;
    }
    if (tid == 0) offsets[E] = T * k;
    if (slots) {
        int before = 0, total = 0;
        for (int w = 0; w < kSelWaves; ++w) {
            before += w < wave ? wne[w] : 0;
            total += wne[w];
        }
        const int pos = before + __popcll(ne & ((1ull << lane) - 1ull));
        if (tid < E && c > 0 && pos < nslots) slots[pos] = make_int4(tid, run, run + c, 0);
        if (tid >= total && tid < nslots) slots[tid] = make_int4(-1, 0, 0, 0);
    }
    __syncthreads();
    if (wave == 0) wave_scatter<true>(ids, 0, T * k, E, bits_for(E), cnt, sorted_pair, pair_to_row);
}

bool topk_permute_fits(int T, int k, int E) { return (long)T * k <= kSmallPairs && E <= 1024; }

hipError_t launch_topk_permute(const float* logits, int T, int E, int k, int32_t* idx, float* topk_logit,
                               float* gate, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_to_row,
                               int4* slots, hipStream_t s) {
    const int vpl = (E + kWave - 1) / kWave;
    const int nslots = T * k < E ? T * k : E;
#define MOE_SEL(V)                                                                                        \
    hipLaunchKernelGGL(topk_permute_kernel<V>, dim3(1), dim3(kSelWaves * kWave), 0, s, logits, T, E, k, idx, \
                       topk_logit, gate, offsets, sorted_pair, pair_to_row, slots, nslots)
    if (vpl <= 1) MOE_SEL(1);
    else if (vpl <= 2) MOE_SEL(2);
    else if (vpl <= 4) MOE_SEL(4);
    else if (vpl <= 8) MOE_SEL(8);
    else MOE_SEL(16);
#undef MOE_SEL
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Screened routing for many tokens.
//
// 1. Approximate logits la = x . w (bf16 MFMA, fp32 accumulation) for all
//    (token, expert) pairs.
// 2. A bound on |la - L|, L the exact real logit, that assumes nothing about
//    the order or the number of roundings inside the MFMA:
//    - a product of two bf16 values is exact in fp32 (8-bit significands);
//    - one K-step adds 32 products to the fp32 accumulator P.  However it
//      does so (up to 32 two-operand fp32 additions, each rounded to nearest
//      or toward zero: relative error < 2^-23 each; or all 33 terms aligned
//      to the largest exponent and truncated to 24 bits: < 2^-23 of the
//      largest term each), the step's error is below
//      33 * 2^-23 (|P| + sum_step |p|) < 2^-17 (|P| + sum_step |p|);
//    - with |P| <= sum |p| (1 + O(2^-17 S)) over S = H/32 steps, the total is
//      below 2^-17 (S + 1) sum_h |x_h w_h| (the +1 absorbs the second-order
//      terms);
//    - one more 2^-17 sum |x w| covers the fp32 rounding of L (<= 2^-24 |L|),
//      so an expert whose exact fp32 logit could tie the K-th is a candidate;
//    - sum_h |x_h w_h| <= ||x|| ||w_e|| (Cauchy-Schwarz), norms in fp64;
//    - products or partial sums that fall below the fp32 normal range and
//      are flushed lose < 2^-126 each: H 2^-100 covers them;
//    - a bf16 input that is itself denormal might be flushed by the MFMA,
//      an error the bound does not cover: a router row with a denormal entry
//      gets an infinite bound (always a candidate) and a token with one is
//      recomputed exactly for every expert.
//    So |la - L| <= delta = 2^-17 (S + 2) ||x|| ||w_e|| + H 2^-100.
// 3. Experts whose upper bound la + delta reaches the K-th largest lower
//    bound are the only ones that can be in the exact top K; their logits are
//    recomputed exactly (fp64 FMAs, one fp32 rounding) and ranked exactly.
//    When more than 64 experts qualify (near-degenerate logits) the token is
//    recomputed for all experts.
// ---------------------------------------------------------------------------
// 16-byte loads, kQuadBatch of them in flight per lane
constexpr int kQuadBatch = 5;

__global__ __launch_bounds__(256) void row_norms_kernel(const uint16_t* __restrict__ w, int E, int H,
                                                        double* __restrict__ norm) {
    const int lane = threadIdx.x % kWave;
    const int e = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (e >= E) return;
    const uint4* wv = reinterpret_cast<const uint4*>(w + (size_t)e * H);
    double s = 0.0;
    bool den = false;
    for (int c0 = lane; c0 < H / 8; c0 += kWave * kQuadBatch) {
        uint4 w4[kQuadBatch];
#pragma unroll
        for (int u = 0; u < kQuadBatch; ++u) w4[u] = wv[min(c0 + kWave * u, H / 8 - 1)];
#pragma unroll
        for (int u = 0; u < kQuadBatch; ++u) {
            if (c0 + kWave * u >= H / 8) break;
            const uint32_t ww[4] = {w4[u].x, w4[u].y, w4[u].z, w4[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const double lo = (double)bf16_to_f32(ww[i] & 0xFFFFu), hi = (double)bf16_to_f32(ww[i] >> 16);
                s = fma(lo, lo, s);
                s = fma(hi, hi, s);
                den |= bf16x2_has_denormal(ww[i]);
            }
        }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) s += shfl_xor_f64(s, m);
    const bool any_den = __ballot(den) != 0;
    if (lane == 0) norm[e] = any_den ? INFINITY : sqrt(s) * (1.0 + 1e-12);
}

// Exact fp32 logit of one (token, expert): fp64 FMAs over the wave, one rounding.
__device__ __forceinline__ float wave_exact_logit(const uint16_t* __restrict__ xr,
                                                  const uint16_t* __restrict__ wr, int H) {
    const int lane = threadIdx.x % kWave;
    double acc = 0.0;
    for (int c = lane; c < H / 8; c += kWave) {
        const uint4 x4 = reinterpret_cast<const uint4*>(xr)[c];
        const uint4 w4 = reinterpret_cast<const uint4*>(wr)[c];
        const uint32_t xx[4] = {x4.x, x4.y, x4.z, x4.w};
        const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = fma((double)bf16_to_f32(xx[i] & 0xFFFFu), (double)bf16_to_f32(ww[i] & 0xFFFFu), acc);
            acc = fma((double)bf16_to_f32(xx[i] >> 16), (double)bf16_to_f32(ww[i] >> 16), acc);
        }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) acc += shfl_xor_f64(acc, m);
    return (float)acc;
}

// Exact fp32 logits of four (token, expert) pairs at once: lane group
// g = lane / 16 takes expert e_g (e_g < 0: none) and 16 lanes split the
// hidden dimension; fp64 FMAs, a 16-lane tree, one rounding.  Every lane
// returns its group's logit.  Loads go out kQuadBatch vectors at a time
// before any of them is used.
__device__ __forceinline__ float quad_exact_logit(const uint16_t* __restrict__ xr,
                                                  const uint16_t* __restrict__ wr, int H, int e_g) {
    const int l16 = threadIdx.x % 16;
    double acc = 0.0;
    if (e_g >= 0) {
        const uint4* wv = reinterpret_cast<const uint4*>(wr + (size_t)e_g * H);
        const uint4* xv = reinterpret_cast<const uint4*>(xr);
        const int nvec = H / 8;
        for (int c0 = l16; c0 < nvec; c0 += 16 * kQuadBatch) {
            uint4 x4[kQuadBatch], w4[kQuadBatch];
#pragma unroll
            for (int u = 0; u < kQuadBatch; ++u) {
                const int c = c0 + 16 * u;
                if (c < nvec) {
                    x4[u] = xv[c];
                    w4[u] = wv[c];
                }
            }
#pragma unroll
            for (int u = 0; u < kQuadBatch; ++u) {
                if (c0 + 16 * u >= nvec) break;
                const uint32_t xx[4] = {x4[u].x, x4[u].y, x4[u].z, x4[u].w};
                const uint32_t ww[4] = {w4[u].x, w4[u].y, w4[u].z, w4[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc = fma((double)bf16_to_f32(xx[i] & 0xFFFFu), (double)bf16_to_f32(ww[i] & 0xFFFFu), acc);
                    acc = fma((double)bf16_to_f32(xx[i] >> 16), (double)bf16_to_f32(ww[i] >> 16), acc);
                }
            }
        }
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) acc += shfl_xor_f64(acc, m);
    return (float)acc;
}

// Rank-ordered top K of n <= 64 distinct 64-bit keys held one per lane
// (lanes >= n hold nothing): each lane counts the keys above its own through
// the wave's LDS copy.  Writes the experts and logits of ranks < K and, with
// gate, the renormalised gates of ranks < k.
__device__ __forceinline__ void rank_emit(uint64_t key, int n, uint64_t* kbuf, float* lbuf, int K,
                                          int k, int32_t* idx, float* topk_logit, float* gate,
                                          size_t t) {
    const int lane = threadIdx.x % kWave;
    if (lane < n) kbuf[lane] = key;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int rank = kWave;
    if (lane < n) {
        rank = 0;
        for (int i = 0; i < n; ++i) rank += kbuf[i] > key;
    }
    const int e = (int)(~(uint32_t)key);
    const float l = float_from_order_key((uint32_t)(key >> 32));
    if (rank < K) {
        idx[t * K + rank] = e;
        if (topk_logit) topk_logit[t * K + rank] = l;
    }
    if (gate) {
        // the selected logits move to lane = rank, so that the gates are
        // summed in the same order as the per-token top-k kernel sums them
        if (rank < k) lbuf[rank] = l;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const float my_l = lane < k ? lbuf[lane] : 0.0f;
        const float l0 = lbuf[0];
        const float p = lane < k ? expf(my_l - l0) : 0.0f;
        const float z = wave_sum_f32(p);
        if (lane < k) gate[t * k + lane] = p / z;
    }
}

// XV > 0: H == 512 * XV, and token t's inputs stay in registers as fp64
// (vector c = lane + 64 u of 8 inputs, u < XV) while the candidates' exact
// logits are formed one per wave pass; XV = 0: four candidates at a time with
// 16 lanes each (quad_exact_logit), any H.
template <int VPL, int XV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(XV == 5 && VPL <= 8 ? (VPL == 8 ? 3 : 4) : 1))) void route_refine_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, float* __restrict__ la,
    const double* __restrict__ wnorm, int T, int H, int E, int K, int k, int32_t* __restrict__ idx,
    float* __restrict__ topk_logit, float* __restrict__ gate) {
    __shared__ int cand[4][kWave];
    __shared__ double lmax[4][kWave];
    __shared__ uint64_t kbuf[4][kWave];
    __shared__ float lbuf[4][kWave];
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;  // whole wave; no block barrier below
    const uint16_t* xr = x + (size_t)t * H;
    float* lrow = la + (size_t)t * E;

    // ||x_t|| (fp64) and the bound factor
    double xs = 0.0;
    bool xden = false;
    for (int c0 = lane; c0 < H / 8; c0 += kWave * kQuadBatch) {
        uint4 x4[kQuadBatch];
#pragma unroll
        for (int u = 0; u < kQuadBatch; ++u) x4[u] = reinterpret_cast<const uint4*>(xr)[min(c0 + kWave * u, H / 8 - 1)];
#pragma unroll
        for (int u = 0; u < kQuadBatch; ++u) {
            if (c0 + kWave * u >= H / 8) break;
            const uint32_t xx[4] = {x4[u].x, x4[u].y, x4[u].z, x4[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const double a = (double)bf16_to_f32(xx[i] & 0xFFFFu), b = (double)bf16_to_f32(xx[i] >> 16);
                xs = fma(a, a, xs);
                xs = fma(b, b, xs);
                xden |= bf16x2_has_denormal(xx[i]);
            }
        }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) xs += shfl_xor_f64(xs, m);
    const double S = (double)((H + 31) / 32);
    const double fac = ldexp(S + 2.0, -17) * sqrt(xs) * (1.0 + 1e-12);
    const double dabs = (double)H * ldexp(1.0, -100);
    // a denormal input may have been flushed by the MFMA: no bound holds
    const bool x_denormal = __ballot(xden) != 0;

    double lo[VPL], hi[VPL];
    double mylo = -INFINITY;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int e = v * kWave + lane;
        if (e < E) {
            const double wn = wnorm[e];
            const double d = wn == INFINITY ? INFINITY : fac * wn + dabs;
            const double l = (double)lrow[e];
            lo[v] = l - d;
            hi[v] = l + d;
        } else {
            lo[v] = -INFINITY;
            hi[v] = -INFINITY;
        }
        mylo = fmax(mylo, lo[v]);
    }
    // tau: the K-th largest of the 64 lanes' largest lower bounds.  At least K
    // lower bounds (those K lane maxima) reach it, so it does not exceed the
    // K-th largest lower bound, and every expert that can be in the exact top
    // K has an upper bound >= tau.
    double tau = -INFINITY;
    if (K <= kWave) {
        lmax[wv][lane] = mylo;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        int rank = 0;
        for (int i = 0; i < kWave; ++i) {
            const double o = lmax[wv][i];
            rank += (o > mylo) || (o == mylo && i < lane);
        }
        const uint64_t hit = __ballot(rank == K - 1);
        tau = lmax[wv][__ffsll((long long)hit) - 1];
    }
    // candidates: hi >= tau
    int ncand = 0;
    bool overflow = false;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const bool c = (v * kWave + lane < E) && hi[v] >= tau;
        const uint64_t m = __ballot(c);
        const int n = __popcll(m);
        if (!overflow && ncand + n <= kWave) {
            if (c) cand[wv][ncand + __popcll(m & ((1ull << lane) - 1ull))] = v * kWave + lane;
        } else {
            overflow = true;
        }
        ncand += n;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (ncand > kWave || x_denormal) overflow = true;

    if (!overflow && XV > 0) {
        // exact logits of the candidates, one per pass of the whole wave over
        // the fp64 inputs; candidate j's logit ends in lane j
        const uint4* xv = reinterpret_cast<const uint4*>(xr);
        double xd[XV > 0 ? XV : 1][8];
#pragma unroll
        for (int u = 0; u < XV; ++u) {
            const uint4 x4 = xv[lane + kWave * u];
            const uint32_t xx[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xd[u][2 * i] = (double)bf16_to_f32(xx[i] & 0xFFFFu);
                xd[u][2 * i + 1] = (double)bf16_to_f32(xx[i] >> 16);
            }
        }
        float mine = 0.0f;
        // 512 experts (eight a lane): candidate j + 1's router row loads
        // while candidate j's logit forms, at three waves a SIMD for the
        // second row buffer (4096 tokens: layer 0.842 -> 0.833 ms); with
        // fewer experts the rows load one candidate at a time, at four waves
        // (the prefetch measured slower there)
        uint4 wa[XV > 0 ? XV : 1], wb[XV > 0 ? XV : 1];
        auto load_row = [&](uint4 (&w4)[XV > 0 ? XV : 1], int j) {
            const uint4* wv4 = reinterpret_cast<const uint4*>(wr + (size_t)cand[wv][j] * H);
#pragma unroll
            for (int u = 0; u < XV; ++u) w4[u] = wv4[lane + kWave * u];
        };
        auto logit = [&](const uint4 (&w4)[XV > 0 ? XV : 1], int j) {
            double acc = 0.0;
#pragma unroll
            for (int u = 0; u < XV; ++u) {
                const uint32_t ww[4] = {w4[u].x, w4[u].y, w4[u].z, w4[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc = fma(xd[u][2 * i], (double)bf16_to_f32(ww[i] & 0xFFFFu), acc);
                    acc = fma(xd[u][2 * i + 1], (double)bf16_to_f32(ww[i] >> 16), acc);
                }
            }
            const float lj = (float)wave_sum_f64(acc);  // every lane takes part
            if (lane == j) mine = lj;
        };
        if constexpr (VPL == 8) {
            if (ncand > 0) load_row(wa, 0);
            for (int j = 0; j < ncand; j += 2) {
                if (j + 1 < ncand) load_row(wb, j + 1);
                logit(wa, j);
                if (j + 2 < ncand) load_row(wa, j + 2);
                if (j + 1 < ncand) logit(wb, j + 1);
            }
        } else {
            for (int j = 0; j < ncand; ++j) {
                load_row(wa, j);
                logit(wa, j);
            }
        }
        uint64_t key = 0;
        if (lane < ncand) key = ((uint64_t)float_order_key(mine) << 32) | (uint32_t)(~cand[wv][lane]);
        rank_emit(key, ncand, kbuf[wv], lbuf[wv], K, k, idx, topk_logit, gate, (size_t)t);
        return;
    }
    if (!overflow) {
        // exact logits of the candidates, four at a time; candidate j's logit
        // ends in lane j
        float mine = 0.0f;
        for (int j0 = 0; j0 < ncand; j0 += 4) {
            const int j = j0 + lane / 16;
            const float l = quad_exact_logit(xr, wr, H, j < ncand ? cand[wv][j] : -1);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float lg = __shfl(l, g * 16, kWave);
                if (lane == j0 + g) mine = lg;
            }
        }
        uint64_t key = 0;
        if (lane < ncand) key = ((uint64_t)float_order_key(mine) << 32) | (uint32_t)(~cand[wv][lane]);
        rank_emit(key, ncand, kbuf[wv], lbuf[wv], K, k, idx, topk_logit, gate, (size_t)t);
        return;
    }
    // fallback: every logit of this token exactly (kept in the owning lane's
    // registers), then the plain top-K
    uint32_t keys[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) keys[v] = 0;
    for (int e = 0; e < E; ++e) {
        const uint32_t kk = expert_key(wave_exact_logit(xr, wr + (size_t)e * H, H));
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            if (v * kWave + lane == e) keys[v] = kk;
    }
    int my_e = 0;
    float my_l = 0.0f;
    wave_topk<VPL>(keys, K, lane, my_e, my_l);
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

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t route_filter_ws_bytes(int T, int E, int H) {
    (void)H;
    return align256((size_t)T * E * sizeof(float)) + align256((size_t)E * sizeof(double)) +
           dense_gemm_ws_bytes(T);
}

hipError_t launch_route_filter(const uint16_t* x, const uint16_t* wr, int T, int H, int E, int k,
                               int extra, int32_t* idx, float* topk_logit, float* gate, void* ws,
                               hipStream_t s) {
    char* p = static_cast<char*>(ws);
    float* la = reinterpret_cast<float*>(p);
    p += align256((size_t)T * E * sizeof(float));
    double* wn = reinterpret_cast<double*>(p);
    p += align256((size_t)E * sizeof(double));
    hipLaunchKernelGGL(row_norms_kernel, dim3((E + 3) / 4), dim3(256), 0, s, wr, E, H, wn);
    hipError_t err = launch_dense_gemm_f32(x, T, H, wr, E, la, p, s);
    if (err != hipSuccess) return err;
    const int K = k + extra;
    const int vpl = (E + kWave - 1) / kWave;
    dim3 grid((T + 3) / 4), block(256);
#define MOE_REFINE_XV(V, XV) \
    hipLaunchKernelGGL((route_refine_kernel<V, XV>), grid, block, 0, s, x, wr, la, wn, T, H, E, K, k, idx, \
                       topk_logit, gate)
#define MOE_REFINE(V)                          \
    do {                                       \
        if (H == 2560) MOE_REFINE_XV(V, 5);    \
        else if (H == 512) MOE_REFINE_XV(V, 1); \
        else MOE_REFINE_XV(V, 0);              \
    } while (0)
    if (vpl <= 2) MOE_REFINE(2);
    else if (vpl <= 4) MOE_REFINE(4);
    else if (vpl <= 8) MOE_REFINE(8);
    else MOE_REFINE(16);
#undef MOE_REFINE
#undef MOE_REFINE_XV
    return hipGetLastError();
}

}  // namespace moe

// Grouped SwiGLU experts for few rows per expert (decode): weight streaming.
//
// Qwen3.8-Flash-Next architecture sheet, FFN / MoE entries: SwiGLU experts
// (gate, up, down), no bias, no clamp.  AWQ-g32 card, "Checkpoint":
// asymmetric W4A16, group 32 along the input, integer zeros, fp16 scales,
// GEMM packing.  With a handful of tokens per expert the work is a stream of
// the touched experts' weights from HBM; each weight is read once and used
// for every row of its expert.
//
// AWQ path: a word holds 8 output columns of one input row.  Two words of
// consecutive input rows i, i+1 are merged byte by byte (v_perm) so that each
// 32-bit register holds the codes of one column for rows i and i+1; OR-ing
// the exponent pattern 0x4300 makes each half the bf16 value 128 + q.  One
// v_dot2_f32_bf16 with the activation pair (x_i, x_{i+1}) accumulates
// sum x (128 + q); per group of 32 rows the column result is
//   s * (acc - (128 + z) * sum_group(x)) = s * sum x (q - z).
// Threads own one word column (8 output columns) and whole groups, so the
// zero/scale correction is paid once per group.
#include "ffn_internal.h"
#include "nvfp4.h"

namespace moe {

constexpr int kAwqNib[8] = {0, 2, 4, 6, 1, 3, 5, 7};  // nibble j holds column 8c + kAwqNib[j]
constexpr int kGemvMaxKPairs = 1024;                  // LDS activation pairs per row (2048 inputs)
constexpr int kGemvMaxSplit = 8;  // input splits of the non-AWQ gate/up pass (more measured slower)

__device__ __forceinline__ int row_token(const int32_t* sorted_pair, int k, int r) {
    return sorted_pair ? sorted_pair[r] / k : r;
}

// Registers of one group of one word column: 32 code words (input rows
// 32g..32g+31), the packed zero word and the 8 fp16 scales.
struct AwqGroupRegs {
    uint32_t w[32];
    uint32_t z;
    u32x4_t s;  // a native vector (HIP's uint4 class can keep a copy in scratch)
};

__device__ __forceinline__ void awq_load_group(const int32_t* __restrict__ qw,
                                               const int32_t* __restrict__ qz,
                                               const uint16_t* __restrict__ sc, int O, int OW, int c,
                                               int g, AwqGroupRegs& r) {
    const int32_t* wp = qw + (size_t)g * 32 * OW + c;
#pragma unroll
    for (int q = 0; q < 32; ++q) r.w[q] = (uint32_t)wp[(size_t)q * OW];
    r.z = (uint32_t)qz[(size_t)g * OW + c];
    r.s = *reinterpret_cast<const u32x4_t*>(sc + (size_t)g * O + 8 * c);
}

template <int RCH>
__device__ __forceinline__ void awq_group_dot(const AwqGroupRegs& r, const uint32_t* xs, int npairs,
                                              const float* xsum, int ngroups, int lg,
                                              float (&res)[8][RCH]) {
    float acc[8][RCH];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < RCH; ++i) acc[j][i] = 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const uint32_t w0 = r.w[2 * q], w1 = r.w[2 * q + 1];
        uint32_t v[8];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            // bytes: [w0.b, 0, w1.b, 0]
            const uint32_t t = __builtin_amdgcn_perm(w1, w0, 0x0C000C00u | b | ((4u + b) << 16));
            v[2 * b] = and_or(t, 0x000F000Fu, 0x43004300u);
            v[2 * b + 1] = and_or(t >> 4, 0x000F000Fu, 0x43004300u);
        }
#pragma unroll
        for (int i = 0; i < RCH; ++i) {
            const uint32_t xp = xs[i * npairs + lg * 16 + q];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j][i] = dot2_bf16(v[j], xp, acc[j][i]);
        }
    }
    const uint32_t sw[4] = {r.s[0], r.s[1], r.s[2], r.s[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int col = kAwqNib[j];
        const float s = f16_to_f32((sw[col / 2] >> (16 * (col % 2))) & 0xFFFFu);
        const float zc = 128.0f + (float)((r.z >> (4 * j)) & 15u);
#pragma unroll
        for (int i = 0; i < RCH; ++i)
            res[j][i] = fmaf(s, fmaf(-zc, xsum[i * ngroups + lg], acc[j][i]), res[j][i]);
    }
}

// Accumulate the AWQ GEMV of groups [g_begin, g_end) stepping by g_step for one
// word column c of a projection (I inputs, OW = O/8 words per input row).
// xs: activation pairs [RCH][npairs] (row pairs relative to group g_base),
// xsum: [RCH][ngroups] group sums.  res[j][i]: column 8c + kAwqNib[j], row i.
// One group's 37 loads are in flight at a time per thread; the other waves of
// the compute unit cover the latency (a second register set for the next
// group costs occupancy and measured slower).
template <int RCH>
__device__ __forceinline__ void awq_gemv_groups(const int32_t* __restrict__ qw,
                                                const int32_t* __restrict__ qz,
                                                const uint16_t* __restrict__ sc, int O, int OW,
                                                int c, int g_base, int g_begin, int g_end,
                                                int g_step, const uint32_t* xs, int npairs,
                                                const float* xsum, int ngroups,
                                                float (&res)[8][RCH]) {
    for (int g = g_begin; g < g_end; g += g_step) {
        AwqGroupRegs cur;
        awq_load_group(qw, qz, sc, O, OW, c, g, cur);
        awq_group_dot<RCH>(cur, xs, npairs, xsum, ngroups, g - g_base, res);
    }
}

template <int R>
struct RowsTag {
    static constexpr int value = R;
};

// Calls body(RowsTag<R>) with the smallest R in {1, 2, 4, RCH} that covers nr
// rows, so that experts with one or two rows do not pay for RCH.
template <int RCH, class Body>
__device__ __forceinline__ void dispatch_rows(int nr, Body&& body) {
    if (nr <= 1) body(RowsTag<1>{});
    else if (nr <= 2 || RCH < 4) body(RowsTag<(RCH < 2 ? RCH : 2)>{});
    else if (nr <= 4 || RCH < 8) body(RowsTag<(RCH < 4 ? RCH : 4)>{});
    else body(RowsTag<RCH>{});
}

// Group sums of the staged activation pairs.
template <int RCH>
__device__ __forceinline__ void stage_group_sums(const uint32_t* xs, int npairs, int ngroups,
                                                 float* xsum) {
    for (int it = threadIdx.x; it < RCH * ngroups; it += blockDim.x) {
        const int i = it / ngroups, g = it % ngroups;
        float s = 0.0f;
        for (int q = 0; q < 16; ++q) {
            const uint32_t v = xs[i * npairs + g * 16 + q];
            s += bf16_to_f32(v & 0xFFFFu) + bf16_to_f32(v >> 16);
        }
        xsum[it] = s;
    }
}

// Deterministic reduction of per-row-phase results into red[RCH][8*OWC]:
// phases add in order 0, 1, ..., RP-1.
template <int RCH>
__device__ __forceinline__ void reduce_phases(const float (&res)[8][RCH], int cl, int rp, int RP,
                                              int ncols, float* red) {
    for (int q = 0; q < RP; ++q) {
        if (rp == q) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < RCH; ++i) {
                    float* d = &red[i * ncols + 8 * cl + kAwqNib[j]];
                    *d = q == 0 ? res[j][i] : *d + res[j][i];
                }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// AWQ gate/up: grid (2*KS, expert slot); block = OW * RP threads.
// part[ks][r][mat*F + col] (fp32 partial over the WG's groups).
// ---------------------------------------------------------------------------
template <int RCH>
__global__ __launch_bounds__(512) void awq_gateup_kernel(GroupedArgs a, int KS, float* __restrict__ part) {
    __shared__ uint32_t xs[RCH * kGemvMaxKPairs];
    __shared__ float xsum[RCH * 64];
    extern __shared__ float red[];  // [RCH][F]
    int r0, r1;
    const int e = a.offsets ? slot_expert(a.slots, blockIdx.y, &r0, &r1) : 0;
    if (!a.offsets) { r0 = 0; r1 = a.T; }
    if (e < 0) return;
    const int mat = blockIdx.x / KS, ks = blockIdx.x % KS;
    const int H = a.H, F = a.F, OW = F / 8, G = H / 32;
    const int g0 = ks * G / KS, g1 = (ks + 1) * G / KS, ng = g1 - g0, npairs = ng * 16;
    const int c = threadIdx.x % OW, rp = threadIdx.x / OW, RP = blockDim.x / OW;
    const ProjDev& pj = mat ? a.up : a.gate;
    const int32_t* qw = pj.qweight + (size_t)e * H * OW;
    const int32_t* qz = pj.qzeros + (size_t)e * G * OW;
    const uint16_t* sc = pj.scales + (size_t)e * G * F;
    for (int rc = r0; rc < r1; rc += RCH) {
        const int nr = min(RCH, r1 - rc);
        __syncthreads();
        for (int it = threadIdx.x; it < RCH * npairs; it += blockDim.x) {
            const int i = it / npairs, q = it % npairs;
            uint32_t v = 0;
            if (i < nr) {
                const int t = row_token(a.sorted_pair, a.k, rc + i);
                v = reinterpret_cast<const uint32_t*>(a.x + (size_t)t * H + g0 * 32)[q];
            }
            xs[it] = v;
        }
        __syncthreads();
        stage_group_sums<RCH>(xs, npairs, ng, xsum);
        __syncthreads();
        auto body = [&](auto rtag) {
            constexpr int R = decltype(rtag)::value;
            float res[8][R];
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < R; ++i) res[j][i] = 0.0f;
            awq_gemv_groups<R>(qw, qz, sc, F, OW, c, g0, g0 + rp, g1, RP, xs, npairs, xsum, ng, res);
            reduce_phases<R>(res, c, rp, RP, F, red);
        };
        dispatch_rows<RCH>(nr, body);
        for (int it = threadIdx.x; it < nr * F; it += blockDim.x) {
            const int i = it / F, col = it % F;
            part[((size_t)ks * a.P + rc + i) * (2 * F) + mat * F + col] = red[i * F + col];
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 gate/up: grid (F/32 column chunks, expert slot, KS input splits);
// block 256 (4 waves).  Waves 0,1: gate columns c0..c0+31, waves 2,3: up.
// 16 lanes per weight row.  part[ks][r][mat*F + col].
// ---------------------------------------------------------------------------
constexpr int kBfChunkK = 2048;
// NVFP4 GEMV shape: rows per lane and lanes per row of the down pass, lanes
// per row of the gate/up pass, vectors each lane loads before using them
// (0: the software-pipelined stream)
constexpr int kNvDownRows = 2, kNvDownUnroll = 0, kNvDownLanes = 4, kNvGateLanes = 8, kNvGateUnroll = 2;

// Dot products of NR weight rows (16-byte vectors, 16 lanes per row, vector
// v of a row at rows[n][v]) with R activation rows staged in LDS (xs[i*xstride
// + v]).  U vectors of every row are loaded before any is used, so NR*U loads
// per lane are in flight.
template <int R, int NR, int U, int RA>
__device__ __forceinline__ void bf16_stream_dot(const uint4* const (&rows)[NR], int nv, int l16,
                                                const uint4* xs, int xstride, float (&acc)[4][RA]) {
    int v = l16;
    for (; v + 16 * (U - 1) < nv; v += 16 * U) {
        uint4 w[U][NR];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int n = 0; n < NR; ++n) w[u][n] = ld_stream(&rows[n][v + 16 * u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const uint4 xv = xs[i * xstride + v + 16 * u];
#pragma unroll
                for (int n = 0; n < NR; ++n) {
                    float t = acc[n][i];
                    t = dot2_bf16(w[u][n].x, xv.x, t);
                    t = dot2_bf16(w[u][n].y, xv.y, t);
                    t = dot2_bf16(w[u][n].z, xv.z, t);
                    t = dot2_bf16(w[u][n].w, xv.w, t);
                    acc[n][i] = t;
                }
            }
    }
    for (; v < nv; v += 16) {
        uint4 w[NR];
#pragma unroll
        for (int n = 0; n < NR; ++n) w[n] = ld_stream(&rows[n][v]);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const uint4 xv = xs[i * xstride + v];
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                float t = acc[n][i];
                t = dot2_bf16(w[n].x, xv.x, t);
                t = dot2_bf16(w[n].y, xv.y, t);
                t = dot2_bf16(w[n].z, xv.z, t);
                t = dot2_bf16(w[n].w, xv.w, t);
                acc[n][i] = t;
            }
        }
    }
}

template <int R, int RA>
__device__ __forceinline__ void bf16_rows_dot(const uint16_t* __restrict__ W, int H, int k0, int nv,
                                              int c0, int wave, int sub, int l16, const uint4* xs,
                                              float (&acc)[4][RA]) {
    const uint4* rows[4];
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
        const int col = c0 + (wave % 2) * 16 + ps * 4 + sub;
        rows[ps] = reinterpret_cast<const uint4*>(W + (size_t)col * H + k0);
    }
    bf16_stream_dot<R, 4, 2>(rows, nv, l16, xs, kBfChunkK / 8, acc);
}

template <int RCH>
__global__ __launch_bounds__(256) void bf16_gateup_kernel(GroupedArgs a, int KS, float* __restrict__ part) {
    __shared__ uint4 xs[RCH * kBfChunkK / 8];
    __shared__ float outv[64][RCH];
    int r0, r1;
    const int e = a.offsets ? slot_expert(a.slots, blockIdx.y, &r0, &r1) : 0;
    if (!a.offsets) { r0 = 0; r1 = a.T; }
    if (e < 0) return;
    const int H = a.H, F = a.F;
    const int ks = blockIdx.z;
    const int kb = (int)((long)H / 8 * ks / KS) * 8, ke = (int)((long)H / 8 * (ks + 1) / KS) * 8;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int sub = lane / 16, l16 = lane % 16;  // 4 rows per pass, 16 lanes each
    const int c0 = blockIdx.x * 32;
    const int mat = wave / 2;
    const uint16_t* W = (mat ? a.up.w : a.gate.w) + (size_t)e * F * H;
    for (int rc = r0; rc < r1; rc += RCH) {
        const int nr = min(RCH, r1 - rc);
        float acc[4][RCH];
#pragma unroll
        for (int ps = 0; ps < 4; ++ps)
#pragma unroll
            for (int i = 0; i < RCH; ++i) acc[ps][i] = 0.0f;
        for (int k0 = kb; k0 < ke; k0 += kBfChunkK) {
            const int kl = min(kBfChunkK, ke - k0), nv = kl / 8;
            __syncthreads();
            for (int it = threadIdx.x; it < nr * nv; it += blockDim.x) {
                const int i = it / nv, v = it % nv;
                const int t = row_token(a.sorted_pair, a.k, rc + i);
                xs[i * (kBfChunkK / 8) + v] = reinterpret_cast<const uint4*>(a.x + (size_t)t * H + k0)[v];
            }
            __syncthreads();
            auto body = [&](auto rtag) {
                constexpr int R = decltype(rtag)::value;
                bf16_rows_dot<R, RCH>(W, H, k0, nv, c0, wave, sub, l16, xs, acc);
            };
            dispatch_rows<RCH>(nr, body);
        }
#pragma unroll
        for (int ps = 0; ps < 4; ++ps)
#pragma unroll
            for (int i = 0; i < RCH; ++i) {
                float v = acc[ps][i];
                v += __shfl_xor(v, 1, kWave);
                v += __shfl_xor(v, 2, kWave);
                v += __shfl_xor(v, 4, kWave);
                v += __shfl_xor(v, 8, kWave);
                if (l16 == 0) outv[wave * 16 + ps * 4 + sub][i] = v;
            }
        __syncthreads();
        for (int it = threadIdx.x; it < 64 * nr; it += blockDim.x) {
            const int o = it % 64, i = it / 64;
            const int m = o / 32, col = c0 + o % 32;
            part[((size_t)ks * a.P + rc + i) * (2 * F) + m * F + col] = outv[o][i];
        }
    }
}

// ---------------------------------------------------------------------------
// FP8 E4M3 experts with 128 x 128 block scales (AWQ-g32 card, "Optional FP8
// MTP": routed experts in E4M3 with explicit block scales).  Same mapping as
// the bf16 kernels, 16 lanes per weight row, but a 16-byte vector holds 16
// weights: v_cvt_pk_f32_fp8 widens two codes at a time (every E4M3 value is
// exactly a bf16 value), v_cvt_pk_bf16_f32 packs them and v_dot2_f32_bf16
// takes the activation pairs; the vector's dot product is scaled by its
// block's scale (a vector never crosses a 128-input block).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void fp8_to_bf16x8(uint4 c, uint32_t (&o)[8]) {
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[i], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[i], true);
        o[2 * i] = pack_bf16x2(lo[0], lo[1]);
        o[2 * i + 1] = pack_bf16x2(hi[0], hi[1]);
    }
}

// Dot products of NR FP8 weight rows (row n: codes rows[n], scales srow[n]
// per 128-input block, first input k0) with R activation rows in LDS
// (xs[i * xstride + v], 8 bf16 per uint4, input 8v relative to k0), 16 lanes
// per row.  U vectors per lane and row are loaded before any is used (vector
// indices past the row's end are clamped for the loads and skipped in the
// sums), so that a short row (F = 640 inputs: 40 vectors, 2 or 3 per lane)
// costs one memory round trip instead of one per vector (FP8 decode routed
// call 0.149 -> 0.138 ms with U = 3 for the down rows and U = 2 for gate/up).
template <int R, int NR, int RA, int U>
__device__ __forceinline__ void fp8_stream_dot(const uint4* const (&rows)[NR],
                                                       const float* const (&srow)[NR], int k0, int nv, int l16,
                                                       const uint4* xs, int xstride, float (&acc)[4][RA]) {
    for (int v0 = l16; v0 < nv; v0 += 16 * U) {
        uint4 w[U][NR];
        float sc[U][NR];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = min(v0 + 16 * u, nv - 1);
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                w[u][n] = ld_stream(&rows[n][v]);
                sc[u][n] = srow[n][(k0 + 16 * v) >> 7];
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // keeps the scheduler from sinking the loads to their uses
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + 16 * u;
            if (v < nv) {
#pragma unroll
                for (int n = 0; n < NR; ++n) {
                    uint32_t wb[8];
                    fp8_to_bf16x8(w[u][n], wb);
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        const uint4 x0 = xs[i * xstride + 2 * v], x1 = xs[i * xstride + 2 * v + 1];
                        float t = 0.0f;
                        t = dot2_bf16(wb[0], x0.x, t);
                        t = dot2_bf16(wb[1], x0.y, t);
                        t = dot2_bf16(wb[2], x0.z, t);
                        t = dot2_bf16(wb[3], x0.w, t);
                        t = dot2_bf16(wb[4], x1.x, t);
                        t = dot2_bf16(wb[5], x1.y, t);
                        t = dot2_bf16(wb[6], x1.z, t);
                        t = dot2_bf16(wb[7], x1.w, t);
                        acc[n][i] = fmaf(sc[u][n], t, acc[n][i]);
                    }
                }
            }
        }
    }
}

// FP8 gate/up: grid (F/32 column chunks, expert slot, KS input splits);
// block 256 (4 waves).  Waves 0,1: gate columns c0..c0+31, waves 2,3: up.
template <int RCH>
__global__ __launch_bounds__(256) void fp8_gateup_kernel(GroupedArgs a, int KS, float* __restrict__ part) {
    __shared__ uint4 xs[RCH * kBfChunkK / 8];
    __shared__ float outv[64][RCH];
    int r0, r1;
    const int e = a.offsets ? slot_expert(a.slots, blockIdx.y, &r0, &r1) : 0;
    if (!a.offsets) { r0 = 0; r1 = a.T; }
    if (e < 0) return;
    const int H = a.H, F = a.F;
    const int ks = blockIdx.z;
    // input split on 16-weight vectors
    const int kb = (int)((long)H / 16 * ks / KS) * 16, ke = (int)((long)H / 16 * (ks + 1) / KS) * 16;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int sub = lane / 16, l16 = lane % 16;
    const int c0 = blockIdx.x * 32;
    const int mat = wave / 2;
    const ProjDev& pj = mat ? a.up : a.gate;
    const uint8_t* W = pj.codes + (size_t)e * F * H;
    const float* S = pj.bscales + (size_t)e * (F / 128) * (H / 128);
    for (int rc = r0; rc < r1; rc += RCH) {
        const int nr = min(RCH, r1 - rc);
        float acc[4][RCH];
#pragma unroll
        for (int ps = 0; ps < 4; ++ps)
#pragma unroll
            for (int i = 0; i < RCH; ++i) acc[ps][i] = 0.0f;
        for (int k0 = kb; k0 < ke; k0 += kBfChunkK) {
            const int kl = min(kBfChunkK, ke - k0), nx = kl / 8;
            __syncthreads();
            for (int it = threadIdx.x; it < nr * nx; it += blockDim.x) {
                const int i = it / nx, v = it % nx;
                const int t = row_token(a.sorted_pair, a.k, rc + i);
                xs[i * (kBfChunkK / 8) + v] = reinterpret_cast<const uint4*>(a.x + (size_t)t * H + k0)[v];
            }
            __syncthreads();
            const uint4* rows[4];
            const float* srow[4];
#pragma unroll
            for (int ps = 0; ps < 4; ++ps) {
                const int col = c0 + (wave % 2) * 16 + ps * 4 + sub;
                rows[ps] = reinterpret_cast<const uint4*>(W + (size_t)col * H + k0);
                srow[ps] = S + (size_t)(col / 128) * (H / 128);
            }
            auto body = [&](auto rtag) {
                constexpr int R = decltype(rtag)::value;
                fp8_stream_dot<R, 4, RCH, 2>(rows, srow, k0, kl / 16, l16, xs, kBfChunkK / 8, acc);
            };
            dispatch_rows<RCH>(nr, body);
        }
#pragma unroll
        for (int ps = 0; ps < 4; ++ps)
#pragma unroll
            for (int i = 0; i < RCH; ++i) {
                float v = acc[ps][i];
                v += __shfl_xor(v, 1, kWave);
                v += __shfl_xor(v, 2, kWave);
                v += __shfl_xor(v, 4, kWave);
                v += __shfl_xor(v, 8, kWave);
                if (l16 == 0) outv[wave * 16 + ps * 4 + sub][i] = v;
            }
        __syncthreads();
        for (int it = threadIdx.x; it < 64 * nr; it += blockDim.x) {
            const int o = it % 64, i = it / 64;
            const int m = o / 32, col = c0 + o % 32;
            part[((size_t)ks * a.P + rc + i) * (2 * F) + m * F + col] = outv[o][i];
        }
    }
}

// ---------------------------------------------------------------------------
// NVFP4 experts (W4A4): the activations arrive quantised (e2m1 * block
// scale, as bf16).  A 16-byte weight vector holds 32 E2M1 codes, inputs
// 32v..32v+31 of one row, i.e. two groups of 16 with one E4M3 scale each.
// v_cvt_scalef32_pk_bf16_fp4 with scale 1 gives a byte's two codes exactly
// as a bf16 pair (low nibble first: the even input) and v_dot2_f32_bf16
// takes the activation pair; each group's dot product is
// then scaled by its E4M3 scale.  The global factors (activation and weight
// global scales) are applied to the row sums.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void fp4_to_bf16x4(uint32_t w, uint32_t (&o)[4]) {
    // v_cvt_scalef32_pk_bf16_fp4: the two codes of byte b (low nibble first)
    // as a bf16 pair; E2M1 values are exact in bf16 and the scale 1 is exact
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
}

// One weight vector (32 inputs, two groups) of one row against R staged
// activation rows: xv[i * xstride .. + 3] are the vector's 32 inputs of row i.
template <int R, int RA>
__device__ __forceinline__ void nvfp4_vec_dot(uint4 w, uint32_t sc2, const uint4* xv, int xstride,
                                              float (&acc)[RA]) {
    const auto sv = __builtin_amdgcn_cvt_pk_f32_fp8((int)sc2, false);  // the two E4M3 group scales
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    uint32_t wb[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t o[4];
        fp4_to_bf16x4(ww[q], o);
#pragma unroll
        for (int b = 0; b < 4; ++b) wb[4 * q + b] = o[b];
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const uint4* x = xv + i * xstride;
        float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint4 a = x[c], b = x[c + 2];
            t0 = dot2_bf16(wb[4 * c + 0], a.x, t0);
            t0 = dot2_bf16(wb[4 * c + 1], a.y, t0);
            t0 = dot2_bf16(wb[4 * c + 2], a.z, t0);
            t0 = dot2_bf16(wb[4 * c + 3], a.w, t0);
            t1 = dot2_bf16(wb[4 * c + 8], b.x, t1);
            t1 = dot2_bf16(wb[4 * c + 9], b.y, t1);
            t1 = dot2_bf16(wb[4 * c + 10], b.z, t1);
            t1 = dot2_bf16(wb[4 * c + 11], b.w, t1);
        }
        acc[i] = fmaf(sv[1], t1, fmaf(sv[0], t0, acc[i]));
    }
}

// Dot products of NR NVFP4 weight rows with R activation rows staged in LDS.
// LPR lanes share a row, lane lr taking vectors lr, lr + LPR, ...; vector v
// of row n is rows[n][v] with its two group scales at srow[n] + (k0 + 32 v) / 16.
// U vectors of every row are loaded before any is used (NR * U loads in flight).
template <int R, int NR, int U, int LPR, int RA>
__device__ __forceinline__ void nvfp4_stream_dot(const uint4* const (&rows)[NR], const uint8_t* const (&srow)[NR],
                                                 int k0, int nv, int lr, const uint4* xs, int xstride,
                                                 float (&acc)[4][RA]) {
    int v = lr;
    for (; v + LPR * (U - 1) < nv; v += LPR * U) {
        uint4 w[U][NR];
        uint32_t sc[U][NR];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                const int vv = v + LPR * u;
                w[u][n] = ld_stream(&rows[n][vv]);
                sc[u][n] = *reinterpret_cast<const uint16_t*>(srow[n] + ((k0 + 32 * vv) >> 4));
            }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int n = 0; n < NR; ++n) nvfp4_vec_dot<R, RA>(w[u][n], sc[u][n], xs + 4 * (v + LPR * u), xstride, acc[n]);
    }
    for (; v < nv; v += LPR) {
        uint4 w[NR];
        uint32_t sc[NR];
#pragma unroll
        for (int n = 0; n < NR; ++n) {
            w[n] = ld_stream(&rows[n][v]);
            sc[n] = *reinterpret_cast<const uint16_t*>(srow[n] + ((k0 + 32 * v) >> 4));
        }
#pragma unroll
        for (int n = 0; n < NR; ++n) nvfp4_vec_dot<R, RA>(w[n], sc[n], xs + 4 * v, xstride, acc[n]);
    }
}

// Software-pipelined form: the loads of the lane's next vector are issued
// before the current one is used, so NR loads stay in flight behind the
// arithmetic.  wn / sn hold the lane's first vector (v = lr) and its scales,
// loaded by the caller (before it stages the activations) when lr < nv.
template <int NR>
__device__ __forceinline__ void nvfp4_load_vec(const uint4* const (&rows)[NR], const uint8_t* const (&srow)[NR],
                                               int k0, int v, uint4 (&w)[NR], uint32_t (&sc)[NR]) {
#pragma unroll
    for (int n = 0; n < NR; ++n) {
        w[n] = ld_stream(&rows[n][v]);
        sc[n] = *reinterpret_cast<const uint16_t*>(srow[n] + ((k0 + 32 * v) >> 4));
    }
}

template <int R, int NR, int LPR, int RA>
__device__ __forceinline__ void nvfp4_stream_dot_pf(const uint4* const (&rows)[NR], const uint8_t* const (&srow)[NR],
                                                    int k0, int nv, int lr, const uint4* xs, int xstride,
                                                    float (&acc)[4][RA], uint4 (&wn)[NR], uint32_t (&sn)[NR]) {
    for (int v = lr; v < nv; v += LPR) {
        uint4 w[NR];
        uint32_t sc[NR];
#pragma unroll
        for (int n = 0; n < NR; ++n) { w[n] = wn[n]; sc[n] = sn[n]; }
        if (v + LPR < nv) nvfp4_load_vec<NR>(rows, srow, k0, v + LPR, wn, sn);
#pragma unroll
        for (int n = 0; n < NR; ++n) nvfp4_vec_dot<R, RA>(w[n], sc[n], xs + 4 * v, xstride, acc[n]);
    }
}

// Lanes sharing one NVFP4 weight row, and the gate (or up) columns a gate/up
// workgroup covers: two waves per matrix, four passes of 64 / LPR rows each.
__host__ __device__ constexpr int nv_gate_cols(int lpr) { return 2 * 4 * (64 / lpr); }

// NVFP4 gate/up: grid (F / nv_gate_cols(LPR) column chunks, expert slot, KS
// input splits); block 256 (4 waves).  Waves 0,1: gate columns, waves 2,3 the
// same up columns; LPR lanes stream one row (a row is H/2 bytes: 80 vectors
// at H = 2560), so a workgroup covers 512 / LPR columns of each matrix per
// staging of the activation rows.
template <int RCH, int LPR>
__global__ __launch_bounds__(256) void nvfp4_gateup_kernel(GroupedArgs a, int KS, float* __restrict__ part) {
    constexpr int RPW = 64 / LPR;                  // rows per wave per pass
    constexpr int CW = 4 * RPW;                    // columns per wave
    constexpr int CPB = nv_gate_cols(LPR);         // columns per matrix per workgroup
    constexpr int CK = RCH <= 2 ? 2 * kBfChunkK : kBfChunkK;  // inputs staged at once
    __shared__ uint4 xs[RCH * CK / 8];
    __shared__ float outv[2 * CPB][RCH];
    int r0, r1;
    const int e = a.offsets ? slot_expert(a.slots, blockIdx.y, &r0, &r1) : 0;
    if (!a.offsets) { r0 = 0; r1 = a.T; }
    if (e < 0) return;
    const int H = a.H, F = a.F;
    const int ks = blockIdx.z;
    const int kb = (int)((long)H / 32 * ks / KS) * 32, ke = (int)((long)H / 32 * (ks + 1) / KS) * 32;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int sub = lane / LPR, lr = lane % LPR;
    const int c0 = blockIdx.x * CPB;
    const int mat = wave / 2;
    const uint8_t* W = (mat ? a.up.codes : a.gate.codes) + (size_t)e * F * (H / 2);
    const uint8_t* S = (mat ? a.up.gscales : a.gate.gscales) + (size_t)e * F * (H / 16);
    const float gscale = a.gate.act * (mat ? a.up.wglobal : a.gate.wglobal)[e];
    for (int rc = r0; rc < r1; rc += RCH) {
        const int nr = min(RCH, r1 - rc);
        float acc[4][RCH];
#pragma unroll
        for (int ps = 0; ps < 4; ++ps)
#pragma unroll
            for (int i = 0; i < RCH; ++i) acc[ps][i] = 0.0f;
        for (int k0 = kb; k0 < ke; k0 += CK) {
            const int kl = min(CK, ke - k0), nx = kl / 8;
            const uint4* rows[4];
            const uint8_t* srow[4];
#pragma unroll
            for (int ps = 0; ps < 4; ++ps) {
                const int col = c0 + (wave % 2) * CW + ps * RPW + sub;
                rows[ps] = reinterpret_cast<const uint4*>(W + (size_t)col * (H / 2) + k0 / 2);
                srow[ps] = S + (size_t)col * (H / 16);
            }
            uint4 wn[4];
            uint32_t sn[4];
            if (kNvGateUnroll == 0 && lr < kl / 32)
                nvfp4_load_vec<4>(rows, srow, k0, lr, wn, sn);  // in flight during the staging
            __syncthreads();
            for (int it = threadIdx.x; it < nr * nx; it += blockDim.x) {
                const int i = it / nx, v = it % nx;
                const int t = row_token(a.sorted_pair, a.k, rc + i);
                xs[i * (CK / 8) + v] = reinterpret_cast<const uint4*>(a.x + (size_t)t * H + k0)[v];
            }
            __syncthreads();
            auto body = [&](auto rtag) {
                constexpr int R = decltype(rtag)::value;
                if constexpr (kNvGateUnroll == 0)
                    nvfp4_stream_dot_pf<R, 4, LPR, RCH>(rows, srow, k0, kl / 32, lr, xs, CK / 8, acc, wn, sn);
                else
                    nvfp4_stream_dot<R, 4, kNvGateUnroll, LPR, RCH>(rows, srow, k0, kl / 32, lr, xs, CK / 8, acc);
            };
            dispatch_rows<RCH>(nr, body);
        }
#pragma unroll
        for (int ps = 0; ps < 4; ++ps)
#pragma unroll
            for (int i = 0; i < RCH; ++i) {
                float v = acc[ps][i];
#pragma unroll
                for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m, kWave);
                if (lr == 0) outv[wave * CW + ps * RPW + sub][i] = v * gscale;
            }
        __syncthreads();
        for (int it = threadIdx.x; it < 2 * CPB * nr; it += blockDim.x) {
            const int o = it % (2 * CPB), i = it / (2 * CPB);
            const int m = o / CPB, col = c0 + o % CPB;
            part[((size_t)ks * a.P + rc + i) * (2 * F) + m * F + col] = outv[o][i];
        }
    }
}

// SwiGLU of the gate/up partials summed over the KS input splits: one bf16
// pair (the product rounded once) per thread, h[r][F/2].
// A pair of SwiGLU values to bf16; with qa > 0 (NVFP4) they are first
// quantised with activation global scale qa in their group of 16, which
// eight consecutive lanes hold (every lane of the group must take part).
__device__ __forceinline__ uint32_t pack_h_pair(float h0, float h1, float qa) {
    if (qa > 0.0f) {
        float amax = fmaxf(fabsf(h0), fabsf(h1));
        amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
        amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
        amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
        const float sc = nvfp4_group_scale(amax, qa);
        h0 = nvfp4_qv(h0, sc, qa);
        h1 = nvfp4_qv(h1, sc, qa);
    }
    return pack_bf16x2(h0, h1);
}

__device__ __forceinline__ uint32_t swiglu_pair(const float* __restrict__ part, int KS, int P, int F,
                                                int r, int f, float qa) {
    float hv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        float g = 0.0f, up = 0.0f;
        for (int ks = 0; ks < KS; ++ks) {
            const float* pp = part + ((size_t)ks * P + r) * (2 * F);
            g += pp[f + u];
            up += pp[F + f + u];
        }
        hv[u] = silu(g) * up;
    }
    return pack_h_pair(hv[0], hv[1], qa);
}

// With several input splits the SwiGLU is formed once per row here, instead of
// in every down-projection workgroup that reads the row.  Groups of 16 values
// (8 lanes) never straddle the end, so whole groups leave together.
__global__ __launch_bounds__(256) void swiglu_reduce_kernel(const float* __restrict__ part, int KS,
                                                            int P, int F, float qa, uint32_t* __restrict__ h) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)P * (F / 2)) return;
    const int r = (int)(i / (F / 2)), f = 2 * (int)(i % (F / 2));
    h[i] = swiglu_pair(part, KS, P, F, r, f, qa);
}

hipError_t launch_swiglu_reduce(const float* part, int KS, int P, int F, uint32_t* h, hipStream_t s) {
    const long pairs = (long)P * (F / 2);
    hipLaunchKernelGGL(swiglu_reduce_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, s, part, KS, P, F,
                       0.0f, h);
    return hipGetLastError();
}

// Rows [rc, rc+nr) of h into LDS as bf16 pairs h2[RCH][F/2]: copied from hsrc
// when the SwiGLU was formed by swiglu_reduce_kernel, else formed here.
template <int RCH>
__device__ __forceinline__ void stage_swiglu(const float* __restrict__ part,
                                             const uint32_t* __restrict__ hsrc, int KS, int P,
                                             int F, int rc, int nr, uint32_t* h2, float qa = 0.0f) {
    if (hsrc) {
        for (int it = threadIdx.x; it < RCH * (F / 2); it += blockDim.x) {
            const int i = it / (F / 2);
            h2[it] = i < nr ? hsrc[(size_t)(rc + i) * (F / 2) + it % (F / 2)] : 0u;
        }
        return;
    }
    for (int it = threadIdx.x; it < RCH * (F / 2); it += blockDim.x) {
        const int i = it / (F / 2), f = 2 * (it % (F / 2));
        float hv[2] = {0.0f, 0.0f};
        if (i < nr) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float g = 0.0f, up = 0.0f;
                for (int ks = 0; ks < KS; ++ks) {
                    const float* pp = part + ((size_t)ks * P + rc + i) * (2 * F);
                    g += pp[f + u];
                    up += pp[F + f + u];
                }
                hv[u] = silu(g) * up;
            }
        }
        h2[it] = pack_h_pair(hv[0], hv[1], qa);  // rows >= nr: zeros, quantised to zeros
    }
}

// ---------------------------------------------------------------------------
// AWQ down: grid (OW/OWC column chunks, expert slot); block = OWC * RP.
// ---------------------------------------------------------------------------
template <int RCH>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void awq_down_kernel(GroupedArgs a, int KS, int OWC,
                                                       const float* __restrict__ part,
                                                       const uint32_t* __restrict__ hsrc) {
    __shared__ uint32_t xs[RCH * kGemvMaxKPairs];
    __shared__ float xsum[RCH * 64];
    extern __shared__ float red[];  // [RCH][8*OWC]
    int r0, r1;
    const int e = a.offsets ? slot_expert(a.slots, blockIdx.y, &r0, &r1) : 0;
    if (!a.offsets) { r0 = 0; r1 = a.T; }
    if (e < 0) return;
    const int H = a.H, F = a.F, OW = H / 8, G = F / 32, npairs = F / 2;
    const int cl = threadIdx.x % OWC, rp = threadIdx.x / OWC, RP = blockDim.x / OWC;
    const int c = blockIdx.x * OWC + cl;
    const int32_t* qw = a.down.qweight + (size_t)e * F * OW;
    const int32_t* qz = a.down.qzeros + (size_t)e * G * OW;
    const uint16_t* sc = a.down.scales + (size_t)e * G * H;
    for (int rc = r0; rc < r1; rc += RCH) {
        const int nr = min(RCH, r1 - rc);
        __syncthreads();
        stage_swiglu<RCH>(part, hsrc, KS, a.P, F, rc, nr, xs);
        __syncthreads();
        stage_group_sums<RCH>(xs, npairs, G, xsum);
        __syncthreads();
        auto body = [&](auto rtag) {
            constexpr int R = decltype(rtag)::value;
            float res[8][R];
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < R; ++i) res[j][i] = 0.0f;
            awq_gemv_groups<R>(qw, qz, sc, H, OW, c, 0, rp, G, RP, xs, npairs, xsum, G, res);
            reduce_phases<R>(res, cl, rp, RP, 8 * OWC, red);
        };
        dispatch_rows<RCH>(nr, body);
        const int ncol = 8 * OWC;
        for (int it = threadIdx.x; it < nr * ncol; it += blockDim.x) {
            const int i = it / ncol, col = it % ncol;
            const size_t o = (size_t)(rc + i) * H + (size_t)blockIdx.x * ncol + col;
            const float v = red[i * ncol + col];
            if (a.out_f32) static_cast<float*>(a.rows)[o] = v;
            else static_cast<uint16_t*>(a.rows)[o] = (uint16_t)f32_to_bf16_bits(v);
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 down: grid (H/(16*npass) row chunks, expert slot); block 256; 16 lanes
// per weight row; each WG covers 16*npass output rows.
// ---------------------------------------------------------------------------
template <int R, int NPASS, int RA>
__device__ __forceinline__ void bf16_down_dot(const uint16_t* __restrict__ W, int F, int o0,
                                              int wave, int sub, int l16, const uint4* hv,
                                              float (&acc)[4][RA]) {
    const uint4* rows[NPASS];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps)
        rows[ps] = reinterpret_cast<const uint4*>(W + (size_t)(o0 + ps * 16 + wave * 4 + sub) * F);
    bf16_stream_dot<R, NPASS, (NPASS >= 4 ? 2 : 4)>(rows, F / 8, l16, hv, F / 8, acc);
}

// The down projection of bf16 (WF 0) or FP8 (WF 2) experts.
template <int RCH, int NPASS, int WF = 0>
__global__ __launch_bounds__(256) void bf16_down_kernel(GroupedArgs a, int KS,
                                                        const float* __restrict__ part,
                                                        const uint32_t* __restrict__ hsrc) {
    constexpr int npass = NPASS;
    __shared__ uint32_t h2[RCH * kGemvMaxKPairs];
    __shared__ float outv[64][RCH];
    int r0, r1;
    const int e = a.offsets ? slot_expert(a.slots, blockIdx.y, &r0, &r1) : 0;
    if (!a.offsets) { r0 = 0; r1 = a.T; }
    if (e < 0) return;
    const int H = a.H, F = a.F;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int sub = lane / 16, l16 = lane % 16;
    const int o0 = blockIdx.x * 16 * npass;
    const uint16_t* W = a.down.w + (size_t)e * H * F;
    const uint4* hv = reinterpret_cast<const uint4*>(h2);
    for (int rc = r0; rc < r1; rc += RCH) {
        const int nr = min(RCH, r1 - rc);
        __syncthreads();
        stage_swiglu<RCH>(part, hsrc, KS, a.P, F, rc, nr, h2);
        __syncthreads();
        float acc[4][RCH];
#pragma unroll
        for (int ps = 0; ps < 4; ++ps)
#pragma unroll
            for (int i = 0; i < RCH; ++i) acc[ps][i] = 0.0f;
        auto body = [&](auto rtag) {
            constexpr int R = decltype(rtag)::value;
            if constexpr (WF == 2) {
                const uint4* rows[NPASS];
                const float* srow[NPASS];
                const uint8_t* C = a.down.codes + (size_t)e * H * F;
                const float* S = a.down.bscales + (size_t)e * (H / 128) * (F / 128);
#pragma unroll
                for (int ps = 0; ps < NPASS; ++ps) {
                    const int o = o0 + ps * 16 + wave * 4 + sub;
                    rows[ps] = reinterpret_cast<const uint4*>(C + (size_t)o * F);
                    srow[ps] = S + (size_t)(o / 128) * (F / 128);
                }
                fp8_stream_dot<R, NPASS, RCH, 3>(rows, srow, 0, F / 16, l16, hv, F / 8, acc);
            } else {
                bf16_down_dot<R, NPASS, RCH>(W, F, o0, wave, sub, l16, hv, acc);
            }
        };
        dispatch_rows<RCH>(nr, body);
#pragma unroll
        for (int ps = 0; ps < 4; ++ps)
#pragma unroll
            for (int i = 0; i < RCH; ++i) {
                float v = acc[ps][i];
                v += __shfl_xor(v, 1, kWave);
                v += __shfl_xor(v, 2, kWave);
                v += __shfl_xor(v, 4, kWave);
                v += __shfl_xor(v, 8, kWave);
                if (l16 == 0 && ps < npass) outv[ps * 16 + wave * 4 + sub][i] = v;
            }
        __syncthreads();
        const int nrows = 16 * npass;
        for (int it = threadIdx.x; it < nrows * nr; it += blockDim.x) {
            const int o = it % nrows, i = it / nrows;
            const size_t idx = (size_t)(rc + i) * H + o0 + o;
            const float v = outv[o][i];
            if (a.out_f32) static_cast<float*>(a.rows)[idx] = v;
            else static_cast<uint16_t*>(a.rows)[idx] = (uint16_t)f32_to_bf16_bits(v);
        }
    }
}

// NVFP4 down: a row of W_down is F/2 bytes (20 vectors at F = 640), so LPR
// lanes (few) share a row and a wave covers 64 / LPR rows per pass.  Grid
// (H / rows per workgroup, expert slot); block 256; lane q = lane / LPR of
// wave w takes rows o0 + p * 4 * (64 / LPR) + w * (64 / LPR) + q, p < NP.  The
// SwiGLU product is staged (quantised) in LDS once per row chunk; the global
// factor act_scale * global_scale[e] scales the sums.
__host__ __device__ constexpr int nv_down_rows(int np, int lpr) { return np * 4 * (64 / lpr); }

template <int RCH, int NP, int U, int LPR>
__global__ __launch_bounds__(256) void nvfp4_down_kernel(GroupedArgs a, int KS, const float* __restrict__ part,
                                                         const uint32_t* __restrict__ hsrc) {
    constexpr int RPW = 64 / LPR, RPP = 4 * RPW, NROWS = nv_down_rows(NP, LPR);
    __shared__ uint32_t h2[RCH * kGemvMaxKPairs];
    __shared__ float outv[NROWS][RCH];
    int r0, r1;
    const int e = a.offsets ? slot_expert(a.slots, blockIdx.y, &r0, &r1) : 0;
    if (!a.offsets) { r0 = 0; r1 = a.T; }
    if (e < 0) return;
    const int H = a.H, F = a.F;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int q = lane / LPR, lr = lane % LPR;
    const int o0 = blockIdx.x * NROWS;
    const int nrows = min(NROWS, H - o0);
    const float oscale = a.down.act * a.down.wglobal[e];
    const uint8_t* C = a.down.codes + (size_t)e * H * (F / 2);
    const uint8_t* S = a.down.gscales + (size_t)e * H * (F / 16);
    const uint4* rows[NP];
    const uint8_t* srow[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int o = min(o0 + p * RPP + wave * RPW + q, H - 1);  // rows past H repeat the last, unused
        rows[p] = reinterpret_cast<const uint4*>(C + (size_t)o * (F / 2));
        srow[p] = S + (size_t)o * (F / 16);
    }
    const uint4* hv = reinterpret_cast<const uint4*>(h2);
    for (int rc = r0; rc < r1; rc += RCH) {
        const int nr = min(RCH, r1 - rc);
        uint4 wn[NP];
        uint32_t sn[NP];
        if (lr < F / 32) nvfp4_load_vec<NP>(rows, srow, 0, lr, wn, sn);  // in flight during the staging
        __syncthreads();
        stage_swiglu<RCH>(part, hsrc, KS, a.P, F, rc, nr, h2, a.down.act);
        __syncthreads();
        float acc[4][RCH];
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int i = 0; i < RCH; ++i) acc[p][i] = 0.0f;
        auto body = [&](auto rtag) {
            constexpr int R = decltype(rtag)::value;
            if constexpr (U == 0)
                nvfp4_stream_dot_pf<R, NP, LPR, RCH>(rows, srow, 0, F / 32, lr, hv, F / 8, acc, wn, sn);
            else
                nvfp4_stream_dot<R, NP, U, LPR, RCH>(rows, srow, 0, F / 32, lr, hv, F / 8, acc);
        };
        dispatch_rows<RCH>(nr, body);
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int i = 0; i < RCH; ++i) {
                float v = acc[p][i];
#pragma unroll
                for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m, kWave);
                if (lr == 0) outv[p * RPP + wave * RPW + q][i] = v * oscale;
            }
        __syncthreads();
        for (int it = threadIdx.x; it < nrows * nr; it += blockDim.x) {
            const int o = it % nrows, i = it / nrows;
            const size_t idx = (size_t)(rc + i) * H + o0 + o;
            const float v = outv[o][i];
            if (a.out_f32) static_cast<float*>(a.rows)[idx] = v;
            else static_cast<uint16_t*>(a.rows)[idx] = (uint16_t)f32_to_bf16_bits(v);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// Input splits of the gate/up pass.  AWQ: groups per workgroup bounded by the
// LDS activation stage (16 groups at H = 2560).  bf16: enough workgroups when
// few experts are active (the shared expert is a single expert).
int gemv_ksplit(const GroupedArgs& a) {
    if (!a.awq) {
        const int slots = a.offsets ? (a.P < a.E ? a.P : a.E) : 1;
        const int cols = a.nvfp4 && a.F % nv_gate_cols(kNvGateLanes) == 0 ? nv_gate_cols(kNvGateLanes) : 32;
        const long wgs = (long)slots * (a.F / cols);
        int ks = 1;
        while (wgs * ks < 1024 && ks < kGemvMaxSplit && (a.H / 8) % (ks * 2) == 0) ks *= 2;
        return ks;
    }
    const int G = a.H / 32;
    int ks = 5;                            // 16 groups per workgroup at H = 2560
    while (ks > 1 && G % ks) --ks;
    while ((G + ks - 1) / ks * 16 > kGemvMaxKPairs) ++ks;  // LDS bound
    return ks;
}

static size_t slot_table_bytes(int P) { return ((size_t)P * sizeof(int4) + 255) & ~(size_t)255; }

static size_t part_bytes(int P, int F, int ks) {
    return ((size_t)ks * P * 2 * F * sizeof(float) + 255) & ~(size_t)255;
}

size_t gemv_ws_bytes(int P, int H, int F, int awq, int E) {
    int ks = kGemvMaxSplit;  // bf16, FP8, NVFP4 bound
    (void)E;
    if (awq) {
        GroupedArgs a{};
        a.H = H;
        a.awq = awq;
        ks = gemv_ksplit(a);
    }
    // slot table, partial sums, then h [P][F] bf16
    return slot_table_bytes(P) + part_bytes(P, F, ks) + (size_t)P * F * sizeof(uint16_t);
}

static int down_owc(int OW) {
    const int cand[5] = {64, 32, 16, 8, 4};
    if (OW <= 64) return OW;
    for (int c : cand)
        if (OW % c == 0) return c;
    return 4;
}

// Row phases for OW word columns: about 256 threads, a whole number of waves.
static int row_phases(int OW) {
    int rp = 256 / OW;
    if (rp < 1) rp = 1;
    while ((OW * rp) % kWave != 0 && OW * (rp + 1) <= 512) ++rp;
    return rp;
}

// Grids put the column (or row) chunk along x and the expert slot along y, so
// workgroups that are dispatched one after another stream adjacent parts of
// one expert's weights (measured faster than slot-major order).
template <int RCH>
static hipError_t launch_gemv_rch(const GroupedArgs& a, void* ws, hipStream_t s) {
    const int slots = a.offsets ? (a.P < a.E ? a.P : a.E) : 1;
    const int F = a.F, H = a.H;
    const int KS = gemv_ksplit(a);
    float* part = static_cast<float*>(ws);
    uint32_t* hbuf = nullptr;
    if (KS > 1) hbuf = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + part_bytes(a.P, F, KS));
    if (a.awq) {
      if constexpr (RCH <= 2) {
        const int OW = F / 8;
        const int RP = row_phases(OW);
        const size_t red_bytes = (size_t)RCH * F * sizeof(float);
        hipLaunchKernelGGL(awq_gateup_kernel<RCH>, dim3(2 * KS, slots), dim3(OW * RP), red_bytes, s,
                           a, KS, part);
        const int OWd = H / 8, OWC = down_owc(OWd);
        // few down workgroups share a row (5 at H = 2560): each forms the
        // SwiGLU from the partial sums itself, which costs less than a launch
        if (OWd / OWC <= 8) hbuf = nullptr;
        if (hbuf) {
            const long pairs = (long)a.P * (F / 2);
            hipLaunchKernelGGL(swiglu_reduce_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0,
                               s, (const float*)part, KS, a.P, F, 0.0f, hbuf);
        }
        const int RPd = row_phases(OWC);
        hipLaunchKernelGGL(awq_down_kernel<RCH>, dim3(OWd / OWC, slots), dim3(OWC * RPd),
                           (size_t)RCH * 8 * OWC * sizeof(float), s, a, KS, OWC,
                           (const float*)part, (const uint32_t*)hbuf);
      } else {
        return hipErrorInvalidValue;  // AWQ takes at most two rows per pass
      }
    } else if (a.nvfp4) {
      if constexpr (RCH <= 8) {
        if (F % nv_gate_cols(kNvGateLanes) == 0)
            hipLaunchKernelGGL((nvfp4_gateup_kernel<RCH, kNvGateLanes>), dim3(F / nv_gate_cols(kNvGateLanes), slots, KS),
                               dim3(256), 0, s, a, KS, part);
        else
            hipLaunchKernelGGL((nvfp4_gateup_kernel<RCH, 16>), dim3(F / nv_gate_cols(16), slots, KS), dim3(256), 0,
                               s, a, KS, part);
        if (hbuf) {
            const long pairs = (long)a.P * (F / 2);
            hipLaunchKernelGGL(swiglu_reduce_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0,
                               s, (const float*)part, KS, a.P, F, a.down.act, hbuf);
        }
        constexpr int DR = nv_down_rows(kNvDownRows, kNvDownLanes);
        hipLaunchKernelGGL((nvfp4_down_kernel<RCH, kNvDownRows, kNvDownUnroll, kNvDownLanes>),
                           dim3((H + DR - 1) / DR, slots), dim3(256), 0, s, a, KS, (const float*)part,
                           (const uint32_t*)hbuf);
      } else {
        return hipErrorInvalidValue;  // NVFP4 takes at most eight rows per pass
      }
    } else if (a.fp8) {
        hipLaunchKernelGGL(fp8_gateup_kernel<RCH>, dim3(F / 32, slots, KS), dim3(256), 0, s, a, KS, part);
        if (hbuf) {
            const long pairs = (long)a.P * (F / 2);
            hipLaunchKernelGGL(swiglu_reduce_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0,
                               s, (const float*)part, KS, a.P, F, 0.0f, hbuf);
        }
        if ((long)slots * (H / 64) >= 1024)
            hipLaunchKernelGGL((bf16_down_kernel<RCH, 4, 2>), dim3(H / 64, slots), dim3(256), 0, s, a, KS,
                               (const float*)part, (const uint32_t*)hbuf);
        else
            hipLaunchKernelGGL((bf16_down_kernel<RCH, 1, 2>), dim3(H / 16, slots), dim3(256), 0, s, a, KS,
                               (const float*)part, (const uint32_t*)hbuf);
    } else {
        hipLaunchKernelGGL(bf16_gateup_kernel<RCH>, dim3(F / 32, slots, KS), dim3(256), 0, s, a, KS,
                           part);
        if (hbuf) {
            const long pairs = (long)a.P * (F / 2);
            hipLaunchKernelGGL(swiglu_reduce_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0,
                               s, (const float*)part, KS, a.P, F, 0.0f, hbuf);
        }
        // rows per down workgroup: 64, or 16 when few experts are active
        if ((long)slots * (H / 64) >= 1024)
            hipLaunchKernelGGL((bf16_down_kernel<RCH, 4>), dim3(H / 64, slots), dim3(256), 0, s, a, KS,
                               (const float*)part, (const uint32_t*)hbuf);
        else
            hipLaunchKernelGGL((bf16_down_kernel<RCH, 1>), dim3(H / 16, slots), dim3(256), 0, s, a, KS,
                               (const float*)part, (const uint32_t*)hbuf);
    }
    return hipGetLastError();
}

// Slot table of a grouped call: slot i (< nslots) = the i-th non-empty expert
// in index order with its row range; later slots get expert -1.  One block of
// 1024 threads (E <= 1024): a ballot prefix count of the non-empty experts.
__global__ __launch_bounds__(1024) void slot_table_kernel(const int32_t* __restrict__ offsets, int E, int nslots,
                                                          int4* __restrict__ slots) {
    __shared__ int wsum[16];
    const int e = threadIdx.x, lane = e % kWave, wave = e / kWave;
    int r0 = 0, r1 = 0;
    if (e < E) {
        r0 = offsets[e];
        r1 = offsets[e + 1];
    }
    const bool ne = r1 > r0;
    const unsigned long long m = __ballot(ne);
    if (lane == 0) wsum[wave] = __popcll(m);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        before += w < wave ? wsum[w] : 0;
        total += wsum[w];
    }
    const int pos = before + __popcll(m & ((1ull << lane) - 1ull));
    if (ne && pos < nslots) slots[pos] = make_int4(e, r0, r1, 0);
    if (e >= total && e < nslots) slots[e] = make_int4(-1, 0, 0, 0);
}

int4* launch_slot_table(const int32_t* offsets, int E, int P, int4* tab, hipStream_t s) {
    hipLaunchKernelGGL(slot_table_kernel, dim3(1), dim3(1024), 0, s, offsets, E, P < E ? P : E, tab);
    return tab;
}

hipError_t launch_gemv(const GroupedArgs& a0, void* ws, hipStream_t s) {
    GroupedArgs a = a0;
    if (a.offsets) {
        int4* tab = static_cast<int4*>(ws);
        ws = static_cast<char*>(ws) + slot_table_bytes(a.P);
        if (!a0.slots) a.slots = launch_slot_table(a.offsets, a.E, a.P, tab, s);
    } else {
        a.slots = nullptr;
    }
    // rows per pass: a bf16 shared expert sees every token (all of a decode
    // batch in one pass); a routed expert at decode sees one or two, and the
    // AWQ kernels keep two rows per pass to hold the next group's words in
    // registers; FP8 and NVFP4 shared experts take eight rows per pass
    if (!a.offsets && a.T > 2 && !a.awq && !a.fp8 && !a.nvfp4) return launch_gemv_rch<16>(a, ws, s);
    if (!a.offsets && a.T > 2 && (a.fp8 || a.nvfp4)) return launch_gemv_rch<8>(a, ws, s);
    return launch_gemv_rch<2>(a, ws, s);
}

}  // namespace moe

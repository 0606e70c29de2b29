// The shared expert of a decode step: one bf16 SwiGLU expert applied to a
// handful of tokens (at most 16), as a split-K skinny GEMM on the 16x16x32
// bf16 MFMA.
//
// Qwen3.8-Flash-Next architecture sheet, FFN / MoE entries: one always-on
// shared expert, SwiGLU, no bias, no clamp.  Its 2 x F x H + H x F bf16
// weights are a few MB, read once; a 16 x 16 MFMA tile holds every token
// row, so each weight row's 16-byte runs go from HBM straight into a lane's
// B operand (lane l: column l % 16, inputs 8 (l / 16) .. +7 of a 32-input
// step; A: token row l % 16, the same inputs; the product: rows
// 4 (l / 16) .. +3 of column l % 16).  Rows past T read as zero.
//
// Gate/up: a wave takes 16 of the 2F gate-then-up columns over one of KS
// input splits and writes fp32 partial sums part[ks][t][2F]; the SwiGLU
// reduction (swiglu_reduce_kernel, shared with the streaming kernels) adds
// the splits in order and rounds h to bf16.  Down: a wave takes 16 output
// columns over all F inputs and writes the rows.  Every load of a wave is
// issued before its first MFMA.
#include "ffn_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));

constexpr int kSkWaves = 4;
constexpr int kSkMaxRows = 16;
constexpr int kSkMaxSteps = 20;  // 32-input MFMA steps a wave (all loads in flight)

__device__ __forceinline__ bf16x8_v sk_load(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_t*>(p));
}

// 16 columns x steps 32-input MFMA steps: the weight rows w_of(col) and the
// token rows x[row * ld] (rows >= T read as zero), inputs k0 + 32 m + ...
template <int NS>
__device__ __forceinline__ f32x4_t sk_tile(const uint16_t* wrow, const uint16_t* xrow, bool row_ok, int k0) {
    const int lane = threadIdx.x % kWave, kq = 8 * (lane / 16);
    bf16x8_v B[NS], A[NS];
#pragma unroll
    for (int m = 0; m < NS; ++m) {
        B[m] = sk_load(wrow + k0 + 32 * m + kq);
        A[m] = row_ok ? sk_load(xrow + k0 + 32 * m + kq) : bf16x8_v{};
    }
    f32x4_t d0 = {0.0f, 0.0f, 0.0f, 0.0f}, d1 = d0;
#pragma unroll
    for (int m = 0; m < NS; m += 2) {
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[m], B[m], d0, 0, 0, 0);
        if (m + 1 < NS) d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[m + 1], B[m + 1], d1, 0, 0, 0);
    }
    return d0 + d1;
}

// grid (2F / (16 kSkWaves), KS); part[ks][t][2F] fp32.
template <int NS>
__global__ __launch_bounds__(kSkWaves * kWave) void sk_gateup_kernel(GroupedArgs a, int KS, float* __restrict__ part) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int F = a.F, H = a.H, T = a.T;
    const int c = (blockIdx.x * kSkWaves + wave) * 16 + lane % 16;  // column of [gate | up]
    if (c >= 2 * F) return;                                            // whole wave (2F % 16 == 0)
    const int ks = blockIdx.y, k0 = ks * (H / KS);
    const uint16_t* wrow = (c < F ? a.gate.w + (size_t)c * H : a.up.w + (size_t)(c - F) * H);
    const int row = lane % 16;
    const f32x4_t d = sk_tile<NS>(wrow, a.x + (size_t)row * H, row < T, k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * (lane / 16) + i;
        if (r < T) part[((size_t)ks * T + r) * (2 * F) + c] = d[i];
    }
}

// grid (H / (16 kSkWaves)); h [T][F] bf16 -> rows [T][H].
template <int NS>
__global__ __launch_bounds__(kSkWaves * kWave) void sk_down_kernel(GroupedArgs a, const uint16_t* __restrict__ h) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int F = a.F, H = a.H, T = a.T;
    const int c = (blockIdx.x * kSkWaves + wave) * 16 + lane % 16;
    if (c >= H) return;  // whole wave (H % 16 == 0)
    const int row = lane % 16;
    const f32x4_t d = sk_tile<NS>(a.down.w + (size_t)c * F, h + (size_t)row * F, row < T, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * (lane / 16) + i;
        if (r >= T) continue;
        const size_t o = (size_t)r * H + c;
        if (a.out_f32) static_cast<float*>(a.rows)[o] = d[i];
        else static_cast<uint16_t*>(a.rows)[o] = (uint16_t)f32_to_bf16_bits(d[i]);
    }
}

// Input splits of the gate/up pass: the most of 8, 4, 2, 1 that leave a
// whole number of 32-input steps, at most kSkMaxSteps of them.
int sk_splits(int H) {
    for (int ks = 8; ks >= 1; ks >>= 1)
        if (H % (32 * ks) == 0 && H / (32 * ks) <= kSkMaxSteps) return ks;
    return 0;
}

size_t sk_part_bytes(int T, int F, int KS) { return ((size_t)KS * T * 2 * F * sizeof(float) + 255) & ~(size_t)255; }

}  // namespace

bool skinny_supported(int T, int H, int F) {
    return T >= 1 && T <= kSkMaxRows && H % 32 == 0 && F % 32 == 0 && F / 32 <= kSkMaxSteps && sk_splits(H) > 0;
}

size_t skinny_ws_bytes(int T, int H, int F) {
    return sk_part_bytes(T, F, sk_splits(H)) + (size_t)T * F * sizeof(uint16_t);
}

hipError_t launch_skinny(const GroupedArgs& a, void* ws, hipStream_t s) {
    const int KS = sk_splits(a.H), ns = a.H / KS / 32, nd = a.F / 32;
    float* part = static_cast<float*>(ws);
    uint16_t* h = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + sk_part_bytes(a.T, a.F, KS));
    const dim3 g1((2 * a.F / 16 + kSkWaves - 1) / kSkWaves, KS);
    switch (ns) {
#define MOE_SK(N) \
    case N: hipLaunchKernelGGL(sk_gateup_kernel<N>, g1, dim3(kSkWaves * kWave), 0, s, a, KS, part); break;
        MOE_SK(1) MOE_SK(2) MOE_SK(3) MOE_SK(4) MOE_SK(5) MOE_SK(6) MOE_SK(7) MOE_SK(8) MOE_SK(9) MOE_SK(10)
        MOE_SK(11) MOE_SK(12) MOE_SK(13) MOE_SK(14) MOE_SK(15) MOE_SK(16) MOE_SK(17) MOE_SK(18) MOE_SK(19) MOE_SK(20)
#undef MOE_SK
        default: return hipErrorInvalidValue;
    }
    hipError_t err = launch_swiglu_reduce(part, KS, a.T, a.F, reinterpret_cast<uint32_t*>(h), s);
    if (err != hipSuccess) return err;
    const dim3 g2((a.H / 16 + kSkWaves - 1) / kSkWaves);
    switch (nd) {
#define MOE_SK(N) \
    case N: hipLaunchKernelGGL(sk_down_kernel<N>, g2, dim3(kSkWaves * kWave), 0, s, a, (const uint16_t*)h); break;
        MOE_SK(1) MOE_SK(2) MOE_SK(3) MOE_SK(4) MOE_SK(5) MOE_SK(6) MOE_SK(7) MOE_SK(8) MOE_SK(9) MOE_SK(10)
        MOE_SK(11) MOE_SK(12) MOE_SK(13) MOE_SK(14) MOE_SK(15) MOE_SK(16) MOE_SK(17) MOE_SK(18) MOE_SK(19) MOE_SK(20)
#undef MOE_SK
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moe

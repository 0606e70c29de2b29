// NVFP4 activation quantisation of bf16 rows (NVFP4 release card, precision
// table: W4A4 experts, FP4 values in groups of 16 with FP8 block scales and
// FP32 global scales).  One thread per group of 16 inputs: the group's scale
// is the E4M3 rounding of amax / (6 ga), each input the E2M1 rounding of
// v / (s ga); the output is e2m1 * s as bf16 (exact: at most 6 significant
// bits), the global factor ga being applied after the dot products.
#include "kernels.h"
#include "nvfp4.h"

namespace moe {

__global__ __launch_bounds__(256) void nvfp4_quantize_kernel(const uint16_t* __restrict__ x, long groups,
                                                             float ga, uint16_t* __restrict__ out) {
    const long g = (long)blockIdx.x * 256 + threadIdx.x;
    if (g >= groups) return;
    const uint4* src = reinterpret_cast<const uint4*>(x) + 2 * g;
    const uint4 a = src[0], b = src[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float v[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
    }
    const float s = nvfp4_group_scale(amax, ga);
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = pack_bf16x2(nvfp4_qv(v[2 * i], s, ga), nvfp4_qv(v[2 * i + 1], s, ga));
    uint4* dst = reinterpret_cast<uint4*>(out) + 2 * g;
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

hipError_t launch_nvfp4_quantize(const uint16_t* x, int T, int n, float act_scale, uint16_t* out,
                                 hipStream_t s) {
    const long groups = (long)T * n / 16;
    hipLaunchKernelGGL(nvfp4_quantize_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, x,
                       groups, act_scale, out);
    return hipGetLastError();
}

}  // namespace moe

// Internal interface between the grouped-expert dispatcher (ffn.hip) and its
// two kernel families: streaming GEMV kernels for few rows per expert
// (ffn_gemv.hip) and MFMA grouped GEMM kernels for many (ffn_gemm.hip).
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// Device-side view of one projection of a bank.
struct ProjDev {
    const uint16_t* w;        // bf16 [E][out][in]
    const int32_t* qweight;   // awq  [E][in][out/8]
    const int32_t* qzeros;    // awq  [E][in/32][out/8]
    const uint16_t* scales;   // awq  [E][in/32][out] fp16
    const uint8_t* codes;     // fp8  [E][out][in] E4M3; nvfp4 [E][out][in/2] E2M1 pairs
    const float* bscales;     // fp8  [E][out/128][in/128]
    const uint8_t* gscales;   // nvfp4 [E][out][in/16] E4M3
    const float* wglobal;     // nvfp4 [E]
    float act;                // nvfp4: global scale of the projection's input
};

struct GroupedArgs {
    const uint16_t* x;          // [T][H] bf16
    int T, k, H, F, E, P;       // P = T*k rows
    int awq;                    // 1: AWQ g32, 0: bf16 or fp8
    int fp8;                    // 1: FP8 E4M3 with 128 x 128 block scales
    int nvfp4;                  // 1: NVFP4 W4A4 (x already quantised)
    const int32_t* offsets;     // [E+1] or nullptr (identity: E == 1, row r = token r)
    const int32_t* sorted_pair; // [P] or nullptr
    ProjDev gate, up, down;
    int out_f32;
    void* rows;                 // [P][H]
};

// GEMV family: gate/up partial sums [KS][P][2F] fp32 in `part`, then the down
// projection (whose prologue finishes SwiGLU) writes `rows`.
int gemv_ksplit(const GroupedArgs& a);
size_t gemv_ws_bytes(int P, int H, int F, int awq);
hipError_t launch_gemv(const GroupedArgs& a, void* ws, hipStream_t s);

// MFMA family: h [P][F] bf16 in the workspace, then rows.
size_t gemm_ws_bytes(int P, int F, int E);
hipError_t launch_gemm(const GroupedArgs& a, void* ws, hipStream_t s);

// Dense fp32 GEMM on the same kernels (used by the router's screening pass).
size_t dense_gemm_ws_bytes(int M);
hipError_t launch_dense_gemm_f32(const uint16_t* A, int M, int K, const uint16_t* B, int N, float* C,
                                 void* ws, hipStream_t s);

// Find the expert of work slot `slot` among the non-empty experts of
// offsets[0..E] (slot-th non-empty expert in index order).  Block-wide; every
// thread gets the same answer.  Returns -1 when there is no such expert.
__device__ __forceinline__ int slot_expert(const int32_t* offsets, int E, int slot, int* r0,
                                           int* r1) {
    __shared__ unsigned long long s_mask[16];
    __shared__ int s_e, s_r0, s_r1;
    const int tid = threadIdx.x;
    // ballots from complete waves only (a partial wave would see a partial mask)
    const int lane = tid % kWave, wave = tid / kWave, nfull = blockDim.x / kWave;
    if (wave < nfull) {
        for (int chunk = wave; chunk < 16; chunk += nfull) {
            const int e = chunk * kWave + lane;
            const bool ne = e < E && offsets[e + 1] > offsets[e];
            const unsigned long long m = __ballot(ne);
            if (lane == 0) s_mask[chunk] = m;
        }
    }
    __syncthreads();
    if (tid == 0) {
        int found = -1, left = slot;
        for (int chunk = 0; chunk < 16 && found < 0; ++chunk) {
            unsigned long long m = s_mask[chunk];
            const int c = __popcll(m);
            if (left < c) {
                for (int i = 0; i < left; ++i) m &= m - 1;  // drop lowest set bits
                found = chunk * kWave + __ffsll((long long)m) - 1;
            } else {
                left -= c;
            }
        }
        s_e = found;
        s_r0 = found >= 0 ? offsets[found] : 0;
        s_r1 = found >= 0 ? offsets[found + 1] : 0;
    }
    __syncthreads();
    *r0 = s_r0;
    *r1 = s_r1;
    return s_e;
}

}  // namespace moe

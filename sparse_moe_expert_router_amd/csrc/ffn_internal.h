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
    const int4* slots;          // GEMV work slots: (expert, first row, end row), expert -1 = none
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

// Expert and rows of GEMV work slot `slot` (workgroup index along x): one
// uniform 16-byte load from the slot table built for the call.  Returns -1
// for a slot past the last non-empty expert.
__device__ __forceinline__ int slot_expert(const int4* slots, int slot, int* r0, int* r1) {
    const int4 t = slots[slot];
    *r0 = t.y;
    *r1 = t.z;
    return t.x;
}

}  // namespace moe

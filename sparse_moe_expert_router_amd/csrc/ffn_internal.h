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
    const int32_t* pair_expert; // [P] expert of pair p, rows indexed by pair (offsets == nullptr), or nullptr
    ProjDev gate, up, down;
    int out_f32;
    void* rows;                 // [P][H]
};

// GEMV family: gate/up partial sums [KS][P][2F] fp32 in `part`, then the down
// projection (whose prologue finishes SwiGLU) writes `rows`.
int gemv_ksplit(const GroupedArgs& a);
size_t gemv_ws_bytes(int P, int H, int F, int awq, int E);
hipError_t launch_gemv(const GroupedArgs& a, void* ws, hipStream_t s);

// MFMA family: h [P][F] bf16 in the workspace, then rows.
size_t gemm_ws_bytes(int P, int F, int E);
hipError_t launch_gemm(const GroupedArgs& a, void* ws, hipStream_t s);

// Tile table of a grouped GEMM (tiles[0] = count, then (expert, first row)
// pairs, ceil(rows / BM) tiles per expert); tiles_bytes(P, E) bounds its size
// for any BM >= 64.
size_t tiles_bytes(int P, int E);
void launch_tile_table(const int32_t* offsets, int E, int P, int BM, int32_t* tiles, hipStream_t s);

// Workgroup b runs on XCD b % 8.  The grid is an upper bound on the work (the
// tile count is only known on the device); the `total` real work items are
// split into 8 contiguous ranges, XCD x taking range x with its lowest-numbered
// workgroups, so every XCD gets an equal share and the surplus workgroups of
// every XCD exit.  Returns -1 for a surplus workgroup.  Needs gridDim a
// multiple of 8 and at least total rounded up to a multiple of 8.
constexpr int kXcd = 8;
__device__ __forceinline__ int xcd_remap(int b, int total) {
    const int q = (total + kXcd - 1) / kXcd;
    const int x = b % kXcd, i = b / kXcd;
    if (i >= q) return -1;
    const int l = x * q + i;
    return l < total ? l : -1;
}

// Grouped GEMM on AWQ g32 codes stored output-major (ffn_gemm_om.hip): h [P][F]
// bf16 in the workspace after the tile table, then rows.
size_t om_gemm_ws_bytes(int P, int F, int E);
hipError_t launch_om_gemm(const GroupedArgs& a, void* ws, hipStream_t s);

// Streaming GEMV on AWQ g32 codes stored output-major (ffn_gemv_om.hip): the
// slot table, then h [P][F] bf16 in the workspace, then rows.
bool om_gemv_supported(int H, int F);
size_t om_gemv_ws_bytes(int P, int F);
hipError_t launch_om_gemv(const GroupedArgs& a, void* ws, hipStream_t s);

// h = bf16(silu(sum_ks gate) * sum_ks up) of fp32 partial sums
// part[KS][P][2F] (splits added in order), as bf16 pairs [P][F/2] (ffn_gemv.hip).
hipError_t launch_swiglu_reduce(const float* part, int KS, int P, int F, uint32_t* h, hipStream_t s);

// A one-expert bf16 call of at most 16 tokens (the shared expert at decode):
// split-K MFMA GEMM (ffn_skinny.hip); workspace: partial sums, then h.
bool skinny_supported(int T, int H, int F);
size_t skinny_ws_bytes(int T, int H, int F);
hipError_t launch_skinny(const GroupedArgs& a, void* ws, hipStream_t s);

// Slot table of a grouped GEMV call (ffn_gemv.hip) into `tab` (min(P, E)
// entries); returns tab.
int4* launch_slot_table(const int32_t* offsets, int E, int P, int4* tab, hipStream_t s);

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

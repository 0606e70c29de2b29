// Host-side launchers of the libmoe kernels (internal; the ABI is include/moe.h).
// Each launcher enqueues on `s` and returns the launch status.  Shapes are
// validated by the caller (api.cpp) before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---- routing (route.hip)
hipError_t launch_exact_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E,
                               float* logits, hipStream_t s);
hipError_t launch_topk(const float* logits, int T, int E, int k, int extra, int32_t* idx,
                       float* topk_logit, float* gate, hipStream_t s);
// top-k followed by the permutation, one workgroup (when topk_permute_fits);
// `slots` (nullable, min(T*k, E) entries) also receives the GEMV slot table
bool topk_permute_fits(int T, int k, int E);
hipError_t launch_topk_permute(const float* logits, int T, int E, int k, int32_t* idx, float* topk_logit,
                               float* gate, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_to_row,
                               int4* slots, hipStream_t s);
size_t route_filter_ws_bytes(int T, int E, int H);
hipError_t launch_route_filter(const uint16_t* x, const uint16_t* wr, int T, int H, int E, int k,
                               int extra, int32_t* idx, float* topk_logit, float* gate, void* ws,
                               hipStream_t s);

// ---- permutation (permute.hip)
size_t permute_ws_bytes(int T, int k, int E);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_to_row, void* ws, hipStream_t s);

// ---- grouped experts (ffn_gemv.hip, ffn_gemm.hip)
struct FfnArgs {
    const uint16_t* x;            // [T][H] bf16
    int T, k, H, F, E;
    const moe_experts* ex;        // host struct of device pointers
    const int32_t* offsets;       // [E+1], or nullptr (identity, E == 1)
    const int32_t* sorted_pair;   // [T*k], or nullptr
    int out_f32;                  // 1: rows are fp32, else bf16
    void* rows;                   // [T*k][H]
    const int4* slots = nullptr;  // GEMV slot table already built (see launch_topk_permute), or nullptr
    // [T*k] expert of each (token, slot) pair, with offsets == nullptr: rows
    // are indexed by pair (row p = pair p), no permutation (see pair_mode_fits)
    const int32_t* pair_expert = nullptr;
};
size_t ffn_ws_bytes(int T, int k, int E, int H, int F, int fmt);
// whether a grouped call of P rows over E experts runs the streaming GEMV
// kernels (which read a slot table) rather than an MFMA GEMM
bool ffn_takes_gemv(int P, int E, int H, int F, int fmt);
// whether a call of T tokens x k slots over E experts of format fmt can take
// its rows by pair (FfnArgs::pair_expert): the output-major streaming GEMV,
// at most kPairModeMaxT tokens and kPairModeMaxP pairs
constexpr int kPairModeMaxT = 256, kPairModeMaxP = 1024;
bool pair_mode_fits(int T, int k, int E, int H, int F, int fmt);
// hidden and inter sizes the output-major AWQ GEMM takes
bool om_gemm_supported(int H, int F);
hipError_t launch_awq_to_om(const int32_t* src, int32_t* dst, int E, int K, int N, hipStream_t s);

// ---- NVFP4 activation quantisation (quant.hip)
hipError_t launch_nvfp4_quantize(const uint16_t* x, int T, int n, float act_scale, uint16_t* out,
                                 hipStream_t s);
hipError_t launch_ffn(const FfnArgs& a, void* ws, hipStream_t s);

// ---- combine (combine.hip); pair_to_row == nullptr: row of pair p is p
hipError_t launch_combine(const void* rows, int rows_f32, const int32_t* pair_to_row,
                          const float* gate, int T, int k, int H, const uint16_t* shared,
                          const float* shared_scale, uint16_t* y, hipStream_t s);

// ---- Refill-RMS, keep policies, pruning (refill.hip, slice.hip)
size_t refill_ws_bytes(int T, int k);
hipError_t launch_refill_score(const float* rows, const int32_t* offsets, const int32_t* sorted_pair,
                               const int32_t* pair_to_row, const float* tl,
                               const uint8_t* valid, int T, int k, int H, int E, float* stat_sum,
                               uint32_t* stat_count, void* ws, hipStream_t s);
hipError_t launch_refill_finalize(const float* stat_sum, const uint32_t* stat_count, int E, int H,
                                  int keep, float* score, uint8_t* mask, int32_t* keep_idx,
                                  hipStream_t s);
hipError_t launch_router_norm_keep(const uint16_t* wr, int E, int H, int keep, float* norm,
                                   int32_t* keep_idx, hipStream_t s);
hipError_t launch_gather_slabs(const int32_t* keep_idx, int n_keep, int src_n, const void* src, void* dst,
                               size_t slab_bytes, hipStream_t s);

}  // namespace moe

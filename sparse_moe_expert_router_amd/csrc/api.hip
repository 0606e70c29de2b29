// C ABI of libmoe (declared in include/moe.h): host-side argument validation,
// workspace accounting and dispatch to the kernel launchers.  Nothing is
// enqueued unless every check passes.
#include <stdint.h>

#include "kernels.h"
#include "moe.h"

namespace {

thread_local int32_t g_last_hip = 0;

moe_status hip_status(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip = (int32_t)e;
        return MOE_ERR_HIP;
    }
    return MOE_OK;
}

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p % 16) == 0; }

constexpr int kMaxE = 1024;

// Screened routing (approximate MFMA logits + exact recompute of candidates)
// for batches of at least kFilterMinT tokens and E a multiple of 256;
// otherwise every logit is computed exactly.
constexpr int kFilterMinT = 64;
bool route_filtered(int T, int H, int E) { return T >= kFilterMinT && E % 256 == 0 && H % 32 == 0; }

size_t route_ws(int T, int E, int H) {
    if (route_filtered(T, H, E)) return moe::route_filter_ws_bytes(T, E, H);
    return (size_t)T * E * sizeof(float);
}

bool proj_ok(const moe_proj& p, int fmt, int in_dim, int out_dim, int E, moe_status* st) {
    if (p.fmt != fmt || p.in_dim != in_dim || p.out_dim != out_dim) {
        *st = MOE_ERR_SHAPE;
        return false;
    }
    if (fmt == MOE_W_BF16) {
        if (!p.w) { *st = MOE_ERR_NULL; return false; }
        if (!aligned16(p.w)) { *st = MOE_ERR_UNSUPPORTED; return false; }
    } else if (fmt == MOE_W_AWQ_G32) {
        if (!p.qweight || !p.qzeros || !p.scales) { *st = MOE_ERR_NULL; return false; }
        if (in_dim % 32 || out_dim % 32) { *st = MOE_ERR_UNSUPPORTED; return false; }
        if (!aligned16(p.qweight) || !aligned16(p.scales) || ((uintptr_t)p.qzeros % 4)) {
            *st = MOE_ERR_UNSUPPORTED;
            return false;
        }
    } else if (fmt == MOE_W_NVFP4) {
        if (!p.codes || !p.group_scales || !p.global_scale) { *st = MOE_ERR_NULL; return false; }
        if (in_dim % 32 || out_dim % 32) { *st = MOE_ERR_UNSUPPORTED; return false; }
        if (!(p.act_scale > 0.0f) || !(p.act_scale < 3.0e38f)) { *st = MOE_ERR_SHAPE; return false; }
        if (!aligned16(p.codes) || ((uintptr_t)p.group_scales % 2) || ((uintptr_t)p.global_scale % 4)) {
            *st = MOE_ERR_UNSUPPORTED;
            return false;
        }
    } else if (fmt == MOE_W_FP8_BLOCK) {
        if (!p.codes || !p.block_scales) { *st = MOE_ERR_NULL; return false; }
        if (in_dim % 128 || out_dim % 128) { *st = MOE_ERR_UNSUPPORTED; return false; }
        if (!aligned16(p.codes) || ((uintptr_t)p.block_scales % 4)) {
            *st = MOE_ERR_UNSUPPORTED;
            return false;
        }
    } else {
        *st = MOE_ERR_UNSUPPORTED;
        return false;
    }
    (void)E;
    return true;
}

bool bank_ok(const moe_experts* ex, moe_status* st) {
    if (!ex) { *st = MOE_ERR_NULL; return false; }
    const int E = ex->num_experts, H = ex->hidden, F = ex->inter;
    if (E < 1 || H < 1 || F < 1) { *st = MOE_ERR_SHAPE; return false; }
    if (E > kMaxE || H % 64 || F % 32 || H > 16384 || F > 2048) { *st = MOE_ERR_UNSUPPORTED; return false; }
    const int fmt = ex->gate.fmt;
    if (!(proj_ok(ex->gate, fmt, H, F, E, st) && proj_ok(ex->up, fmt, H, F, E, st) &&
          proj_ok(ex->down, fmt, F, H, E, st)))
        return false;
    if (fmt == MOE_W_NVFP4 && ex->gate.act_scale != ex->up.act_scale) { *st = MOE_ERR_SHAPE; return false; }
    return true;
}

// Workspace of moe_route_permute: the two calls run one after the other on
// one stream, so they share it.
size_t route_permute_ws(int T, int k, int E, int H) {
    const size_t a = route_ws(T, E, H), b = moe::permute_ws_bytes(T, k, E);
    return a > b ? a : b;
}

}  // namespace

extern "C" {

moe_status moe_route(const uint16_t* x, const uint16_t* w_router, int32_t T, int32_t H, int32_t E,
                     int32_t k, int32_t extra, int32_t* topk_idx, float* topk_logit,
                     float* topk_gate, float* logits, void* ws, size_t ws_bytes, void* stream) {
    if (T < 0 || H < 1 || E < 1 || k < 1 || extra < 0 || extra > 1 || k + extra > E)
        return MOE_ERR_SHAPE;
    if (E > kMaxE || H % 8 || k + extra > 64) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !topk_idx) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!logits && route_filtered(T, H, E)) {
        if (ws_bytes < route_ws(T, E, H)) return MOE_ERR_WORKSPACE;
        if (!ws) return MOE_ERR_NULL;
        if (!aligned16(ws)) return MOE_ERR_UNSUPPORTED;
        return hip_status(moe::launch_route_filter(x, w_router, T, H, E, k, extra, topk_idx,
                                                   topk_logit, topk_gate, ws, s));
    }
    float* lbuf = logits;
    if (!lbuf) {
        if (ws_bytes < route_ws(T, E, H)) return MOE_ERR_WORKSPACE;
        if (!ws) return MOE_ERR_NULL;
        lbuf = static_cast<float*>(ws);
    }
    moe_status st = hip_status(moe::launch_exact_logits(x, w_router, T, H, E, lbuf, s));
    if (st != MOE_OK) return st;
    return hip_status(moe::launch_topk(lbuf, T, E, k, extra, topk_idx, topk_logit, topk_gate, s));
}

moe_status moe_permute(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                       int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_to_row,
                       void* ws, size_t ws_bytes, void* stream) {
    if (T < 0 || k < 1 || E < 1) return MOE_ERR_SHAPE;
    if (E > kMaxE || (int64_t)T * k > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!topk_idx || !expert_offsets || !sorted_pair || !pair_to_row) return MOE_ERR_NULL;
    const size_t need = moe::permute_ws_bytes(T, k, E);
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (need && !ws) return MOE_ERR_NULL;
    return hip_status(moe::launch_permute(topk_idx, T, k, E, expert_offsets, sorted_pair,
                                          pair_to_row, ws, static_cast<hipStream_t>(stream)));
}

moe_status moe_route_permute(const uint16_t* x, const uint16_t* w_router, int32_t T, int32_t H, int32_t E,
                             int32_t k, int32_t* topk_idx, float* topk_logit, float* topk_gate,
                             int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_to_row, void* ws,
                             size_t ws_bytes, void* stream) {
    if (T < 0 || H < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_SHAPE;
    if (E > kMaxE || H % 8 || k > 64 || (int64_t)T * k > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !topk_idx || !expert_offsets || !sorted_pair || !pair_to_row) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_UNSUPPORTED;
    if (ws_bytes < route_permute_ws(T, k, E, H)) return MOE_ERR_WORKSPACE;
    if (!ws) return MOE_ERR_NULL;
    if (!aligned16(ws)) return MOE_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!route_filtered(T, H, E) && moe::topk_permute_fits(T, k, E)) {
        float* lbuf = static_cast<float*>(ws);
        moe_status st = hip_status(moe::launch_exact_logits(x, w_router, T, H, E, lbuf, s));
        if (st != MOE_OK) return st;
        return hip_status(moe::launch_topk_permute(lbuf, T, E, k, topk_idx, topk_logit, topk_gate,
                                                   expert_offsets, sorted_pair, pair_to_row, s));
    }
    moe_status st = moe_route(x, w_router, T, H, E, k, 0, topk_idx, topk_logit, topk_gate, nullptr, ws,
                              ws_bytes, stream);
    if (st != MOE_OK) return st;
    return moe_permute(topk_idx, T, k, E, expert_offsets, sorted_pair, pair_to_row, ws, ws_bytes, stream);
}

moe_status moe_grouped_ffn(const uint16_t* x, int32_t T, int32_t k, const moe_experts* ex,
                           const int32_t* expert_offsets, const int32_t* sorted_pair,
                           int32_t out_dtype, void* rows, void* ws, size_t ws_bytes,
                           void* stream) {
    moe_status st = MOE_OK;
    if (T < 0 || k < 1) return MOE_ERR_SHAPE;
    if (!bank_ok(ex, &st)) return st;
    if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32) return MOE_ERR_UNSUPPORTED;
    const bool identity = expert_offsets == nullptr && sorted_pair == nullptr;
    if (!identity && (expert_offsets == nullptr || sorted_pair == nullptr)) return MOE_ERR_NULL;
    if (identity && (ex->num_experts != 1 || k != 1)) return MOE_ERR_SHAPE;
    if ((int64_t)T * k > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !rows) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(rows)) return MOE_ERR_UNSUPPORTED;
    const int E = ex->num_experts, H = ex->hidden, F = ex->inter;
    const size_t need = moe::ffn_ws_bytes(T, k, E, H, F, ex->gate.fmt == MOE_W_NVFP4);
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (need && !ws) return MOE_ERR_NULL;
    if (!aligned16(ws)) return MOE_ERR_UNSUPPORTED;
    moe::FfnArgs f;
    f.x = x;
    f.T = T;
    f.k = k;
    f.H = H;
    f.F = F;
    f.E = E;
    f.ex = ex;
    f.offsets = expert_offsets;
    f.sorted_pair = sorted_pair;
    f.out_f32 = out_dtype == MOE_OUT_F32;
    f.rows = rows;
    return hip_status(moe::launch_ffn(f, ws, static_cast<hipStream_t>(stream)));
}

moe_status moe_combine(const void* rows, int32_t rows_dtype, const int32_t* pair_to_row,
                       const float* topk_gate, int32_t T, int32_t k, int32_t H,
                       const uint16_t* shared, const float* shared_scale, uint16_t* y,
                       void* stream) {
    if (T < 0 || k < 1 || H < 1) return MOE_ERR_SHAPE;
    if (rows_dtype != MOE_OUT_BF16 && rows_dtype != MOE_OUT_F32) return MOE_ERR_UNSUPPORTED;
    if (H % 8) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!rows || !pair_to_row || !topk_gate || !y) return MOE_ERR_NULL;
    if (!aligned16(rows) || !aligned16(shared) || !aligned16(y)) return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_combine(rows, rows_dtype == MOE_OUT_F32, pair_to_row, topk_gate, T,
                                          k, H, shared, shared_scale, y,
                                          static_cast<hipStream_t>(stream)));
}

moe_status moe_refill_score(const float* rows, const int32_t* expert_offsets,
                            const int32_t* sorted_pair, const int32_t* pair_to_row,
                            const int32_t* topk_idx, const float* topk_logit,
                            const uint8_t* token_valid, int32_t T, int32_t k, int32_t H,
                            int32_t E, float* stat_sum, uint32_t* stat_count, void* ws,
                            size_t ws_bytes, void* stream) {
    if (T < 0 || k < 1 || H < 1 || E < k + 1) return MOE_ERR_SHAPE;
    if (E > kMaxE || k + 1 > 32) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!rows || !expert_offsets || !sorted_pair || !pair_to_row || !topk_logit || !stat_sum ||
        !stat_count)
        return MOE_ERR_NULL;
    if (ws_bytes < moe::refill_ws_bytes(T, k)) return MOE_ERR_WORKSPACE;
    if (!ws) return MOE_ERR_NULL;
    return hip_status(moe::launch_refill_score(rows, expert_offsets, sorted_pair, pair_to_row,
                                               topk_idx, topk_logit, token_valid, T, k, H, E,
                                               stat_sum, stat_count, ws,
                                               static_cast<hipStream_t>(stream)));
}

moe_status moe_refill_finalize(const float* stat_sum, const uint32_t* stat_count, int32_t E,
                               int32_t H, int32_t keep, float* score, uint8_t* keep_mask,
                               int32_t* keep_idx, void* stream) {
    if (E < 1 || H < 1 || keep < 0 || keep > E) return MOE_ERR_SHAPE;
    if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
    if (!stat_sum || !stat_count || !score || !keep_mask || (keep > 0 && !keep_idx))
        return MOE_ERR_NULL;
    return hip_status(moe::launch_refill_finalize(stat_sum, stat_count, E, H, keep, score, keep_mask,
                                                  keep_idx, static_cast<hipStream_t>(stream)));
}

moe_status moe_prune_slice(const int32_t* keep_idx, int32_t n_keep, const uint16_t* w_router_src,
                           uint16_t* w_router_dst, int32_t H, const moe_experts* src,
                           const moe_experts* dst, void* stream) {
    moe_status st = MOE_OK;
    if (n_keep < 0 || H < 1) return MOE_ERR_SHAPE;
    if (!src || !dst) return MOE_ERR_NULL;
    if (!bank_ok(src, &st) || !bank_ok(dst, &st)) return st;
    if (dst->num_experts != n_keep || src->hidden != dst->hidden || src->inter != dst->inter ||
        src->gate.fmt != dst->gate.fmt || src->hidden != H || n_keep > src->num_experts)
        return MOE_ERR_SHAPE;
    if ((w_router_src == nullptr) != (w_router_dst == nullptr)) return MOE_ERR_NULL;
    if (n_keep == 0) return MOE_OK;
    if (!keep_idx) return MOE_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int F = src->inter;
    if (w_router_src) {
        st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, w_router_src, w_router_dst,
                                                 (size_t)H * sizeof(uint16_t), s));
        if (st != MOE_OK) return st;
    }
    const moe_proj* sp[3] = {&src->gate, &src->up, &src->down};
    const moe_proj* dp[3] = {&dst->gate, &dst->up, &dst->down};
    for (int m = 0; m < 3; ++m) {
        const size_t in = sp[m]->in_dim, out = sp[m]->out_dim;
        (void)F;
        if (sp[m]->fmt == MOE_W_BF16) {
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, sp[m]->w, const_cast<uint16_t*>(dp[m]->w),
                                                     in * out * sizeof(uint16_t), s));
            if (st != MOE_OK) return st;
        } else if (sp[m]->fmt == MOE_W_NVFP4) {
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, sp[m]->codes,
                                                     const_cast<uint8_t*>(dp[m]->codes), in / 2 * out, s));
            if (st != MOE_OK) return st;
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, sp[m]->group_scales,
                                                     const_cast<uint8_t*>(dp[m]->group_scales), in / 16 * out, s));
            if (st != MOE_OK) return st;
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, sp[m]->global_scale,
                                                     const_cast<float*>(dp[m]->global_scale), sizeof(float), s));
            if (st != MOE_OK) return st;
        } else if (sp[m]->fmt == MOE_W_FP8_BLOCK) {
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, sp[m]->codes,
                                                     const_cast<uint8_t*>(dp[m]->codes), in * out, s));
            if (st != MOE_OK) return st;
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, sp[m]->block_scales,
                                                     const_cast<float*>(dp[m]->block_scales),
                                                     (in / 128) * (out / 128) * sizeof(float), s));
            if (st != MOE_OK) return st;
        } else {
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, sp[m]->qweight,
                                                     const_cast<int32_t*>(dp[m]->qweight),
                                                     in * (out / 8) * sizeof(int32_t), s));
            if (st != MOE_OK) return st;
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, sp[m]->qzeros,
                                                     const_cast<int32_t*>(dp[m]->qzeros),
                                                     (in / 32) * (out / 8) * sizeof(int32_t), s));
            if (st != MOE_OK) return st;
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, sp[m]->scales,
                                                     const_cast<uint16_t*>(dp[m]->scales),
                                                     (in / 32) * out * sizeof(uint16_t), s));
            if (st != MOE_OK) return st;
        }
    }
    return MOE_OK;
}

moe_status moe_router_norm_keep(const uint16_t* w_router, int32_t E, int32_t H, int32_t keep,
                                float* norm, int32_t* keep_idx, void* stream) {
    if (E < 1 || H < 1 || keep < 0 || keep > E) return MOE_ERR_SHAPE;
    if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
    if (!w_router || !norm || (keep > 0 && !keep_idx)) return MOE_ERR_NULL;
    return hip_status(moe::launch_router_norm_keep(w_router, E, H, keep, norm, keep_idx,
                                                   static_cast<hipStream_t>(stream)));
}

moe_status moe_nvfp4_quantize(const uint16_t* x, int32_t T, int32_t n, float act_scale, uint16_t* out,
                              void* stream) {
    if (T < 0 || n < 1) return MOE_ERR_SHAPE;
    if (n % 16) return MOE_ERR_UNSUPPORTED;
    if (!(act_scale > 0.0f) || !(act_scale < 3.0e38f)) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!x || !out) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(out)) return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_nvfp4_quantize(x, T, n, act_scale, out, static_cast<hipStream_t>(stream)));
}

size_t moe_workspace_bytes(int32_t op, int32_t T, int32_t k, int32_t E, int32_t H, int32_t F) {
    if (T <= 0 || k <= 0 || E <= 0) return 0;
    switch (op) {
        case MOE_OP_ROUTE: return route_ws(T, E, H);
        case MOE_OP_PERMUTE: return moe::permute_ws_bytes(T, k, E);
        case MOE_OP_GROUPED_FFN: return moe::ffn_ws_bytes(T, k, E, H, F, false);
        case MOE_OP_GROUPED_FFN_NVFP4: return moe::ffn_ws_bytes(T, k, E, H, F, true);
        case MOE_OP_ROUTE_PERMUTE: return route_permute_ws(T, k, E, H);
        case MOE_OP_REFILL_SCORE: return moe::refill_ws_bytes(T, k);
        default: return 0;
    }
}

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "inconsistent sizes";
        case MOE_ERR_UNSUPPORTED: return "unsupported size, format or alignment";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "a HIP call failed";
        default: return "unknown status";
    }
}

int32_t moe_last_hip_error(void) { return g_last_hip; }

}  // extern "C"

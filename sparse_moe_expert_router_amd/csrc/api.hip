// C ABI of libmoe (declared in include/moe.h): host-side argument validation,
// workspace accounting and dispatch to the kernel launchers.  Nothing is
// enqueued unless every check passes.
#include <stdint.h>

#include <mutex>

#include "kernels.h"
#include "moe.h"

// Device scratch of moe_grouped_ffn_noalloc (16 MiB per GPU; see below).
static __device__ __align__(256) unsigned char scratch[(size_t)16 << 20];

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
    } else if (fmt == MOE_W_AWQ_G32 || fmt == MOE_W_AWQ_G32_OM) {
        if (!p.qweight || !p.qzeros || !p.scales) { *st = MOE_ERR_NULL; return false; }
        if (in_dim % 32 || out_dim % 32) { *st = MOE_ERR_UNSUPPORTED; return false; }
        if (fmt == MOE_W_AWQ_G32_OM &&
            (in_dim % 64 || out_dim % 64 || (uint64_t)E * in_dim * out_dim / 2 >= (1ull << 32))) {
            *st = MOE_ERR_UNSUPPORTED;
            return false;
        }
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
    if (fmt == MOE_W_AWQ_G32_OM && !moe::om_gemm_supported(H, F)) { *st = MOE_ERR_UNSUPPORTED; return false; }
    return true;
}

// Validation shared by moe_grouped_ffn and moe_grouped_ffn_noalloc: fills the
// launch arguments and the scratch bytes the call needs.  T == 0 passes.
moe_status ffn_prepare(const uint16_t* x, int32_t T, int32_t k, const moe_experts* ex,
                       const int32_t* expert_offsets, const int32_t* sorted_pair, int32_t out_dtype,
                       void* rows, moe::FfnArgs* f, size_t* need) {
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
    if (ex->gate.fmt == MOE_W_AWQ_G32_OM &&
        ((uint64_t)T * H * 2 >= (1ull << 32) || (uint64_t)T * k * F * 2 >= (1ull << 32)))
        return MOE_ERR_UNSUPPORTED;
    *need = moe::ffn_ws_bytes(T, k, E, H, F, ex->gate.fmt);
    f->x = x;
    f->T = T;
    f->k = k;
    f->H = H;
    f->F = F;
    f->E = E;
    f->ex = ex;
    f->offsets = expert_offsets;
    f->sorted_pair = sorted_pair;
    f->out_f32 = out_dtype == MOE_OUT_F32;
    f->rows = rows;
    return MOE_OK;
}

// Scratch of moe_grouped_ffn_noalloc: one array per GPU, resident for the life
// of the process.  Host code never uses the array's name as an address (on
// the host it is only a handle); each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = sizeof(scratch);

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status scratch_address(hipStream_t s, void** out) {
    int dev = -1;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return hip_status(e);
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return hip_status(e);
        if (!p) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// Workspace of moe_route_permute: the two calls run one after the other on
// one stream, so they share it.
size_t route_permute_ws(int T, int k, int E, int H) {
    const size_t a = route_ws(T, E, H), b = moe::permute_ws_bytes(T, k, E);
    return a > b ? a : b;
}

// ---- the whole layer in one call (moe_layer)

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace regions of moe_layer, in order; every offset is a multiple of 256.
struct LayerLayout {
    size_t idx, tl, gate, off, sp, p2r, slots, rows, srows, rp_ws, ffn_ws, sh_ws, total;
};

LayerLayout layer_layout(int T, int k, const moe_experts* ex, const moe_experts* sh) {
    const int E = ex->num_experts, H = ex->hidden, F = ex->inter;
    const size_t P = (size_t)T * k;
    LayerLayout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += align256(bytes);
        return at;
    };
    L.idx = take(P * 4);
    L.tl = take(P * 4);
    L.gate = take(P * 4);
    L.off = take(((size_t)E + 1) * 4);
    L.sp = take(P * 4);
    L.p2r = take(P * 4);
    L.slots = take(P * 16);
    L.rows = take(P * H * 2);
    L.srows = take(sh ? (size_t)T * H * 2 : 0);
    L.rp_ws = take(route_permute_ws(T, k, E, H));
    L.ffn_ws = take(moe::ffn_ws_bytes(T, k, E, H, F, ex->gate.fmt));
    L.sh_ws = take(sh ? moe::ffn_ws_bytes(T, 1, 1, H, sh->inter, sh->gate.fmt) : 0);
    L.total = o;
    return L;
}

// Fork and join events of the shared expert's side stream, one pair per
// thread and device (a call records and waits on them from its own thread).
struct SideEvents {
    hipEvent_t fork = nullptr, join = nullptr;
};
thread_local SideEvents t_side[kMaxDevices];

moe_status side_events(hipStream_t s, SideEvents** out) {
    int dev = -1;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    SideEvents& ev = t_side[dev];
    if (!ev.fork) {
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_status(e);
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
        hipEvent_t a = nullptr, b = nullptr;
        e = hipEventCreateWithFlags(&a, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&b, hipEventDisableTiming);
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) {
            if (a) (void)hipEventDestroy(a);
            if (b) (void)hipEventDestroy(b);
            return hip_status(e);
        }
        ev.fork = a;
        ev.join = b;
    }
    *out = &ev;
    return MOE_OK;
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
                                                   expert_offsets, sorted_pair, pair_to_row, nullptr, s));
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
    moe::FfnArgs f;
    size_t need = 0;
    moe_status st = ffn_prepare(x, T, k, ex, expert_offsets, sorted_pair, out_dtype, rows, &f, &need);
    if (st != MOE_OK || T == 0) return st;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (need && !ws) return MOE_ERR_NULL;
    if (!aligned16(ws)) return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_ffn(f, ws, static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_ffn_noalloc(const uint16_t* x, int32_t T, int32_t k, const moe_experts* ex,
                                   const int32_t* expert_offsets, const int32_t* sorted_pair,
                                   int32_t out_dtype, void* rows, void* stream) {
    moe::FfnArgs f;
    size_t need = 0;
    moe_status st = ffn_prepare(x, T, k, ex, expert_offsets, sorted_pair, out_dtype, rows, &f, &need);
    if (st != MOE_OK || T == 0) return st;
    if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    st = scratch_address(s, &ws);
    if (st != MOE_OK) return st;
    return hip_status(moe::launch_ffn(f, ws, s));
}

size_t moe_grouped_ffn_noalloc_max_bytes(void) { return kScratchBytes; }

size_t moe_layer_workspace_bytes(int32_t T, int32_t k, const moe_experts* experts, const moe_experts* shared) {
    moe_status st = MOE_OK;
    if (T <= 0 || k < 1 || !bank_ok(experts, &st) || (shared && !bank_ok(shared, &st))) return 0;
    return layer_layout(T, k, experts, shared).total;
}

moe_status moe_layer(const uint16_t* x, int32_t T, const uint16_t* w_router, int32_t k,
                     const moe_experts* experts, const moe_experts* shared, const float* shared_scale,
                     uint16_t* y, int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream,
                     void* side_stream, void* const* routed_events) {
    moe_status st = MOE_OK;
    if (T < 0 || k < 1) return MOE_ERR_SHAPE;
    if (!bank_ok(experts, &st)) return st;
    const int E = experts->num_experts, H = experts->hidden;
    if (k > E) return MOE_ERR_SHAPE;
    if (k > 64 || (int64_t)T * k > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
    if (shared) {
        if (!bank_ok(shared, &st)) return st;
        if (shared->num_experts != 1 || shared->hidden != H) return MOE_ERR_SHAPE;
    } else if (shared_scale) {
        return MOE_ERR_SHAPE;
    }
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !y) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(y)) return MOE_ERR_UNSUPPORTED;
    if (experts->gate.fmt == MOE_W_AWQ_G32_OM &&
        ((uint64_t)T * H * 2 >= (1ull << 32) || (uint64_t)T * k * experts->inter * 2 >= (1ull << 32)))
        return MOE_ERR_UNSUPPORTED;
    const LayerLayout L = layer_layout(T, k, experts, shared);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (!ws) return MOE_ERR_NULL;
    if (!aligned16(ws)) return MOE_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipStream_t side = static_cast<hipStream_t>(side_stream);
    SideEvents* ev = nullptr;
    if (shared && side) {
        if (side == s) return MOE_ERR_SHAPE;
        if ((st = side_events(s, &ev)) != MOE_OK) return st;
    }
    char* w = static_cast<char*>(ws);
    int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(w + L.idx);
    float* tl = reinterpret_cast<float*>(w + L.tl);
    float* gate = reinterpret_cast<float*>(w + L.gate);
    int32_t* off = reinterpret_cast<int32_t*>(w + L.off);
    int32_t* sp = reinterpret_cast<int32_t*>(w + L.sp);
    int32_t* p2r = reinterpret_cast<int32_t*>(w + L.p2r);
    int4* slots = reinterpret_cast<int4*>(w + L.slots);
    uint16_t* rows = reinterpret_cast<uint16_t*>(w + L.rows);
    uint16_t* srows = shared ? reinterpret_cast<uint16_t*>(w + L.srows) : nullptr;

    moe::FfnArgs sf{};
    if (shared) {
        sf.x = x; sf.T = T; sf.k = 1; sf.H = H; sf.F = shared->inter; sf.E = 1; sf.ex = shared;
        sf.offsets = nullptr; sf.sorted_pair = nullptr; sf.out_f32 = 0; sf.rows = srows;
    }
    // the shared expert needs only x: with a side stream it runs beside the
    // routing and the routed experts (fork here, join before the combine)
    if (ev) {
        if ((st = hip_status(hipEventRecord(ev->fork, s))) != MOE_OK) return st;
        if ((st = hip_status(hipStreamWaitEvent(side, ev->fork, 0))) != MOE_OK) return st;
        if ((st = hip_status(moe::launch_ffn(sf, w + L.sh_ws, side))) != MOE_OK) return st;
        if ((st = hip_status(hipEventRecord(ev->join, side))) != MOE_OK) return st;
    }
    // routing and permutation.  Few tokens on output-major codes: the
    // streaming kernels take their rows by (token, slot) pair, so the top-k
    // runs one wave per token and there is no permutation; otherwise the
    // single-workgroup selection permutes too, and writes the GEMV slot table
    // when the routed call streams
    const int P = T * k;
    const int fmt = experts->gate.fmt;
    const bool fused = !route_filtered(T, H, E) && moe::topk_permute_fits(T, k, E);
    const bool pairs = fused && moe::pair_mode_fits(T, k, E, H, experts->inter, fmt);
    const bool pre_slots = fused && !pairs && moe::ffn_takes_gemv(P, E, H, experts->inter, fmt);
    if (fused) {
        float* lbuf = reinterpret_cast<float*>(w + L.rp_ws);
        if ((st = hip_status(moe::launch_exact_logits(x, w_router, T, H, E, lbuf, s))) != MOE_OK) return st;
        if (pairs)
            st = hip_status(moe::launch_topk(lbuf, T, E, k, 0, idx, tl, gate, s));
        else
            st = hip_status(moe::launch_topk_permute(lbuf, T, E, k, idx, tl, gate, off, sp, p2r,
                                                     pre_slots ? slots : nullptr, s));
    } else {
        st = moe_route_permute(x, w_router, T, H, E, k, idx, tl, gate, off, sp, p2r, w + L.rp_ws,
                               route_permute_ws(T, k, E, H), stream);
    }
    if (st != MOE_OK) return st;
    // routed experts
    moe::FfnArgs f{};
    f.x = x; f.T = T; f.k = k; f.H = H; f.F = experts->inter; f.E = E; f.ex = experts;
    f.offsets = pairs ? nullptr : off; f.sorted_pair = pairs ? nullptr : sp; f.out_f32 = 0; f.rows = rows;
    f.slots = pre_slots ? slots : nullptr;
    f.pair_expert = pairs ? idx : nullptr;
    if (routed_events && routed_events[0] &&
        (st = hip_status(hipEventRecord(static_cast<hipEvent_t>(routed_events[0]), s))) != MOE_OK)
        return st;
    if ((st = hip_status(moe::launch_ffn(f, w + L.ffn_ws, s))) != MOE_OK) return st;
    if (routed_events && routed_events[1] &&
        (st = hip_status(hipEventRecord(static_cast<hipEvent_t>(routed_events[1]), s))) != MOE_OK)
        return st;
    if (shared && !ev && (st = hip_status(moe::launch_ffn(sf, w + L.sh_ws, s))) != MOE_OK) return st;
    if (ev && (st = hip_status(hipStreamWaitEvent(s, ev->join, 0))) != MOE_OK) return st;
    return hip_status(moe::launch_combine(rows, 0, pairs ? nullptr : p2r, gate, T, k, H, srows, shared_scale, y, s));
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
                            const float* topk_logit,
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
    if (!aligned16(ws)) return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_refill_score(rows, expert_offsets, sorted_pair, pair_to_row,
                                               topk_logit, token_valid, T, k, H, E,
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
        st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, src->num_experts, w_router_src, w_router_dst,
                                                 (size_t)H * sizeof(uint16_t), s));
        if (st != MOE_OK) return st;
    }
    const moe_proj* sp[3] = {&src->gate, &src->up, &src->down};
    const moe_proj* dp[3] = {&dst->gate, &dst->up, &dst->down};
    for (int m = 0; m < 3; ++m) {
        const size_t in = sp[m]->in_dim, out = sp[m]->out_dim;
        (void)F;
        if (sp[m]->fmt == MOE_W_BF16) {
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, src->num_experts, sp[m]->w, const_cast<uint16_t*>(dp[m]->w),
                                                     in * out * sizeof(uint16_t), s));
            if (st != MOE_OK) return st;
        } else if (sp[m]->fmt == MOE_W_NVFP4) {
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, src->num_experts, sp[m]->codes,
                                                     const_cast<uint8_t*>(dp[m]->codes), in / 2 * out, s));
            if (st != MOE_OK) return st;
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, src->num_experts, sp[m]->group_scales,
                                                     const_cast<uint8_t*>(dp[m]->group_scales), in / 16 * out, s));
            if (st != MOE_OK) return st;
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, src->num_experts, sp[m]->global_scale,
                                                     const_cast<float*>(dp[m]->global_scale), sizeof(float), s));
            if (st != MOE_OK) return st;
        } else if (sp[m]->fmt == MOE_W_FP8_BLOCK) {
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, src->num_experts, sp[m]->codes,
                                                     const_cast<uint8_t*>(dp[m]->codes), in * out, s));
            if (st != MOE_OK) return st;
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, src->num_experts, sp[m]->block_scales,
                                                     const_cast<float*>(dp[m]->block_scales),
                                                     (in / 128) * (out / 128) * sizeof(float), s));
            if (st != MOE_OK) return st;
        } else {
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, src->num_experts, sp[m]->qweight,
                                                     const_cast<int32_t*>(dp[m]->qweight),
                                                     in * (out / 8) * sizeof(int32_t), s));
            if (st != MOE_OK) return st;
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, src->num_experts, sp[m]->qzeros,
                                                     const_cast<int32_t*>(dp[m]->qzeros),
                                                     (in / 32) * (out / 8) * sizeof(int32_t), s));
            if (st != MOE_OK) return st;
            st = hip_status(moe::launch_gather_slabs(keep_idx, n_keep, src->num_experts, sp[m]->scales,
                                                     const_cast<uint16_t*>(dp[m]->scales),
                                                     (in / 32) * out * sizeof(uint16_t), s));
            if (st != MOE_OK) return st;
        }
    }
    return MOE_OK;
}

moe_status moe_awq_to_output_major(const moe_experts* src, const moe_experts* dst, void* stream) {
    moe_status st = MOE_OK;
    if (!src || !dst) return MOE_ERR_NULL;
    if (src->gate.fmt != MOE_W_AWQ_G32 || dst->gate.fmt != MOE_W_AWQ_G32_OM) return MOE_ERR_SHAPE;
    if (src->num_experts != dst->num_experts || src->hidden != dst->hidden || src->inter != dst->inter)
        return MOE_ERR_SHAPE;
    if (!bank_ok(src, &st) || !bank_ok(dst, &st)) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int E = src->num_experts;
    const moe_proj* sp[3] = {&src->gate, &src->up, &src->down};
    const moe_proj* dp[3] = {&dst->gate, &dst->up, &dst->down};
    for (int m = 0; m < 3; ++m) {
        const size_t I = sp[m]->in_dim, O = sp[m]->out_dim;
        const size_t qb = (size_t)E * I * O / 2;
        const char* sq = reinterpret_cast<const char*>(sp[m]->qweight);
        const char* dq = reinterpret_cast<const char*>(dp[m]->qweight);
        if (sq < dq + qb && dq < sq + qb) return MOE_ERR_SHAPE;  // overlapping codes
    }
    for (int m = 0; m < 3; ++m) {
        const int I = sp[m]->in_dim, O = sp[m]->out_dim;
        st = hip_status(moe::launch_awq_to_om(sp[m]->qweight, const_cast<int32_t*>(dp[m]->qweight), E, I, O, s));
        if (st != MOE_OK) return st;
        const size_t zb = (size_t)E * (I / 32) * (O / 8) * sizeof(int32_t);
        const size_t sb = (size_t)E * (I / 32) * O * sizeof(uint16_t);
        if (dp[m]->qzeros != sp[m]->qzeros) {
            st = hip_status(hipMemcpyAsync(const_cast<int32_t*>(dp[m]->qzeros), sp[m]->qzeros, zb,
                                           hipMemcpyDeviceToDevice, s));
            if (st != MOE_OK) return st;
        }
        if (dp[m]->scales != sp[m]->scales) {
            st = hip_status(hipMemcpyAsync(const_cast<uint16_t*>(dp[m]->scales), sp[m]->scales, sb,
                                           hipMemcpyDeviceToDevice, s));
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
        case MOE_OP_GROUPED_FFN: return moe::ffn_ws_bytes(T, k, E, H, F, MOE_W_AWQ_G32_OM);
        case MOE_OP_GROUPED_FFN_NVFP4: return moe::ffn_ws_bytes(T, k, E, H, F, MOE_W_NVFP4);
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

// Grouped-expert dispatcher: picks the weight-streaming GEMV kernels when an
// expert sees only a few rows (decode) and the MFMA grouped GEMM otherwise.
#include "ffn_internal.h"

namespace moe {

// Average rows per non-empty expert at or above which the MFMA path is used.
constexpr int kGemmMinRows = 32;

static bool use_gemm(int P, int E, int H, int F) {
    const int active = P < E ? P : E;
    if (active <= 0) return false;
    if (F % 128 != 0 || H % 256 != 0) return false;
    return P / active >= kGemmMinRows;
}

// Workspace for T*k rows, monotone in T: the GEMV path (taken below
// kGemmMinRows rows per expert) needs at most its size at that bound.
// An NVFP4 bank adds the quantised input rows [T][H] bf16 in front.
static size_t quant_x_bytes(int T, int H) { return ((size_t)T * H * sizeof(uint16_t) + 255) & ~(size_t)255; }

size_t ffn_ws_bytes(int T, int k, int E, int H, int F, bool nvfp4) {
    if (nvfp4) return quant_x_bytes(T, H) + ffn_ws_bytes(T, k, E, H, F, false);
    const long P = (long)T * k;
    // shapes the GEMM does not take stream every row through the GEMV
    const bool gemm_ok = F % 128 == 0 && H % 256 == 0;
    const long Pg = (gemm_ok && P >= (long)kGemmMinRows * E) ? (long)kGemmMinRows * E : P;
    const size_t g1 = gemv_ws_bytes((int)Pg, H, F, 1), g0 = gemv_ws_bytes((int)Pg, H, F, 0);
    size_t need = g1 > g0 ? g1 : g0;
    if (F % 128 == 0 && H % 256 == 0 && P >= (long)kGemmMinRows * E) {
        const size_t gm = gemm_ws_bytes((int)P, F, E);
        if (gm > need) need = gm;
    }
    return need;
}

hipError_t launch_ffn(const FfnArgs& f, void* ws, hipStream_t s) {
    GroupedArgs a{};
    a.x = f.x;
    a.T = f.T;
    a.k = f.k;
    a.H = f.H;
    a.F = f.F;
    a.E = f.E;
    a.P = f.T * f.k;
    a.awq = f.ex->gate.fmt == MOE_W_AWQ_G32;
    a.fp8 = f.ex->gate.fmt == MOE_W_FP8_BLOCK;
    a.nvfp4 = f.ex->gate.fmt == MOE_W_NVFP4;
    a.offsets = f.offsets;
    a.sorted_pair = f.sorted_pair;
    auto pj = [](const moe_proj& p) {
        ProjDev d;
        d.w = p.w;
        d.qweight = p.qweight;
        d.qzeros = p.qzeros;
        d.scales = p.scales;
        d.codes = p.codes;
        d.bscales = p.block_scales;
        d.gscales = p.group_scales;
        d.wglobal = p.global_scale;
        d.act = p.act_scale;
        return d;
    };
    a.gate = pj(f.ex->gate);
    a.up = pj(f.ex->up);
    a.down = pj(f.ex->down);
    a.out_f32 = f.out_f32;
    a.rows = f.rows;
    if (a.nvfp4) {
        // W4A4: the experts read the quantised input rows
        uint16_t* xq = static_cast<uint16_t*>(ws);
        const hipError_t err = launch_nvfp4_quantize(f.x, f.T, f.H, a.gate.act, xq, s);
        if (err != hipSuccess) return err;
        a.x = xq;
        ws = static_cast<char*>(ws) + quant_x_bytes(f.T, f.H);
    }
    if (use_gemm(a.P, a.offsets ? a.E : 1, a.H, a.F)) return launch_gemm(a, ws, s);
    return launch_gemv(a, ws, s);
}

}  // namespace moe

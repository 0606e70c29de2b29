/*
 * moe.h -- C ABI of the MI355X (gfx950) routed mixture-of-experts
 * feed-forward layer library (libmoe.so).
 *
 * The layer (Qwen3.8-Flash-Next architecture sheet, FFN / MoE entries): a
 * softmax router over E expert logits, the top-k experts per token with their
 * gates renormalised to sum to 1, routed SwiGLU experts (gate, up, down; no
 * bias, no clamp), one always-on shared expert, and the gate-weighted sum.
 * Routed experts are stored either in bf16 or in asymmetric AWQ W4A16 with
 * group size 32 along the input dimension, integer zero points and fp16 scales
 * in GEMM packing (Qwen3.8-Flash-Next-AWQ-g32 card, "Checkpoint").  Expert
 * pruning keeps a subset of experts by slicing router rows and expert tensors
 * (RAZOR E256of512 card, property table and "Selection and calibration"),
 * and the Refill-RMS pass scores experts to choose that subset (same card,
 * "Selection and calibration").
 *
 * Conventions for every call:
 *  - Every pointer argument is a DEVICE pointer unless its comment says host.
 *    bf16 and fp16 values are passed as their uint16_t bit patterns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    on it; nothing is waited for.  Device-side faults surface at the
 *    caller's next synchronisation.
 *  - All argument validation happens on the host before anything is enqueued.
 *    On any error nothing is enqueued and the status says why.  A failed
 *    launch returns MOE_ERR_HIP; moe_last_hip_error() then gives the
 *    hipError_t of the calling thread's last failed HIP call.
 *  - The library never allocates device memory (moe_grouped_ffn_noalloc's
 *    static array aside) and keeps no state between calls except cached
 *    device properties and, for moe_layer with a side stream, two HIP events
 *    per calling thread and device.  The caller owns every buffer, including
 *    the scratch workspace `ws` whose size comes from moe_workspace_bytes()
 *    or moe_layer_workspace_bytes().  Calls on different streams need
 *    distinct workspaces.
 *  - Results are deterministic: the same inputs give the same bits.
 *  - T = 0 is a valid no-op for every call.
 *
 * Layouts (row-major, all contiguous):
 *  x           [T][H]        bf16 hidden states (already normalised)
 *  w_router    [E][H]        bf16, one row per expert, no bias
 *  topk_idx    [T][k+extra]  int32 expert ids, rank order
 *  pair id     p = t*kk + slot for kk pairs per token (kk = k, or k+1 for
 *              Refill-RMS); "rows" are expert outputs in grouped order:
 *              row r holds the output of pair sorted_pair[r].
 *  bf16 experts: gate, up [E][F][H]; down [E][H][F]  (row per output feature)
 *  FP8 experts:  codes [E][O][I] uint8, OCP FP8 E4M3 (bias 7, max 448, no
 *                infinities, S.1111.111 = NaN); block_scales [E][O/128][I/128]
 *                fp32; w[e][o][i] = e4m3(codes[e][o][i]) * block_scales[e][o/128][i/128]
 *                (the optional FP8 draft of the AWQ-g32 card stores routed
 *                experts in E4M3 with explicit block scales; the 128 x 128
 *                block is this library's reading).  I and O multiples of 128.
 *  NVFP4 experts (W4A4; the NVFP4 release card's precision table: group
 *                16, FP8 block scales, FP32 global scales; the layouts and the
 *                activation recipe below are this library's reading):
 *                codes [E][O][I/2]: byte j holds inputs 2j (bits 0..3) and
 *                2j+1 (bits 4..7) as E2M1 (sign bit 3, exponent bits 2..1
 *                with bias 1, mantissa bit 0); group_scales [E][O][I/16] E4M3;
 *                global_scale [E] fp32:
 *                  w[e][o][i] = e2m1 * e4m3(group_scales[e][o][i/16]) * global_scale[e].
 *                Every input row of every projection is quantised the same
 *                way, per 16 consecutive inputs, all in fp32: with g =
 *                act_scale, the group's scale code is the E4M3 rounding
 *                (nearest, ties to even, saturating at 448) of amax / (6 g);
 *                with s its value, each input v becomes the E2M1 rounding
 *                (nearest, ties to even, saturating at 6) of v / (s g); the
 *                projection then sees e2m1 * s * g.  Gate and up share their
 *                input and must carry the same act_scale; the down
 *                projection's input (the SwiGLU product) is quantised with
 *                down.act_scale.  I and O multiples of 32.
 *  AWQ experts:  for a projection with input dim I and output dim O
 *                  qweight [E][I][O/8] int32, qzeros [E][I/32][O/8] int32,
 *                  scales [E][I/32][O] fp16;
 *                nibble j (bits 4j..4j+3) of word c holds column
 *                8c + {0,2,4,6,1,3,5,7}[j];  w[e][o][i] = (q - z) * s.
 *  AWQ experts, output-major codes (MOE_W_AWQ_G32_OM): the same codes,
 *                zeros and scales, with only the codes rearranged so that
 *                one word holds 8 consecutive inputs of one output column:
 *                  qweight [E][O][I/8] int32, nibble j of word w = code of
 *                  input 8w + j;  qzeros and scales as above.
 *                The bytes per expert are those of the AWQ layout.  This is
 *                the layout the MFMA path reads without restaging: one word
 *                is one lane's operand of a bf16 MFMA.  moe_awq_to_output_major
 *                converts an AWQ bank.  Requires I and O multiples of 64,
 *                hidden % 256 == 0 and inter % 128 == 0, and every tensor, x
 *                and the intermediate [T*k][inter] bf16 product below 4 GiB.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                    */
    MOE_ERR_SHAPE = 2,       /* sizes inconsistent (k > E, negative T, ...)    */
    MOE_ERR_UNSUPPORTED = 3, /* valid but not supported (E > 1024, H % 32, ...) */
    MOE_ERR_WORKSPACE = 4,   /* ws_bytes smaller than moe_workspace_bytes()   */
    MOE_ERR_HIP = 5          /* a HIP call failed; see moe_last_hip_error()   */
} moe_status;

typedef enum { MOE_W_BF16 = 0, MOE_W_AWQ_G32 = 1, MOE_W_FP8_BLOCK = 2, MOE_W_NVFP4 = 3,
               MOE_W_AWQ_G32_OM = 4 } moe_wfmt;
typedef enum { MOE_OUT_BF16 = 0, MOE_OUT_F32 = 1 } moe_dtype;

/* One projection of a bank of experts, input dim in_dim, output dim out_dim. */
typedef struct {
    int32_t fmt;              /* moe_wfmt                                     */
    int32_t in_dim, out_dim;
    const uint16_t *w;        /* BF16: [E][out][in]                           */
    const int32_t *qweight;   /* AWQ:  [E][in][out/8]                         */
    const int32_t *qzeros;    /* AWQ:  [E][in/32][out/8]                      */
    const uint16_t *scales;   /* AWQ:  [E][in/32][out] fp16                   */
    const uint8_t *codes;     /* FP8:  [E][out][in] E4M3 (OCP)                */
                              /* NVFP4: [E][out][in/2] two E2M1 codes a byte  */
    const float *block_scales;/* FP8:  [E][out/128][in/128] fp32              */
    const uint8_t *group_scales; /* NVFP4: [E][out][in/16] E4M3               */
    const float *global_scale;   /* NVFP4: [E] fp32 weight global scale       */
    float act_scale;             /* NVFP4: global scale of this projection's
                                    input activations (host value, > 0)       */
} moe_proj;

/* A bank of SwiGLU experts: gate, up: hidden -> inter; down: inter -> hidden.
 * The three projections share one format. */
typedef struct {
    int32_t num_experts, hidden, inter;
    moe_proj gate, up, down;
} moe_experts;

/* Operation ids for moe_workspace_bytes(). */
enum { MOE_OP_ROUTE = 0, MOE_OP_PERMUTE = 1, MOE_OP_GROUPED_FFN = 2, MOE_OP_REFILL_SCORE = 3,
       MOE_OP_GROUPED_FFN_NVFP4 = 4, /* grouped FFN of an NVFP4 bank (adds the quantised input) */
       MOE_OP_ROUTE_PERMUTE = 5 };

/*
 * Router: logits, softmax, top-k, renormalised gates.
 * (architecture sheet: softmax gating over the expert logits, 10 of 512
 * routed experts per token, selected weights renormalised to sum to 1.)
 *
 * logit[t][e] = the correctly rounded fp32 value of the exact dot product
 * x[t] . w_router[e].  Experts are ranked by logit descending, ties to the
 * lower index (-0.0 == +0.0).  topk_idx[t] lists the first k+extra experts
 * in rank order; extra = 1 adds the highest-ranked unselected expert used by
 * Refill-RMS.  topk_gate[t][j] = exp(l_j) / sum_{i<k} exp(l_i) over the
 * first k (fp32).  topk_logit (nullable) gets the exact logits of the listed
 * experts.  logits (nullable, [T][E]) gets every exact logit (slower; meant
 * for tests).  Requires 1 <= k, k + extra <= E <= 1024, extra in {0,1},
 * H % 8 == 0.
 */
moe_status moe_route(const uint16_t *x, const uint16_t *w_router, int32_t T, int32_t H,
                     int32_t E, int32_t k, int32_t extra, int32_t *topk_idx, float *topk_logit,
                     float *topk_gate, float *logits, void *ws, size_t ws_bytes, void *stream);

/*
 * Permutation of (token, slot) pairs by expert (architecture sheet, FFN /
 * MoE entries: each token's hidden state goes to the k experts it selected,
 * so every expert processes the group of rows routed to it): a stable
 * counting sort of the pair ids p = t*k + slot by topk_idx[p].
 *   expert_offsets [E+1]: rows of expert e are [offsets[e], offsets[e+1])
 *   sorted_pair    [T*k]: pair id held by each row, ascending within an expert
 *   pair_to_row    [T*k]: inverse of sorted_pair
 * Entries of topk_idx must lie in [0, E); out-of-range ids are not detected
 * (the row assignment is then undefined but stays inside the buffers).
 */
moe_status moe_permute(const int32_t *topk_idx, int32_t T, int32_t k, int32_t E,
                       int32_t *expert_offsets, int32_t *sorted_pair, int32_t *pair_to_row,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * moe_route (extra = 0) followed by moe_permute of its topk_idx, in one call;
 * the outputs and the requirements are those of the two calls (topk_logit
 * and topk_gate nullable).  For decode-sized batches (T < 64, T * k <= 4096)
 * the selection and the permutation share one single-workgroup kernel after
 * the logits, saving a launch on the layer's critical path; otherwise the
 * two calls run as they are.  Workspace: moe_workspace_bytes(
 * MOE_OP_ROUTE_PERMUTE, T, k, E, H, 0).
 */
moe_status moe_route_permute(const uint16_t *x, const uint16_t *w_router, int32_t T, int32_t H,
                             int32_t E, int32_t k, int32_t *topk_idx, float *topk_logit,
                             float *topk_gate, int32_t *expert_offsets, int32_t *sorted_pair,
                             int32_t *pair_to_row, void *ws, size_t ws_bytes, void *stream);

/*
 * Grouped SwiGLU experts: for every row r with pair p = sorted_pair[r],
 * token t = p / k, expert e (the group r falls in):
 *   rows[r] = W_down[e] ( silu(W_gate[e] x[t]) * (W_up[e] x[t]) )
 * (architecture sheet: SwiGLU, no FFN bias, no GLU clamp).
 * With sorted_pair == NULL and expert_offsets == NULL the bank must hold one
 * expert applied to every token (the shared expert): rows[t] = expert(x[t]),
 * and k must be 1.  `ex` is a HOST pointer to a struct of device pointers.
 * rows is [T*k][H] of out_dtype.  Intermediates: fp32 accumulation, the
 * SwiGLU product rounded to bf16 before the down projection (NVFP4: x and
 * the SwiGLU product are quantised as described under "NVFP4 experts").
 * An AWQ_OM bank always runs the MFMA path (any number of rows per expert;
 * for one or two rows per expert the AWQ layout's streaming kernels are the
 * faster choice).
 * AWQ and NVFP4 require hidden % 32 == 0 and inter % 32 == 0, FP8 multiples
 * of 128.  x, rows, ws and the bf16 / AWQ / FP8 / NVFP4 code arrays must be
 * 16-byte aligned, FP8 block scales and NVFP4 global scales 4-byte aligned,
 * NVFP4 group scales 2-byte aligned (MOE_ERR_UNSUPPORTED otherwise).  A bad
 * NVFP4 act_scale (not in (0, 3e38)) or gate/up act_scales that differ give
 * MOE_ERR_SHAPE.
 */
moe_status moe_grouped_ffn(const uint16_t *x, int32_t T, int32_t k, const moe_experts *ex,
                           const int32_t *expert_offsets, const int32_t *sorted_pair,
                           int32_t out_dtype, void *rows, void *ws, size_t ws_bytes,
                           void *stream);

/*
 * moe_grouped_ffn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * moe_grouped_ffn; the scratch it needs lives in a device array of
 * moe_grouped_ffn_noalloc_max_bytes() bytes (16 MiB) that the library holds
 * on every GPU it runs on until the process ends.  A call whose scratch need,
 * moe_workspace_bytes(MOE_OP_GROUPED_FFN or MOE_OP_GROUPED_FFN_NVFP4, ...),
 * exceeds that size returns MOE_ERR_WORKSPACE and enqueues nothing (at the
 * full layer geometry, hidden 2560, width 640, 512 experts, top-10: up to
 * about 40 tokens).  The call allocates nothing.  Every call on one GPU uses
 * that GPU's one array, so calls that may run at the same time on one GPU
 * (on different streams, or from different threads) race and give undefined
 * results; serialise them.  The first call on a device looks the array's
 * address up (a HIP symbol query, no allocation) with that device current.
 */
moe_status moe_grouped_ffn_noalloc(const uint16_t *x, int32_t T, int32_t k, const moe_experts *ex,
                                   const int32_t *expert_offsets, const int32_t *sorted_pair,
                                   int32_t out_dtype, void *rows, void *stream);

/* Bytes of the per-GPU scratch array of moe_grouped_ffn_noalloc. */
size_t moe_grouped_ffn_noalloc_max_bytes(void);

/*
 * The whole MoE feed-forward layer of one batch in one call (architecture
 * sheet, FFN / MoE entries: router top-k with renormalised gates, routed
 * SwiGLU experts, the always-on shared expert, gate-weighted sum):
 *   y = moe_combine(rows, pair_to_row, topk_gate, shared(x), shared_scale)
 * where rows = moe_grouped_ffn(x, k, experts, ...) (bf16 rows) over the
 * permutation that moe_route_permute(x, w_router, ...) gives.  The results
 * are bit-identical to those four calls made one after the other; the call
 * exists so that a decode step costs one host call instead of four and the
 * small steps between the kernels can be merged (for decode-sized batches
 * the selection kernel also builds the routed call's work table).
 *   x [T][H] bf16, w_router [E][H] bf16 with E = experts->num_experts and
 *   H = experts->hidden, y [T][H] bf16 (may not overlap x).  experts and
 *   shared are HOST pointers to structs of device pointers; shared (nullable)
 *   must hold one expert of hidden H (any format, any inter); shared_scale
 *   (nullable, [T] fp32) needs shared.  topk_idx (nullable, [T][k] int32)
 *   also receives the routing decisions.
 *   side_stream (nullable): a hipStream_t other than `stream` on which the
 *   shared expert runs beside the routed path (it waits for the work already
 *   on `stream`, and `stream` waits for it before the combine); NULL runs
 *   everything on `stream`.  The fork and join use two events per calling
 *   thread and device, created on the first such call.
 *   routed_events (nullable, HOST array of two hipEvent_t): recorded on
 *   `stream` right before and right after the routed grouped-expert call,
 *   for timing it inside the layer; either entry may be NULL.
 *   ws: moe_layer_workspace_bytes(T, k, experts, shared) bytes, 16-byte
 *   aligned; it holds every intermediate (routing, permutation, rows).
 * Requirements and errors: those of the four calls; k <= min(E, 64);
 * side_stream == stream or a shared bank with more than one expert or a
 * different hidden size -> MOE_ERR_SHAPE.
 */
moe_status moe_layer(const uint16_t *x, int32_t T, const uint16_t *w_router, int32_t k,
                     const moe_experts *experts, const moe_experts *shared, const float *shared_scale,
                     uint16_t *y, int32_t *topk_idx, void *ws, size_t ws_bytes, void *stream,
                     void *side_stream, void *const *routed_events);

/* Workspace bytes of moe_layer (0 for T <= 0 or an invalid bank).  Grows
 * with T; a workspace sized for the largest T serves every smaller call. */
size_t moe_layer_workspace_bytes(int32_t T, int32_t k, const moe_experts *experts,
                                 const moe_experts *shared);

/*
 * Weighted combine (architecture sheet: routed outputs weighted by the
 * renormalised gates, plus the always-on shared expert):
 *   y[t] = sum_{j<k} topk_gate[t][j] * rows[pair_to_row[t*k+j]]
 *          + shared_scale[t] * shared[t]
 * accumulated in fp32 in slot order, rounded once to bf16.  shared (nullable)
 * is [T][H] bf16; shared_scale (nullable) defaults to 1.  rows_dtype gives
 * the element type of rows.
 */
moe_status moe_combine(const void *rows, int32_t rows_dtype, const int32_t *pair_to_row,
                       const float *topk_gate, int32_t T, int32_t k, int32_t H,
                       const uint16_t *shared, const float *shared_scale, uint16_t *y,
                       void *stream);

/*
 * Refill-RMS statistics (RAZOR E256of512 card, "Selection and calibration"):
 * for each valid token t and each selected slot j < k, drop the slot's
 * expert, promote the expert of slot k (the highest-ranked unselected
 * expert), renormalise the gates over the new set, and add the squared L2
 * norm of the change of the routed output to stat_sum[e] and 1 to
 * stat_count[e], e the dropped expert.  The shared expert cancels in the
 * change and is not needed.  Inputs come from moe_route with extra = 1 and
 * moe_permute over its k+1 slots: rows are the fp32 expert outputs of that
 * permutation (expert_offsets [E+1], sorted_pair and pair_to_row over
 * T*(k+1) pairs), topk_logit is [T][k+1].  The expert of every pair is the
 * group its row falls in (expert_offsets), so the expert ids themselves are
 * not an input.  token_valid (nullable = all valid) is [T] uint8.  stat_sum
 * (fp32 [E]) and stat_count (uint32 [E]) are ADDED to, so batches
 * accumulate; each expert's additions are summed in a fixed order (64
 * strided partial sums over the expert's rows in grouped order, then a fixed
 * tree) and added once per call, so results are reproducible.  Workspace:
 * moe_workspace_bytes(MOE_OP_REFILL_SCORE, T, k, E, H, 0) bytes, 16-byte
 * aligned (MOE_ERR_UNSUPPORTED otherwise).  Requires E >= k + 1,
 * k + 1 <= 32, E <= 1024.
 */
moe_status moe_refill_score(const float *rows, const int32_t *expert_offsets,
                            const int32_t *sorted_pair, const int32_t *pair_to_row,
                            const float *topk_logit,
                            const uint8_t *token_valid, int32_t T, int32_t k, int32_t H,
                            int32_t E, float *stat_sum, uint32_t *stat_count, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * Refill-RMS keep-set (same card and section): score[e] =
 * sqrt(stat_sum[e] / (stat_count[e] * H)), 0 for experts never routed; rank
 * by score descending, ties to the lower index; keep the first `keep`.
 * keep_mask [E] uint8 (1 = kept); keep_idx [keep] lists the kept experts in
 * ascending original index.  E <= 1024, 0 <= keep <= E.
 */
moe_status moe_refill_finalize(const float *stat_sum, const uint32_t *stat_count, int32_t E,
                               int32_t H, int32_t keep, float *score, uint8_t *keep_mask,
                               int32_t *keep_idx, void *stream);

/*
 * Expert pruning by slicing (RAZOR cards: surviving router rows and expert
 * weights are slices of the base, in the keep-set's order):
 *   w_router_dst[j] = w_router_src[keep_idx[j]]        (may be NULL to skip)
 *   every tensor of dst expert j = that of src expert keep_idx[j]
 * keep_idx is a device array of n_keep ids in [0, src->num_experts) (an id
 * outside that range is clamped into it, so no access leaves the source
 * buffers; the copied slab is then that of the clamped id); src and
 * dst are HOST pointers to structs of device pointers with the same format
 * and sizes, dst->num_experts == n_keep.
 */
moe_status moe_prune_slice(const int32_t *keep_idx, int32_t n_keep, const uint16_t *w_router_src,
                           uint16_t *w_router_dst, int32_t H, const moe_experts *src,
                           const moe_experts *dst, void *stream);

/*
 * Rearranges the codes of an AWQ bank (MOE_W_AWQ_G32) into the output-major
 * layout (MOE_W_AWQ_G32_OM, see Layouts): for each projection, dst qweight
 * [E][O][I/8] gets, in nibble j of word w of column o, the code of input
 * 8w + j, exactly (a bit permutation).  dst qzeros and scales must hold the
 * same bytes as src's: they may point to src's own arrays (nothing is
 * copied) or to arrays of the same size, into which src's are copied.  src
 * and dst are HOST pointers to structs of device pointers with equal
 * num_experts, hidden and inter; dst qweight may not overlap src's.  A setup
 * step (one pass over the codes), not part of the layer's hot path.
 * Errors: a format other than AWQ / AWQ_OM, or sizes that differ ->
 * MOE_ERR_SHAPE; sizes the output-major layout does not support ->
 * MOE_ERR_UNSUPPORTED; a null pointer -> MOE_ERR_NULL.
 */
moe_status moe_awq_to_output_major(const moe_experts *src, const moe_experts *dst, void *stream);

/*
 * Router-norm keep policy (RAZOR E256of512 card, "Selection and
 * calibration": the rule used for the layer that calibration text never
 * executes): norm[e] = L2 norm of router row e (fp32 of an fp64 sum); rank
 * descending, ties to the lower index; keep_idx [keep] lists the first
 * `keep` in ascending index.  E <= 1024.
 */
moe_status moe_router_norm_keep(const uint16_t *w_router, int32_t E, int32_t H, int32_t keep,
                                float *norm, int32_t *keep_idx, void *stream);

/*
 * NVFP4 activation quantisation (the recipe under "NVFP4 experts" above) of
 * a [T][n] bf16 matrix, row by row in groups of 16 (n % 16 == 0): out[t][i]
 * = e2m1(code) * s as bf16 (exact), without the global factor act_scale.
 * moe_grouped_ffn applies it to NVFP4 banks by itself; this call exposes it
 * for checking.  x and out are device pointers, 16-byte aligned, owned by
 * the caller (out may not overlap x).  Errors: T < 0, n < 1 or act_scale not
 * in (0, 3e38) -> MOE_ERR_SHAPE; n % 16 or misalignment ->
 * MOE_ERR_UNSUPPORTED; a null pointer with T > 0 -> MOE_ERR_NULL.
 */
moe_status moe_nvfp4_quantize(const uint16_t *x, int32_t T, int32_t n, float act_scale,
                              uint16_t *out, void *stream);

/* Scratch bytes an operation needs (0 when none).  For MOE_OP_GROUPED_FFN,
 * k is the pairs per token and E the bank's expert count; an NVFP4 bank needs
 * MOE_OP_GROUPED_FFN_NVFP4.  Sizes grow with T; a workspace sized for the
 * largest T of a run serves every smaller call. */
size_t moe_workspace_bytes(int32_t op, int32_t T, int32_t k, int32_t E, int32_t H, int32_t F);

/* Static text for a status code. */
const char *moe_status_string(moe_status s);

/* hipError_t (as int) of the calling thread's last failed HIP call, 0 if none. */
int32_t moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */

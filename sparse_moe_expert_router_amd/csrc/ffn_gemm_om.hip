// Grouped SwiGLU experts for many rows per expert on AWQ W4A16 g32 codes
// stored output-major (and on FP8 and NVFP4 codes and bf16 weights, which are
// output-major as stored): bf16 MFMA with the weights dequantised in registers.
//
// Qwen3.8-Flash-Next architecture sheet, FFN / MoE entries: SwiGLU experts
// (gate, up, down), no bias, no clamp.  AWQ-g32 card, "Checkpoint": asymmetric
// W4A16, group 32 along the input, integer zeros, fp16 scales, w = (q - z) s.
// NVFP4 release card, precision table: W4A4 experts, E2M1 values in groups of
// 16 with E4M3 group scales and fp32 global scales (the layout and the
// activation recipe are this library's reading, as in nvfp4.h).  The AWQ-g32
// card's optional FP8 draft: routed experts in E4M3 with explicit block
// scales (128 x 128 blocks: this library's reading).
//
// Code layout: qweight [E][out][in/8] int32, nibble j of word w holds input
// 8w + j of that output column (the AWQ codes rearranged once by
// moe_awq_to_output_major); zeros [E][in/32][out/8] and scales [E][in/32][out]
// keep the AWQ layout.  A lane of the B operand of a 32x32x16 bf16 MFMA holds
// 8 consecutive inputs of one output column: exactly one code word, so B goes
// from HBM straight into registers and is dequantised there; no B tile passes
// through LDS.
//
// Workgroup: 256 threads, 4 waves (one per SIMD; two workgroups per compute
// unit for tiles of up to 128 rows).  Tile: BM = 32 TM rows x
// 256 B-columns (gate/up: 128 gate columns and the same 128 up columns; down:
// 256 output columns); wave w takes all BM rows x its 64 B-columns (gate/up:
// 32 gate + the matching 32 up columns, so SwiGLU is applied in registers),
// TM x 2 MFMA tiles of 32 x 32 (256 fp32 accumulators a lane at TM = 8).
//
// K advances 64 inputs (two AWQ groups) per step, in four MFMA k-chunks of 16.
// In k-chunk h, lane group g = lane / 32 of both operands takes inputs
// 32 g + 8 h .. +7 of the step (any assignment of inputs to lanes gives the
// same dot products as long as A and B agree): a lane's B words for the four
// k-chunks are the consecutive words 8 j + 4 g .. +3 of its column (one 16-byte
// load per step and fragment), all in AWQ group 2 j + g.
//
// Dequantisation of a code q with scale s and zero z: one v_and_or_b32 places
// the nibbles q_b, q_{b+4} of a code word in the low mantissa bits of two fp16
// of exponent 2^10, giving 1024 + q exactly for two inputs at once; a mixed
// precision fma (v_fma_mix_f32 reads the fp16 half directly) gives
// fma(1024 + q, s, -(1024 + z) s) = (q - z) s exactly (the product has 22
// significant bits, the result 16), then one RNE to bf16 for the MFMA.  That
// is 2.4 VALU instructions a weight (3.0 with an fp32 of exponent 2^4 built
// by a v_perm per weight: pruned layer 4.40 -> 4.34 ms, 4096-token prefill
// routed call 0.70 -> 0.67 ms).
//
// A (token rows gathered through sorted_pair, or h rows) goes from global
// memory straight into LDS (16-byte buffer loads to LDS, two steps ahead),
// four stages, one barrier a step.  LDS rows are 128 bytes (64 inputs), their
// 16-byte chunks XOR-swizzled by row (om_swz).
//
// Row tiles: an expert's rows are split into ceil(rows / BM) tiles of equal
// size (a multiple of 32), so that no tile is mostly padding; a tile that
// needs fewer 32-row blocks may run a copy of the loop compiled for fewer
// (om_gemm_kernel).  (Skipping the MFMAs of 32-row blocks past a tile's end
// with a branch inside the step measured 14% slower than computing them.)
//
// Pipeline: a step is 4 TM pieces (k-chunk h = piece / TM, A fragment mi =
// piece % TM), each 2 MFMAs plus a share of the dequantisation of the next
// k-chunk's B words (k-chunk 3: step j+1's first), with the A fragment of the
// piece three ahead read from LDS, across k-chunk and step boundaries.  After
// k-chunk 1 of step j, once this wave's loads of step j+1's A have landed, one
// barrier publishes that stage (so the last pieces of step j can already read
// step j+1's fragments) and step j+3's A is requested into the stage step j-1
// used; after k-chunk 2 the B words of step j+2 are requested.  Loads use raw buffer resources: a per-lane 32-bit
// offset fixed for the whole loop plus a uniform step offset.
#include <type_traits>

#include "ffn_internal.h"
#include "nvfp4.h"

namespace moe {

namespace {

constexpr int kOmThreads = 256;
constexpr int kOmBN = 256;  // B-columns per workgroup
constexpr int kOmKS = 64;   // inputs per step
constexpr int kOmTN = 2;    // 32-column MFMA tiles per wave

enum { OM_GATEUP = 0, OM_DOWN = 1 };

typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int TM>
struct OmShape {
    static constexpr int BM = 32 * TM;           // rows per tile
    static constexpr int AP = TM;                // 16-byte A chunks per thread per step
    static constexpr int STAGE = BM * kOmKS;     // bf16 elements per LDS stage
    // waves per SIMD: tiles up to 128 rows keep their accumulators in VGPRs
    // (at most 256 registers a lane) and run two workgroups per compute unit
    static constexpr int MINW = TM <= 4 ? 2 : 1;
    // epilogue staging: 4 waves x 32 rows x (64 + 4) floats, in bf16 elements
    static constexpr int STG = 4 * 32 * (64 + 4) * 2;
    static constexpr int SMEM = 4 * STAGE > STG ? 4 * STAGE : STG;
};

// LDS row swizzle: the 16-byte chunk c of row r sits at chunk c ^ om_swz(r),
// om_swz(r) = (r & 7) ^ ((r >> 3) & 1).  Eight consecutive rows then take eight
// different chunks, and so do the eight even (or odd) rows of sixteen
// consecutive rows, whether the LDS serves a 16-byte read 8 or 16 lanes at a
// time (rocprofv3: SQ_LDS_BANK_CONFLICT 14x lower than with r & 7 alone).
// om_swz(r + 32 i) == om_swz(r) for every i.
__device__ __forceinline__ int om_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// LDS element offset of 16-byte chunk c of row r (128-byte rows).
__device__ __forceinline__ int om_lds(int r, int c) { return r * kOmKS + ((c ^ om_swz(r)) << 3); }

// Nibble position of column (c mod 8) in an AWQ zero word (packing order
// {0,2,4,6,1,3,5,7}: nibble j holds column perm(j)).
__device__ __forceinline__ int awq_nib(int c8) { return (c8 & 1) ? 4 + (c8 >> 1) : (c8 >> 1); }

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// 0x000F000F in a VGPR the compiler cannot fold into a literal, so that
// (v & m) | c stays one v_and_or_b32 (a VOP3 instruction takes no literal).
// The result of this asm feeds no MFMA directly: the v_and_or_b32 that reads
// it is plain C, so the compiler inserts the VALU -> MFMA wait states.
__device__ __forceinline__ uint32_t om_mask() {
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(m));
    return m;
}

// One code word (8 consecutive inputs) -> 8 bf16 (q - z) s, input i in element
// i, in parts: om_quad once, then om_pair(b) for the inputs 2b, 2b+1.
// om_quad: pq[b] = fp16 pair (1024 + q_b, 1024 + q_{b+4}), b = 0..3.
__device__ __forceinline__ void om_quad(uint32_t w, uint32_t m, uint32_t (&pq)[4]) {
#pragma unroll
    for (int b = 0; b < 4; ++b) pq[b] = ((w >> (4 * b)) & m) | 0x64006400u;
}
__device__ __forceinline__ uint32_t om_pair(int b, const uint32_t (&pq)[4], float s, float c) {
    const f16x2_t e = __builtin_bit_cast(f16x2_t, pq[(2 * b) & 3]);      // input 2b
    const f16x2_t o = __builtin_bit_cast(f16x2_t, pq[(2 * b + 1) & 3]);  // input 2b + 1
    const float lo = fmaf((float)(b < 2 ? e.x : e.y), s, c);
    const float hi = fmaf((float)(b < 2 ? o.x : o.y), s, c);
    return pack_bf16x2(lo, hi);
}

// Raw buffer resource over `bytes` bytes at p (gfx9 family: word 3 = 0x00020000,
// 32-bit data, no stride).  Loads through it take a per-lane 32-bit byte
// offset and a uniform byte offset; an offset past `bytes` reads 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t om_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// NVFP4 (W4A4) codes in the same place: codes [E][out][in/2], byte j of a
// column's row holding inputs 2j (bits 0..3) and 2j+1 (bits 4..7) as E2M1, so
// a 32-bit word is again 8 consecutive inputs; E4M3 group scales
// [E][out][in/16].  A lane's 32 inputs of a step span two groups (words 0-1
// and 2-3).  Both factors of a weight e2m1 * s go into fp16 exactly:
// nv_quad: pq[b] = the pair of inputs 2b, 2b+1 as fp16 e2m1 * 2^8, by the
// gfx950 scaled conversion (its scale operand acts as a power of two only: a
// probe over every byte value and byte position matched
// bf16(e2m1 * 2^floor(log2 s)) everywhere, so 2^8 is exact and the E4M3
// mantissa cannot go there); nv_scales: the two E4M3 bytes of a step moved
// into the two halves of an fp16 pair, whose value is then s * 2^-8 exactly
// (exponent field e, mantissa m: 2^(e-15) (1 + m/8), and for e = 0 the fp16
// subnormal m 2^-17, as E4M3 has 2^(e-7) (1 + m/8) and m 2^-9); nv_pair(b):
// one mixed-precision fma a weight reads both halves, + -0 (a register, so
// that the fma is not folded into a multiply) keeps the sign of a zero
// product, then one RNE to bf16 (exact: at most 6 significant bits).  The
// global factors are applied to the accumulators.
__device__ __forceinline__ void nv_quad(uint32_t w, uint32_t (&pq)[4]) {
    pq[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0));
    pq[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1));
    pq[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2));
    pq[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3));
}
__device__ __forceinline__ uint32_t nv_scales(uint32_t sbits) {
    return ((sbits & 0x7Fu) << 7) | ((sbits & 0x80u) << 8) | ((sbits & 0x7F00u) << 15) | ((sbits & 0x8000u) << 16);
}
__device__ __forceinline__ uint32_t nv_pair(int b, const uint32_t (&pq)[4], uint32_t sc, bool hi, float nz) {
    const f16x2_t v = __builtin_bit_cast(f16x2_t, pq[b]);
    const f16x2_t s2 = __builtin_bit_cast(f16x2_t, sc);
    const float s = (float)(hi ? s2.y : s2.x);
    return pack_bf16x2(fmaf((float)v.x, s, nz), fmaf((float)v.y, s, nz));
}
__device__ __forceinline__ float om_neg_zero() {
    float z;
    asm volatile("v_mov_b32 %0, 0x80000000" : "=v"(z));
    return z;
}

// FP8 E4M3 codes [E][out][in] with fp32 block scales [E][out/128][in/128]: a
// k-chunk's 8 inputs are 8 bytes of the column's row (two words), and a
// step's 64 inputs lie in one scale block.  f8_pair(b): inputs 2b, 2b+1
// widened by v_cvt_pk_f32_fp8, times the block scale in fp32, rounded once to
// bf16 (the arithmetic the first GEMM applies to FP8 tiles).
__device__ __forceinline__ uint32_t f8_pair(int b, uint32_t w0, uint32_t w1, float s) {
    const int w = (int)(b < 2 ? w0 : w1);
    const auto v = (b & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    return pack_bf16x2(v[0] * s, v[1] * s);
}

// (s, -(1024 + z) s) of a lane's column from its raw scale bits and zero word.
__device__ __forceinline__ void om_params(uint32_t sbits, uint32_t zw, int znib, float& s, float& c) {
    s = f16_to_f32(sbits & 0xFFFFu);
    const float z = (float)((zw >> (4 * znib)) & 15u);
    c = -(1024.0f + z) * s;
}

// WF: weight format, 1 = AWQ g32 codes output-major, 2 = FP8, 3 = NVFP4, 0 =
// bf16 [E][out][in] (a lane's 8 inputs are 16 contiguous bytes of its weight
// row; no dequant).
// One row tile (rows m0 .. m1 - 1 of expert e, at most 32 TM) x B-column tile
// nt, computed as TM blocks of 32 rows.
template <int MODE, int WF, int TM>
__device__ __forceinline__ void om_gemm_tile(const GroupedArgs& a, uint16_t* __restrict__ smem,
                                             uint16_t* __restrict__ hbuf, int e, int m0, int m1, int nt) {
    using S = OmShape<TM>;
    constexpr int AP = S::AP;
    constexpr bool AQ = WF == 1, F8 = WF == 2, NV = WF == 3;
    constexpr bool W4 = AQ || F8 || NV;  // codes dequantised in registers
    constexpr int LB = NV ? 4 : 6;  // W4: loads a load_b issues (codes, scales and, AWQ, zero words)

    const int tid = threadIdx.x, lane = tid & 63, wn = tid >> 6;
    const int H = a.H, F = a.F;
    const int K = MODE == OM_GATEUP ? H : F;      // inputs of the projection(s)
    const int N = MODE == OM_GATEUP ? F : H;      // outputs of one projection
    const int NJ = K / kOmKS;

    // ---- A: chunk q = tid + 256 i is row (tid >> 3) + 32 i, chunk tid & 7 of the step
    const rsrc_t ra = MODE == OM_GATEUP ? om_rsrc(a.x, (uint32_t)a.T * (uint32_t)H * 2u)
                                        : om_rsrc(hbuf, (uint32_t)a.P * (uint32_t)F * 2u);
    // Load i of wave wn fills LDS slots 64 (4 i + wn) .. +63 of the stage (one
    // 16-byte slot a lane): row r = 32 i + 8 wn + lane / 8, physical chunk
    // lane & 7, so logical chunk (lane & 7) ^ om_swz(r) of that row.
    uint32_t aoff[AP];  // byte offset of the lane's source chunk in step 0
#pragma unroll
    for (int i = 0; i < AP; ++i) {
        const int r = 32 * i + 8 * wn + (lane >> 3);
        const int gr = min(m0 + r, m1 - 1);
        uint32_t row;
        if (MODE == OM_GATEUP) row = (uint32_t)(a.sorted_pair ? a.sorted_pair[gr] / a.k : gr);
        else row = (uint32_t)gr;
        aoff[i] = row * (uint32_t)K * 2u + (uint32_t)((((lane & 7) ^ om_swz(r))) * 16);
    }

    // ---- B: fragment f of the wave (32 columns), lane column lane & 31,
    // lane group g = lane / 32.  Gate/up: fragment 0 reads the gate tensors,
    // fragment 1 the up tensors.
    const int g = lane >> 5;
    const ProjDev& p0 = MODE == OM_GATEUP ? a.gate : a.down;
    const ProjDev& p1 = MODE == OM_GATEUP ? a.up : a.down;
    const uint32_t qbytes = (AQ || NV) ? (uint32_t)a.E * (uint32_t)N * (uint32_t)(K / 2)
                                       : (uint32_t)a.E * (uint32_t)N * (uint32_t)K * (F8 ? 1u : 2u);
    const uint32_t sbytes = NV ? (uint32_t)a.E * (uint32_t)N * (uint32_t)(K / 16)
                          : F8 ? (uint32_t)a.E * (uint32_t)(N / 128) * (uint32_t)(K / 128) * 4u
                               : (uint32_t)a.E * (uint32_t)(K / 32) * (uint32_t)N * 2u;
    const uint32_t zbytes = AQ ? sbytes / 4u : 0u;
    auto qsrc = [&](const ProjDev& p) {
        return (NV || F8) ? (const void*)p.codes : AQ ? (const void*)p.qweight : (const void*)p.w;
    };
    auto ssrc = [&](const ProjDev& p) {
        return NV ? (const void*)p.gscales : F8 ? (const void*)p.bscales : (const void*)p.scales;
    };
    const rsrc_t rq0 = om_rsrc(qsrc(p0), qbytes), rq1 = om_rsrc(qsrc(p1), qbytes);
    const rsrc_t rs0 = om_rsrc(ssrc(p0), W4 ? sbytes : 0u), rs1 = om_rsrc(ssrc(p1), W4 ? sbytes : 0u);
    const rsrc_t rz0 = om_rsrc(p0.qzeros, zbytes), rz1 = om_rsrc(p1.qzeros, zbytes);
    uint32_t boff[kOmTN];   // byte offset of the lane's B data in step 0
    uint32_t soff[kOmTN];   // W4: byte offset of its scale (NVFP4: its two group scales; FP8: block scale) in step 0
    uint32_t zoff[kOmTN];   // W4: byte offset of its zero word in step 0
    int znib[kOmTN];
#pragma unroll
    for (int f = 0; f < kOmTN; ++f) {
        const int col = MODE == OM_GATEUP ? nt * (kOmBN / 2) + 32 * wn + (lane & 31)
                                          : nt * kOmBN + 64 * wn + 32 * f + (lane & 31);
        const uint32_t grp0 = (uint32_t)e * (uint32_t)(K / 32) + (uint32_t)g;
        const uint32_t row = (uint32_t)e * (uint32_t)N + (uint32_t)col;
        boff[f] = (AQ || NV) ? (row * (uint32_t)(K / 8) + 4u * (uint32_t)g) * 4u   // 4 code words
                : F8 ? row * (uint32_t)K + 32u * (uint32_t)g                       // 32 E4M3 codes
                     : (row * (uint32_t)K + 32u * (uint32_t)g) * 2u;               // 32 bf16 inputs
        soff[f] = NV ? row * (uint32_t)(K / 16) + 2u * (uint32_t)g
                : F8 ? ((uint32_t)e * (uint32_t)(N / 128) + (uint32_t)(col / 128)) * (uint32_t)(K / 128) * 4u
                     : (grp0 * (uint32_t)N + (uint32_t)col) * 2u;
        zoff[f] = (grp0 * (uint32_t)(N / 8) + (uint32_t)(col >> 3)) * 4u;
        znib[f] = awq_nib(col & 7);
    }
    const uint32_t sstep = NV ? 4u : 4u * (uint32_t)N, zstep = (uint32_t)N;  // bytes per step (AWQ: two groups; NVFP4: four)
    const int bstep = (AQ || NV) ? 32 : F8 ? kOmKS : 2 * kOmKS;   // B bytes per step and lane

    f32x16_t acc[TM][kOmTN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int f = 0; f < kOmTN; ++f) acc[i][f] = f32x16_t{};

    // W4: raw B of two steps (buffer = step parity): four code words, scale
    // bits, zero word.  bf16: the current step's 4 k-chunks of B, each
    // refilled with the next step's once its MFMAs have issued.
    u32x4_t cw[W4 ? 2 : 1][kOmTN][F8 ? 2 : 1];  // FP8: 32 codes in two vectors
    uint32_t sb[2][kOmTN], zw[2][kOmTN];
    u32x4_t braw[W4 ? 1 : 4][kOmTN];
    auto load_b = [&](int buf, int j) {
#pragma unroll
        for (int f = 0; f < kOmTN; ++f) {
            const bool hi = MODE == OM_GATEUP && f == 1;
            cw[buf][f][0] = __builtin_amdgcn_raw_buffer_load_b128(hi ? rq1 : rq0, (int)boff[f], j * bstep, 0);
            if (F8) {
                cw[buf][f][F8 ? 1 : 0] = __builtin_amdgcn_raw_buffer_load_b128(hi ? rq1 : rq0, (int)boff[f] + 16, j * bstep, 0);
                // the step's 64 inputs lie in block j / 2 of 128
                sb[buf][f] = __builtin_amdgcn_raw_buffer_load_b32(hi ? rs1 : rs0, (int)soff[f], (j >> 1) * 4, 0);
            } else {
                sb[buf][f] = __builtin_amdgcn_raw_buffer_load_b16(hi ? rs1 : rs0, (int)soff[f], (int)(sstep * (uint32_t)j), 0);
            }
            if (AQ) zw[buf][f] = __builtin_amdgcn_raw_buffer_load_b32(hi ? rz1 : rz0, (int)zoff[f], (int)(zstep * (uint32_t)j), 0);
        }
    };
    auto load_braw = [&](int h, int j) {
#pragma unroll
        for (int f = 0; f < kOmTN; ++f) {
            const bool hi = MODE == OM_GATEUP && f == 1;
            braw[W4 ? 0 : h][f] = __builtin_amdgcn_raw_buffer_load_b128(hi ? rq1 : rq0, (int)boff[f] + 16 * h, j * bstep, 0);
        }
    };
    // A of step j straight into LDS stage st (buffer load to LDS: lane L's 16
    // bytes land at the wave's base + 16 L)
    auto load_a = [&](uint16_t* st, int j) {
#pragma unroll
        for (int i = 0; i < AP; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(st + (4 * i + wn) * 512),
                                                     16, (int)aoff[i], j * kOmKS * 2, 0, 0);
    };
    // wait until at most n vector-memory loads of this wave are outstanding
    // (s_waitcnt: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima)
    auto wait_vm = [](auto n) {
        constexpr int v = decltype(n)::value;
        __builtin_amdgcn_s_waitcnt((v & 15) | ((v >> 4) << 14) | 0x70 | 0xF00);
    };
    // A fragment (h, mi): row 32 mi + (lane & 31), logical chunk 4 g + h
    int afr[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) afr[h] = (lane & 31) * kOmKS + (((4 * g + h) ^ om_swz(lane & 31)) << 3);

    u32x4_t bfr[2][kOmTN];        // W4: dequantised B of two k-chunks (bf16 pairs)
    float ps[kOmTN], pc[kOmTN];   // W4: (s, c) of the step being dequantised (NVFP4: ps = its two group scales)
    uint32_t pq[kOmTN][4];        // W4: fp16 pairs of the code word being dequantised
    const uint32_t msk = om_mask();

    // A fragments of the pieces in flight: piece p uses af[p % 4]; the read of
    // piece p + kAD is issued in piece p.
    constexpr int kAD = 3;
    constexpr int NP = 4 * TM;                      // pieces per step
    constexpr int PPC = (4 * kOmTN + TM - 1) / TM;  // dequant parts per piece (8 per k-chunk)
    bf16x8_t af[4];
    auto read_af = [&](const uint16_t* A, int q) {
        af[q % 4] = *reinterpret_cast<const bf16x8_t*>(A + 32 * (q % TM) * kOmKS + afr[q / TM]);
    };

    // ---- prologue.  Vector-memory loads complete in issue order for the
    // s_waitcnt counter, and each step issues them in one fixed order:
    //   W4:   [mid step m: A(m+3)] [piece 3 TM - 1: B(m+2)]
    //   bf16: [k-chunk h end: its B of step m+1] with A(m+3) at mid step
    // so at the mid-step wait of step j at most 2 LB + TM loads issued after
    // A(j+1) can be outstanding (W4; 12 + TM is a stricter wait for bf16).  The prologue issues steps 0..2's loads in the
    // order the two steps before step 0 would have, so that this holds from
    // step 0 on.
    auto stg = [&](int i) { return smem + i * S::STAGE; };
    load_a(stg(0), 0);
    load_a(stg(1), min(1, NJ - 1));
    if (W4) {
        load_b(0, 0);
        load_a(stg(2), min(2, NJ - 1));
        load_b(1, min(1, NJ - 1));
        wait_vm(std::integral_constant<int, 2 * LB + 2 * TM>{});   // A(0)
    } else {
        load_braw(0, 0);
        load_braw(1, 0);
        load_a(stg(2), min(2, NJ - 1));
        load_braw(2, 0);
        load_braw(3, 0);
        wait_vm(std::integral_constant<int, 8 + 2 * TM>{});    // A(0)
    }
    // NVFP4: the two group scales of a lane's step as an fp16 pair (in ps)
    const float nz = NV ? om_neg_zero() : 0.0f;
    auto nv_params = [](uint32_t sbits, float& s01, float&) { s01 = __uint_as_float(nv_scales(sbits)); };
    if (W4) {
#pragma unroll
        for (int f = 0; f < kOmTN; ++f) {
            if (F8) {
                ps[f] = __uint_as_float(sb[0][f]);
#pragma unroll
                for (int b = 0; b < 4; ++b) bfr[0][f][b] = f8_pair(b, cw[0][f][0][0], cw[0][f][0][1], ps[f]);
            } else if (NV) {
                nv_params(sb[0][f], ps[f], pc[f]);
                nv_quad(cw[0][f][0][0], pq[f]);
#pragma unroll
                for (int b = 0; b < 4; ++b) bfr[0][f][b] = nv_pair(b, pq[f], __float_as_uint(ps[f]), false, nz);
            } else {
                om_params(sb[0][f], zw[0][f], znib[f], ps[f], pc[f]);
                om_quad(cw[0][f][0][0], msk, pq[f]);
#pragma unroll
                for (int b = 0; b < 4; ++b) bfr[0][f][b] = om_pair(b, pq[f], ps[f], pc[f]);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kAD; ++q) read_af(stg(0), q);

    auto step = [&](int j, int cur) {
        const int nxt = cur ^ 1;
        const uint16_t* A = stg(j & 3);
        const uint16_t* An = stg((j + 1) & 3);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int h = p / TM, mi = p % TM;
            const int q = p + kAD;
            if (q < NP) read_af(A, q);
            else read_af(An, q - NP);  // published by this step's barrier (q - NP < kAD <= 2 TM)
#pragma unroll
                for (int f = 0; f < kOmTN; ++f)
                    acc[mi][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        af[p % 4], __builtin_bit_cast(bf16x8_t, W4 ? bfr[h & 1][f] : braw[W4 ? 0 : h][f]), acc[mi][f], 0, 0, 0);
            if (W4) {
                // a share of the next k-chunk's B: words h + 1 of step j, or word 0 of step j+1
#pragma unroll
                for (int u = mi * PPC; u < (mi + 1) * PPC && u < 4 * kOmTN; ++u) {
                    const int f = u / 4, b = u % 4;
                    const uint32_t w = h < 3 ? cw[cur][f][0][(h + 1) & 3] : cw[W4 ? nxt : 0][f][0][0];
                    if (F8) {
                        // k-chunk (h + 1) mod 4: words 2 kc, 2 kc + 1 of the step's eight
                        const int kc = (h + 1) & 3;
                        const u32x4_t& v = cw[h < 3 ? cur : (W4 ? nxt : 0)][f][(kc >> 1) & (F8 ? 1 : 0)];
                        bfr[(h + 1) & 1][f][b] = f8_pair(b, v[2 * (kc & 1)], v[2 * (kc & 1) + 1], ps[f]);
                    } else if (NV) {
                        // words 0-1 of a step take its first group scale, 2-3 the second
                        if (b == 0) nv_quad(w, pq[f]);
                        bfr[(h + 1) & 1][f][b] = nv_pair(b, pq[f], __float_as_uint(ps[f]), h == 1 || h == 2, nz);
                    } else {
                        if (b == 0) om_quad(w, msk, pq[f]);
                        bfr[(h + 1) & 1][f][b] = om_pair(b, pq[f], ps[f], pc[f]);
                    }
                }
            } else if (mi == TM - 1) {
                load_braw(h, min(j + 1, NJ - 1));  // k-chunk h of step j+1 into the registers just used
            }
            if (p == 2 * TM - 1) {
                // A(j+1) has landed in its stage: publish it, then request A(j+3)
                // into the stage step j-1 used (every wave is past step j-1 here)
                wait_vm(std::integral_constant<int, (W4 ? 2 * LB : 12) + TM>{});
                __syncthreads();
                load_a(stg((j + 3) & 3), min(j + 3, NJ - 1));
            }
            if (W4 && p == 3 * TM - 1) {
                // step j's words are all dequantised: request step j+2's; step
                // j+1's parameters for k-chunk 3's share
                load_b(cur, min(j + 2, NJ - 1));
#pragma unroll
                for (int f = 0; f < kOmTN; ++f) {
                    if (F8) ps[f] = __uint_as_float(sb[nxt][f]);
                    else if (NV) nv_params(sb[nxt][f], ps[f], pc[f]);
                    else om_params(sb[nxt][f], zw[nxt][f], znib[f], ps[f], pc[f]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // two steps per trip so that the register buffers are addressed statically
    int j = 0;
    for (; j + 1 < NJ; j += 2) {
        step(j, 0);
        step(j + 1, 1);
    }
    if (j < NJ) step(j, 0);
    // no load may still be writing a stage when the epilogue reuses the LDS
    wait_vm(std::integral_constant<int, 0>{});
    __syncthreads();

    // ---- epilogue: element 4 i + r of a lane's 32 x 32 tile is
    // C[8 i + 4 (lane / 32) + r][lane % 32].  Each wave passes 32 rows at a
    // time through its own LDS region (the A stages are free after the last
    // barrier) as fp32 and writes whole 16-byte vectors of a row.
    constexpr int LD = 64 + 4;  // floats per staged row
    float* st = reinterpret_cast<float*>(smem) + wn * 32 * LD;
    static_assert(S::SMEM * sizeof(uint16_t) >= 4 * 32 * LD * sizeof(float), "epilogue staging");
    const int nrows = m1 - m0;
    const int col = lane & 31;
    // NVFP4: the global factors (input scale x weight scale) of the
    // accumulators of fragment 0 and 1
    float cf0 = 1.0f, cf1 = 1.0f;
    if (NV) {
        cf0 = (MODE == OM_GATEUP ? a.gate.act : a.down.act) * p0.wglobal[e];
        cf1 = (MODE == OM_GATEUP ? a.gate.act : a.down.act) * p1.wglobal[e];
    }
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
        if (MODE == OM_GATEUP) {
#pragma unroll
            for (int k = 0; k < 16; ++k)
                st[(8 * (k >> 2) + 4 * g + (k & 3)) * LD + col] =
                    NV ? silu(acc[mi][0][k] * cf0) * (acc[mi][1][k] * cf1) : silu(acc[mi][0][k]) * acc[mi][1][k];
        } else {
#pragma unroll
            for (int f = 0; f < kOmTN; ++f)
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    st[(8 * (k >> 2) + 4 * g + (k & 3)) * LD + 32 * f + col] = NV ? acc[mi][f][k] * cf0 : acc[mi][f][k];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (MODE == OM_GATEUP) {
            const int hcol = nt * (kOmBN / 2) + 32 * wn;
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {  // 16 rows x 4 chunks of 8 h columns
                const int rr = pass * 16 + (lane >> 2), ch = lane & 3;
                const int row = 32 * mi + rr;
                float4 v0 = *reinterpret_cast<const float4*>(&st[rr * LD + ch * 8]);
                float4 v1 = *reinterpret_cast<const float4*>(&st[rr * LD + ch * 8 + 4]);
                if (NV) {
                    // the down projection's input quantised in groups of 16 h
                    // columns (chunks 0-1 and 2-3 of the row's lanes 4i .. 4i+3)
                    float am = fmaxf(fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))),
                                     fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)), fmaxf(fabsf(v1.z), fabsf(v1.w))));
                    am = fmaxf(am, __shfl_xor(am, 1, kWave));
                    const float qa = a.down.act, sc = nvfp4_group_scale(am, qa);
                    v0 = make_float4(nvfp4_qv(v0.x, sc, qa), nvfp4_qv(v0.y, sc, qa), nvfp4_qv(v0.z, sc, qa),
                                     nvfp4_qv(v0.w, sc, qa));
                    v1 = make_float4(nvfp4_qv(v1.x, sc, qa), nvfp4_qv(v1.y, sc, qa), nvfp4_qv(v1.z, sc, qa),
                                     nvfp4_qv(v1.w, sc, qa));
                }
                if (row < nrows)
                    st_stream(&hbuf[(size_t)(m0 + row) * F + hcol + ch * 8],
                              u32x4_t{pack_bf16x2(v0.x, v0.y), pack_bf16x2(v0.z, v0.w), pack_bf16x2(v1.x, v1.y),
                                      pack_bf16x2(v1.z, v1.w)});
            }
        } else if (a.out_f32) {
            float* out = static_cast<float*>(a.rows);
            const int ocol = nt * kOmBN + 64 * wn;
#pragma unroll
            for (int pass = 0; pass < 8; ++pass) {  // 4 rows x 16 chunks of 4 floats
                const int rr = pass * 4 + (lane >> 4), ch = lane & 15;
                const int row = 32 * mi + rr;
                const float4 v = *reinterpret_cast<const float4*>(&st[rr * LD + ch * 4]);
                if (row < nrows) *reinterpret_cast<float4*>(&out[(size_t)(m0 + row) * H + ocol + ch * 4]) = v;
            }
        } else {
            uint16_t* out = static_cast<uint16_t*>(a.rows);
            const int ocol = nt * kOmBN + 64 * wn;
#pragma unroll
            for (int pass = 0; pass < 4; ++pass) {  // 8 rows x 8 chunks of 8 values
                const int rr = pass * 8 + (lane >> 3), ch = lane & 7;
                const int row = 32 * mi + rr;
                const float4 v0 = *reinterpret_cast<const float4*>(&st[rr * LD + ch * 8]);
                const float4 v1 = *reinterpret_cast<const float4*>(&st[rr * LD + ch * 8 + 4]);
                if (row < nrows)
                    st_stream(&out[(size_t)(m0 + row) * H + ocol + ch * 8],
                              u32x4_t{pack_bf16x2(v0.x, v0.y), pack_bf16x2(v0.z, v0.w), pack_bf16x2(v1.x, v1.y),
                                      pack_bf16x2(v1.z, v1.w)});
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// The grouped GEMM over a tile table.  A tile of fewer rows than 32 TM may
// run a copy of the loop with fewer row blocks (chosen per tile, outside the
// K loop, so that every copy keeps a static schedule): an expert whose rows
// just exceed a multiple of 32 TM is split into tiles one block short, and
// its last tile is often shorter still.
template <int MODE, int WF, int TM>
__global__ __launch_bounds__(kOmThreads) __attribute__((amdgpu_waves_per_eu(OmShape<TM>::MINW, OmShape<TM>::MINW)))
void om_gemm_kernel(GroupedArgs a, const int32_t* __restrict__ tiles, uint16_t* __restrict__ hbuf, int NT) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[OmShape<TM>::SMEM];
    // tiles == nullptr: one expert (identity mode), split as the tile table
    // splits an expert: ceil(P / 32 TM) tiles of equal size, a multiple of 32
    const int ntl = tiles ? tiles[0] : (a.P + 32 * TM - 1) / (32 * TM);
    const int l = xcd_remap(blockIdx.x, ntl * NT);
    if (l < 0) return;
    const int tile = l / NT, nt = l % NT;
    const int isz = tiles ? 0 : ((a.P + ntl - 1) / ntl + 31) / 32 * 32;
    const int e = tiles ? tiles[1 + 3 * tile] : 0;
    const int m0 = tiles ? tiles[2 + 3 * tile] : tile * isz;
    const int m1 = tiles ? tiles[3 + 3 * tile] : min(m0 + isz, a.P);
    const int tv = (m1 - m0 + 31) >> 5;  // row blocks the tile needs, 1 .. TM
    // gate/up tiles of 192 or 256 rows: copies one and two blocks short.
    // Down tiles of 128 rows (two workgroups a compute unit): one copy of two
    // blocks, for an expert's last tile of at most 64 rows (copies of two and
    // three blocks measured slower than none)
    constexpr bool VAR = MODE == OM_GATEUP && TM >= 6;
    constexpr bool VD = MODE == OM_DOWN && TM == 4;
    constexpr int T1 = VAR ? TM - 1 : VD ? 2 : TM, T2 = VAR ? TM - 2 : VD ? 2 : TM;
    if constexpr (T1 == TM) {
        om_gemm_tile<MODE, WF, TM>(a, smem, hbuf, e, m0, m1, nt);
    } else if constexpr (T2 == T1) {
        if (tv > T1) om_gemm_tile<MODE, WF, TM>(a, smem, hbuf, e, m0, m1, nt);
        else om_gemm_tile<MODE, WF, T1>(a, smem, hbuf, e, m0, m1, nt);
    } else {
        if (tv > T1) om_gemm_tile<MODE, WF, TM>(a, smem, hbuf, e, m0, m1, nt);
        else if (tv > T2) om_gemm_tile<MODE, WF, T1>(a, smem, hbuf, e, m0, m1, nt);
        else om_gemm_tile<MODE, WF, T2>(a, smem, hbuf, e, m0, m1, nt);
    }
}

// Tile table: tiles[0] = number of tiles, then (expert, first row, end row)
// triples.  An expert with n rows gets t = ceil(n / BM) tiles of equal size
// ceil(n / t) rounded up to 32 (the last one shorter).
__global__ __launch_bounds__(1024) void om_tile_table_kernel(const int32_t* __restrict__ offsets, int E, int P, int BM,
                                                             int32_t* __restrict__ tiles) {
    __shared__ int scan[1024];
    const int e = threadIdx.x;
    int cnt = 0, r0 = 0;
    if (offsets) {
        if (e < E) {
            r0 = offsets[e];
            cnt = offsets[e + 1] - r0;
        }
    } else if (e == 0) {
        cnt = P;
    }
    const int nt = (cnt + BM - 1) / BM;
    const int sz = nt ? ((cnt + nt - 1) / nt + 31) / 32 * 32 : 0;
    scan[e] = nt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int v = e >= off ? scan[e - off] : 0;
        __syncthreads();
        scan[e] += v;
        __syncthreads();
    }
    const int start = scan[e] - nt;
    for (int i = 0; i < nt; ++i) {
        tiles[1 + 3 * (start + i)] = e;
        tiles[2 + 3 * (start + i)] = r0 + i * sz;
        tiles[3 + 3 * (start + i)] = min(r0 + (i + 1) * sz, r0 + cnt);
    }
    if (e == 1023) tiles[0] = scan[1023];
}

// Output-major code words from AWQ codes: word w of column o of expert e holds
// inputs 8w..8w+7, input 8w + j in nibble j.  One thread per output word.
__global__ __launch_bounds__(256) void awq_to_om_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                                        int E, int K, int N) {
    const size_t words = (size_t)E * N * (K / 8);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x) {
        const int w = (int)(i % (K / 8));
        const size_t en = i / (K / 8);
        const int n = (int)(en % N);
        const size_t e = en / N;
        const int sh = 4 * awq_nib(n & 7);
        const uint32_t* s = src + (e * K + 8 * (size_t)w) * (N / 8) + n / 8;
        uint32_t out = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) out |= ((s[(size_t)j * (N / 8)] >> sh) & 15u) << (4 * j);
        dst[i] = out;
    }
}

template <int TM>
dim3 om_grid(int P, int E, int ntile) {
    const long mt = (long)(P + 32 * TM - 1) / (32 * TM) + E;
    return dim3((unsigned)((mt * ntile + kXcd - 1) / kXcd * kXcd));
}

template <int MODE, int WF, int TM>
void launch_om_tm(const GroupedArgs& a, const int32_t* tiles, uint16_t* hbuf, int E, hipStream_t s) {
    const int NT = MODE == OM_GATEUP ? a.F / (kOmBN / 2) : a.H / kOmBN;
    hipLaunchKernelGGL((om_gemm_kernel<MODE, WF, TM>), om_grid<TM>(a.P, E, NT), dim3(kOmThreads), 0, s, a, tiles,
                       hbuf, NT);
}

template <int MODE, int WF>
void launch_om_wf(const GroupedArgs& a, const int32_t* tiles, uint16_t* hbuf, int E, int TM, hipStream_t s) {
    switch (TM) {
        case 8: launch_om_tm<MODE, WF, 8>(a, tiles, hbuf, E, s); break;
        case 6: launch_om_tm<MODE, WF, 6>(a, tiles, hbuf, E, s); break;
        case 4: launch_om_tm<MODE, WF, 4>(a, tiles, hbuf, E, s); break;
        case 3: launch_om_tm<MODE, WF, 3>(a, tiles, hbuf, E, s); break;
        default: launch_om_tm<MODE, WF, 2>(a, tiles, hbuf, E, s); break;
    }
}

// Rows per tile from the average rows per non-empty expert: one tile should
// hold most experts whole.
int om_pick_tm(int P, int E) {
    const int active = P < E ? P : E;
    const int avg = active > 0 ? P / active : 0;
    return avg >= 192 ? 8 : avg >= 128 ? 6 : avg >= 96 ? 4 : avg >= 64 ? 3 : 2;
}

}  // namespace

bool om_gemm_supported(int H, int F) { return H % kOmBN == 0 && F % (kOmBN / 2) == 0 && H % kOmKS == 0 && F % kOmKS == 0; }

// Tile table bytes: at most P / 64 + E tiles (BM >= 64) of 3 ints, plus the count.
static size_t om_tiles_bytes(int P, int E) { return (((size_t)(1 + 3 * ((P + 63) / 64 + E)) * sizeof(int32_t)) + 255) & ~(size_t)255; }

size_t om_gemm_ws_bytes(int P, int F, int E) { return 2 * om_tiles_bytes(P, E) + (size_t)P * F * sizeof(uint16_t); }

hipError_t launch_om_gemm(const GroupedArgs& a, void* ws, hipStream_t s) {
    const int E = a.offsets ? a.E : 1;
    // gate/up: the row tile that holds most experts whole; down (K = inter,
    // few steps per tile): at most 128 rows, two workgroups per compute unit,
    // so that one tile's prologue and epilogue overlap another's main loop.
    // One bf16 expert over many rows (the shared expert) keeps 256-row down
    // tiles: every tile reads the same weights, and the larger tile reads
    // them half as often (32768 rows: 178.7 -> 147.6 us alone)
    const int TMG = om_pick_tm(a.P, E);
    const bool one_bf16 = !a.offsets && !a.awq && !a.fp8 && !a.nvfp4;
    const int TMD = (one_bf16 && TMG == 8) ? 8 : TMG > 4 ? 4 : TMG;
    int32_t* tiles = static_cast<int32_t*>(ws);
    int32_t* tiles_d = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + om_tiles_bytes(a.P, E));
    uint16_t* hbuf = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + 2 * om_tiles_bytes(a.P, E));
    if (!a.offsets) {
        // one expert: the kernels derive their tiles from the block index
        tiles = nullptr;
        tiles_d = nullptr;
    } else {
        hipLaunchKernelGGL(om_tile_table_kernel, dim3(1), dim3(1024), 0, s, a.offsets, E, a.P, 32 * TMG, tiles);
        if (TMD != TMG)
            hipLaunchKernelGGL(om_tile_table_kernel, dim3(1), dim3(1024), 0, s, a.offsets, E, a.P, 32 * TMD, tiles_d);
        else tiles_d = tiles;
    }
    if (a.nvfp4) {
        launch_om_wf<OM_GATEUP, 3>(a, tiles, hbuf, E, TMG, s);
        launch_om_wf<OM_DOWN, 3>(a, tiles_d, hbuf, E, TMD, s);
    } else if (a.fp8) {
        launch_om_wf<OM_GATEUP, 2>(a, tiles, hbuf, E, TMG, s);
        launch_om_wf<OM_DOWN, 2>(a, tiles_d, hbuf, E, TMD, s);
    } else if (a.awq) {
        launch_om_wf<OM_GATEUP, 1>(a, tiles, hbuf, E, TMG, s);
        launch_om_wf<OM_DOWN, 1>(a, tiles_d, hbuf, E, TMD, s);
    } else {
        launch_om_wf<OM_GATEUP, 0>(a, tiles, hbuf, E, TMG, s);
        launch_om_wf<OM_DOWN, 0>(a, tiles_d, hbuf, E, TMD, s);
    }
    return hipGetLastError();
}

hipError_t launch_awq_to_om(const int32_t* src, int32_t* dst, int E, int K, int N, hipStream_t s) {
    const size_t words = (size_t)E * N * (K / 8);
    if (words == 0) return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(awq_to_om_kernel, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const uint32_t*>(src),
                       reinterpret_cast<uint32_t*>(dst), E, K, N);
    return hipGetLastError();
}

}  // namespace moe

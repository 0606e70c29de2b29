// Grouped SwiGLU experts for few rows per expert (decode) on AWQ W4A16 g32
// codes stored output-major: weight streaming, with the dot products on the
// 4x4x4 bf16 MFMA (16 independent 4 x 4 blocks a wave), which the streaming
// otherwise leaves idle.
//
// Qwen3.8-Flash-Next architecture sheet, FFN / MoE entries: SwiGLU experts
// (gate, up, down), no bias, no clamp.  AWQ-g32 card, "Checkpoint": asymmetric
// W4A16, group 32 along the input, integer zeros, fp16 scales, w = (q - z) s.
// With a handful of tokens per expert the work is a stream of the touched
// experts' codes from HBM; each code is read once and used for every row.
//
// Lane l of a wave is lane j = l % 4 of block b = l / 4.  For the MFMA, lane l
// supplies row j of its block's A (4 consecutive k), column j of its block's
// B, and receives rows 0..3 of column j of its block's product.  Block
// b = cq NG + gb takes, in pass p, AWQ group g = gb + NG p of column
// c = base + 4 cq + j: a wave covers 64 / NG columns, and the G = in / 32
// groups of a column take PS = G / NG passes.  The 32 codes of (c, g) are 16
// contiguous bytes of the output-major layout (one load a lane and pass).
//
// Unpacking: a code word w (8 inputs) gives the bf16 pairs (n0,n4), (n1,n5),
// (n2,n6), (n3,n7) as 128 + q, one v_and_or each (after a shift for the last
// three); (n0,n4),(n1,n5) feed one MFMA and (n2,n6),(n3,n7) the next.  The A
// rows (token rows gathered through sorted_pair, or taken by (token, slot)
// pair, for gate/up; h rows for down; at most 4 a chunk) are staged in LDS
// with every 8 inputs in the order 0,4,1,5,2,6,3,7 so that a 16-byte LDS read
// is the A operand of two MFMAs.  The codes stream with the non-temporal hint;
// the scales and zero words of a workgroup's columns go to LDS once, by
// buffer loads to LDS issued with the first codes.
// 8 MFMAs give, per block, D = sum_{i in g} x_i (128 + q_i) for the 4 rows;
// the group's contribution s (D - (128 + z) sum_{i in g} x_i) is added in
// fp32 for the chunk's real rows only, then the NG blocks of a column are
// summed across lanes in a fixed order (results are deterministic).
//
// Gate/up (MODE 0): workgroups of the gate and of the up projection each
// write their columns in fp32 (4 columns a set at in = 2560, NG = 16); the
// down pass (MODE 1, 16 columns a set at in = 640, NG = 4) forms
// h = bf16(silu(gate) up) while staging its rows, and writes the output rows.
// No partial sums leave a wave.
#include "ffn_internal.h"

namespace moe {

namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kOvWaves = 4;
constexpr int kOvThreads = kOvWaves * kWave;
constexpr int kOvMaxIn = 4096;  // LDS holds 4 rows of at most this many inputs
constexpr int kOvMaxPass = 8;
constexpr int kOvSetsPerWave = 8;

// Raw buffer resource over `bytes` bytes at p (gfx9 family: word 3 = 0x00020000).
__device__ __forceinline__ rsrc_t ov_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ f32x4_t ov_mfma(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4_t c) {
    const s16x4_t A = __builtin_bit_cast(s16x4_t, u32x2_t{a0, a1});
    const s16x4_t B = __builtin_bit_cast(s16x4_t, u32x2_t{b0, b1});
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(A, B, c, 0, 0, 0);
}

// bf16 pair 128 + q of the nibbles at bits 0..3 and 16..19 of v, written in
// plain C (one v_and_or_b32 with the mask m in a VGPR, see ov_mask): the
// result is an MFMA operand, and the compiler's hazard tracking, which
// inserts the wait states between a VALU write and an MFMA read of a
// register, does not see into inline assembly.
__device__ __forceinline__ uint32_t ov_pair(uint32_t v, uint32_t m) { return (v & m) | 0x43004300u; }

// 0x000F000F in a VGPR the compiler cannot fold into a literal, so that
// (v & m) | c stays one v_and_or_b32 (a VOP3 instruction takes no literal).
__device__ __forceinline__ uint32_t ov_mask() {
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(m));
    return m;
}

// Nibble position of column (c mod 8) in an AWQ zero word (packing order
// {0,2,4,6,1,3,5,7}: nibble j holds column perm(j)).
__device__ __forceinline__ int ov_nib(int c8) { return (c8 & 1) ? 4 + (c8 >> 1) : (c8 >> 1); }

// D of one group for this lane's block: the 8 MFMAs over its 4 code words,
// alternating between two accumulators (D = d0 + d1) so that each MFMA
// depends on the one two back rather than on the previous.
__device__ __forceinline__ void ov_group(const u32x4_t& cw, const uint32_t* xa, uint32_t m, f32x4_t& d0,
                                         f32x4_t& d1) {
    d0 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    d1 = d0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xa + 4 * w);
        const uint32_t q = cw[w];
        d0 = ov_mfma(xv.x, xv.y, ov_pair(q, m), ov_pair(q >> 4, m), d0);
        d1 = ov_mfma(xv.z, xv.w, ov_pair(q >> 8, m), ov_pair(q >> 12, m), d1);
    }
}

// res[i] += s (d0[i] + d1[i] - (128 + z) xsum[i]) for the R rows.
template <int R>
__device__ __forceinline__ void ov_correct(const f32x4_t& d0, const f32x4_t& d1, uint32_t sbits, uint32_t zw,
                                           int znib, const f32x4_t& xs4, float (&res)[R]) {
    const float s = f16_to_f32(sbits & 0xFFFFu);
    const float zc = 128.0f + (float)((zw >> (4 * znib)) & 15u);
#pragma unroll
    for (int i = 0; i < R; ++i) res[i] = fmaf(s, fmaf(-zc, xs4[i], d0[i] + d1[i]), res[i]);
}

// Code words of one column set: PS passes.
template <int PS>
struct OvCodes {
    u32x4_t c[PS];
};

// Cache policy of the code loads: non-temporal (the codes are read once per
// call; 104 -> 96 us for the 16-token decode layer's routed call).
constexpr int kOvCodePolicy = 2;

template <int PS>
__device__ __forceinline__ void ov_load(OvCodes<PS>& cd, rsrc_t cw, uint32_t vc, int NG) {
#pragma unroll
    for (int p = 0; p < PS; ++p)
        cd.c[p] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(cw, vc, 16 * NG * p, kOvCodePolicy));
}

// Shapes of one launch: I inputs, O output columns a projection, G = I / 32
// groups, NG blocks a column, CS = 64 / NG columns a set, SPW sets a wave,
// CW = 4 SPW CS columns a workgroup, NWG workgroups a projection, NM
// projections (gate and up, or down).
struct OvShape {
    int I, O, G, NG, CS, SPW, CW, NWG, NM;
};

// LDS of a workgroup: the A rows [4][I/2] (bf16 pairs), their group sums
// [G][4], and the scales [G][CW] (fp16) and zero words [G][CW/8] of the
// workgroup's columns.
__host__ __device__ inline size_t ov_lds_bytes(const OvShape& h) {
    return (size_t)4 * h.I * 2 + (size_t)h.G * 16 + (size_t)h.G * h.CW * 2 + (size_t)h.G * h.CW / 2;
}

// One column set (column c of projection m, local column cl) of the chunk's
// rows: MFMAs, corrections, the reduction over the NG blocks of a column,
// and the write of the real rows: MODE 0 writes gate (m = 0) or up (m = 1)
// in fp32 to gu [P][2 O]; MODE 1 writes the rows.
template <int MODE, int PS, int R>
__device__ __forceinline__ void ov_compute(const GroupedArgs& a, const OvShape& h, const OvCodes<PS>& cd, int m,
                                           int c, int cl, int gb, int rc, int nr, const int* prow,
                                           const uint32_t* xrow, const float* xsum, const uint16_t* ssc,
                                           const uint32_t* szr, uint32_t msk, float* __restrict__ gu) {
    const int znib = ov_nib(c & 7);
    float r[R];
#pragma unroll
    for (int i = 0; i < R; ++i) r[i] = 0.0f;
#pragma unroll
    for (int p = 0; p < PS; ++p) {
        const int g = gb + h.NG * p;
        const f32x4_t xs4 = *reinterpret_cast<const f32x4_t*>(xsum + 4 * g);
        const uint32_t sb = ssc[g * h.CW + cl];
        const uint32_t zw = szr[g * (h.CW / 8) + cl / 8];
        f32x4_t d0, d1;
        ov_group(cd.c[p], xrow + 16 * g, msk, d0, d1);
        ov_correct<R>(d0, d1, sb, zw, znib, xs4, r);
        // one pass's unpacked operands live at a time (the scheduler would
        // otherwise unpack every pass ahead and spill)
        __builtin_amdgcn_sched_barrier(0);
    }
    // the NG blocks of a column: lane bits 2 .. 2 + log2(NG)
    for (int s = 4; s < 4 * h.NG; s <<= 1) {
#pragma unroll
        for (int i = 0; i < R; ++i) r[i] += __shfl_xor(r[i], s, kWave);
    }
    if (gb == 0) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            if (i >= nr) break;
            const int rid = prow ? prow[rc + i] : rc + i;
            if constexpr (MODE == 0) {
                gu[(size_t)rid * (2 * h.O) + m * h.O + c] = r[i];
            } else {
                const size_t o = (size_t)rid * h.O + c;
                if (a.out_f32) static_cast<float*>(a.rows)[o] = r[i];
                else static_cast<uint16_t*>(a.rows)[o] = (uint16_t)f32_to_bf16_bits(r[i]);
            }
        }
    }
}

// The wave's column sets [st0, st1) with the codes of the next set in flight
// while the current one computes (A holds st0's codes on entry).
template <int MODE, int PS, int R>
__device__ __forceinline__ void ov_run(const GroupedArgs& a, const OvShape& h, OvCodes<PS>& A, rsrc_t cw, int m,
                                       int st0, int st1, int cb, int cq, int j, int gb, int rc, int nr,
                                       const int* prow, const uint32_t* xrow, const float* xsum, const uint16_t* ssc,
                                       const uint32_t* szr, uint32_t msk, float* __restrict__ gu) {
    OvCodes<PS> B;
    auto col = [&](int st) { return st * h.CS + 4 * cq + j; };
    auto voff = [&](int st) { return (uint32_t)col(st) * (h.I / 2) + 16u * gb; };
    for (int st = st0; st < st1; st += 2) {
        if (st + 1 < st1) ov_load<PS>(B, cw, voff(st + 1), h.NG);
        ov_compute<MODE, PS, R>(a, h, A, m, col(st), col(st) - cb, gb, rc, nr, prow, xrow, xsum, ssc, szr, msk, gu);
        if (st + 2 < st1) ov_load<PS>(A, cw, voff(st + 2), h.NG);
        if (st + 1 < st1)
            ov_compute<MODE, PS, R>(a, h, B, m, col(st + 1), col(st + 1) - cb, gb, rc, nr, prow, xrow, xsum, ssc, szr,
                                    msk, gu);
    }
}

// Rows by pair (one wave): the pairs q with pe[q] == e, ascending, into
// prow; info[0] = their count, info[1] = whether one precedes pair p.
__device__ __forceinline__ void ov_pair_rows(const int32_t* __restrict__ pe, int P, int p, int e, int lane,
                                             int* prow, int* info) {
    constexpr int kB = 4;  // 64-pair chunks loaded at a time
    const uint64_t below = lane ? (~0ull >> (kWave - lane)) : 0ull;
    int n = 0;
    bool dup = false;
    for (int u0 = 0; u0 * kWave < P; u0 += kB) {
        int v[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) v[u] = pe[min((u0 + u) * kWave + lane, P - 1)];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int q = (u0 + u) * kWave + lane;
            const bool hit = q < P && v[u] == e;
            const uint64_t mk = __ballot(hit);
            dup |= __ballot(hit && q < p) != 0;
            const int pos = n + __popcll(mk & below);
            if (hit && pos < kPairModeMaxT) prow[pos] = q;
            n += __popcll(mk);
        }
    }
    if (lane == 0) {
        info[0] = min(n, kPairModeMaxT);
        info[1] = dup;
    }
}

// Waves per SIMD: four (128 registers) unless the codes of two sets in flight
// need more (from 3 passes), then three or two, rather than spilling.
constexpr int ov_waves_per_simd(int PS) { return PS >= 6 ? 2 : PS >= 3 ? 3 : 4; }

// grid (NM x NWG column chunks, expert slot); block 4 waves, each wave SPW
// consecutive column sets of one projection.  MODE 0: gate and up -> gu
// [P][2F] fp32; MODE 1: h = bf16(silu(gate) up), formed while staging, ->
// rows.  Dynamic LDS of ov_lds_bytes(h).
template <int MODE, int PS>
__global__ __launch_bounds__(kOvThreads) __attribute__((amdgpu_waves_per_eu(ov_waves_per_simd(PS))))
void ov_kernel(GroupedArgs a, OvShape h, float* __restrict__ gu) {
    extern __shared__ __attribute__((aligned(16))) uint32_t ov_lds[];
    __shared__ int prow_lds[kPairModeMaxT];  // rows by pair: this expert's pairs, ascending
    __shared__ int pinfo[2];                 // their count, and whether an earlier pair has the expert
    uint32_t* xs = ov_lds;                                              // [4][I/2]
    float* xsum = reinterpret_cast<float*>(ov_lds + 2 * h.I);           // [G][4]
    uint16_t* ssc = reinterpret_cast<uint16_t*>(xsum + 4 * h.G);        // [G][CW]
    uint32_t* szr = reinterpret_cast<uint32_t*>(ssc + (size_t)h.G * h.CW);  // [G][CW/8]
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    int r0 = 0, r1 = a.T, e = 0;
    const int* prow = nullptr;
    if (a.pair_expert) {
        // workgroup y = pair p: it runs only when p is the first pair of its
        // expert, and then takes every pair of that expert in ascending order
        // (the rows a stable sort by expert would give it).  The pairs are
        // scanned while the first codes are in flight (below); until then the
        // workgroup has one row.
        e = a.pair_expert[blockIdx.y];
        r1 = 1;
        prow = prow_lds;
    } else if (a.offsets) {
        e = slot_expert(a.slots, blockIdx.y, &r0, &r1);
        if (e < 0) return;  // whole workgroup
    }
    const int I = h.I, O = h.O, G = h.G, nb8 = I / 8, nsets = O / h.CS;
    const int m = blockIdx.x / h.NWG, chunk = blockIdx.x % h.NWG;
    const int j = lane & 3, b = lane >> 2, gb = b % h.NG, cq = b / h.NG;
    const int cb = chunk * h.CW;
    const int st0 = (chunk * kOvWaves + wave) * h.SPW, st1 = min(st0 + h.SPW, nsets);
    // this projection's arrays as plain pointers (taking the address of a
    // kernel argument would copy the arguments to scratch memory)
    const int32_t* qw = MODE == 1 ? a.down.qweight : m ? a.up.qweight : a.gate.qweight;
    const int32_t* qz = MODE == 1 ? a.down.qzeros : m ? a.up.qzeros : a.gate.qzeros;
    const uint16_t* sc = MODE == 1 ? a.down.scales : m ? a.up.scales : a.gate.scales;
    const rsrc_t cw = ov_rsrc(qw + (size_t)e * O * (I / 8), (uint32_t)O * (I / 2));
    const uint32_t msk = ov_mask();
    // Staging: the scales and zero words of the workgroup's columns go from
    // memory straight into LDS (16- and 4-byte buffer loads to LDS: item
    // it = g sv + v of a wave lands at its LDS base + lane x size), all in
    // flight at once and in no register; the rows go through registers in
    // batches whose loads are all issued before the first is used.  (A
    // load-then-store loop waited a memory round trip per item: five for the
    // scales and zero words, two for the rows.)
    constexpr int kXB = MODE == 0 ? 2 : 1;  // row items a thread loads at once
    static_assert(MODE != 0 || kOvMaxIn / 8 <= kOvThreads * kXB, "a row's items fit one batch");
    const int sv = h.CW / 8;                // 16-byte scale vectors, and zero words, a group row
    const int nst = G * sv;
    const rsrc_t rsc = ov_rsrc(sc + (size_t)e * G * O, (uint32_t)G * O * 2u);
    const rsrc_t rzr = ov_rsrc(qz + (size_t)e * G * (O / 8), (uint32_t)G * (O / 8) * 4u);
    auto stage_scales = [&]() {
        if (nst % kOvThreads == 0) {
            // every wave's 64 items exist; columns past O read the next group
            // row or, past the last, 0 (those columns are never computed)
            for (int u0 = 0; u0 < nst; u0 += kOvThreads) {
                const int it = u0 + threadIdx.x, g = it / sv, c0 = cb + 8 * (it % sv);
                const int wb = u0 + wave * kWave;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (__attribute__((address_space(3))) void*)(ssc + 8 * wb), 16,
                                                         (g * O + c0) * 2, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rzr, (__attribute__((address_space(3))) void*)(szr + wb), 4,
                                                         (g * (O / 8) + c0 / 8) * 4, 0, 0, 0);
            }
        } else {
            for (int it = threadIdx.x; it < nst; it += kOvThreads) {
                const int g = it / sv, v = it % sv, c0 = cb + 8 * v;
                u32x4_t val = {0u, 0u, 0u, 0u};
                if (c0 < O) val = *reinterpret_cast<const u32x4_t*>(sc + ((size_t)e * G + g) * O + c0);
                *reinterpret_cast<u32x4_t*>(ssc + g * h.CW + 8 * v) = val;
                szr[g * sv + v] = c0 < O ? (uint32_t)qz[((size_t)e * G + g) * (O / 8) + c0 / 8] : 0u;
            }
        }
    };
    for (int rc = r0; rc < r1; rc += 4) {
        OvCodes<PS> A;
        // the first set's codes, the scales and the zero words are in flight
        // while the workgroup finds its rows and stages them
        if (st0 < st1) ov_load<PS>(A, cw, (uint32_t)(st0 * h.CS + 4 * cq + j) * (I / 2) + 16u * gb, h.NG);
        if (rc == r0) stage_scales();
        // stage item (row i, inputs 8 w8 .. +7) from its 8 bf16 inputs v: LDS
        // in the order 0,4,1,5,2,6,3,7, and the group sums (a thread sums its
        // 8 inputs in order, then the 4 threads of a group, consecutive lanes
        // all active together, add theirs in a fixed order)
        auto stage_item = [&](int i, int w8, const u32x4_t& v) {
            u32x4_t o;
            o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // (x0, x4)
            o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // (x1, x5)
            o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);  // (x2, x6)
            o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);  // (x3, x7)
            *reinterpret_cast<u32x4_t*>(&xs[i * (I / 2) + 4 * w8]) = o;
            float sum = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) sum += bf16_to_f32(v[q] & 0xFFFFu) + bf16_to_f32(v[q] >> 16);
            sum += __shfl_xor(sum, 1, kWave);
            sum += __shfl_xor(sum, 2, kWave);
            if ((w8 & 3) == 0) xsum[4 * (w8 >> 2) + i] = sum;
        };
        // gate/up: the first row's token is known before the pair scan (the
        // workgroup's own pair, or the slot's first row), so its inputs load
        // with the first codes and are staged before the barrier (no earlier
        // chunk reads the stage); wave 0 scans the pairs first
        int first = 0;  // first item staged after the barrier
        if constexpr (MODE == 0) {
            if (rc == r0) {
                const int t0 = prow ? (int)blockIdx.y / a.k : a.sorted_pair ? a.sorted_pair[r0] / a.k : r0;
                u32x4_t pre[kXB];
#pragma unroll
                for (int u = 0; u < kXB; ++u) {
                    const int it = threadIdx.x + kOvThreads * u;
                    if (it < nb8) pre[u] = *reinterpret_cast<const u32x4_t*>(a.x + (size_t)t0 * I + 8 * it);
                }
                if (prow && wave == 0) ov_pair_rows(a.pair_expert, a.P, (int)blockIdx.y, e, lane, prow_lds, pinfo);
#pragma unroll
                for (int u = 0; u < kXB; ++u) {
                    const int it = threadIdx.x + kOvThreads * u;
                    if (it < nb8) stage_item(0, it, pre[u]);
                }
                first = nb8;
            }
        }
        if (MODE != 0 && prow && rc == r0 && wave == 0)
            ov_pair_rows(a.pair_expert, a.P, (int)blockIdx.y, e, lane, prow_lds, pinfo);
        __syncthreads();  // the previous chunk's rows have been read; the pair scan is done
        if (prow && rc == r0) {
            if (pinfo[1]) {
                // whole workgroup: an earlier pair has the expert.  Its loads
                // to LDS land before it ends, so that none writes the LDS of
                // a workgroup that takes its place
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
                return;
            }
            r1 = pinfo[0];
        }
        const int nr = min(4, r1 - rc);
        // the chunk's other rows, in batches whose loads all go out first
        const int nx = nr * nb8;
        for (int x0 = first; x0 < nx; x0 += kOvThreads * kXB) {
            u32x4_t ld[kXB][MODE == 0 ? 1 : 4];
#pragma unroll
            for (int u = 0; u < kXB; ++u) {
                const int it = x0 + threadIdx.x + kOvThreads * u;
                if (it < nx) {
                    const int i = it / nb8, w8 = it % nb8;
                    if constexpr (MODE == 0) {
                        const int t = prow ? prow[rc + i] / a.k : a.sorted_pair ? a.sorted_pair[rc + i] / a.k : rc + i;
                        ld[u][0] = *reinterpret_cast<const u32x4_t*>(a.x + (size_t)t * I + 8 * w8);
                    } else {
                        const float* gr = gu + (size_t)(prow ? prow[rc + i] : rc + i) * (2 * I) + 8 * w8;
                        ld[u][0] = *reinterpret_cast<const u32x4_t*>(gr);
                        ld[u][1] = *reinterpret_cast<const u32x4_t*>(gr + 4);
                        ld[u][2] = *reinterpret_cast<const u32x4_t*>(gr + I);
                        ld[u][3] = *reinterpret_cast<const u32x4_t*>(gr + I + 4);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kXB; ++u) {
                const int it = x0 + threadIdx.x + kOvThreads * u;
                if (it >= nx) continue;  // whole groups of 4 lanes (nb8 % 4 == 0)
                const int i = it / nb8, w8 = it % nb8;
                u32x4_t v;  // x0x1 x2x3 x4x5 x6x7
                if constexpr (MODE == 0) {
                    v = ld[u][0];
                } else {
                    const f32x4_t g0 = __builtin_bit_cast(f32x4_t, ld[u][0]), g1 = __builtin_bit_cast(f32x4_t, ld[u][1]);
                    const f32x4_t u0 = __builtin_bit_cast(f32x4_t, ld[u][2]), u1 = __builtin_bit_cast(f32x4_t, ld[u][3]);
                    v.x = pack_bf16x2(silu(g0.x) * u0.x, silu(g0.y) * u0.y);
                    v.y = pack_bf16x2(silu(g0.z) * u0.z, silu(g0.w) * u0.w);
                    v.z = pack_bf16x2(silu(g1.x) * u1.x, silu(g1.y) * u1.y);
                    v.w = pack_bf16x2(silu(g1.z) * u1.z, silu(g1.w) * u1.w);
                }
                stage_item(i, w8, v);
            }
        }
        // every load of this wave has landed (the scales and zero words in
        // LDS among them) before the barrier publishes the stage
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) (bits 3:0 and 15:14), expcnt and lgkmcnt at their maxima
        __syncthreads();
        if (st0 < st1) {
            const uint32_t* xrow = xs + min(j, nr - 1) * (I / 2);  // rows past nr repeat the last
            if (nr == 1)
                ov_run<MODE, PS, 1>(a, h, A, cw, m, st0, st1, cb, cq, j, gb, rc, nr, prow, xrow, xsum, ssc, szr, msk, gu);
            else if (nr == 2)
                ov_run<MODE, PS, 2>(a, h, A, cw, m, st0, st1, cb, cq, j, gb, rc, nr, prow, xrow, xsum, ssc, szr, msk, gu);
            else
                ov_run<MODE, PS, 4>(a, h, A, cw, m, st0, st1, cb, cq, j, gb, rc, nr, prow, xrow, xsum, ssc, szr, msk, gu);
        }
    }
}

// Blocks per column (NG) for G groups: the largest of 16, 8, 4, 2, 1 dividing
// G with at most kOvMaxPass passes; 0 when none does.
int ov_blocks(int G) {
    for (int ng = 16; ng >= 1; ng >>= 1)
        if (G % ng == 0 && G / ng <= kOvMaxPass) return ng;
    return 0;
}

size_t ov_table_bytes(int P) { return ((size_t)P * sizeof(int4) + 255) & ~(size_t)255; }

constexpr size_t kOvMaxLds = 64 << 10;

// Launch shape of one projection pass (SPW halved until the LDS fits).
OvShape ov_shape(int MODE, int I, int O) {
    OvShape h;
    h.I = I;
    h.O = O;
    h.G = I / 32;
    h.NG = ov_blocks(h.G);
    h.CS = h.NG ? 64 / h.NG : 0;
    h.NM = MODE == 0 ? 2 : 1;
    h.SPW = kOvSetsPerWave;
    for (;;) {
        h.CW = kOvWaves * h.SPW * h.CS;
        if (h.SPW == 1 || ov_lds_bytes(h) <= kOvMaxLds) break;
        h.SPW /= 2;
    }
    h.NWG = h.CS ? (O / h.CS + kOvWaves * h.SPW - 1) / (kOvWaves * h.SPW) : 0;
    return h;
}

template <int MODE>
hipError_t ov_launch(const GroupedArgs& a, int I, int O, int slots, float* gu, hipStream_t s) {
    const OvShape h = ov_shape(MODE, I, O);
    const size_t lds = ov_lds_bytes(h);
    if (!h.NG || lds > kOvMaxLds) return hipErrorInvalidValue;
    const dim3 grid(h.NM * h.NWG, slots);
    switch (h.G / h.NG) {
#define MOE_OV(N) \
    case N: hipLaunchKernelGGL((ov_kernel<MODE, N>), grid, dim3(kOvThreads), lds, s, a, h, gu); break;
        MOE_OV(1) MOE_OV(2) MOE_OV(3) MOE_OV(4) MOE_OV(5) MOE_OV(6) MOE_OV(7) MOE_OV(8)
#undef MOE_OV
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool om_gemv_supported(int H, int F) {
    if (H % 64 || F % 64 || H > kOvMaxIn || F > kOvMaxIn) return false;
    const OvShape g = ov_shape(0, H, F), d = ov_shape(1, F, H);
    return g.NG && d.NG && ov_lds_bytes(g) <= kOvMaxLds && ov_lds_bytes(d) <= kOvMaxLds;
}

// slot table, then gu [P][2F] fp32
size_t om_gemv_ws_bytes(int P, int F) { return ov_table_bytes(P) + (size_t)P * 2 * F * sizeof(float); }

hipError_t launch_om_gemv(const GroupedArgs& a0, void* ws, hipStream_t s) {
    GroupedArgs a = a0;
    char* w = static_cast<char*>(ws);
    if (a.pair_expert) {
        a.slots = nullptr;  // one workgroup slot per pair
    } else if (a.offsets) {
        if (!a.slots) a.slots = launch_slot_table(a.offsets, a.E, a.P, reinterpret_cast<int4*>(w), s);
    } else {
        a.slots = nullptr;
    }
    float* gu = reinterpret_cast<float*>(w + ov_table_bytes(a.P));
    const int slots = a.pair_expert ? a.P : a.offsets ? (a.P < a.E ? a.P : a.E) : 1;
    hipError_t err = ov_launch<0>(a, a.H, a.F, slots, gu, s);
    if (err != hipSuccess) return err;
    return ov_launch<1>(a, a.F, a.H, slots, gu, s);
}

}  // namespace moe

// Grouped SwiGLU experts for many rows per expert (prefill): bf16 MFMA GEMM.
//
// Qwen3.8-Flash-Next architecture sheet, FFN / MoE entries: SwiGLU experts
// (gate, up, down), no bias, no clamp.  AWQ-g32 card, "Checkpoint" and
// "Calibration": asymmetric W4A16, group 32 along the input, integer zeros,
// fp16 scales, GEMM packing, w = (q - z) * s.
//
// Two passes per bank, both a grouped GEMM over the rows of each expert:
//   gate/up: h[r] = silu(W_gate x_t) * (W_up x_t)   A = gathered token rows
//   down:    rows[r] = W_down h[r]                  A = h rows (contiguous)
// Workgroup tile: BM rows (64, 128 or 256, from the average rows per expert)
// x 128 B-columns, K step 32 (= one AWQ group), BM/32 waves as BM/64 (rows)
// x 2 (columns), each wave 64 x 64 on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  For gate/up the 128
// B-columns are 64 gate and the same 64 up columns, so SwiGLU is applied in
// registers.  A and B tiles are staged in LDS, double buffered through
// registers.
//
// AWQ B tile: each thread owns one input row of one packed word (8 columns).
// A code q is placed in the top mantissa bits of an fp32 with exponent 2^4,
// giving m = 16 + q exactly; with c = -(16 + z) * s (exact: 5 x 11 bits),
// fma(m, s, c) = (q - z) * s exactly, then one RNE to bf16.  s and c per
// column of the group are computed once per K step by 128 threads into LDS.
//
// Tiles are enumerated per expert (ceil(rows / BM) each) by a small kernel;
// workgroup ids are remapped so that each XCD (ids are dealt round-robin over
// 8 XCDs) works on a contiguous range of tiles with the column tiles of one
// row tile adjacent: the A rows and the expert's weights are then reused from
// that XCD's L2.
#include "ffn_internal.h"

namespace moe {

constexpr int kBN = 128, kBK = 32, kLDK = kBK + 8;  // LDS row stride (bf16)
constexpr int kXcd = 8;

enum { MODE_GATEUP = 0, MODE_DOWN = 1 };

// ---------------------------------------------------------------------------
// Tile table: tiles[0] = number of tiles, then pairs (expert, first row).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ offsets, int E,
                                                         int P, int BM, int32_t* __restrict__ tiles) {
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
        tiles[1 + 2 * (start + i)] = e;
        tiles[2 + 2 * (start + i)] = r0 + i * BM;
    }
    if (e == 1023) tiles[0] = scan[1023];
}

__device__ __forceinline__ int xcd_remap(int p, int G) {
    const int q = G / kXcd, r = G % kXcd;
    const int x = p % kXcd, i = p / kXcd;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// Packing order {0,2,4,6,1,3,5,7}: nibble j holds column awq_perm(j) of its word.
__device__ __forceinline__ int awq_perm(int j) { return (j < 4) ? 2 * j : 2 * (j - 4) + 1; }
__device__ __forceinline__ int awq_nibble_of_col(int c8) { return (c8 & 1) ? 4 + (c8 >> 1) : (c8 >> 1); }

template <int MODE, bool AWQ, int BM>
__global__ __launch_bounds__(2 * BM) void grouped_gemm_kernel(GroupedArgs a,
                                                                    const int32_t* __restrict__ tiles,
                                                                    uint16_t* __restrict__ hbuf,
                                                                    int NT) {
    constexpr int kThreads = 2 * BM;  // waves: (BM/64) along rows x 2 along columns
    constexpr int kBPer = kBN * kBK / 8 / kThreads;  // B items per thread
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kLDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kLDK];
    __shared__ __attribute__((aligned(16))) float2 Ps[2][kBN];  // AWQ (s, -(16+z)s) per column

    const int l = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = l / NT, nt = l % NT;
    if (tile >= tiles[0]) return;
    const int e = tiles[1 + 2 * tile];
    const int m0 = tiles[2 + 2 * tile];
    const int m1 = a.offsets ? min(m0 + BM, (int)a.offsets[e + 1]) : min(m0 + BM, a.P);

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / 2, wn = wave % 2;
    const int H = a.H, F = a.F;
    const int K = MODE == MODE_GATEUP ? H : F;       // reduction dim
    const int NOUT = MODE == MODE_GATEUP ? F : H;    // output dim of the projection(s)
    const int n0 = MODE == MODE_GATEUP ? nt * (kBN / 2) : nt * kBN;
    const int nk = K / kBK;

    // ---- A sources: 2 x 16-byte chunks per thread: chunk q -> row q/4, k-offset (q%4)*8
    const uint16_t* asrc[2];
    int arow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = tid + i * kThreads;
        const int row = q / 4, kc = q % 4;
        arow[i] = row;
        const int gr = min(m0 + row, m1 - 1);
        if (MODE == MODE_GATEUP) {
            const int t = a.sorted_pair ? a.sorted_pair[gr] / a.k : gr;
            asrc[i] = a.x + (size_t)t * H + kc * 8;
        } else {
            asrc[i] = hbuf + (size_t)gr * F + kc * 8;
        }
    }
    // ---- B sources, kBPer items per thread (item u = tid + i*kThreads)
    // bf16: a 16-byte chunk: B-column bc = u/4, k-offset (u%4)*8
    // awq : one packed word: k-row kr = u/16, word column wc = u%16
    const uint16_t* bsrc[kBPer];
    const int32_t* wsrc[kBPer];
    const int32_t* zsrc = nullptr;
    const uint16_t* ssrc = nullptr;
    int pcol = 0;  // AWQ: the B-column whose (s, c) this thread prepares (tid < kBN)
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
        const int u = tid + i * kThreads;
        if (!AWQ) {
            const int bc = u / 4, kc = u % 4;
            const uint16_t* W;
            int col;
            if (MODE == MODE_GATEUP) {
                W = (bc < kBN / 2 ? a.gate.w : a.up.w) + (size_t)e * F * H;
                col = n0 + bc % (kBN / 2);
            } else {
                W = a.down.w + (size_t)e * H * F;
                col = n0 + bc;
            }
            bsrc[i] = W + (size_t)col * K + kc * 8;
            wsrc[i] = nullptr;
        } else {
            const int kr = u / 16, wc = u % 16;
            const ProjDev& pj = MODE == MODE_GATEUP ? (wc < 8 ? a.gate : a.up) : a.down;
            const int OW = NOUT / 8;
            const int word = MODE == MODE_GATEUP ? n0 / 8 + wc % 8 : n0 / 8 + wc;
            wsrc[i] = pj.qweight + (size_t)e * K * OW + (size_t)kr * OW + word;
            bsrc[i] = nullptr;
        }
    }
    if (AWQ && tid < kBN) {
        pcol = tid;
        const ProjDev& pp = MODE == MODE_GATEUP ? (tid < 64 ? a.gate : a.up) : a.down;
        const int col = MODE == MODE_GATEUP ? n0 + tid % 64 : n0 + tid;
        const int OW = NOUT / 8;
        zsrc = pp.qzeros + (size_t)e * (K / 32) * OW + col / 8;
        ssrc = pp.scales + (size_t)e * (K / 32) * NOUT + col;
    }

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    uint4 areg[2];
    uint4 breg[kBPer];
    uint32_t wreg[kBPer];

    auto load_global = [&](int kt) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < 2; ++i) areg[i] = *reinterpret_cast<const uint4*>(asrc[i] + k0);
#pragma unroll
        for (int i = 0; i < kBPer; ++i) {
            if (!AWQ) breg[i] = *reinterpret_cast<const uint4*>(bsrc[i] + k0);
            else wreg[i] = (uint32_t)wsrc[i][(size_t)k0 * (NOUT / 8)];
        }
    };
    // AWQ per-column parameters of group kt into Ps[buf]
    auto make_params = [&](int kt, int buf) {
        if (AWQ && tid < kBN) {
            const int OW = NOUT / 8;
            const uint32_t zw = (uint32_t)zsrc[(size_t)kt * OW];
            const int c8 = (MODE == MODE_GATEUP ? n0 + pcol % 64 : n0 + pcol) % 8;
            const float z = (float)((zw >> (4 * awq_nibble_of_col(c8))) & 15u);
            const float s = f16_to_f32(ssrc[(size_t)kt * NOUT]);
            Ps[buf][pcol] = make_float2(s, -(16.0f + z) * s);
        }
    };
    auto store_lds = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = tid + i * kThreads;
            *reinterpret_cast<uint4*>(&As[buf][arow[i] * kLDK + (q % 4) * 8]) = areg[i];
        }
#pragma unroll
        for (int ii = 0; ii < kBPer; ++ii) {
            const int u = tid + ii * kThreads;
            if (!AWQ) {
                const int bc = u / 4, kc = u % 4;
                *reinterpret_cast<uint4*>(&Bs[buf][bc * kLDK + kc * 8]) = breg[ii];
            } else {
                const int kr = u / 16, wc = u % 16;
                const int cbase = MODE == MODE_GATEUP ? (wc / 8) * 64 + (wc % 8) * 8 : wc * 8;
                const float4* pv = reinterpret_cast<const float4*>(&Ps[buf][cbase]);
                float s[8], c[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 v = pv[i];
                    s[2 * i] = v.x; c[2 * i] = v.y; s[2 * i + 1] = v.z; c[2 * i + 1] = v.w;
                }
                // bytes with the code in bits 3..6 and bit 7 set (the exponent LSB)
                const uint32_t even = ((wreg[ii] << 3) & 0x78787878u) | 0x80808080u;  // nibbles 0,2,4,6
                const uint32_t odd = ((wreg[ii] >> 1) & 0x78787878u) | 0x80808080u;   // nibbles 1,3,5,7
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t src = (j & 1) ? odd : even;
                    const int b = j >> 1;
                    // float bits 0x41 | byte | 00 | 00  ->  16 + q
                    const uint32_t mbits =
                        __builtin_amdgcn_perm(0x41000000u, src, 0x07000C0Cu | ((uint32_t)b << 16));
                    const int col = awq_perm(j);
                    const float w = fmaf(__uint_as_float(mbits), s[col], c[col]);
                    const __bf16 wb = (__bf16)w;
                    Bs[buf][(cbase + col) * kLDK + kr] = __builtin_bit_cast(uint16_t, wb);
                }
            }
        }
    };

    // prologue: step 0
    load_global(0);
    make_params(0, 0);
    __syncthreads();
    store_lds(0);

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1, nxt = cur ^ 1;
        __syncthreads();  // As/Bs[cur] complete; all reads of [nxt] done
        const bool more = kt + 1 < nk;
        if (more) {
            load_global(kt + 1);
            make_params(kt + 1, nxt);
        }
        // MFMA on the current tiles
        bf16x8_t af[4], bfr[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            af[mi] = *reinterpret_cast<const bf16x8_t*>(
                &As[cur][(wm * 64 + mi * 16 + lane % 16) * kLDK + (lane / 16) * 8]);
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
            const int bcol = MODE == MODE_GATEUP ? (nj / 2) * 64 + wn * 32 + (nj % 2) * 16
                                                 : wn * 64 + nj * 16;
            bfr[nj] = *reinterpret_cast<const bf16x8_t*>(
                &Bs[cur][(bcol + lane % 16) * kLDK + (lane / 16) * 8]);
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int nj = 0; nj < 4; ++nj)
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[nj], acc[mi][nj], 0, 0, 0);
        if (more) {
            if (AWQ) __syncthreads();  // Ps[nxt] visible to every thread
            store_lds(nxt);
        }
    }

    // ---- epilogue: lane holds C[4*(lane/16) + r][lane%16] of each 16x16 tile
    const int rbase = m0 + wm * 64 + 4 * (lane / 16);
    if (MODE == MODE_GATEUP) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int nj = 0; nj < 2; ++nj) {
                const int col = n0 + wn * 32 + nj * 16 + lane % 16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = rbase + mi * 16 + r;
                    if (row < m1) {
                        const float g = acc[mi][nj][r], u = acc[mi][nj + 2][r];
                        hbuf[(size_t)row * F + col] = (uint16_t)f32_to_bf16_bits(silu(g) * u);
                    }
                }
            }
    } else {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int nj = 0; nj < 4; ++nj) {
                const int col = n0 + wn * 64 + nj * 16 + lane % 16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = rbase + mi * 16 + r;
                    if (row < m1) {
                        const float v = acc[mi][nj][r];
                        const size_t o = (size_t)row * H + col;
                        if (a.out_f32) static_cast<float*>(a.rows)[o] = v;
                        else static_cast<uint16_t*>(a.rows)[o] = (uint16_t)f32_to_bf16_bits(v);
                    }
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int max_tiles(int P, int E, int BM) { return (P + BM - 1) / BM + E; }

// Row tile from the average rows per non-empty expert.
static int pick_bm(int P, int E) {
    const int active = P < E ? P : E;
    const int avg = active > 0 ? P / active : 0;
    return avg >= 192 ? 256 : (avg >= 96 ? 128 : 64);
}

size_t gemm_ws_bytes(int P, int F, int E) {
    const size_t tiles = (size_t)(1 + 2 * max_tiles(P, E, 64)) * sizeof(int32_t);
    const size_t tiles_al = (tiles + 255) & ~(size_t)255;
    return tiles_al + (size_t)P * F * sizeof(uint16_t);
}

template <int BM>
static void launch_gemm_bm(const GroupedArgs& a, const int32_t* tiles, uint16_t* hbuf, int mt,
                           hipStream_t s) {
    const int NT1 = a.F / (kBN / 2), NT2 = a.H / kBN;
    if (a.awq) {
        hipLaunchKernelGGL((grouped_gemm_kernel<MODE_GATEUP, true, BM>), dim3(mt * NT1), dim3(2 * BM), 0,
                           s, a, tiles, hbuf, NT1);
        hipLaunchKernelGGL((grouped_gemm_kernel<MODE_DOWN, true, BM>), dim3(mt * NT2), dim3(2 * BM), 0,
                           s, a, tiles, hbuf, NT2);
    } else {
        hipLaunchKernelGGL((grouped_gemm_kernel<MODE_GATEUP, false, BM>), dim3(mt * NT1), dim3(2 * BM), 0,
                           s, a, tiles, hbuf, NT1);
        hipLaunchKernelGGL((grouped_gemm_kernel<MODE_DOWN, false, BM>), dim3(mt * NT2), dim3(2 * BM), 0,
                           s, a, tiles, hbuf, NT2);
    }
}

hipError_t launch_gemm(const GroupedArgs& a, void* ws, hipStream_t s) {
    const int E = a.offsets ? a.E : 1;
    const int BM = pick_bm(a.P, E);
    const int mt = max_tiles(a.P, E, BM);
    int32_t* tiles = static_cast<int32_t*>(ws);
    const size_t tiles_al =
        (((size_t)(1 + 2 * max_tiles(a.P, E, 64)) * sizeof(int32_t)) + 255) & ~(size_t)255;
    uint16_t* hbuf = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + tiles_al);
    hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, s, a.offsets, E, a.P, BM, tiles);
    if (BM == 256) launch_gemm_bm<256>(a, tiles, hbuf, mt, s);
    else if (BM == 128) launch_gemm_bm<128>(a, tiles, hbuf, mt, s);
    else launch_gemm_bm<64>(a, tiles, hbuf, mt, s);
    return hipGetLastError();
}

}  // namespace moe

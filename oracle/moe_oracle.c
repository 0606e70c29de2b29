/*
 * CPU oracle for the routed mixture-of-experts feed-forward layer.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load this library.  It shares
 * no code, header, table or helper with the HIP library; it reads the raw
 * input bytes (bf16 / fp16 bit patterns, packed int32 words) and decodes them
 * itself.
 *
 * Every floating-point step is plain IEEE double arithmetic with no blocking,
 * fusion or reordering beyond the definition being followed.  Build with
 * -ffp-contract=off so that no multiply-add is fused behind our back.
 *
 * Sources (web pages; cited by title and section):
 *  [ARCH]  "Qwen3.8-Flash-Next" architecture sheet, FFN / MoE entries:
 *          SwiGLU, no FFN bias, no GLU clamp, 512 routed experts, top-10,
 *          1 shared expert, expert width 640, softmax gating, selected
 *          weights renormalised to sum to 1.
 *  [AWQ]   "Qwen3.8-Flash-Next-AWQ-g32" card, sections "Checkpoint" and
 *          "Calibration": asymmetric W4A16, group 32, integer zero points,
 *          FP16 scales, codes clip(round(w/scale + zero), 0, 15), GEMM packing.
 *  [FP8]   "Qwen3.8-Flash-Next-AWQ-g32" card, "Optional FP8 MTP": routed
 *          experts stored in FP8 E4M3 with explicit block scales (the
 *          128 x 128 block and fp32 scales are this oracle's reading).
 *  [NVFP4] "cleyesode/Qwen3.8-Flash-Next-RAZOR-96B-A6B-NVFP4" card, precision
 *          table: routed experts NVFP4 W4A4, group 16, FP8 block scales,
 *          FP32 global scales (layouts and the activation recipe are this
 *          oracle's reading).
 *  [RAZOR] "Qwen3.8-Flash-Next-RAZOR-65B-A6B-E256of512" card, section
 *          "Selection and calibration": Refill-RMS saliency, RMS conditional on
 *          the tokens routed to each expert, additive statistics, keep-set in
 *          original-index order.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - router logits are the correctly rounded fp32 value of the exact dot
 *    product of the bf16 hidden state with the bf16 router row;
 *  - ranking is by logit descending, ties to the lower expert index
 *    (-0.0 and +0.0 compare equal);
 *  - AWQ GEMM packing: codes [E][in][out/8], zeros [E][in/32][out/8] int32,
 *    scales [E][in/32][out] fp16; nibble j (bits 4j..4j+3) of a word holds
 *    column 8c + PERM[j] with PERM = {0,2,4,6,1,3,5,7};
 *  - bf16 expert weights are stored [E][out][in] (row per output feature).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Bit-pattern decoding                                                       */
/* ------------------------------------------------------------------------- */

/* bf16 is the top half of an IEEE binary32; widening to double is exact. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16 decoded field by field; exact in double. */
static double fp16_value(uint16_t bits)
{
    int sign = bits >> 15;
    int expo = (bits >> 10) & 31;
    int frac = bits & 1023;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);                 /* subnormal */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), expo - 25);  /* normal */
    return sign ? -mag : mag;
}

/* ------------------------------------------------------------------------- */
/* O1: router logits, correctly rounded fp32 of the exact dot product         */
/* ------------------------------------------------------------------------- */

/*
 * Fast path: accumulate the exact bf16 x bf16 products in double and use the
 * TwoSum error term to certify that no addition rounded.  When every error
 * term is zero the double sum IS the exact sum, and one conversion to float
 * (round to nearest even) gives the answer.
 */
static int dot_certified(const uint16_t *a, const uint16_t *b, int64_t n, double *out)
{
    double s = 0.0;
    int exact = 1;
    for (int64_t i = 0; i < n; ++i) {
        double p = bf16_value(a[i]) * bf16_value(b[i]);  /* exact: 8b x 8b significands */
        double t = s + p;
        double bv = t - s;
        double err = (s - (t - bv)) + (p - bv);          /* Knuth TwoSum */
        if (err != 0.0)
            exact = 0;
        s = t;
    }
    *out = s;
    return exact;
}

/*
 * Plain definition: a fixed-point (Kulisch) accumulator wide enough to hold
 * any sum of bf16 x bf16 products exactly, then a single round-to-nearest-even
 * to binary32.
 *
 * A bf16 value is m * 2^q with integer 0 <= m < 256 and q = max(E,1) - 134
 * (E = biased exponent field).  A product is (m1*m2) * 2^(q1+q2) with
 * q1+q2 in [-266, 240] and m1*m2 < 2^16.  Bit i of the accumulator weighs
 * 2^(i - KUL_BIAS); 640 bits cover 2^31 terms with room to spare.
 */
#define KUL_LIMBS 10
#define KUL_BIAS 300

static void bf16_split(uint16_t bits, int *neg, uint32_t *mant, int *q)
{
    int e = (bits >> 7) & 0xFF;
    uint32_t f = bits & 0x7F;
    *neg = bits >> 15;
    if (e == 0) {
        *mant = f;
        *q = -133;
    } else {
        *mant = 128 + f;
        *q = e - 134;
    }
}

static void kul_add_shifted(uint64_t acc[KUL_LIMBS], uint64_t v, int shift, int negative)
{
    /* v < 2^16 placed at bit `shift`; spans at most two limbs. */
    int limb = shift / 64, off = shift % 64;
    uint64_t lo = v << off;
    uint64_t hi = off ? (v >> (64 - off)) : 0;
    uint64_t addend[KUL_LIMBS];
    memset(addend, 0, sizeof addend);
    addend[limb] = lo;
    if (limb + 1 < KUL_LIMBS)
        addend[limb + 1] = hi;
    if (!negative) {
        uint64_t carry = 0;
        for (int i = 0; i < KUL_LIMBS; ++i) {
            uint64_t s = acc[i] + addend[i];
            uint64_t c1 = s < acc[i];
            uint64_t s2 = s + carry;
            uint64_t c2 = s2 < s;
            acc[i] = s2;
            carry = c1 | c2;
        }
    } else {
        uint64_t borrow = 0;
        for (int i = 0; i < KUL_LIMBS; ++i) {
            uint64_t d = acc[i] - addend[i];
            uint64_t b1 = acc[i] < addend[i];
            uint64_t d2 = d - borrow;
            uint64_t b2 = d < borrow;
            acc[i] = d2;
            borrow = b1 | b2;
        }
    }
}

static int kul_bit(const uint64_t acc[KUL_LIMBS], int i)
{
    return (int)((acc[i / 64] >> (i % 64)) & 1u);
}

static float kul_round_f32(const uint64_t acc_in[KUL_LIMBS])
{
    uint64_t acc[KUL_LIMBS];
    memcpy(acc, acc_in, sizeof acc);
    int negative = (int)(acc[KUL_LIMBS - 1] >> 63);
    if (negative) { /* two's complement negate */
        uint64_t carry = 1;
        for (int i = 0; i < KUL_LIMBS; ++i) {
            uint64_t v = ~acc[i] + carry;
            carry = (carry && v == 0) ? 1 : 0;
            acc[i] = v;
        }
    }
    int top = -1;
    for (int i = KUL_LIMBS * 64 - 1; i >= 0; --i)
        if (kul_bit(acc, i)) { top = i; break; }
    if (top < 0)
        return 0.0f;
    /* binary32 keeps 24 significant bits; its smallest ulp is 2^-149. */
    int lsb = top - 23;
    if (lsb < KUL_BIAS - 149)
        lsb = KUL_BIAS - 149;
    uint64_t mant = 0;
    for (int i = top; i >= lsb; --i)
        mant = (mant << 1) | (uint64_t)kul_bit(acc, i);
    int guard = lsb - 1 >= 0 ? kul_bit(acc, lsb - 1) : 0;
    int sticky = 0;
    for (int i = lsb - 2; i >= 0; --i)
        if (kul_bit(acc, i)) { sticky = 1; break; }
    if (guard && (sticky || (mant & 1u)))
        mant += 1;
    double mag = ldexp((double)mant, lsb - KUL_BIAS); /* exact: mant <= 2^24 */
    float r = (float)mag;                              /* exact, or overflow to inf */
    return negative ? -r : r;
}

static float dot_exact_kulisch(const uint16_t *a, const uint16_t *b, int64_t n)
{
    uint64_t acc[KUL_LIMBS];
    memset(acc, 0, sizeof acc);
    for (int64_t i = 0; i < n; ++i) {
        int na, nb, qa, qb;
        uint32_t ma, mb;
        bf16_split(a[i], &na, &ma, &qa);
        bf16_split(b[i], &nb, &mb, &qb);
        uint64_t m = (uint64_t)ma * mb;
        if (m == 0)
            continue;
        kul_add_shifted(acc, m, qa + qb + KUL_BIAS, na ^ nb);
    }
    return kul_round_f32(acc);
}

/* Exported for the tests: the plain definition on one pair of vectors. */
float oracle_dot_exact_f32(const uint16_t *a, const uint16_t *b, int64_t n)
{
    return dot_exact_kulisch(a, b, n);
}

/* Exported for the tests: the certified fast path; returns 1 when certified. */
int oracle_dot_certified(const uint16_t *a, const uint16_t *b, int64_t n, double *out)
{
    return dot_certified(a, b, n, out);
}

/*
 * logits[t][e] = RNE_fp32( sum_h x[t][h] * w_router[e][h] ), exactly.
 * Router rows are experts ([ARCH]: softmax gating over the expert logits; the
 * router has one row per expert and no bias -- pinned by the parameter counts).
 * Returns the number of logits that needed the fixed-point path.
 */
int64_t oracle_router_logits(const uint16_t *x, const uint16_t *w_router,
                             int64_t T, int64_t H, int64_t E, float *logits)
{
    int64_t fallbacks = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : fallbacks)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            double s;
            const uint16_t *xr = x + t * H, *wr = w_router + e * H;
            if (dot_certified(xr, wr, H, &s)) {
                logits[t * E + e] = (float)s;
            } else {
                logits[t * E + e] = dot_exact_kulisch(xr, wr, H);
                fallbacks += 1;
            }
        }
    }
    return fallbacks;
}

/* ------------------------------------------------------------------------- */
/* O2: ranking -- logit descending, ties to the lower expert index            */
/* ------------------------------------------------------------------------- */

/*
 * idx[t][0..n-1] = the first n experts of the total order.  Selection by
 * repeated arg-max; a strict '>' keeps the first (lowest) index on ties, and
 * -0.0 == +0.0 under '>'.  [ARCH] top-k routing; the tiny workload fixes ties
 * to the lowest index.  For Refill-RMS, position n-1 = k is the
 * "highest-ranked unselected expert" of [RAZOR].
 */
void oracle_rank(const float *logits, int64_t T, int64_t E, int64_t n, int32_t *idx)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        char *taken = (char *)calloc((size_t)E, 1);
        const float *l = logits + t * E;
        for (int64_t r = 0; r < n; ++r) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || l[e] > l[best])
                    best = e;
            }
            taken[best] = 1;
            idx[t * n + r] = (int32_t)best;
        }
        free(taken);
    }
}

/* ------------------------------------------------------------------------- */
/* O3: gates -- softmax over all experts, then renormalise the selected ones  */
/* ------------------------------------------------------------------------- */

/*
 * p_e = exp(l_e - max l) / sum_e' exp(l_e' - max l) over all E experts, then
 * g_j = p_{idx_j} / sum_{i in top-k} p_i ([ARCH]: softmax gating; selected
 * weights renormalised to sum to 1).  idx has row stride idx_stride >= k.
 */
void oracle_gates(const float *logits, const int32_t *idx, int64_t T, int64_t E,
                  int64_t k, int64_t idx_stride, double *gates)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        double m = -INFINITY;
        for (int64_t e = 0; e < E; ++e)
            if ((double)l[e] > m)
                m = (double)l[e];
        double denom = 0.0;
        for (int64_t e = 0; e < E; ++e)
            denom += exp((double)l[e] - m);
        double sel = 0.0;
        for (int64_t j = 0; j < k; ++j)
            sel += exp((double)l[idx[t * idx_stride + j]] - m) / denom;
        for (int64_t j = 0; j < k; ++j)
            gates[t * k + j] = (exp((double)l[idx[t * idx_stride + j]] - m) / denom) / sel;
    }
}

/* ------------------------------------------------------------------------- */
/* O4: permutation of (token, slot) pairs by expert                           */
/* ------------------------------------------------------------------------- */

/*
 * Stable counting sort of pair ids p = t*k + slot by expert idx[p]:
 * offsets[e] = number of pairs routed to experts < e (offsets[E] = T*k);
 * sorted_pair lists the pairs of expert 0, then expert 1, ..., each group in
 * ascending pair id; pair_to_row is its inverse.  The pages route each token
 * to its experts without spelling the grouping out; this is the plain one.
 */
void oracle_permute(const int32_t *idx, int64_t T, int64_t k, int64_t E,
                    int32_t *offsets, int32_t *sorted_pair, int32_t *pair_to_row)
{
    int64_t P = T * k;
    int64_t *count = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    for (int64_t p = 0; p < P; ++p)
        count[idx[p]] += 1;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + (int32_t)count[e];
    int64_t *cursor = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    for (int64_t e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (int64_t p = 0; p < P; ++p) {
        int64_t row = cursor[idx[p]]++;
        sorted_pair[row] = (int32_t)p;
        pair_to_row[p] = (int32_t)row;
    }
    free(count);
    free(cursor);
}

/* ------------------------------------------------------------------------- */
/* O5/O6: one SwiGLU expert, bf16 or AWQ W4 weights                           */
/* ------------------------------------------------------------------------- */

enum { ORA_BF16 = 0, ORA_AWQ = 1, ORA_FP8 = 2, ORA_NVFP4 = 3, ORA_AWQ_OM = 4 };

/* One projection of a bank of experts (out x in per expert). */
typedef struct {
    int32_t fmt;
    int32_t in_dim, out_dim;
    const uint16_t *w;       /* bf16: [E][out][in]                  */
    const int32_t *qweight;  /* awq:  [E][in][out/8]                */
                             /* awq, output-major codes: [E][out][in/8], nibble j
                                of word w holds input 8w + j            */
    const int32_t *qzeros;   /* awq:  [E][in/32][out/8]             */
    const uint16_t *scales;  /* awq:  [E][in/32][out] fp16          */
    const uint8_t *codes;    /* fp8:  [E][out][in] E4M3              */
                             /* nvfp4: [E][out][in/2], two E2M1 codes */
    const float *bscales;    /* fp8:  [E][out/128][in/128] fp32      */
    const uint8_t *gscales;  /* nvfp4: [E][out][in/16] E4M3          */
    const float *wglobal;    /* nvfp4: [E] fp32 weight global scale  */
    float aglobal;           /* nvfp4: activation global scale       */
} ora_proj;

typedef struct {
    int32_t num_experts, hidden, inter;
    ora_proj gate, up, down;
} ora_bank;

/* Nibble position that holds column (o mod 8) of a packed word: the inverse
 * of PERM = {0,2,4,6,1,3,5,7}. */
static int awq_nibble_of_column(int c8)
{
    return (c8 % 2 == 0) ? c8 / 2 : 4 + c8 / 2;
}

/* OCP FP8 E4M3 code to its exact value: sign bit, 4 exponent bits with bias
 * 7, 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); exponent
 * field 15 with mantissa 7 is NaN (there are no infinities, so 448 is the
 * largest finite magnitude). */
static double e4m3_value(uint8_t c)
{
    int sign = c >> 7, ex = (c >> 3) & 15, m = c & 7;
    double v;
    if (ex == 15 && m == 7)
        return NAN;
    if (ex == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, ex - 7);
    return sign ? -v : v;
}

/* Exported for the tests: the value of every E4M3 code. */
double oracle_e4m3_value(int code)
{
    return e4m3_value((uint8_t)code);
}

/* ---- NVFP4 ([NVFP4]: routed experts W4A4, FP4 values in groups of 16 with
 * FP8 E4M3 block scales and FP32 global scales). */

/* E2M1 code (sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0) to
 * its value; exponent field 0 is subnormal: 0 or 0.5. */
static double e2m1_value(int c)
{
    int sign = (c >> 3) & 1, ex = (c >> 1) & 3, m = c & 1;
    double v = ex == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, ex - 1);
    return sign ? -v : v;
}

/* Nearest E2M1 code to v (fp32), ties to the even code, magnitudes above 6
 * saturating to 6; a result of magnitude 0 is +0. */
static int e2m1_round(float v)
{
    static const float grid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    float a = fabsf(v);
    int best = 0;
    if (a > 6.0f)  /* saturation; past 2^22 the fp32 distances below would tie */
        return v < 0.0f ? 15 : 7;
    for (int c = 1; c < 8; ++c) {
        float dc = fabsf(a - grid[c]), db = fabsf(a - grid[best]);
        if (dc < db || (dc == db && (c & 1) == 0))
            best = c;
    }
    return (best != 0 && v < 0.0f) ? (best | 8) : best;
}

/* Nearest E4M3 code to f >= 0 (fp32), ties to even, saturating at 448:
 * the value grid is 2^-9 * k for k < 8 (subnormal) and (8 + m) * 2^(e - 10)
 * for exponent field e in 1..15 (the top code 15/7 excluded). */
static int e4m3_round(float f)
{
    if (!(f > 0.0f))
        return 0;
    if (f >= 448.0f)
        return 0x7E;
    double x = (double)f;  /* exact */
    int e = 0;
    frexp(x, &e);          /* x = r * 2^e, r in [0.5, 1) */
    int ex = e - 1 + 7;    /* exponent field if normal */
    double step = ex >= 1 ? ldexp(1.0, ex - 7 - 3) : ldexp(1.0, -9);
    double k = x / step;   /* exact: a power-of-two division */
    double kf = floor(k);
    double r = k - kf;
    double kr = (r > 0.5 || (r == 0.5 && fmod(kf, 2.0) != 0.0)) ? kf + 1.0 : kf;
    if (ex < 1) {          /* subnormal: k in [0, 8] */
        int ki = (int)kr;
        return ki >= 8 ? 0x08 : ki;  /* 8 * 2^-9 = 2^-6: exponent 1, mantissa 0 */
    }
    int ki = (int)kr;      /* in [8, 16] */
    if (ki == 16) { ki = 8; ex += 1; }
    if (ex > 15 || (ex == 15 && ki - 8 == 7))
        return 0x7E;
    return (ex << 3) | (ki - 8);
}

/* Exported for the tests. */
double oracle_e2m1_value(int code) { return e2m1_value(code); }
int oracle_e2m1_round(float v) { return e2m1_round(v); }
int oracle_e4m3_round(float f) { return e4m3_round(f); }

/* NVFP4 quantisation of n values (n a multiple of 16) with activation
 * global scale ga, every decision in fp32: per group of 16, the block scale
 * code is the E4M3 rounding of amax / (6 * ga); with block scale s, each
 * value's code is the E2M1 rounding of v / (s * ga).  out[i] receives
 * e2m1(code) * s (exact), i.e. the value without the global factor ga. */
void oracle_nvfp4_quantize(const float *v, int64_t n, float ga, double *out)
{
    for (int64_t g = 0; g < n; g += 16) {
        float amax = 0.0f;
        for (int i = 0; i < 16; ++i)
            amax = fmaxf(amax, fabsf(v[g + i]));
        float sf = amax / (6.0f * ga);
        double s = e4m3_value((uint8_t)e4m3_round(sf));
        for (int i = 0; i < 16; ++i) {
            if (s == 0.0) {
                out[g + i] = 0.0;
            } else {
                float d = (float)s * ga;
                out[g + i] = e2m1_value(e2m1_round(v[g + i] / d)) * s;
            }
        }
    }
}

/* Weight W[e][o][i] of a projection, decoded to an exact double.
 * AWQ: w = (q - z) * s, q and z integers in 0..15, s fp16 ([AWQ]).
 * FP8: w = e4m3(code) * block scale of the 128 x 128 block holding (o, i),
 * the product of a 4-bit and a 24-bit significand, exact in double. */
static double proj_weight(const ora_proj *p, int64_t e, int64_t o, int64_t i)
{
    if (p->fmt == ORA_BF16)
        return bf16_value(p->w[(e * p->out_dim + o) * p->in_dim + i]);
    if (p->fmt == ORA_FP8) {
        int64_t ob = p->out_dim / 128, ib = p->in_dim / 128;
        double s = (double)p->bscales[(e * ob + o / 128) * ib + i / 128];
        return e4m3_value(p->codes[(e * p->out_dim + o) * p->in_dim + i]) * s;
    }
    if (p->fmt == ORA_NVFP4) {
        uint8_t byte = p->codes[(e * p->out_dim + o) * (p->in_dim / 2) + i / 2];
        int c = (i % 2) ? (byte >> 4) : (byte & 15);
        double s = e4m3_value(p->gscales[(e * p->out_dim + o) * (p->in_dim / 16) + i / 16]);
        return e2m1_value(c) * s * (double)p->wglobal[e];
    }
    int64_t words = p->out_dim / 8, groups = p->in_dim / 32;
    int nib = awq_nibble_of_column((int)(o % 8));
    uint32_t qw;
    int qnib = nib;
    if (p->fmt == ORA_AWQ_OM) {
        /* the same codes stored with one word per 8 consecutive inputs of an
         * output column; zeros and scales as in the AWQ layout */
        qw = (uint32_t)p->qweight[(e * p->out_dim + o) * (p->in_dim / 8) + i / 8];
        qnib = (int)(i % 8);
    } else {
        qw = (uint32_t)p->qweight[(e * p->in_dim + i) * words + o / 8];
    }
    uint32_t zw = (uint32_t)p->qzeros[(e * groups + i / 32) * words + o / 8];
    int q = (int)((qw >> (4 * qnib)) & 15u);
    int z = (int)((zw >> (4 * nib)) & 15u);
    double s = fp16_value(p->scales[(e * groups + i / 32) * p->out_dim + o]);
    return (double)(q - z) * s;
}

/* Exported for the tests: dequantised weight W[e][o][i] of one projection. */
double oracle_proj_weight(const ora_proj *p, int64_t e, int64_t o, int64_t i)
{
    return proj_weight(p, e, o, i);
}

/* silu(a) = a / (1 + exp(-a)) */
static double silu(double a)
{
    return a / (1.0 + exp(-a));
}

/*
 * out = W_down[e] ( silu(W_gate[e] x) * (W_up[e] x) ), all in double with no
 * intermediate rounding ([ARCH]: SwiGLU, no bias, no clamp).
 */
static void expert_forward(const ora_bank *b, int64_t e, const double *x, double *out)
{
    int64_t H = b->hidden, F = b->inter;
    double *h = (double *)malloc((size_t)F * sizeof(double));
    const double *xin = x;
    double *xq = NULL;
    double ga_in = 1.0, ga_h = 1.0;
    if (b->gate.fmt == ORA_NVFP4) {
        /* W4A4: the input is quantised once for gate and up (shared
         * activation global scale of the gate/up pair) */
        float *xf = (float *)malloc((size_t)H * sizeof(float));
        xq = (double *)malloc((size_t)H * sizeof(double));
        for (int64_t i = 0; i < H; ++i)
            xf[i] = (float)x[i];  /* bf16 values: exact */
        oracle_nvfp4_quantize(xf, H, b->gate.aglobal, xq);
        free(xf);
        xin = xq;
        ga_in = (double)b->gate.aglobal;
        ga_h = (double)b->down.aglobal;
    }
    for (int64_t f = 0; f < F; ++f) {
        double a = 0.0, u = 0.0;
        for (int64_t i = 0; i < H; ++i) {
            a += proj_weight(&b->gate, e, f, i) * xin[i];
            u += proj_weight(&b->up, e, f, i) * xin[i];
        }
        h[f] = silu(a * ga_in) * (u * ga_in);
    }
    const double *hin = h;
    double *hq = NULL;
    if (b->gate.fmt == ORA_NVFP4) {
        /* the down projection's input is quantised too; its decisions are
         * taken on h rounded to fp32 */
        float *hf = (float *)malloc((size_t)F * sizeof(float));
        hq = (double *)malloc((size_t)F * sizeof(double));
        for (int64_t f = 0; f < F; ++f)
            hf[f] = (float)h[f];
        oracle_nvfp4_quantize(hf, F, b->down.aglobal, hq);
        free(hf);
        hin = hq;
    }
    for (int64_t o = 0; o < H; ++o) {
        double s = 0.0;
        for (int64_t f = 0; f < F; ++f)
            s += proj_weight(&b->down, e, o, f) * hin[f];
        out[o] = s * ga_h;
    }
    free(h);
    free(xq);
    free(hq);
}

static void x_row(const uint16_t *x, int64_t t, int64_t H, double *xd)
{
    for (int64_t i = 0; i < H; ++i)
        xd[i] = bf16_value(x[t * H + i]);
}

/*
 * Per-pair expert outputs: rows[p][:] = expert idx[p] applied to x[p / k].
 * Pair order p = t*k + slot (not the grouped order).
 */
void oracle_pair_outputs(const uint16_t *x, int64_t T, int64_t k, const int32_t *idx,
                         const ora_bank *bank, double *rows)
{
    int64_t H = bank->hidden;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < T * k; ++p) {
        double *xd = (double *)malloc((size_t)H * sizeof(double));
        x_row(x, p / k, H, xd);
        expert_forward(bank, idx[p], xd, rows + p * H);
        free(xd);
    }
}

/* Shared (always-on) expert applied to every token: s[t] = expert 0 of `shared`. */
void oracle_shared_outputs(const uint16_t *x, int64_t T, const ora_bank *shared, double *s)
{
    int64_t H = shared->hidden;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        double *xd = (double *)malloc((size_t)H * sizeof(double));
        x_row(x, t, H, xd);
        expert_forward(shared, 0, xd, s + t * H);
        free(xd);
    }
}

/* ------------------------------------------------------------------------- */
/* O7: combine                                                                */
/* ------------------------------------------------------------------------- */

/*
 * y[t] = sum_j g[t][j] * rows[t*k + j] + sigma_t * s[t]   (sigma_t = 1 when
 * shared_scale is NULL; s may be NULL for "no shared expert").
 * [ARCH]: the routed experts' outputs weighted by the renormalised gates,
 * plus the always-on expert.
 */
void oracle_combine(const double *rows, const double *gates, const double *s,
                    const double *shared_scale, int64_t T, int64_t k, int64_t H, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t i = 0; i < H; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += gates[t * k + j] * rows[(t * k + j) * H + i];
            if (s)
                acc += (shared_scale ? shared_scale[t] : 1.0) * s[t * H + i];
            y[t * H + i] = acc;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Whole layer, token by token                                                */
/* ------------------------------------------------------------------------- */

/*
 * y = MoE(x) for T tokens: exact logits, top-k, renormalised gates, routed
 * SwiGLU experts, the shared expert (NULL = none), weighted combine.
 * Optional outputs (may be NULL): idx [T][k], gates [T][k].
 */
void oracle_layer(const uint16_t *x, const uint16_t *w_router, int64_t T, int64_t E, int64_t k,
                  const ora_bank *bank, const ora_bank *shared, const double *shared_scale,
                  double *y, int32_t *idx_out, double *gates_out)
{
    int64_t H = bank->hidden;
    float *logits = (float *)malloc((size_t)(T * E) * sizeof(float));
    int32_t *idx = (int32_t *)malloc((size_t)(T * k) * sizeof(int32_t));
    double *gates = (double *)malloc((size_t)(T * k) * sizeof(double));
    double *rows = (double *)malloc((size_t)(T * k * H) * sizeof(double));
    double *s = shared ? (double *)malloc((size_t)(T * H) * sizeof(double)) : NULL;
    oracle_router_logits(x, w_router, T, H, E, logits);
    oracle_rank(logits, T, E, k, idx);
    oracle_gates(logits, idx, T, E, k, k, gates);
    oracle_pair_outputs(x, T, k, idx, bank, rows);
    if (shared)
        oracle_shared_outputs(x, T, shared, s);
    oracle_combine(rows, gates, s, shared_scale, T, k, H, y);
    if (idx_out)
        memcpy(idx_out, idx, (size_t)(T * k) * sizeof(int32_t));
    if (gates_out)
        memcpy(gates_out, gates, (size_t)(T * k) * sizeof(double));
    free(logits);
    free(idx);
    free(gates);
    free(rows);
    free(s);
}

/* ------------------------------------------------------------------------- */
/* O8: Refill-RMS saliency statistics and the keep-set                        */
/* ------------------------------------------------------------------------- */

/*
 * [RAZOR] "Selection and calibration": for each valid token and each selected
 * expert j, remove j, promote the highest-ranked unselected expert r, and
 * measure the change of the layer output.  Full re-evaluation, no shortcut:
 *   y  = sum_{i in S}  g_i  o_i + s,      g  = p / sum_S  p
 *   y' = sum_{i in S'} g'_i o_i + s,      g' = p / sum_S' p,   S' = S - {j} + {r}
 *   sum[j] += ||y' - y||^2,  count[j] += 1.
 * p is the softmax over all E experts (as in oracle_gates).  The statistics
 * are additive: this call adds into sum[] and count[].  valid may be NULL.
 * logits must be the exact router logits [T][E].
 */
void oracle_refill_accumulate(const uint16_t *x, const float *logits, int64_t T, int64_t E,
                              int64_t k, const ora_bank *bank, const ora_bank *shared,
                              const uint8_t *valid, double *sum, int64_t *count)
{
    int64_t H = bank->hidden;
    int64_t K1 = k + 1;
    int32_t *idx = (int32_t *)malloc((size_t)(T * K1) * sizeof(int32_t));
    oracle_rank(logits, T, E, K1, idx);
    double *dsq = (double *)calloc((size_t)(T * k), sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        if (valid && !valid[t])
            continue;
        const float *l = logits + t * E;
        const int32_t *sel = idx + t * K1;
        double *xd = (double *)malloc((size_t)H * sizeof(double));
        double *o = (double *)malloc((size_t)(K1 * H) * sizeof(double));
        double *sv = (double *)calloc((size_t)H, sizeof(double));
        double *y = (double *)malloc((size_t)H * sizeof(double));
        double *y2 = (double *)malloc((size_t)H * sizeof(double));
        double *p = (double *)malloc((size_t)K1 * sizeof(double));
        x_row(x, t, H, xd);
        for (int64_t j = 0; j < K1; ++j)
            expert_forward(bank, sel[j], xd, o + j * H);
        if (shared)
            expert_forward(shared, 0, xd, sv);
        double m = -INFINITY, denom = 0.0;
        for (int64_t e = 0; e < E; ++e)
            if ((double)l[e] > m)
                m = (double)l[e];
        for (int64_t e = 0; e < E; ++e)
            denom += exp((double)l[e] - m);
        for (int64_t j = 0; j < K1; ++j)
            p[j] = exp((double)l[sel[j]] - m) / denom;
        double zs = 0.0;
        for (int64_t j = 0; j < k; ++j)
            zs += p[j];
        for (int64_t i = 0; i < H; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += (p[j] / zs) * o[j * H + i];
            y[i] = acc + sv[i];
        }
        for (int64_t drop = 0; drop < k; ++drop) {
            double z2 = 0.0;
            for (int64_t j = 0; j < K1; ++j)
                if (j != drop)
                    z2 += p[j];
            double d2 = 0.0;
            for (int64_t i = 0; i < H; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < K1; ++j)
                    if (j != drop)
                        acc += (p[j] / z2) * o[j * H + i];
                y2[i] = acc + sv[i];
                double d = y2[i] - y[i];
                d2 += d * d;
            }
            dsq[t * k + drop] = d2;
        }
        free(xd);
        free(o);
        free(sv);
        free(y);
        free(y2);
        free(p);
    }
    /* Serial, token order: the statistics do not depend on the thread count. */
    for (int64_t t = 0; t < T; ++t) {
        if (valid && !valid[t])
            continue;
        for (int64_t j = 0; j < k; ++j) {
            sum[idx[t * K1 + j]] += dsq[t * k + j];
            count[idx[t * K1 + j]] += 1;
        }
    }
    free(dsq);
    free(idx);
}

/*
 * score_e = sqrt(sum_e / (count_e * H)): the RMS of the output change per
 * hidden element over the tokens routed to e ([RAZOR]: RMS conditional on the
 * tokens routed to each expert); experts never routed score 0.  Rank by score
 * descending, ties to the lower index; keep the first `keep`; keep_idx lists
 * the kept original indices in ascending order.
 */
void oracle_refill_finalize(const double *sum, const int64_t *count, int64_t E, int64_t H,
                            int64_t keep, double *score, uint8_t *keep_mask, int32_t *keep_idx)
{
    for (int64_t e = 0; e < E; ++e)
        score[e] = count[e] > 0 ? sqrt(sum[e] / ((double)count[e] * (double)H)) : 0.0;
    char *taken = (char *)calloc((size_t)E, 1);
    for (int64_t r = 0; r < keep; ++r) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || score[e] > score[best]))
                best = e;
        taken[best] = 1;
    }
    int64_t n = 0;
    for (int64_t e = 0; e < E; ++e) {
        keep_mask[e] = (uint8_t)taken[e];
        if (taken[e])
            keep_idx[n++] = (int32_t)e;
    }
    free(taken);
}

/*
 * Router-norm keep policy ([RAZOR] "Selection and calibration", the policy
 * used for the layer the calibration text never executes): rank experts by
 * the L2 norm of their router row, descending, ties to the lower index; keep
 * the first `keep`, listed in ascending index order.
 */
void oracle_router_norm_keep(const uint16_t *w_router, int64_t E, int64_t H, int64_t keep,
                             double *norm, int32_t *keep_idx)
{
    for (int64_t e = 0; e < E; ++e) {
        double s = 0.0;
        for (int64_t i = 0; i < H; ++i) {
            double w = bf16_value(w_router[e * H + i]);
            s += w * w;
        }
        norm[e] = sqrt(s);
    }
    char *taken = (char *)calloc((size_t)E, 1);
    for (int64_t r = 0; r < keep; ++r) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || norm[e] > norm[best]))
                best = e;
        taken[best] = 1;
    }
    int64_t n = 0;
    for (int64_t e = 0; e < E; ++e)
        if (taken[e])
            keep_idx[n++] = (int32_t)e;
    free(taken);
}

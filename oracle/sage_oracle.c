/*
 * Plain CPU oracle for SageAttention2-style quantized attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do. It shares no code with the HIP library.
 *
 * What it computes, and where each step comes from (page title, section):
 *   - "SageAttention: Quantized Attention Library" (topgit.dev), core
 *     features list: INT8 quantization of Q and K for QK^T, FP8 quantization
 *     of P and V for PV, smoothing of K before quantization.
 *   - "thu-ml/SageAttention" README translation (gittoolsai.com), current
 *     features and usage sections: the same steps, HND/NHD inputs, causal.
 *   - stable-diffusion.cpp "SageAttention" doc, kernel-selection table and the
 *     paragraph after it: K is smoothed, V is quantized per channel to FP8 and
 *     padded/permuted; head dims below 64 pad to 64, 65..127 pad to 128, the
 *     original softmax scale is kept and the output is cropped.
 *   - "SageAttention-RDNA4" releases, v0.4.0 notes: the key mean is summed in
 *     fp64; v0.2.0 notes: one INT8 scale per query token.
 *   - "SageAttention 2.2.0 for Blackwell sm_120a" (pirateface.co), accuracy
 *     table, and the README translation, kernel list and performance note
 *     ("8+16"): the INT8-QK / FP16-PV variant, P and V in a 16-bit float
 *     format for the P.V product.
 *
 * The pages give names and properties, not formulas. Where they leave a step
 * open the plainest reading is taken; every reading is listed in the design
 * notes of the repository and restated at the function that implements it.
 *
 * Precision: integer and fp32 steps (means, scales, codes) are the contract
 * the GPU must match bit for bit, so they are written in fp32 exactly as
 * specified (build with -ffp-contract=off, no fast-math). Everything after the
 * int32 logits is computed in fp64.
 *
 * Array conventions: one (batch, head) slice at a time, row-major, token
 * major: x[token * width + channel]. Inputs q/k/v are fp32 arrays holding the
 * exact fp16/bf16 input values (both widen to fp32 without rounding).
 *
 * Parity status of each function is stated in the design notes; all are
 * pinned by tests against closed forms, invariants, brute force or an
 * independent library routine.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.    */
/* Normal values 2^(e-7) * (1 + m/8) for e in 1..15 (except e=15,m=7),       */
/* subnormals 2^-6 * m/8, largest finite 448, codes 0x7F and 0xFF are NaN,   */
/* no infinities. The pages call this format "FP8" (e4m3) for P and V.      */
/* ------------------------------------------------------------------------ */

double oracle_e4m3_decode(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/*
 * Round x to the nearest E4M3FN value, ties to the even mantissa, saturating
 * at +-448 (x is clamped first, as the quantizers below do). The sign of x is
 * kept on zero results (a negative value that rounds to zero gives 0x80).
 * NaN gives 0x7F.
 */
uint8_t oracle_e4m3_encode(double x)
{
    uint8_t sign = 0;
    double a;
    int e, best_code;
    double q, lo, frac;
    if (isnan(x))
        return 0x7F;
    if (signbit(x)) {
        sign = 0x80;
        a = -x;
    } else {
        a = x;
    }
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    /* Exponent of the binade holding a; below 2^-6 the spacing is fixed at 2^-9. */
    if (a < ldexp(1.0, -6)) {
        q = a / ldexp(1.0, -9);          /* exact: scaling by a power of two */
        lo = floor(q);
        frac = q - lo;
        if (frac > 0.5 || (frac == 0.5 && fmod(lo, 2.0) != 0.0))
            lo += 1.0;
        /* lo in 0..8; 8 means the smallest normal 2^-6 (code 0x08). */
        return (uint8_t)(sign | (int)lo);
    }
    e = (int)floor(log2(a));
    /* guard against log2 rounding at binade edges */
    if (ldexp(1.0, e) > a)
        e -= 1;
    if (ldexp(1.0, e + 1) <= a)
        e += 1;
    q = a / ldexp(1.0, e - 3);           /* in [8, 16): 8 + mantissa */
    lo = floor(q);
    frac = q - lo;
    if (frac > 0.5 || (frac == 0.5 && fmod(lo, 2.0) != 0.0))
        lo += 1.0;
    if (lo == 16.0) {                    /* rounded up into the next binade */
        lo = 8.0;
        e += 1;
    }
    best_code = ((e + 7) << 3) | ((int)lo - 8);
    if (best_code > 0x7E)                /* cannot happen below 448, kept as a guard */
        best_code = 0x7E;
    return (uint8_t)(sign | best_code);
}

/* ------------------------------------------------------------------------ */
/* Padded head dimension (stable-diffusion.cpp doc, shape-support paragraph): */
/* D < 64 pads to 64, 65..127 to 128; 64 and 128 stay.                       */
/* ------------------------------------------------------------------------ */
int oracle_padded_dim(int d)
{
    if (d <= 64)
        return 64;
    return 128;
}

/* ------------------------------------------------------------------------ */
/* K mean over tokens for one (batch, kv-head): kbar[d] = mean_j k[j][d].     */
/* RDNA4 releases page, v0.4.0: the key mean is summed in fp64.              */
/* Reading: the sum runs over all Lk real tokens (also when causal); its     */
/* order is fixed so the result is reproducible: tokens are summed in order  */
/* within consecutive chunks of KMEAN_CHUNK tokens, then the chunk sums are   */
/* added in chunk order; one fp64 division by Lk and one rounding to fp32.   */
/* Channels d >= D (padding) get 0.                                          */
/* ------------------------------------------------------------------------ */
#define KMEAN_CHUNK 256

void oracle_k_mean(const float *k, int Lk, int D, int Dp, float *kbar)
{
    int d, j, c0;
    for (d = 0; d < Dp; ++d) {
        double total = 0.0;
        if (d >= D) {
            kbar[d] = 0.0f;
            continue;
        }
        for (c0 = 0; c0 < Lk; c0 += KMEAN_CHUNK) {
            double chunk = 0.0;
            int c1 = c0 + KMEAN_CHUNK < Lk ? c0 + KMEAN_CHUNK : Lk;
            for (j = c0; j < c1; ++j)
                chunk += (double)k[(size_t)j * D + d];
            total += chunk;
        }
        kbar[d] = (float)(total / (double)Lk);
    }
}

/* Symmetric INT8 code of x given the reciprocal step r = 127/amax (fp32):   */
/* round x*r (one fp32 product) to the nearest integer, ties to even, and     */
/* clamp to [-127, 127]. -128 is never used.                                 */
static int8_t int8_code(float x, float r)
{
    float y = x * r;
    float n = rintf(y);
    if (n > 127.0f)
        n = 127.0f;
    if (n < -127.0f)
        n = -127.0f;
    return (int8_t)n;
}

/* ------------------------------------------------------------------------ */
/* Q quantization, one scale per query token.                                */
/* topgit.dev features list (per-token INT8 granularity for QK^T); RDNA4      */
/* releases v0.2.0 (one scale per token).                                    */
/* For token i: a = max_d |q_id|; s_q = a/127 (fp32, correctly rounded);     */
/* r = 127/a (fp32) or 0 when a = 0; code = clamp(rne(q_id * r)).            */
/* Output rows are Dp wide; channels d >= D are 0.                           */
/* ------------------------------------------------------------------------ */
void oracle_quant_q(const float *q, int L, int D, int Dp, int8_t *qhat, float *sq)
{
    int i, d;
    for (i = 0; i < L; ++i) {
        float a = 0.0f, r;
        for (d = 0; d < D; ++d) {
            float t = fabsf(q[(size_t)i * D + d]);
            if (t > a)
                a = t;
        }
        sq[i] = a / 127.0f;
        r = a > 0.0f ? 127.0f / a : 0.0f;
        for (d = 0; d < Dp; ++d)
            qhat[(size_t)i * Dp + d] = d < D ? int8_code(q[(size_t)i * D + d], r) : 0;
    }
}

/* ------------------------------------------------------------------------ */
/* K smoothing and quantization, one scale per block of 64 tokens.           */
/* Smoothing (topgit.dev features; sd.cpp doc): k~ = k - kbar, one fp32      */
/* subtraction, not rounded back to the input type. Quantization granularity */
/* "per block" of the key sequence: blocks of KBLOCK tokens of one           */
/* (batch, kv-head); the last block covers only the real tokens.             */
/* For block b: a = max over its tokens and d < D of |k~|; s_k = a/127;      */
/* r = 127/a or 0; code = clamp(rne(k~ * r)). Channels d >= D are 0.         */
/* ------------------------------------------------------------------------ */
#define KBLOCK 64

void oracle_quant_k(const float *k, const float *kbar, int Lk, int D, int Dp,
                    int8_t *khat, float *sk)
{
    int b, j, d;
    int nblk = (Lk + KBLOCK - 1) / KBLOCK;
    for (b = 0; b < nblk; ++b) {
        int j0 = b * KBLOCK;
        int j1 = j0 + KBLOCK < Lk ? j0 + KBLOCK : Lk;
        float a = 0.0f, r;
        for (j = j0; j < j1; ++j)
            for (d = 0; d < D; ++d) {
                float t = fabsf(k[(size_t)j * D + d] - kbar[d]);
                if (t > a)
                    a = t;
            }
        sk[b] = a / 127.0f;
        r = a > 0.0f ? 127.0f / a : 0.0f;
        for (j = j0; j < j1; ++j)
            for (d = 0; d < Dp; ++d)
                khat[(size_t)j * Dp + d] =
                    d < D ? int8_code(k[(size_t)j * D + d] - kbar[d], r) : 0;
    }
}

/* ------------------------------------------------------------------------ */
/* V quantization to FP8 E4M3, one scale per channel.                        */
/* sd.cpp doc, after the kernel table: V is quantized per channel.           */
/* For channel d: c = max_j |v_jd|; s_v = c/448 (fp32); rho = 448/c or 0;    */
/* code = E4M3(clamp(v_jd * rho, -448, 448)) with the fp32 product.          */
/* The range is the full 448: the 2.25 limit on the same page belongs to an  */
/* FP16 instruction accumulator that this design does not have.              */
/* vhat is token major [Lk][Dp] (no permutation: that is a layout detail of  */
/* the GPU workspace). Channels d >= D get code 0 and scale 0.               */
/* ------------------------------------------------------------------------ */
void oracle_quant_v(const float *v, int Lk, int D, int Dp, uint8_t *vhat, float *sv)
{
    int j, d;
    for (d = 0; d < Dp; ++d) {
        float c = 0.0f, rho;
        if (d < D)
            for (j = 0; j < Lk; ++j) {
                float t = fabsf(v[(size_t)j * D + d]);
                if (t > c)
                    c = t;
            }
        sv[d] = c / 448.0f;
        rho = c > 0.0f ? 448.0f / c : 0.0f;
        for (j = 0; j < Lk; ++j) {
            float y;
            if (d >= D) {
                vhat[(size_t)j * Dp + d] = 0;
                continue;
            }
            y = v[(size_t)j * D + d] * rho;
            if (y > 448.0f)
                y = 448.0f;
            if (y < -448.0f)
                y = -448.0f;
            vhat[(size_t)j * Dp + d] = oracle_e4m3_encode((double)y);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Exact int32 logits A[i][j] = sum_d qhat[i][d] * khat[j][d] ("8+8": INT8   */
/* QK^T, README performance section). |A| <= Dp * 127^2 fits easily.          */
/* ------------------------------------------------------------------------ */
void oracle_qk_int32(const int8_t *qhat, int Lq, const int8_t *khat, int Lk, int Dp,
                     int32_t *out)
{
    int i, j, d;
    for (i = 0; i < Lq; ++i)
        for (j = 0; j < Lk; ++j) {
            int32_t acc = 0;
            for (d = 0; d < Dp; ++d)
                acc += (int32_t)qhat[(size_t)i * Dp + d] * (int32_t)khat[(size_t)j * Dp + d];
            out[(size_t)i * Lk + j] = acc;
        }
}

/* ------------------------------------------------------------------------ */
/* Quantized attention for query rows [r0, r1) of one (batch, q-head).       */
/*                                                                           */
/* The blocked, FlashAttention-style online softmax (topgit.dev, "SageAttention */
/* vs FlashAttention" and problem statement): keys are visited in blocks of  */
/* bk in order. For each block:                                              */
/*   logit_j = A_ij * s_q,i * s_k,blk(j) * sm_scale (fp64), or -inf when     */
/*             masked (causal: j > i, top-left aligned);                     */
/*   m_new   = max(m, max_j logit_j);  alpha = exp(m - m_new);               */
/*   P~_j    = exp(logit_j - m_new);                                         */
/*   P^_j    = E4M3(P~_j * 2^8)      -- P quantized to FP8 with a static     */
/*                                      power-of-two scale (reading);        */
/*   (pref = 1: m_new is not the block maximum itself but the running       */
/*    reference raised by the least whole number of powers of two that     */
/*    reaches it; pref = 2: a lazy reference above the maximum; see         */
/*    softmax_reference below; pref = 0: the maximum)                       */
/*   l       = alpha * l + sum_j dec(P^_j)   -- the normaliser is the sum of */
/*                                      the same quantized weights that      */
/*                                      multiply V (reading);                */
/*   O_d     = alpha * O_d + sum_j dec(P^_j) * dec(v^_jd).                   */
/* Finally out_id = O_d * s_v,d / l for d < D (crop).                        */
/* sm_scale is applied after dequantization; the caller passes 1/sqrt(D) of  */
/* the original head dim by default (sd.cpp doc: original scale kept).       */
/* out is [(r1 - r0)][D], fp64.                                              */
/* ------------------------------------------------------------------------ */
/* ------------------------------------------------------------------------ */
/* The reference the online softmax quantizes P against (topgit.dev,        */
/* "SageAttention vs FlashAttention": blockwise softmax with a running      */
/* maximum; the pages do not say against which value P is rounded).        */
/* Any reference at or above a block's logits gives the same softmax after */
/* normalisation; only the point where P is rounded moves. Two rules:       */
/*   pref = 0: the running maximum itself (m_new = max(m, block max));      */
/*   pref = 1: power-of-two steps. The first block with a visible key sets  */
/*             the reference to its maximum; afterwards, when a block's     */
/*             maximum mb exceeds the reference m, the reference rises by   */
/*             the least whole number n of factors of two that reaches it:  */
/*             n = ceil((mb - m) / ln 2), m_new = m + n ln 2, and the        */
/*             rescale of the running sums is alpha = 2^-n exactly. So the  */
/*             reference stays within one factor of two above the running  */
/*             maximum, every block's largest weight lies in (1/2, 1], and  */
/*             rescaling the sums is exact. Blocks whose maximum does not   */
/*             exceed the reference leave it unchanged under both rules.    */
/*   pref = 2: a lazy reference above the maximum. The first block with a   */
/*             visible key sets the reference to its maximum plus           */
/*             LAZY_OVER factors of two; afterwards the reference stays     */
/*             until a block's maximum passes it by more than LAZY_SLACK    */
/*             factors of two, and is then set to that maximum plus         */
/*             LAZY_OVER factors of two. Every weight stays at most         */
/*             2^LAZY_SLACK (2^8 P <= 430.5, inside E4M3's range), and the  */
/*             running sums are rescaled only on the blocks that move it.   */
/* Returns m_new and sets *alpha = e^(m - m_new) (0 on the first visible    */
/* block). Called only when max(m, mb) is finite.                           */
/* ------------------------------------------------------------------------ */
#define LAZY_OVER 2.0
#define LAZY_SLACK 0.75

static double softmax_reference(double m, double mb, int pref, double *alpha)
{
    double steps, m_new;
    if (m == -INFINITY) {               /* first visible block */
        *alpha = 0.0;
        return pref == 2 ? mb + LAZY_OVER * log(2.0) : mb;
    }
    if (pref == 2) {
        if (mb <= m + LAZY_SLACK * log(2.0)) {
            *alpha = 1.0;
            return m;
        }
        m_new = mb + LAZY_OVER * log(2.0);
        *alpha = exp(m - m_new);
        return m_new;
    }
    if (mb <= m) {
        *alpha = 1.0;
        return m;
    }
    if (pref == 0) {
        *alpha = exp(m - mb);
        return mb;
    }
    steps = ceil((mb - m) / log(2.0));
    if (steps < 1.0)
        steps = 1.0;
    *alpha = ldexp(1.0, -(int)steps);
    return m + steps * log(2.0);
}

void oracle_attn_quantized(const int8_t *qhat, const float *sq, int Lq,
                           const int8_t *khat, const float *sk,
                           const uint8_t *vhat, const float *sv, int Lk,
                           int D, int Dp, double sm_scale, int causal, int bk, int pref,
                           int r0, int r1, double *out)
{
    int i, j, d, j0;
    double *logit = (double *)malloc(sizeof(double) * (size_t)bk);
    double *pdec = (double *)malloc(sizeof(double) * (size_t)bk);
    double *acc = (double *)malloc(sizeof(double) * (size_t)Dp);
    (void)Lq;
    for (i = r0; i < r1; ++i) {
        double m = -INFINITY, l = 0.0;
        for (d = 0; d < Dp; ++d)
            acc[d] = 0.0;
        for (j0 = 0; j0 < Lk; j0 += bk) {
            int j1 = j0 + bk < Lk ? j0 + bk : Lk;
            double mb = -INFINITY, m_new, alpha, psum = 0.0;
            for (j = j0; j < j1; ++j) {
                if (causal && j > i) {
                    logit[j - j0] = -INFINITY;
                } else {
                    int32_t a = 0;
                    for (d = 0; d < Dp; ++d)
                        a += (int32_t)qhat[(size_t)i * Dp + d] * (int32_t)khat[(size_t)j * Dp + d];
                    logit[j - j0] = (double)a * (double)sq[i] * (double)sk[j / KBLOCK] * sm_scale;
                }
                if (logit[j - j0] > mb)
                    mb = logit[j - j0];
            }
            if (mb == -INFINITY && m == -INFINITY)
                continue;               /* nothing visible yet: state stays empty */
            m_new = softmax_reference(m, mb, pref, &alpha);
            for (j = j0; j < j1; ++j) {
                double p = exp(logit[j - j0] - m_new);
                pdec[j - j0] = oracle_e4m3_decode(oracle_e4m3_encode(p * 256.0));
                psum += pdec[j - j0];
            }
            l = alpha * l + psum;
            for (d = 0; d < Dp; ++d) {
                double s = 0.0;
                for (j = j0; j < j1; ++j)
                    s += pdec[j - j0] * oracle_e4m3_decode(vhat[(size_t)j * Dp + d]);
                acc[d] = alpha * acc[d] + s;
            }
            m = m_new;
        }
        for (d = 0; d < D; ++d)
            out[(size_t)(i - r0) * D + d] = acc[d] * (double)sv[d] / l;
    }
    free(logit);
    free(pdec);
    free(acc);
}

/* ------------------------------------------------------------------------ */
/* Rounding to the 16-bit float formats, from their definitions, for the    */
/* INT8-QK / 16-bit-PV variant ("8+16": FP16 PV, README performance note;   */
/* sageattn_qk_int8_pv_fp16 in the kernel list and the sm_120a accuracy      */
/* table). Both round to nearest, ties to even, with gradual underflow:     */
/*   binary16: 5 exponent bits (bias 15), 10 fraction bits, normals down to */
/*             2^-14, subnormal step 2^-24, largest finite 65504, above     */
/*             that infinity;                                                */
/*   bfloat16: 8 exponent bits (bias 127), 7 fraction bits, normals down to */
/*             2^-126, subnormal step 2^-133, largest finite                 */
/*             (2 - 2^-7) * 2^127, above that infinity.                      */
/* x is rounded in one step: it is split into a multiple of the format's    */
/* spacing at its magnitude, and rint (round to nearest even in the default */
/* rounding mode) picks the neighbour.                                       */
/* ------------------------------------------------------------------------ */
static double round_to_format(double x, int frac_bits, int emin, int emax)
{
    double ax, q, r;
    int e;
    if (x != x || x == 0.0 || isinf(x))
        return x;
    ax = fabs(x);
    frexp(ax, &e);                      /* ax = f * 2^e with f in [0.5, 1) */
    e -= 1;                             /* ax in [2^e, 2^(e+1)) */
    if (e < emin)
        e = emin;                       /* subnormal range: fixed spacing */
    q = ldexp(1.0, e - frac_bits);      /* spacing of representable values near ax */
    r = rint(ax / q) * q;               /* ax / q is exact (power-of-two scale) */
    if (r > ldexp(2.0 - ldexp(1.0, -frac_bits), emax))
        r = INFINITY;
    return x < 0.0 ? -r : r;
}

double oracle_round_f16(double x)
{
    return round_to_format(x, 10, -14, 15);
}

double oracle_round_bf16(double x)
{
    return round_to_format(x, 7, -126, 127);
}

/* ------------------------------------------------------------------------ */
/* Quantized attention, INT8-QK / 16-bit-PV variant, rows [r0, r1) of one   */
/* (batch, q-head). Q and K are the same INT8 codes and scales as in the    */
/* FP8 variant (smoothed K); V is not quantized: the 16-bit input values    */
/* themselves (v, [Lk][D], exact in fp32) multiply P. The online softmax is */
/* the same blocked one; P is rounded to the same 16-bit format as the      */
/* inputs (fmt 0: binary16, 1: bfloat16; reading: no scale is needed, P~ in */
/* (0, 1] is in range) and the normaliser is the sum of those rounded       */
/* weights:                                                                  */
/*   P^_j = round16(exp(logit_j - m_new)),  l = alpha * l + sum_j P^_j,     */
/*   O_d  = alpha * O_d + sum_j P^_j * v_jd,  out_id = O_d / l.             */
/* out is [(r1 - r0)][D], fp64.                                              */
/* ------------------------------------------------------------------------ */
void oracle_attn_quantized_pv16(const int8_t *qhat, const float *sq, int Lq,
                                const int8_t *khat, const float *sk,
                                const float *v, int Lk, int D, int Dp, double sm_scale,
                                int causal, int bk, int fmt, int r0, int r1, double *out)
{
    int i, j, d, j0;
    double *logit = (double *)malloc(sizeof(double) * (size_t)bk);
    double *pr = (double *)malloc(sizeof(double) * (size_t)bk);
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    (void)Lq;
    for (i = r0; i < r1; ++i) {
        double m = -INFINITY, l = 0.0;
        for (d = 0; d < D; ++d)
            acc[d] = 0.0;
        for (j0 = 0; j0 < Lk; j0 += bk) {
            int j1 = j0 + bk < Lk ? j0 + bk : Lk;
            double mb = -INFINITY, m_new, alpha, psum = 0.0;
            for (j = j0; j < j1; ++j) {
                if (causal && j > i) {
                    logit[j - j0] = -INFINITY;
                } else {
                    int32_t a = 0;
                    for (d = 0; d < Dp; ++d)
                        a += (int32_t)qhat[(size_t)i * Dp + d] * (int32_t)khat[(size_t)j * Dp + d];
                    logit[j - j0] = (double)a * (double)sq[i] * (double)sk[j / KBLOCK] * sm_scale;
                }
                if (logit[j - j0] > mb)
                    mb = logit[j - j0];
            }
            m_new = mb > m ? mb : m;
            if (m_new == -INFINITY)
                continue;
            alpha = exp(m - m_new);
            for (j = j0; j < j1; ++j) {
                double p = exp(logit[j - j0] - m_new);
                pr[j - j0] = fmt == 0 ? oracle_round_f16(p) : oracle_round_bf16(p);
                psum += pr[j - j0];
            }
            l = alpha * l + psum;
            for (d = 0; d < D; ++d) {
                double s = 0.0;
                for (j = j0; j < j1; ++j)
                    s += pr[j - j0] * (double)v[(size_t)j * D + d];
                acc[d] = alpha * acc[d] + s;
            }
            m = m_new;
        }
        for (d = 0; d < D; ++d)
            out[(size_t)(i - r0) * D + d] = acc[d] / l;
    }
    free(logit);
    free(pr);
    free(acc);
}

/* ------------------------------------------------------------------------ */
/* Key-range splits, causal alignment and the log-sum-exp of the softmax.   */
/* The general form of both quantized variants above, for query rows        */
/* [r0, r1) of one (batch, q-head):                                          */
/*   fmt     -1: FP8 P.V (vhat codes, sv channel scales, P * 2^8 to E4M3);   */
/*            0 / 1: 16-bit P.V (v values, P rounded to binary16/bfloat16);  */
/*   causal  0: none; 1: key j visible to query i iff j <= i (top-left);     */
/*           2: iff j <= i + Lk - Lq (bottom-right, the last query sees every */
/*           key);                                                           */
/*   pref    the reference P is quantized against (softmax_reference):    */
/*           0 the running maximum, 1 power-of-two steps;                    */
/*   nsplit  the keys are cut into nsplit ranges of whole blocks of bk,      */
/*           range s holding blocks [floor(s nb / S), floor((s + 1) nb / S)) */
/*           of nb = ceil(Lk / bk). Each range runs the blocked online       */
/*           softmax on its own (P quantized against its own running max)   */
/*           and yields (m_s, l_s, O_s); the ranges combine exactly:         */
/*           m = max m_s, out = sum_s e^(m_s - m) O_s / sum_s e^(m_s - m) l_s */
/*           (flash-decoding style; nsplit = 1 is the unsplit computation). */
/*   lse     (may be NULL) m + log(sum_s e^(m_s - m) l_s): the log of the    */
/*           softmax normaliser, natural log, in the unit of the weights     */
/*           actually used (dec(P^) / 2^8 for FP8).                          */
/*   bmask   (may be NULL) block-sparse pattern (README translation, news   */
/*           2025-06-19: attention under an arbitrary block-sparse pattern; */
/*           topgit.dev feature list: the sparse variant): key j is visible  */
/*           to query i only if bmask[(i / mbq) * mnk + j / mbk] != 0, i.e.  */
/*           blocks of mbq queries x mbk keys are computed or skipped whole; */
/*           a skipped block is -inf for all its logits. Combined with the   */
/*           causal mask by "and".                                           */
/* A row without any visible key has an empty softmax: out = 0, lse = -inf. */
/* ------------------------------------------------------------------------ */
typedef struct {
    int causal, Lq, Lk;
    const uint8_t *bmask;
    int mbq, mbk, mnk;
} Visibility;

static int key_visible(const Visibility *vis, int i, int j)
{
    if (vis->causal == 1 && j > i)
        return 0;
    if (vis->causal == 2 && (long)j > (long)i + (long)vis->Lk - (long)vis->Lq)
        return 0;
    if (vis->bmask != NULL && vis->bmask[(size_t)(i / vis->mbq) * (size_t)vis->mnk + (size_t)(j / vis->mbk)] == 0)
        return 0;
    return 1;
}

void oracle_attn_general(const int8_t *qhat, const float *sq, int Lq,
                         const int8_t *khat, const float *sk,
                         const uint8_t *vhat, const float *sv, const float *v, int Lk,
                         int D, int Dp, double sm_scale, int causal, int bk, int fmt, int pref,
                         int nsplit, const uint8_t *bmask, int mbq, int mbk, int mnk,
                         int r0, int r1, double *out, double *lse)
{
    int i, j, d, s, j0;
    const int nb = (Lk + bk - 1) / bk;
    const Visibility vis = {causal, Lq, Lk, bmask, mbq, mbk, mnk};
    double *logit = (double *)malloc(sizeof(double) * (size_t)bk);
    double *w = (double *)malloc(sizeof(double) * (size_t)bk);
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    double *tot = (double *)malloc(sizeof(double) * (size_t)D);
    for (i = r0; i < r1; ++i) {
        double M = -INFINITY, Lsum = 0.0;       /* running combination of the ranges */
        for (d = 0; d < D; ++d)
            tot[d] = 0.0;
        for (s = 0; s < nsplit; ++s) {
            const int b0 = (int)(((long)s * nb) / nsplit), b1 = (int)(((long)(s + 1) * nb) / nsplit);
            double m = -INFINITY, l = 0.0;
            for (d = 0; d < D; ++d)
                acc[d] = 0.0;
            for (j0 = b0 * bk; j0 < b1 * bk && j0 < Lk; j0 += bk) {
                int j1 = j0 + bk < Lk ? j0 + bk : Lk;
                double mb = -INFINITY, m_new, alpha, psum = 0.0;
                for (j = j0; j < j1; ++j) {
                    if (!key_visible(&vis, i, j)) {
                        logit[j - j0] = -INFINITY;
                    } else {
                        int32_t a = 0;
                        for (d = 0; d < Dp; ++d)
                            a += (int32_t)qhat[(size_t)i * Dp + d] * (int32_t)khat[(size_t)j * Dp + d];
                        logit[j - j0] = (double)a * (double)sq[i] * (double)sk[j / KBLOCK] * sm_scale;
                    }
                    if (logit[j - j0] > mb)
                        mb = logit[j - j0];
                }
                if (mb == -INFINITY && m == -INFINITY)
                    continue;
                m_new = softmax_reference(m, mb, pref, &alpha);
                for (j = j0; j < j1; ++j) {
                    double p = exp(logit[j - j0] - m_new);
                    if (fmt < 0)
                        w[j - j0] = oracle_e4m3_decode(oracle_e4m3_encode(p * 256.0)) / 256.0;
                    else
                        w[j - j0] = fmt == 0 ? oracle_round_f16(p) : oracle_round_bf16(p);
                    psum += w[j - j0];
                }
                l = alpha * l + psum;
                for (d = 0; d < D; ++d) {
                    double t = 0.0;
                    for (j = j0; j < j1; ++j) {
                        const double vv = fmt < 0 ? oracle_e4m3_decode(vhat[(size_t)j * Dp + d]) * (double)sv[d]
                                                  : (double)v[(size_t)j * D + d];
                        t += w[j - j0] * vv;
                    }
                    acc[d] = alpha * acc[d] + t;
                }
                m = m_new;
            }
            if (m == -INFINITY)
                continue;                       /* no visible key in this range */
            {
                const double Mn = m > M ? m : M;
                const double a_old = exp(M - Mn), a_new = exp(m - Mn);
                for (d = 0; d < D; ++d)
                    tot[d] = a_old * tot[d] + a_new * acc[d];
                Lsum = a_old * Lsum + a_new * l;
                M = Mn;
            }
        }
        for (d = 0; d < D; ++d)
            out[(size_t)(i - r0) * D + d] = Lsum > 0.0 ? tot[d] / Lsum : 0.0;
        if (lse)
            lse[i - r0] = Lsum > 0.0 ? M + log(Lsum) : -INFINITY;
    }
    free(logit);
    free(w);
    free(acc);
    free(tot);
}

/* ------------------------------------------------------------------------ */
/* Exact attention in fp64 for query rows [r0, r1) of one (batch, q-head):   */
/* out_i = sum_j softmax_j(sm_scale * q_i . k_j + M_ij) v_j, with M = -inf   */
/* where causal and j > i (top-left; causal = 2: j > i + Lk - Lq, bottom-  */
/* right), two passes with the row max removed; a row without any visible   */
/* key is 0. bmask (may be NULL) skips blocks of mbq x mbk as in            */
/* oracle_attn_general.                                                      */
/* This is the float64 reference the accuracy table of the sm_120a build    */
/* page compares against. out is [(r1 - r0)][D].                            */
/* ------------------------------------------------------------------------ */
void oracle_attn_exact(const float *q, const float *k, const float *v, int Lq, int Lk,
                       int D, double sm_scale, int causal, const uint8_t *bmask, int mbq, int mbk,
                       int mnk, int r0, int r1, double *out)
{
    int i, j, d;
    double *s = (double *)malloc(sizeof(double) * (size_t)Lk);
    const Visibility vis = {causal, Lq, Lk, bmask, mbq, mbk, mnk};
    for (i = r0; i < r1; ++i) {
        double m = -INFINITY, z = 0.0;
        for (j = 0; j < Lk; ++j) {
            if (!key_visible(&vis, i, j)) {
                s[j] = -INFINITY;
                continue;
            }
            {
                double dot = 0.0;
                for (d = 0; d < D; ++d)
                    dot += (double)q[(size_t)i * D + d] * (double)k[(size_t)j * D + d];
                s[j] = dot * sm_scale;
            }
            if (s[j] > m)
                m = s[j];
        }
        if (m == -INFINITY) {                  /* no visible key: empty softmax */
            for (d = 0; d < D; ++d)
                out[(size_t)(i - r0) * D + d] = 0.0;
            continue;
        }
        for (j = 0; j < Lk; ++j) {
            s[j] = exp(s[j] - m);
            z += s[j];
        }
        for (d = 0; d < D; ++d) {
            double acc = 0.0;
            for (j = 0; j < Lk; ++j)
                acc += s[j] * (double)v[(size_t)j * D + d];
            out[(size_t)(i - r0) * D + d] = acc / z;
        }
    }
    free(s);
}

/*
 * qmv_oracle.c -- CPU oracle for the block-quantized expert-gather GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant with the
 * HIP library: every decoder below is written out here on its own.
 *
 * What it computes: the literal definition "dequantize every weight, then
 * take the dot product", accumulated in fp64:
 *
 *     y[t][j][n] = sum_k  w(e, n, k) * x(t, j, k)     with e = ids[t][j]
 *     y[t][j][n] = 0                                   if e is outside [0, E)
 *
 * plus A[t][j][n] = sum_k |w(e, n, k) * x(t, j, k)|, the scale that the
 * parity tolerance is expressed in.
 *
 * Sources (page title, then the part of the page):
 *  - MXFP4 weights: e2m1 nibbles, one E8M0 byte scale per 32 weights, packed
 *    row-major so that weight k of a row lives in byte k/2 and group k/32:
 *    mlxcel issue "add an mxfp4 arm to the warp-shared gather_qmv kernel for
 *    gpt-oss decode", Current Behavior and Proposed Solution step 1.
 *  - The 2-bit and 3-bit code tables fp2 {-1,0,1,2} and fp3
 *    {0,1,2,4,0,-1,-2,-4}, and the decode contract "code -> value x
 *    half-block scale": lucebox-hub PR "optimize ROCMFPX fp3/fp2 MMVQ on
 *    RDNA", the kernel-level correctness tests in the review reply.
 *  - int8 activations with one scale per 32 (q8_1): the same page, and
 *    geo-lucebox PR "DS4 H200: rocmfp2_mix MoE matvec", "What is now hot".
 *  - An expert id outside [0, E) produces a zero row; a partial last column
 *    block writes nothing: mlxcel issue, Implementation Notes, Edge cases.
 *
 * Readings taken where the pages are silent (each is one line to change):
 *  - e2m1 is the OCP MX FP4 element: sign bit 3, two exponent bits with bias
 *    1, one mantissa bit, subnormal at exponent 0.
 *  - E8M0 scale byte s means 2^(s-127); s = 255 is NaN.
 *  - Nibble order: even k in the low nibble.
 *  - 2-bit codebook: c -> c - 1.5, i.e. the page's fp2 table minus 0.5.
 *  - 3-bit codebook: the page's fp3 table times 0.5 with its redundant
 *    negative zero (code 4) replaced by -3: {0,.5,1,2,-3,-.5,-1,-2}.
 *  - 3-bit codes form one little-endian bit stream per row: bit b of the
 *    stream is bit (b % 8) of byte b/8, and code k is stream bits 3k..3k+2
 *    with bit 3k the least significant.
 *  - 2-bit weights carry one fp16 scale per 32, 3-bit weights one fp16 scale
 *    per 16-weight half-block; an int8 activation carries one fp16 scale per
 *    32 and a half-block uses the scale of the 32-block that contains it.
 *
 * Fused gate/up (oracle_qmv_gather_swiglu_sel): the pages name one matvec
 * kernel for an MoE layer's gate and up expert projections (geo-lucebox PR
 * "DS4 H200: rocmfp2_mix MoE matvec", the per-kernel table and "Why this
 * kernel") but not the activation between them.  Reading taken: the SwiGLU
 * of Shazeer, "GLU Variants Improve Transformer" (2020), silu(g) * u with
 * silu(g) = g / (1 + e^-g), no clamp and no bias.
 *
 * Build: plain C99, gcc -O2, no SIMD intrinsics (build() in oracle/__init__.py).
 *
 * Compile-time ORACLE_MUTANT=<n> plants one deliberate mistake so the tests
 * can show that the pins catch it; the default build plants none.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* Format identifiers; numerically equal to the library's enums by
 * agreement of the two written specifications, not by a shared header. */
enum { OR_W_MXFP4 = 0, OR_W_CB2 = 1, OR_W_CB3 = 2 };
enum { OR_A_BF16 = 0, OR_A_Q8 = 1 };

/* ---------------------------------------------------------------- scalars */

/* e2m1 element value from its closed form (OCP MX FP4). */
double oracle_e2m1(int c)
{
    int s = (c >> 3) & 1;
    int e = (c >> 1) & 3;
    int m = c & 1;
    double mag;
    if (e == 0)
        mag = 0.5 * m;                       /* subnormal: 2^(1-1) * m/2 */
    else
        mag = ldexp(1.0 + 0.5 * m, e - 1);   /* 2^(e-1) * (1 + m/2) */
#if ORACLE_MUTANT == 1
    s = 0;                                   /* mutant: sign dropped */
#endif
    return s ? -mag : mag;
}

/* E8M0 scale byte -> 2^(s-127); 0xFF is NaN. */
double oracle_e8m0(int s)
{
    s &= 0xFF;
    if (s == 255)
        return NAN;
#if ORACLE_MUTANT == 6
    return ldexp(1.0, s - 128);              /* mutant: wrong bias */
#else
    return ldexp(1.0, s - 127);
#endif
}

/* IEEE-754 binary16 bit pattern -> value (bias 15, subnormals, Inf, NaN). */
double oracle_h2d(unsigned h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                  /* 0.f * 2^-14 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
#if ORACLE_MUTANT == 7
        v = ldexp(1024.0 + f, e - 24);              /* mutant: bias off by one */
#else
        v = ldexp(1024.0 + f, e - 25);              /* 1.f * 2^(e-15) */
#endif
    return s ? -v : v;
}

/* bfloat16 bit pattern -> value: bf16 is the upper half of a binary32. */
double oracle_bf16(unsigned b)
{
    uint32_t u = (uint32_t)(b & 0xFFFF) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* 2-bit and 3-bit codebooks (see the readings in the header). */
double oracle_cb2_value(int c)
{
    static const double page_fp2[4] = {-1.0, 0.0, 1.0, 2.0};
#if ORACLE_MUTANT == 4
    return page_fp2[c & 3] - 1.0;            /* mutant: codebook shifted */
#else
    return page_fp2[c & 3] - 0.5;
#endif
}

double oracle_cb3_value(int c)
{
    static const double page_fp3[8] = {0, 1, 2, 4, 0, -1, -2, -4};
    c &= 7;
    if (c == 4)
        return -3.0;
    return 0.5 * page_fp3[c];
}

/* ------------------------------------------------------------ row layout */

long oracle_row_code_bytes(int wfmt, long K)
{
    switch (wfmt) {
    case OR_W_MXFP4: return K / 2;
    case OR_W_CB2:   return K / 4;
    case OR_W_CB3:   return 3 * K / 8;
    }
    return -1;
}

long oracle_row_scale_bytes(int wfmt, long K)
{
    switch (wfmt) {
    case OR_W_MXFP4: return K / 32;          /* one byte per 32 */
    case OR_W_CB2:   return 2 * (K / 32);    /* one fp16 per 32 */
    case OR_W_CB3:   return 2 * (K / 16);    /* one fp16 per 16 */
    }
    return -1;
}

/* Code of weight k in a packed row, read one bit at a time for 3-bit. */
int oracle_code(int wfmt, const uint8_t *row, long k)
{
    switch (wfmt) {
    case OR_W_MXFP4: {
        uint8_t b = row[k >> 1];
#if ORACLE_MUTANT == 2
        return (k & 1) ? (b & 15) : (b >> 4); /* mutant: nibbles swapped */
#else
        return (k & 1) ? (b >> 4) : (b & 15);
#endif
    }
    case OR_W_CB2:
        return (row[k >> 2] >> (2 * (k & 3))) & 3;
    case OR_W_CB3: {
        int c = 0;
        for (int i = 0; i < 3; i++) {
            long bit = 3 * k + i;
            int v = (row[bit >> 3] >> (bit & 7)) & 1;
#if ORACLE_MUTANT == 5
            c |= v << (2 - i);               /* mutant: MSB-first codes */
#else
            c |= v << i;
#endif
        }
        return c;
    }
    }
    return -1;
}

static unsigned le16(const uint8_t *p)
{
    return (unsigned)p[0] | ((unsigned)p[1] << 8);
}

/* Scale that applies to weight k of a row. */
double oracle_weight_scale(int wfmt, const uint8_t *srow, long k)
{
    switch (wfmt) {
    case OR_W_MXFP4:
        return oracle_e8m0(srow[k >> 5]);
    case OR_W_CB2:
        return oracle_h2d(le16(srow + 2 * (k >> 5)));
    case OR_W_CB3:
#if ORACLE_MUTANT == 3
        return oracle_h2d(le16(srow + 2 * ((k >> 5) * 2)));  /* mutant: block, not half-block */
#else
        return oracle_h2d(le16(srow + 2 * (k >> 4)));
#endif
    }
    return NAN;
}

/* Code value (before scaling). */
double oracle_code_value(int wfmt, int c)
{
    switch (wfmt) {
    case OR_W_MXFP4: return oracle_e2m1(c);
    case OR_W_CB2:   return oracle_cb2_value(c);
    case OR_W_CB3:   return oracle_cb3_value(c);
    }
    return NAN;
}

/* Dequantized weight k of a row. */
double oracle_weight(int wfmt, const uint8_t *crow, const uint8_t *srow, long k)
{
    return oracle_code_value(wfmt, oracle_code(wfmt, crow, k)) *
           oracle_weight_scale(wfmt, srow, k);
}

/* Dequantized activation k of one activation vector. */
double oracle_activation(int afmt, const void *xrow, const uint16_t *xsrow, long k)
{
    if (afmt == OR_A_BF16)
        return oracle_bf16(((const uint16_t *)xrow)[k]);
    return (double)((const int8_t *)xrow)[k] * oracle_h2d(xsrow[k >> 5]);
}

/* Dequantize a whole row into w[0..K). */
void oracle_dequant_row(int wfmt, const uint8_t *crow, const uint8_t *srow, long K, double *w)
{
    for (long k = 0; k < K; k++)
        w[k] = oracle_weight(wfmt, crow, srow, k);
}

/*
 * Integer side output of the codebook paths: for every block b of a row,
 * S[b] = sum over the block of (2 * code value) * q.  A block is 32 weights
 * for the 2-bit format and a 16-weight half-block for the 3-bit format;
 * 2 * code value is an integer for both codebooks.
 */
long oracle_block_sums(int wfmt, const uint8_t *crow, const int8_t *q, long K, int64_t *S)
{
    long bs = (wfmt == OR_W_CB2) ? 32 : (wfmt == OR_W_CB3) ? 16 : 0;
    if (bs == 0)
        return -1;
    for (long b = 0; b < K / bs; b++) {
        int64_t s = 0;
        for (long i = 0; i < bs; i++) {
            long k = b * bs + i;
            double v2 = 2.0 * oracle_code_value(wfmt, oracle_code(wfmt, crow, k));
            s += (int64_t)v2 * (int64_t)q[k];
        }
        S[b] = s;
    }
    return K / bs;
}

/* ------------------------------------------------------------- the GEMV */

/* One output: dot of weight row (crow, srow) with activation vector v. */
static void dot_row(int wfmt, const uint8_t *crow, const uint8_t *srow, int afmt,
                    const void *xrow, const uint16_t *xsrow, long K,
                    double *y, double *a)
{
    double acc = 0.0, abs_acc = 0.0;
    for (long k = 0; k < K; k++) {
        double p = oracle_weight(wfmt, crow, srow, k) *
                   oracle_activation(afmt, xrow, xsrow, k);
        acc += p;
        abs_acc += fabs(p);
    }
    *y = acc;
    *a = abs_acc;
}

static const void *x_vector(int afmt, const void *x, long v, long K)
{
    size_t elt = (afmt == OR_A_BF16) ? 2 : 1;
    return (const uint8_t *)x + (size_t)v * (size_t)K * elt;
}

/*
 * Gather GEMV over a selection of outputs.  Output o (flat index into
 * y[M][top_k][N]) is t = o / (top_k N), j = (o / N) % top_k, n = o % N.
 * x is x[M][K] when x_per_slot == 0 and x[M][top_k][K] otherwise (int8 x
 * has scales xs of the same leading shape with K/32 entries per vector).
 * Returns 0, or -1 on a malformed argument.
 */
int oracle_qmv_gather_sel(int wfmt, const uint8_t *codes, const uint8_t *scales, long E,
                          const int32_t *ids, long M, long top_k,
                          int afmt, const void *x, const uint16_t *xs, int x_per_slot,
                          long N, long K, const int64_t *outs, long n_outs,
                          double *y, double *A)
{
    long rcb = oracle_row_code_bytes(wfmt, K), rsb = oracle_row_scale_bytes(wfmt, K);
    if (rcb < 0 || K % 32 != 0)
        return -1;
    for (long i = 0; i < n_outs; i++) {
        int64_t o = outs[i];
        long n = (long)(o % N);
        long p = (long)(o / N);          /* pair index t * top_k + j */
        long t = p / top_k;
        if (t >= M || o < 0)
            return -1;
        long e = ids[p];
#if ORACLE_MUTANT == 8
        e = ((e % E) + E) % E;           /* mutant: invalid ids wrap */
#endif
        if (e < 0 || e >= E) {
            y[i] = 0.0;
            A[i] = 0.0;
            continue;
        }
        long v = x_per_slot ? p : t;
        const uint8_t *crow = codes + ((size_t)e * N + n) * rcb;
        const uint8_t *srow = scales + ((size_t)e * N + n) * rsb;
        const uint16_t *xsrow = xs ? xs + (size_t)v * (K / 32) : NULL;
        dot_row(wfmt, crow, srow, afmt, x_vector(afmt, x, v, K), xsrow, K, &y[i], &A[i]);
    }
    return 0;
}

/* All outputs of a gather call, y and A shaped [M][top_k][N]. */
int oracle_qmv_gather(int wfmt, const uint8_t *codes, const uint8_t *scales, long E,
                      const int32_t *ids, long M, long top_k,
                      int afmt, const void *x, const uint16_t *xs, int x_per_slot,
                      long N, long K, double *y, double *A)
{
    long rcb = oracle_row_code_bytes(wfmt, K), rsb = oracle_row_scale_bytes(wfmt, K);
    if (rcb < 0 || K % 32 != 0)
        return -1;
    for (long t = 0; t < M; t++)
        for (long j = 0; j < top_k; j++) {
            long p = t * top_k + j;
            long e = ids[p];
#if ORACLE_MUTANT == 8
            e = ((e % E) + E) % E;
#endif
            for (long n = 0; n < N; n++) {
                size_t o = (size_t)p * N + n;
                if (e < 0 || e >= E) {
                    y[o] = 0.0;
                    A[o] = 0.0;
                    continue;
                }
                long v = x_per_slot ? p : t;
                const uint8_t *crow = codes + ((size_t)e * N + n) * rcb;
                const uint8_t *srow = scales + ((size_t)e * N + n) * rsb;
                const uint16_t *xsrow = xs ? xs + (size_t)v * (K / 32) : NULL;
                dot_row(wfmt, crow, srow, afmt, x_vector(afmt, x, v, K), xsrow, K, &y[o], &A[o]);
            }
        }
    return 0;
}

/* Dense GEMV: y[m][n] = sum_k w(n, k) * x(m, k). */
int oracle_qmv_dense(int wfmt, const uint8_t *codes, const uint8_t *scales,
                     int afmt, const void *x, const uint16_t *xs,
                     long M, long N, long K, double *y, double *A)
{
    long rcb = oracle_row_code_bytes(wfmt, K), rsb = oracle_row_scale_bytes(wfmt, K);
    if (rcb < 0 || K % 32 != 0)
        return -1;
    for (long m = 0; m < M; m++)
        for (long n = 0; n < N; n++) {
            const uint16_t *xsrow = xs ? xs + (size_t)m * (K / 32) : NULL;
            dot_row(wfmt, codes + (size_t)n * rcb, scales + (size_t)n * rsb, afmt,
                    x_vector(afmt, x, m, K), xsrow, K,
                    &y[(size_t)m * N + n], &A[(size_t)m * N + n]);
        }
    return 0;
}

/*
 * Fused gate/up projection with the SwiGLU activation (Shazeer, "GLU Variants
 * Improve Transformer", 2020): for each selected output o of y[M][top_k][N],
 *     g = gather output of the gate weights,  u = gather output of the up weights
 *     y = silu(g) * u,   silu(g) = g / (1 + e^-g),
 * with the token's activation vector (x[M][K]) and the gather's rules for
 * expert ids (an id outside [0, E) gives g = u = y = 0).  Also returns g, u and
 * their sum |w x| scales Ag, Au.  Any of g, u, Ag, Au may be NULL.
 */
int oracle_qmv_gather_swiglu_sel(int wfmt, const uint8_t *gcodes, const uint8_t *gscales,
                                 const uint8_t *ucodes, const uint8_t *uscales, long E,
                                 const int32_t *ids, long M, long top_k,
                                 int afmt, const void *x, const uint16_t *xs,
                                 long N, long K, const int64_t *outs, long n_outs,
                                 double *y, double *g, double *u, double *Ag, double *Au)
{
    for (long i = 0; i < n_outs; i++) {
        double gi, ui, ag, au;
        if (oracle_qmv_gather_sel(wfmt, gcodes, gscales, E, ids, M, top_k, afmt, x, xs, 0,
                                  N, K, &outs[i], 1, &gi, &ag) != 0 ||
            oracle_qmv_gather_sel(wfmt, ucodes, uscales, E, ids, M, top_k, afmt, x, xs, 0,
                                  N, K, &outs[i], 1, &ui, &au) != 0)
            return -1;
#if ORACLE_MUTANT == 9
        y[i] = ui / (1.0 + exp(-ui)) * gi;
#elif ORACLE_MUTANT == 10
        y[i] = ui / (1.0 + exp(-gi));
#else
        y[i] = gi / (1.0 + exp(-gi)) * ui;
#endif
        if (g) g[i] = gi;
        if (u) u[i] = ui;
        if (Ag) Ag[i] = ag;
        if (Au) Au[i] = au;
    }
    return 0;
}

/*
 * Down projection with the router-weighted top-k combine: for token t and row n
 *     y[t][n] = sum_j  w[t][j] * g(t, j, n)
 * where g is the gather output of slot j (zero for an expert id outside
 * [0, E)) and w[t][j] the router's fp32 weight of that slot.  Also returns
 * A[t][n] = sum_j |w[t][j]| * A_gather(t, j, n), the tolerance scale.
 * Outputs are selected by flat index o = t * N + n.
 */
int oracle_qmv_combine_sel(int wfmt, const uint8_t *codes, const uint8_t *scales, long E,
                           const int32_t *ids, const float *w, long M, long top_k,
                           int afmt, const void *x, const uint16_t *xs, int x_per_slot,
                           long N, long K, const int64_t *outs, long n_outs,
                           double *y, double *A)
{
    for (long i = 0; i < n_outs; i++) {
        long t = (long)(outs[i] / N), n = (long)(outs[i] % N);
        if (t < 0 || t >= M)
            return -1;
        double acc = 0.0, acc_a = 0.0;
#if ORACLE_MUTANT == 12
        for (long j = 0; j + 1 < top_k; j++) {       /* mutant: last slot dropped */
#else
        for (long j = 0; j < top_k; j++) {
#endif
            int64_t o = (int64_t)(t * top_k + j) * N + n;
            double g, a;
            if (oracle_qmv_gather_sel(wfmt, codes, scales, E, ids, M, top_k, afmt, x, xs,
                                      x_per_slot, N, K, &o, 1, &g, &a) != 0)
                return -1;
#if ORACLE_MUTANT == 11
            double wj = (double)w[t * top_k + (j + 1) % top_k];   /* mutant: weights shifted */
#elif ORACLE_MUTANT == 15
            double wj = fabs((double)w[t * top_k + j]);           /* mutant: weight signs dropped */
#else
            double wj = (double)w[t * top_k + j];
#endif
            acc += wj * g;
            acc_a += fabs(wj) * a;
        }
        y[i] = acc;
        if (A) A[i] = acc_a;
    }
    return 0;
}

/* ------------------------------------------------- activation quantizer */

/*
 * binary32 -> IEEE-754 binary16 bit pattern, rounded to nearest, ties to
 * even (subnormals kept, overflow to Inf, NaN to a quiet NaN).  Written out
 * in double arithmetic, where every step below is exact: scale the magnitude
 * to units of the target's last place, round to an integer with nearbyint
 * (the default rounding mode rounds halves to even), and let a mantissa that
 * rounds up to 2^10 carry into the exponent field.
 */
unsigned oracle_f2h(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    unsigned sign = (u >> 31) ? 0x8000u : 0u;
    if (isnan(f))
        return sign | 0x7E00u;
    double a = fabs((double)f);
    if (a >= 65520.0)                       /* halfway above 65504 and beyond: Inf */
        return sign | 0x7C00u;
    if (a < ldexp(1.0, -14)) {              /* subnormal range: units of 2^-24 */
        double m = nearbyint(a * ldexp(1.0, 24));
        return sign | (unsigned)m;          /* m == 1024 encodes 2^-14 exactly */
    }
    int ex;
    frexp(a, &ex);                          /* a = fr * 2^ex, fr in [0.5, 1) */
    int e = ex - 1;                         /* a in [2^e, 2^(e+1)) */
    double m = nearbyint((ldexp(a, -e) - 1.0) * 1024.0);
    if (m >= 1024.0) {
        m = 0.0;
        e += 1;
    }
    return sign | (unsigned)((e + 15) << 10) | (unsigned)m;
}

/*
 * Activation quantizer: bf16 activations -> int8 with one fp16 scale per 32,
 * the q8_1 activation blocks that the integer dot products consume
 * (lucebox-hub PR "optimize ROCMFPX fp3/fp2 MMVQ on RDNA", the MMVQ path;
 * geo-lucebox PR "DS4 H200: rocmfp2_mix MoE matvec", "What is now hot",
 * where quantize_q8_1 runs as its own launch before every matvec).  The
 * pages name the step but print no formula; reading taken, in fp32 (the
 * precision the integer decision is made in on both sides):
 *     amax = max_i |x_i|                     (exact)
 *     d    = amax / 127                      (fp32, nearest even)
 *     d16  = binary16(d)                     (nearest even; the stored scale)
 *     r    = 1 / float(d16)  in fp32, or 0 when d16 is zero or infinite
 *     q_i  = clamp(rint(x_i * r), -127, 127) (x_i * r in fp32; rint ties to even)
 * Activations must be finite.  q: int8 [V][K]; d16: fp16 bits [V][K/32].
 */
int oracle_quantize_q8(const uint16_t *xb, long V, long K, int8_t *q, uint16_t *d16)
{
    if (K % 32 != 0)
        return -1;
    for (long v = 0; v < V; v++)
        for (long b = 0; b < K / 32; b++) {
            const uint16_t *xs = xb + v * K + b * 32;
            float x[32];
            float amax = 0.0f;
            for (int i = 0; i < 32; i++) {
                uint32_t u = (uint32_t)xs[i] << 16;
                memcpy(&x[i], &u, sizeof u);
                float a = fabsf(x[i]);
                if (a > amax)
                    amax = a;
            }
            float d = amax / 127.0f;
            unsigned h = oracle_f2h(d);
            float dd = (float)oracle_h2d(h);
#if ORACLE_MUTANT == 14
            dd = d;                             /* mutant: unrounded scale used for q */
#endif
            float r = (dd > 0.0f && !isinf(dd)) ? 1.0f / dd : 0.0f;
            for (int i = 0; i < 32; i++) {
                float t = x[i] * r;
#if ORACLE_MUTANT == 13
                float qi = roundf(t);           /* mutant: ties away from zero */
#else
                float qi = rintf(t);
#endif
                if (qi > 127.0f) qi = 127.0f;
                if (qi < -127.0f) qi = -127.0f;
                q[v * K + b * 32 + i] = (int8_t)qi;
            }
            d16[v * (K / 32) + b] = (uint16_t)h;
        }
    return 0;
}

int oracle_mutant_id(void) { return ORACLE_MUTANT; }

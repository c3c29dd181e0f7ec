/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for the MoE expert
 * grouped GEMM.  TEST INFRASTRUCTURE ONLY: it is called by the tests, by the
 * smoke check and by the CPU-baseline leg of the benchmark, never by the
 * library.  It shares no code, header, table or constant with the HIP path.
 *
 * What it computes (all arithmetic in IEEE binary64 from the exact values of
 * the stored operands; one rounding to the output type at the very end):
 *
 *  - Grouped forward: one matrix multiply per expert over its own contiguous
 *    run of token rows ("Enabling DeepSeek-V4-Flash Training on AMD Instinct
 *    MI355X GPUs with Primus", section "Expert parallelism: DeepEP and the
 *    grouped GEMM": every expert multiplies its own number of tokens by its own
 *    weights, issued as one kernel over a ragged batch).
 *      C[r,n] = sum_{k<K} A[r,k] * B_g[k,n]     for r in expert g's rows.
 *  - Data gradient:  dX[r,k] = sum_{n<N} dY[r,n] * B_g[k,n].
 *  - Weight gradient, accumulated into an fp32 main_grad ("[Megatron-LM] feat:
 *    add grouped gemm fp4 support, skip cache trans weight and santize code",
 *    section "Changes": the weight gradient is always added into
 *    weight.main_grad):   D_g[k,n] = sum_{r in g} A[r,k] * dY[r,n].
 *  - SwiGLU between FC1 and FC2 (same blog, section "MegaMoE: fusing
 *    communication into the grouped GEMM"; the FC1 weight holds gate + up):
 *      h[r,j] = silu(C[r,j]) * C[r,I+j],  silu(x) = x / (1 + exp(-x)).
 *  - OCP Microscaling quantisation to MXFP8 (E4M3) and MXFP4 (E2M1, two per
 *    byte as in float4_e2m1fn_x2 from the PR's "Changes" section) with one
 *    E8M0 scale per 32 consecutive elements, and exact dequantisation.
 *
 * Every summation runs over its index in increasing order, one product at a
 * time, in binary64.  Output rows are independent, so OpenMP only splits the
 * list of requested rows across threads; it does not change any sum.
 *
 * Element encodings (OCP Microscaling Formats v1.0):
 *   E4M3 (FN): 1 sign, 4 exponent (bias 7), 3 mantissa; exponent 0 is
 *              subnormal; S.1111.111 is NaN; no infinities; max 448.
 *   E2M1:      1 sign, 2 exponent (bias 1), 1 mantissa; exponent 0 is
 *              subnormal; max 6.
 *   E8M0:      unsigned exponent, value 2^(E-127); 0xFF is NaN.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BF16 0
#define ORC_E4M3 1
#define ORC_E2M1 2

/* ---------------------------------------------------------------- decoding */

double orc_bf16_value(uint16_t h)
{
    /* bfloat16 is the upper 16 bits of an IEEE binary32 */
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double orc_e4m3_value(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, 1 - 7);          /* subnormal */
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

double orc_e2m1_value(uint8_t nibble)
{
    int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
    double mag;
    if (e == 0)
        mag = ldexp((double)m / 2.0, 1 - 1);          /* subnormal */
    else
        mag = ldexp(1.0 + (double)m / 2.0, e - 1);
    return s ? -mag : mag;
}

double orc_e8m0_value(uint8_t E)
{
    return E == 255 ? NAN : ldexp(1.0, (int)E - 127);
}

/*
 * Value of element (row, col) of a row-major matrix with `cols` columns.
 * MX matrices carry one E8M0 scale per 32 consecutive columns, scale matrix
 * [rows, cols/32]; E2M1 matrices store two codes per byte, the even column in
 * the low nibble.
 */
static double elem(int dtype, const void *data, const uint8_t *scale,
                   int64_t cols, int64_t row, int64_t col)
{
    if (dtype == ORC_BF16)
        return orc_bf16_value(((const uint16_t *)data)[row * cols + col]);
    double s = orc_e8m0_value(scale[row * (cols / 32) + col / 32]);
    if (dtype == ORC_E4M3)
        return orc_e4m3_value(((const uint8_t *)data)[row * cols + col]) * s;
    uint8_t byte = ((const uint8_t *)data)[row * (cols / 2) + col / 2];
    uint8_t nib = (col & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
    return orc_e2m1_value(nib) * s;
}

/* bytes per row of a stored matrix */
static int64_t row_bytes(int dtype, int64_t cols)
{
    return dtype == ORC_BF16 ? cols * 2 : dtype == ORC_E4M3 ? cols : cols / 2;
}

/* Decode rows x cols to binary64 (exact). */
void orc_decode(int dtype, const void *data, const uint8_t *scale,
                int64_t rows, int64_t cols, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = elem(dtype, data, scale, cols, r, c);
}

/* ---------------------------------------------------------------- rounding */

/* Round a binary64 value to the nearest bfloat16, ties to even. */
uint16_t orc_round_bf16(double x)
{
    const double bf16_max = ldexp(2.0 - ldexp(1.0, -7), 127);
    if (isnan(x))
        return 0x7FC0;
    if (x == 0.0)
        return signbit(x) ? 0x8000 : 0x0000;
    int e;
    frexp(fabs(x), &e);              /* |x| = f*2^e, f in [0.5,1) */
    int q_exp = (e - 1) - 7;         /* 8 significant bits            */
    if (q_exp < -133)
        q_exp = -133;                /* subnormal spacing 2^-133      */
    double v = ldexp(nearbyint(ldexp(x, -q_exp)), q_exp);   /* exact    */
    if (fabs(v) > bf16_max)
        return signbit(x) ? 0xFF80 : 0x7F80;                 /* overflow */
    float f = (float)v;              /* exact: v has <= 8 bits         */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void orc_round_bf16_array(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_round_bf16(x[i]);
}

/* Round to binary32, ties to even (the C conversion under the default mode). */
void orc_round_f32_array(const double *x, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)x[i];
}

/* ------------------------------------------------------------ quantisation */

/* Non-negative finite codes in increasing order of value. */
static int positive_grid(int dtype, double *vals)
{
    int n = 0;
    if (dtype == ORC_E4M3) {
        for (int c = 0; c <= 0x7E; ++c)          /* 0x7F is NaN */
            vals[n++] = orc_e4m3_value((uint8_t)c);
    } else {
        for (int c = 0; c <= 7; ++c)
            vals[n++] = orc_e2m1_value((uint8_t)c);
    }
    return n;
}

/*
 * Code of the grid value nearest to a >= 0; a tie goes to the even code (the
 * code's low bit is the mantissa's low bit); magnitudes above the largest
 * grid value saturate to it.
 */
static int nearest_code(double a, const double *vals, int n)
{
    if (a >= vals[n - 1])
        return n - 1;
    int lo = 0, hi = n - 1;                      /* vals[lo] <= a < vals[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (vals[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - vals[lo], dhi = vals[hi] - a;
    if (dlo < dhi)
        return lo;
    if (dhi < dlo)
        return hi;
    return (lo % 2 == 0) ? lo : hi;
}

/*
 * Shared scale of one block (OCP Microscaling Formats v1.0, conversion of a
 * block of scalars): the scale exponent is floor(log2(max |v|)) minus the element format's largest normal
 * exponent (8 for E4M3, 2 for E2M1), biased by 127 and clamped to the E8M0
 * range [0, 254].  An all-zero block takes E = 0.
 */
static int block_scale(int dtype, const double *v, int n)
{
    double amax = 0.0;
    for (int i = 0; i < n; ++i)
        if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    if (amax == 0.0)
        return 0;
    int e;
    frexp(amax, &e);                             /* floor(log2 amax) = e-1 */
    int emax = dtype == ORC_E4M3 ? 8 : 2;
    int E = (e - 1) - emax + 127;
    if (E < 0)
        E = 0;
    if (E > 254)
        E = 254;
    return E;
}

/*
 * Quantise a bf16 matrix [rows, cols] in blocks of 32 along `axis`
 * (1: along a row, consecutive columns; 0: along a column, consecutive rows).
 *   axis 1: q [rows, cols] (E4M3) or [rows, cols/2] (E2M1), scales [rows, cols/32]
 *   axis 0: q [rows, cols] (E4M3) or [rows/2, cols] (E2M1: row pairs share a
 *           byte, the even row in the low nibble), scales [rows/32, cols]
 * Each element is x = v / 2^(E-127) (exact), then the nearest grid code with
 * ties to even and saturation, sign kept.
 */
int orc_mx_quantize(const uint16_t *x, int64_t rows, int64_t cols, int dtype,
                    int axis, uint8_t *q, uint8_t *scales)
{
    if (dtype != ORC_E4M3 && dtype != ORC_E2M1)
        return 1;
    if ((axis == 1 && cols % 32) || (axis == 0 && rows % 32) || (axis != 0 && axis != 1))
        return 1;
    double vals[128];
    int n = positive_grid(dtype, vals);
    int64_t nblk = axis == 1 ? rows * (cols / 32) : (rows / 32) * cols;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
        int64_t r0, c0, dr, dc;
        if (axis == 1) {
            r0 = b / (cols / 32); c0 = (b % (cols / 32)) * 32; dr = 0; dc = 1;
        } else {
            r0 = (b / cols) * 32; c0 = b % cols; dr = 1; dc = 0;
        }
        double v[32];
        for (int i = 0; i < 32; ++i)
            v[i] = orc_bf16_value(x[(r0 + i * dr) * cols + c0 + i * dc]);
        int E = block_scale(dtype, v, 32);
        scales[b] = (uint8_t)E;
        for (int i = 0; i < 32; ++i) {
            double xi = ldexp(v[i], 127 - E);
            int code = nearest_code(fabs(xi), vals, n);
            int sign = signbit(v[i]) ? 1 : 0;
            int64_t r = r0 + i * dr, c = c0 + i * dc;
            if (dtype == ORC_E4M3) {
                q[r * cols + c] = (uint8_t)((sign << 7) | code);
            } else {
                uint8_t nib = (uint8_t)((sign << 3) | code);
                int64_t byte, hi;
                if (axis == 1) { byte = r * (cols / 2) + c / 2; hi = c & 1; }
                else           { byte = (r / 2) * cols + c;     hi = r & 1; }
                if (hi)
                    q[byte] = (uint8_t)((q[byte] & 0x0F) | (nib << 4));
                else
                    q[byte] = (uint8_t)((q[byte] & 0xF0) | nib);
            }
        }
    }
    return 0;
}

/*
 * FP8 E4M3 with one scale per matrix (current scaling; the rule is the
 * reading stated with the library's pt_fp8_quantize): for each of `batch`
 * matrices of n bf16 values, amax = max |x| (exact in fp32), s = 448 / amax
 * in fp32 (1 when amax is 0; the largest finite fp32 when the quotient
 * overflows), each code = the E4M3 value nearest to fp32(x * s) clamped to
 * +-448 (ties to even), and dequant = fp32(1 / s).  The fp32 steps are
 * written as float arithmetic: every one of them is a single IEEE rounding.
 */
void orc_fp8_quantize(const uint16_t *x, int64_t batch, int64_t n, uint8_t *q, float *amax, float *dequant)
{
    double vals[128];
    int ng = positive_grid(ORC_E4M3, vals);
    for (int64_t b = 0; b < batch; ++b) {
        const uint16_t *xb = x + b * n;
        float m = 0.0f;
        for (int64_t i = 0; i < n; ++i) {
            float v = fabsf((float)orc_bf16_value(xb[i]));
            if (v > m)
                m = v;
        }
        float s = (m == 0.0f) ? 1.0f : 448.0f / m;
        if (isinf(s))
            s = FLT_MAX;
        amax[b] = m;
        dequant[b] = 1.0f / s;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            float v = (float)orc_bf16_value(xb[i]);
            float y = v * s;
            int code = nearest_code(fabs((double)y), vals, ng);
            q[b * n + i] = (uint8_t)(((signbit(v) ? 1 : 0) << 7) | code);
        }
    }
}

/*
 * MX quantisation along tokens for the weight gradient, one expert at a
 * time: expert g's rows [off_g, off_g + len_g) of x [M, cols] form blocks of
 * 32 consecutive rows, the last one partial when len_g % 32 != 0 (its
 * missing rows are simply absent: the block scale comes from the rows that
 * exist), so no block straddles two experts.  Codes keep x's row layout:
 * E4M3 q [M, cols]; E2M1 q [M, cols/2] with column 2c in the low nibble of
 * byte c and column 2c+1 in the high one.  Block j of expert g takes scale
 * row bstart_g + j, bstart_g = sum over earlier experts of ceil(len / 32).
 * Returns the number of scale rows used, or -1 for a bad dtype or an odd
 * E2M1 column count.
 */
static void tokens_block(const uint16_t *x, int64_t cols, int64_t r0, int64_t nr, int64_t c, int dtype,
                         const double *vals, int n, int *codes, uint8_t *scale)
{
    double v[32];
    for (int64_t i = 0; i < nr; ++i)
        v[i] = orc_bf16_value(x[(r0 + i) * cols + c]);
    int E = block_scale(dtype, v, (int)nr);
    *scale = (uint8_t)E;
    const int sbit = dtype == ORC_E4M3 ? 7 : 3;
    for (int64_t i = 0; i < nr; ++i) {
        double xi = ldexp(v[i], 127 - E);
        codes[i] = ((signbit(v[i]) ? 1 : 0) << sbit) | nearest_code(fabs(xi), vals, n);
    }
}

int64_t orc_mx_quantize_tokens(const uint16_t *x, const int64_t *lens, int64_t G, int64_t M, int64_t cols,
                               int dtype, uint8_t *q, uint8_t *scales)
{
    if ((dtype != ORC_E4M3 && dtype != ORC_E2M1) || (dtype == ORC_E2M1 && cols % 2))
        return -1;
    double vals[128];
    int n = positive_grid(dtype, vals);
    int64_t off = 0, bstart = 0;
    for (int64_t g = 0; g < G; ++g) {
        int64_t len = lens[g], nb = (len + 31) / 32;
        for (int64_t j = 0; j < nb; ++j) {
            int64_t r0 = off + 32 * j, nr = len - 32 * j < 32 ? len - 32 * j : 32;
            uint8_t *srow = scales + (bstart + j) * cols;
            if (dtype == ORC_E4M3) {
#pragma omp parallel for schedule(static)
                for (int64_t c = 0; c < cols; ++c) {
                    int codes[32];
                    tokens_block(x, cols, r0, nr, c, dtype, vals, n, codes, srow + c);
                    for (int64_t i = 0; i < nr; ++i)
                        q[(r0 + i) * cols + c] = (uint8_t)codes[i];
                }
            } else {
                /* a byte holds two columns, so one thread takes both */
#pragma omp parallel for schedule(static)
                for (int64_t cp = 0; cp < cols / 2; ++cp) {
                    int lo[32], hi[32];
                    tokens_block(x, cols, r0, nr, 2 * cp, dtype, vals, n, lo, srow + 2 * cp);
                    tokens_block(x, cols, r0, nr, 2 * cp + 1, dtype, vals, n, hi, srow + 2 * cp + 1);
                    for (int64_t i = 0; i < nr; ++i)
                        q[(r0 + i) * (cols / 2) + cp] = (uint8_t)(lo[i] | (hi[i] << 4));
                }
            }
        }
        off += len;
        bstart += nb;
    }
    (void)M;
    return bstart;
}

/* ---------------------------------------------------------------- GEMMs */

/* Expert of global row r: offs[g] <= r < offs[g] + lens[g]; -1 if none. */
static int64_t group_of_row(const int64_t *lens, int64_t G, int64_t r,
                            int64_t *start)
{
    int64_t off = 0;
    for (int64_t g = 0; g < G; ++g) {
        if (r >= off && r < off + lens[g]) {
            *start = off;
            return g;
        }
        off += lens[g];
    }
    return -1;
}

/*
 * Forward, rows listed in `rows` (global row indices):
 *   out[i, n] = sum_k A[rows[i], k] * B_g[k, n]     (binary64, unrounded)
 * B is [G, K, N] (trans_b = 0) or [G, N, K] (trans_b = 1; the only layout for
 * MX operands, whose blocks run along K).
 */
int orc_fwd_rows(int dtype, const void *a, const uint8_t *a_scale,
                 const void *b, const uint8_t *b_scale,
                 const int64_t *lens, int64_t G, int64_t M, int64_t N, int64_t K,
                 int trans_b, const int64_t *rows, int64_t nrows, double *out)
{
    (void)M;
    int bad = 0;
    int64_t bstride = row_bytes(dtype, trans_b ? K : N) * (trans_b ? N : K);
    int64_t sstride = dtype == ORC_BF16 ? 0 : (trans_b ? N * (K / 32) : K * (N / 32));
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t start;
        int64_t g = group_of_row(lens, G, rows[i], &start);
        double *o = out + i * N;
        if (g < 0) { bad = 1; continue; }
        const void *bg = (const uint8_t *)b + g * bstride;
        const uint8_t *bsg = dtype == ORC_BF16 ? NULL : b_scale + g * sstride;
        double *arow = (double *)malloc(sizeof(double) * K);
        for (int64_t k = 0; k < K; ++k)
            arow[k] = elem(dtype, a, a_scale, K, rows[i], k);
        if (trans_b) {
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += arow[k] * elem(dtype, bg, bsg, K, n, k);
                o[n] = acc;
            }
        } else {
            for (int64_t n = 0; n < N; ++n)
                o[n] = 0.0;
            for (int64_t k = 0; k < K; ++k)
                for (int64_t n = 0; n < N; ++n)
                    o[n] += arow[k] * elem(dtype, bg, bsg, N, k, n);
        }
        free(arow);
    }
    return bad;
}

/*
 * Data gradient (bf16 operands), rows listed in `rows`:
 *   out[i, k] = sum_n dY[rows[i], n] * B_g[k, n]
 */
int orc_dgrad_rows(const uint16_t *dy, const uint16_t *b,
                   const int64_t *lens, int64_t G, int64_t M, int64_t N, int64_t K,
                   int trans_b, const int64_t *rows, int64_t nrows, double *out)
{
    (void)M;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t start;
        int64_t g = group_of_row(lens, G, rows[i], &start);
        double *o = out + i * K;
        if (g < 0) { bad = 1; continue; }
        const uint16_t *bg = b + g * K * N;
        double *dyrow = (double *)malloc(sizeof(double) * N);
        for (int64_t n = 0; n < N; ++n)
            dyrow[n] = orc_bf16_value(dy[rows[i] * N + n]);
        if (!trans_b) {                           /* B_g stored [K, N] */
            for (int64_t k = 0; k < K; ++k) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    acc += dyrow[n] * orc_bf16_value(bg[k * N + n]);
                o[k] = acc;
            }
        } else {                                  /* B_g stored [N, K] */
            for (int64_t k = 0; k < K; ++k)
                o[k] = 0.0;
            for (int64_t n = 0; n < N; ++n)
                for (int64_t k = 0; k < K; ++k)
                    o[k] += dyrow[n] * orc_bf16_value(bg[n * K + k]);
        }
        free(dyrow);
    }
    return bad;
}

/*
 * Weight gradient (bf16 operands) for the (expert, k) pairs listed:
 *   out[i, n] = sum_{r in expert gs[i]} A[r, ks[i]] * dY[r, n]
 * An expert with no rows gives an all-zero row.
 */
int orc_wgrad_rows(const uint16_t *a, const uint16_t *dy,
                   const int64_t *lens, int64_t G, int64_t M, int64_t N, int64_t K,
                   const int64_t *gs, const int64_t *ks, int64_t npairs, double *out)
{
    (void)M;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t i = 0; i < npairs; ++i) {
        int64_t g = gs[i], k = ks[i];
        double *o = out + i * N;
        if (g < 0 || g >= G || k < 0 || k >= K) { bad = 1; continue; }
        int64_t off = 0;
        for (int64_t j = 0; j < g; ++j)
            off += lens[j];
        for (int64_t n = 0; n < N; ++n)
            o[n] = 0.0;
        for (int64_t r = off; r < off + lens[g]; ++r) {
            double av = orc_bf16_value(a[r * K + k]);
            for (int64_t n = 0; n < N; ++n)
                o[n] += av * orc_bf16_value(dy[r * N + n]);
        }
    }
    return bad;
}

/*
 * SwiGLU over [gate | up] halves: h[i, j] = silu(g) * u with g = c[i, j],
 * u = c[i, I + j].  With a limit L > 0 (finite) the SwiGLU is clamped first:
 * g = min(g, L) and u = min(max(u, -L), L); limit <= 0 or infinite leaves it
 * plain.
 */
static int clamp_on(double limit) { return limit > 0.0 && isfinite(limit); }

void orc_swiglu(const double *c, int64_t nrows, int64_t N, double limit, double *h)
{
    int64_t I = N / 2;
    const int on = clamp_on(limit);
    for (int64_t i = 0; i < nrows; ++i)
        for (int64_t j = 0; j < I; ++j) {
            double gate = c[i * N + j], up = c[i * N + I + j];
            if (on) {
                gate = gate < limit ? gate : limit;
                up = up < -limit ? -limit : (up > limit ? limit : up);
            }
            h[i * I + j] = gate / (1.0 + exp(-gate)) * up;
        }
}

/* Backward of the SwiGLU above.  h = silu(g) * u with silu(g) = g * s,
 * s = 1 / (1 + e^-g), so dh/du = g * s and dh/dg = u * (s + g * s * (1 - s)),
 * taken at the clamped g and u.  A clamped input gets no gradient: the gate
 * where g > L, the up value where |u| > L (at the limit itself the gradient
 * passes).  dh [nrows, I] and c [nrows, 2I] = [gate | up] in; dc [nrows, 2I]
 * out, the gradient of c in the same [gate | up] layout. */
void orc_swiglu_bwd(const double *dh, const double *c, int64_t nrows, int64_t I, double limit, double *dc)
{
    const int on = clamp_on(limit);
    for (int64_t i = 0; i < nrows; ++i)
        for (int64_t j = 0; j < I; ++j) {
            double g = c[i * 2 * I + j], u = c[i * 2 * I + I + j], d = dh[i * I + j];
            int pass_g = 1, pass_u = 1;
            if (on) {
                if (g > limit) { g = limit; pass_g = 0; }
                if (u > limit) { u = limit; pass_u = 0; }
                if (u < -limit) { u = -limit; pass_u = 0; }
            }
            double s = 1.0 / (1.0 + exp(-g));
            dc[i * 2 * I + j] = pass_g ? d * u * s * (1.0 + g * (1.0 - s)) : 0.0;
            dc[i * 2 * I + I + j] = pass_u ? d * g * s : 0.0;
        }
}

int orc_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * attn_oracle.c -- CPU oracle for single-query decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the GPU path is checked against.  Only the test suite, the
 * package smoke check and the bench's CPU-baseline leg load it; the product
 * path never does.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * What it computes follows the page "Developing Apple Metal Kernels in Rust -
 * A Deep Dive Through Attention", section "The MSL, briefly":
 *
 *   kernel attention_qk_f16 : for each head h and position p,
 *       s[h,p] = (sum_i q[h,i] * k[p,h,i]) * (1 / sqrt(head_dim)),
 *       with the scale applied after the full dot product, and
 *       s[h,p] = -inf for every p > current_pos;
 *   kernel attention_pv_f16 : softmax over positions with the global maximum
 *       subtracted first (m = max s, z = sum exp(s - m), w = exp(s - m) / z),
 *       then out[h,d] = sum_p w[h,p] * v[p,h,d].
 *
 * The decode step around it (the rotary embedding of the page "Tutorial 16:
 * Writing Custom Metal Kernels", and the fp16 rounding of what is stored) is
 * at the end of the file: oracle_rope and oracle_double_to_half.  So is the
 * softmax step on its own (oracle_softmax_rows, the Foundry notes' fm_softmax).
 *
 * Layouts (same section): Q and output [n_heads, head_dim]; K and V caches
 * [seq_len, n_heads, head_dim], element (p,h,i) at (p*n_heads + h)*head_dim + i;
 * scores [n_heads, seq_len].  Inputs are IEEE binary16 bit patterns.
 *
 * Readings where the page leaves a step open:
 *  - Everything here is fp64 (inputs decoded exactly); scores are not rounded
 *    to fp16 as the page's two-dispatch design does between its kernels.
 *  - A masked position has weight exactly 0, so it is skipped: its K and V
 *    values are never read.  For finite values this gives the same sum as
 *    adding 0*v; for non-finite garbage it keeps the output finite.
 *  - current_pos >= seq_len masks nothing (the page's guard only tests
 *    pos > current_pos), so the valid length is L = min(current_pos, seq_len-1)+1.
 *
 * Plain scalar loops, built with -O2 and without -ffast-math.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent 0 encodes zero and subnormals (fraction * 2^-24), exponent
 * 31 encodes infinities (fraction 0) and NaNs.  Every binary16 value is exact
 * in binary64. */
double oracle_half_to_double(uint16_t bits)
{
    const int sign = (bits >> 15) & 1;
    const int expo = (bits >> 10) & 0x1f;
    const int frac = bits & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), expo - 25);   /* (1 + f/1024) * 2^(e-15) */
    return sign ? -mag : mag;
}

void oracle_half_to_double_array(const uint16_t *bits, size_t n, double *out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = oracle_half_to_double(bits[i]);
}

/*
 * Decode attention for heads [head_lo, head_hi) of one sequence.
 *   out     [n_heads, head_dim]  rows head_lo..head_hi-1 are written
 *   scores  NULL or [n_heads, seq_len]: s for p <= current_pos, -inf after
 *   weights NULL or [n_heads, seq_len]: softmax weights, 0 after current_pos
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_attn_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       uint32_t n_heads, uint32_t head_dim, uint32_t seq_len,
                       uint32_t current_pos, uint32_t head_lo, uint32_t head_hi,
                       double *out, double *scores, double *weights)
{
    if (!q || !k || !v || !out || n_heads == 0 || head_dim == 0 || seq_len == 0 ||
        head_lo > head_hi || head_hi > n_heads)
        return -1;

    const size_t H = n_heads, D = head_dim, S = seq_len;
    const size_t L = (current_pos < seq_len - 1 ? (size_t)current_pos : S - 1) + 1;
    const double scale = 1.0 / sqrt((double)D);

    double *s = (double *)malloc(L * sizeof(double));
    double *e = (double *)malloc(L * sizeof(double));
    if (!s || !e) {
        free(s);
        free(e);
        return -1;
    }

    for (size_t h = head_lo; h < head_hi; ++h) {
        /* scaled dot products over the unmasked positions */
        for (size_t p = 0; p < L; ++p) {
            double dot = 0.0;
            for (size_t i = 0; i < D; ++i)
                dot += oracle_half_to_double(q[h * D + i]) *
                       oracle_half_to_double(k[(p * H + h) * D + i]);
            s[p] = dot * scale;
        }

        /* softmax: global max, sum of shifted exponentials, normalised weights */
        double m = s[0];
        for (size_t p = 1; p < L; ++p)
            if (s[p] > m)
                m = s[p];
        double z = 0.0;
        for (size_t p = 0; p < L; ++p) {
            e[p] = exp(s[p] - m);
            z += e[p];
        }

        /* probability-weighted sum of V */
        for (size_t d = 0; d < D; ++d) {
            double acc = 0.0;
            for (size_t p = 0; p < L; ++p)
                acc += (e[p] / z) * oracle_half_to_double(v[(p * H + h) * D + d]);
            out[h * D + d] = acc;
        }

        if (scores) {
            for (size_t p = 0; p < S; ++p)
                scores[h * S + p] = p < L ? s[p] : -INFINITY;
        }
        if (weights) {
            for (size_t p = 0; p < S; ++p)
                weights[h * S + p] = p < L ? e[p] / z : 0.0;
        }
    }

    free(s);
    free(e);
    return 0;
}

/*
 * The second kernel of the page's two-dispatch form (attention_pv_f16,
 * section "The MSL, briefly") on its own: softmax of a stored fp16 score row
 * (global max subtracted, shifted exponentials summed, each weight divided
 * by the sum) and the weighted sum of V.  Scores are read as IEEE binary16
 * bits; a score of -inf has weight exactly 0.  Positions after current_pos
 * are skipped, as in oracle_attn_decode.
 *   scores [n_heads, seq_len] binary16 bits; v [seq_len, n_heads, head_dim];
 *   out [n_heads, head_dim] for heads head_lo..head_hi-1.
 * Returns 0, or -1 on a bad argument, allocation failure or a head whose
 * scores are all -inf.
 */
int oracle_attn_pv_from_scores(const uint16_t *scores, const uint16_t *v, uint32_t n_heads,
                               uint32_t head_dim, uint32_t seq_len, uint32_t current_pos,
                               uint32_t head_lo, uint32_t head_hi, double *out)
{
    if (!scores || !v || !out || n_heads == 0 || head_dim == 0 || seq_len == 0 ||
        head_lo > head_hi || head_hi > n_heads)
        return -1;
    const size_t H = n_heads, D = head_dim, S = seq_len;
    const size_t L = (current_pos < seq_len - 1 ? (size_t)current_pos : S - 1) + 1;
    double *e = (double *)malloc(L * sizeof(double));
    if (!e)
        return -1;
    int rc = 0;
    for (size_t h = head_lo; h < head_hi && rc == 0; ++h) {
        double m = -INFINITY;
        for (size_t p = 0; p < L; ++p) {
            const double s = oracle_half_to_double(scores[h * S + p]);
            if (s > m)
                m = s;
        }
        if (m == -INFINITY) {
            rc = -1;
            break;
        }
        double z = 0.0;
        for (size_t p = 0; p < L; ++p) {
            e[p] = exp(oracle_half_to_double(scores[h * S + p]) - m);
            z += e[p];
        }
        for (size_t d = 0; d < D; ++d) {
            double acc = 0.0;
            for (size_t p = 0; p < L; ++p)
                if (e[p] != 0.0)
                    acc += (e[p] / z) * oracle_half_to_double(v[(p * H + h) * D + d]);
            out[h * D + d] = acc;
        }
    }
    free(e);
    return rc;
}

/*
 * IEEE 754 binary16 encoding of a binary64 value, rounded to nearest with
 * ties to even (the rounding of an fp16 store).  Written from the format's
 * definition: normal numbers are n * 2^(E-10) with 1024 <= n < 2048 and
 * -14 <= E <= 15 (bits (E+15) << 10 | (n - 1024)); below 2^-14 the grid is
 * n * 2^-24 with exponent field 0 (bits n, where n = 1024 is the smallest
 * normal); magnitudes that round past 65504 become infinity; NaN stays NaN.
 */
static double oracle_round_half_even(double y)   /* y >= 0, y < 2^52 */
{
    const double f = floor(y);
    const double r = y - f;   /* exact */
    if (r > 0.5)
        return f + 1.0;
    if (r < 0.5)
        return f;
    return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

uint16_t oracle_double_to_half(double x)
{
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    const double a = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00u);
    if (isinf(x))
        return (uint16_t)(sign | 0x7c00u);
    if (a < ldexp(1.0, -14)) {
        const double n = oracle_round_half_even(ldexp(a, 24));   /* 0 .. 1024 */
        return (uint16_t)(sign | (uint16_t)n);
    }
    int ex;
    (void)frexp(a, &ex);   /* a = m * 2^ex, 0.5 <= m < 1, so 2^(ex-1) <= a < 2^ex */
    int E = ex - 1;
    if (E > 15)
        return (uint16_t)(sign | 0x7c00u);
    double n = oracle_round_half_even(ldexp(a, 10 - E));   /* 1024 .. 2048 */
    if (n == 2048.0) {
        n = 1024.0;
        E += 1;
        if (E > 15)
            return (uint16_t)(sign | 0x7c00u);
    }
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(n - 1024.0));
}

void oracle_double_to_half_array(const double *x, size_t n, uint16_t *out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = oracle_double_to_half(x[i]);
}

/*
 * Rotary position embedding, as the page "Tutorial 16: Writing Custom Metal
 * Kernels" (section "5. Example: Fused RoPE Kernel") describes its FastRoPE
 * (dims, base = 10000, traditional = False, one offset per batch entry): the
 * first `dims` values of a vector are split into pairs and each pair is
 * turned through a 2D rotation whose angle grows with the position.
 * Readings where the page leaves a step open:
 *  - pair i (0 <= i < dims/2) turns by the angle pos * theta_i with
 *    theta_i = base^(-2i/dims), the usual rotary frequencies;
 *  - traditional = 0 pairs element i with element i + dims/2, traditional != 0
 *    pairs elements 2i and 2i+1;
 *  - a pair (a, b) becomes (a cos t - b sin t, a sin t + b cos t);
 *  - elements at index >= dims are passed through unchanged.
 * x: n_rows rows of head_dim binary16 values; pos[r] is row r's position;
 * out: fp64 [n_rows, head_dim], exact up to fp64 rounding.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_rope(const uint16_t *x, uint32_t n_rows, uint32_t head_dim, uint32_t dims, double base,
                int traditional, const uint32_t *pos, double *out)
{
    if (!x || !pos || !out || head_dim == 0 || dims > head_dim || (dims & 1u) || !(base > 0.0))
        return -1;
    const size_t D = head_dim;
    const uint32_t half = dims / 2;
    for (size_t r = 0; r < n_rows; ++r) {
        const uint16_t *row = x + r * D;
        double *o = out + r * D;
        for (size_t d = 0; d < D; ++d)
            o[d] = oracle_half_to_double(row[d]);
        for (uint32_t i = 0; i < half; ++i) {
            const size_t ia = traditional ? 2 * (size_t)i : i;
            const size_t ib = traditional ? 2 * (size_t)i + 1 : (size_t)i + half;
            const double theta = pow(base, -(2.0 * i) / (double)dims);
            const double t = (double)pos[r] * theta;
            const double c = cos(t), s = sin(t);
            const double a = oracle_half_to_double(row[ia]);
            const double b = oracle_half_to_double(row[ib]);
            o[ia] = a * c - b * s;
            o[ib] = a * s + b * c;
        }
    }
    return 0;
}

/*
 * Softmax over the last dimension of a [rows, cols] fp32 tensor, as the
 * Foundry notes' fm_softmax (section "API Reference", custom compute kernels:
 * x [rows, cols] -> out [rows, cols]) computes it, with the same max-shifted
 * form as the page "Developing Apple Metal Kernels in Rust - A Deep Dive
 * Through Attention" (section "The MSL, briefly", attention_pv_f16):
 *   m = max_c x[r,c];  z = sum_c exp(x[r,c] - m);  out[r,c] = exp(x[r,c] - m) / z.
 * Inputs are converted to fp64 exactly.  A -inf entry gets exactly 0.  The
 * plain definition is kept where it breaks down: a row of -inf only gives NaN
 * (m = -inf), and a NaN anywhere in a row makes the row NaN.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_softmax_rows(const float *x, uint32_t rows, uint32_t cols, double *out)
{
    if (!x || !out || cols == 0)
        return -1;
    const size_t C = cols;
    for (size_t r = 0; r < rows; ++r) {
        const float *row = x + r * C;
        double *o = out + r * C;
        double m = (double)row[0];
        for (size_t c = 1; c < C; ++c)
            if ((double)row[c] > m)
                m = (double)row[c];
        double z = 0.0;
        for (size_t c = 0; c < C; ++c) {
            o[c] = exp((double)row[c] - m);
            z += o[c];
        }
        for (size_t c = 0; c < C; ++c)
            o[c] = o[c] / z;
    }
    return 0;
}

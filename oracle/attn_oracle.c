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

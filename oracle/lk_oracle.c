/*
 * lk_oracle.c -- plain, slow, single-threaded CPU oracle for the lightning-indexer
 * hot path (key/query quantization, index score, mask, per-row top-k).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls
 * this file.  Only the test suite, the package smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant generator with
 * the HIP path.
 *
 * Sources (the DeepSeek-V3.2-Exp explainer pages and the Trainium NKI page):
 *   - page "Index scores": the score formula S = 1/(sqrt(64) sqrt(128)) sum_h w_h
 *     ReLU(Qbar_h . kbar_s); the fp8_index docstring excerpt (fp8 q @ fp8 k ->
 *     fp32 logits, relu, times folded weights, head sum, times the e8m0 key scale);
 *     the Indexer.forward excerpt (rotate, act_quant, cache write, weight fold,
 *     mask add, top-k).
 *   - page "Hadamard rotation": kbar = ktilde (1/sqrt(128)) H_128, bf16 in/out,
 *     scale = hidden_size ** -0.5, followed by fp8 quantization in 128-feature groups.
 *   - page "Index key cache": fp8 e4m3fn cache with one float32 scale per 128 features.
 *   - NKI page "DeepSeek-V3.2 Sparse Indexer Kernel API Reference": top-k returned as
 *     an unordered int32 set.
 *
 * Readings where the pages are silent (each written out where it is used):
 *   R1 rotate_activation returns bf16 (it asserts a bf16 input; its output feeds
 *      act_quant directly).
 *   R2 H_128 is Sylvester's natural-order Hadamard matrix H[j][i] = (-1)^popcount(i&j).
 *   R3 the rotation is the exact sum, then ONE fp64 multiply by fl64(d ** -0.5),
 *      then round-to-nearest-even straight from fp64 to bf16.
 *   R4 the e8m0 scale is the smallest power of two 2^j (j >= -126) with
 *      amax <= 448 * 2^j; each value is then encoded as e4m3fn(y * 2^-j).
 *   R5 e4m3fn encoding is round-to-nearest-even, keeps the sign (a negative value
 *      that rounds to zero is 0x80), never saturates (unreachable) and never writes NaN.
 *      An exact zero of the rotation is the real number zero and encodes as +0.
 *   R6 the weight fold is w_eff = fl32(fl32(w * q_scale) * fl32(d ** -0.5)), in that
 *      order, where w already carries the 1/sqrt(64) factor.
 *   R7 the key scale multiplies the head sum; masked slots are exactly -inf.
 *   R8 a row's valid keys are the prefix [0, L) with
 *      L = min(T, seq_len_b if given, start_pos + t + 1 if causal).
 *   R9 top-k returns the min(k, L) largest scores of the valid prefix, ties to the
 *      lower index, -0 equal to +0, unused slots -1.
 *
 *   R12 RoPE (Indexer.forward: "rope in indexer is not interleaved"; NKI page: RoPE
 *      rotates the leading rope_dim features, cos and sin tables hold rope_dim/2
 *      entries per token) rotates the pairs (i, i + h), h = rope_dim / 2, i < h:
 *        y_i   = fl32( fl32(x_i c_i) - fl32(x_{i+h} s_i) ),
 *        y_i+h = fl32( fl32(x_i s_i) + fl32(x_{i+h} c_i) ),
 *      each then rounded to bf16 (nearest-even); features >= rope_dim are unchanged.
 *      rope_dim is 64 for the indexer's 128-feature heads.
 *
 *   R13 sparse MLA decode (page "Join query parts", MQA-decode excerpt): for one
 *      decode row and head h, s_t = scale * (qc_h . c_t + qr_h . r_t) over the selected
 *      set I only (the index mask is -inf elsewhere), p = softmax over I,
 *      o_h = sum_{t in I} p_t c_t (the 512-wide latent; the output projection is out of
 *      scope).  Queries, latent cache c and rotary cache r are bf16; the oracle works
 *      in fp64.  Entries -1 of the index list are unused slots; the others are
 *      distinct.  A row whose index list is empty returns zeros.
 *
 * Parity with DeepSeek's own act_quant / fp8_index bytes is unpinned: the pages print
 * no numbers, so R1-R5 cannot be checked against the reference's outputs.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared lk_oracle.c -o liblk_oracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LKO_OK 0
#define LKO_E_RANGE -1   /* input outside the oracle's exact contract */
#define LKO_E_ARG -2     /* bad argument */

/* ------------------------------------------------------------------------- */
/* fp8 e4m3fn (OCP 8-bit floating point): 1 sign, 4 exponent bits (bias 7),   */
/* 3 mantissa bits, no infinities, S.1111.111 is NaN, max finite 448.         */
/* ------------------------------------------------------------------------- */
double lko_e4m3_decode(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);          /* subnormal: 0.m * 2^-6 */
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7); /* normal: 1.m * 2^(e-7) */
    return sign ? -mag : mag;
}

/* Nearest finite e4m3fn code to v by exhaustive search over the 127 non-negative
 * finite codes (they are ordered by magnitude); on a tie the code whose mantissa
 * LSB is 0 wins; the sign bit copies v's sign.  |v| must not exceed 448. */
static double e4m3_pos_tab[0x7F];
static int e4m3_pos_tab_ready = 0;

int lko_e4m3_encode(double v, uint8_t *out)
{
    double a = fabs(v), best_d = INFINITY;
    int best = -1;
    if (!(a <= 448.0))
        return LKO_E_RANGE;
    if (!e4m3_pos_tab_ready) {             /* the 127 non-negative finite values, by code */
        for (int c = 0; c <= 0x7E; c++)
            e4m3_pos_tab[c] = lko_e4m3_decode((uint8_t)c);
        e4m3_pos_tab_ready = 1;
    }
    for (int c = 0; c <= 0x7E; c++) {
        double d = fabs(e4m3_pos_tab[c] - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best_d = d;
            best = c;
        }
    }
    *out = (uint8_t)(best | (signbit(v) ? 0x80 : 0));
    return LKO_OK;
}

/* ------------------------------------------------------------------------- */
/* bfloat16: the upper 16 bits of an IEEE binary32.                           */
/* ------------------------------------------------------------------------- */
double lko_bf16_decode(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, in ONE rounding (no
 * detour through binary32).  bf16 keeps 8 significant bits; below 2^-126 the
 * spacing stays 2^-133 (subnormals).  Returns the bf16 bit pattern. */
int lko_bf16_round(double p, uint16_t *out)
{
    int e;
    double q, y;
    float f;
    uint32_t u;
    if (!isfinite(p))
        return LKO_E_RANGE;
    if (p == 0.0) {
        *out = signbit(p) ? 0x8000 : 0x0000;
        return LKO_OK;
    }
    (void)frexp(fabs(p), &e);
    e -= 1;                        /* 2^e <= |p| < 2^(e+1) */
    if (e < -126)
        e = -126;                  /* subnormal range: fixed spacing */
    q = ldexp(p, 7 - e);           /* exact: p in units of the bf16 spacing */
    q = nearbyint(q);              /* round half to even (default mode) */
    y = ldexp(q, e - 7);
    if (fabs(y) > 3.3895313892515355e38) /* largest finite bf16 */
        return LKO_E_RANGE;
    f = (float)y;                  /* exact: y is a bf16 value */
    memcpy(&u, &f, 4);
    *out = (uint16_t)(u >> 16);
    return LKO_OK;
}

/* ------------------------------------------------------------------------- */
/* Hadamard rotation (page "Hadamard rotation": kbar = ktilde (1/sqrt d) H_d). */
/* ------------------------------------------------------------------------- */
static int popcount_u32(uint32_t x)
{
    int n = 0;
    while (x) {
        n += (int)(x & 1u);
        x >>= 1;
    }
    return n;
}

/* Entry (j, i) of Sylvester's natural-order Hadamard matrix (reading R2). */
int lko_hadamard_entry(int j, int i)
{
    return (popcount_u32((uint32_t)(i & j)) & 1) ? -1 : 1;
}

/* fl64(d ** -0.5), the `scale=hidden_size ** -0.5` argument of rotate_activation.
 * glibc's pow is correctly rounded, as is Python's float power on this platform. */
double lko_rotation_scale(int d)
{
    return pow((double)d, -0.5);
}

static int is_pow2(int d) { return d > 0 && (d & (d - 1)) == 0; }

/* Rotate one row before any rounding to bf16: p_j = fl64(r_j * C) with
 * r_j = sum_i H[j][i] x_i summed exactly (reading R3).  The fp64 sum is exact when
 * the row's nonzero magnitudes span at most 2^38 (8-bit significands, at most
 * 7 bits of carry, 53-bit accumulator); wider rows return LKO_E_RANGE.  d <= 512.
 * Not thread-safe (the matrix table is shared). */
static double hadamard_tab[512 * 512];
static int hadamard_d = 0;

int lko_rotate_row(const uint16_t *x_bf16, int d, double *p_out)
{
    int emin = 100000, emax = -100000;
    double C, xd[512];
    if (!is_pow2(d) || d > 512)
        return LKO_E_ARG;
    for (int i = 0; i < d; i++) {
        double v = lko_bf16_decode(x_bf16[i]);
        int e;
        if (!isfinite(v) || fabs(v) >= 0x1p120)
            return LKO_E_RANGE;
        if (v != 0.0) {
            (void)frexp(v, &e);
            if (e < emin) emin = e;
            if (e > emax) emax = e;
        }
    }
    if (emax >= emin && emax - emin > 38)
        return LKO_E_RANGE;
    C = lko_rotation_scale(d);
    for (int i = 0; i < d; i++)
        xd[i] = lko_bf16_decode(x_bf16[i]);
    if (hadamard_d != d) {                 /* tabulate H_d once from its definition */
        for (int j = 0; j < d; j++)
            for (int i = 0; i < d; i++)
                hadamard_tab[j * d + i] = (double)lko_hadamard_entry(j, i);
        hadamard_d = d;
    }
    for (int j = 0; j < d; j++) {
        double r = 0.0;
        for (int i = 0; i < d; i++)
            r += hadamard_tab[j * d + i] * xd[i];
        if (r == 0.0)
            r = 0.0;               /* the exact sum zero is the real zero: +0 (R5) */
        p_out[j] = r * C;
    }
    return LKO_OK;
}

/* Smallest j >= -126 with A <= 448 * 2^j (reading R4), by direct search. */
int lko_scale_exponent(double amax)
{
    int j = -126;
    while (!(amax <= ldexp(448.0, j)))
        j++;
    return j;
}

/* act_quant of one rotated row (pages "Hadamard rotation" and "Index key cache"):
 * rotate (R1-R3), amax, power-of-two scale (R4), e4m3fn codes (R5).
 * codes[d] receives the bytes, *scale the float32 scale 2^j. */
int lko_quantize_row(const uint16_t *x_bf16, int d, uint8_t *codes, float *scale)
{
    double p[512], y[512], amax = 0.0;
    int rc, j;
    rc = lko_rotate_row(x_bf16, d, p);
    if (rc != LKO_OK)
        return rc;
    for (int i = 0; i < d; i++) {
        uint16_t b;
        rc = lko_bf16_round(p[i], &b);
        if (rc != LKO_OK)
            return rc;
        y[i] = lko_bf16_decode(b);
        if (fabs(y[i]) > amax)
            amax = fabs(y[i]);
    }
    j = lko_scale_exponent(amax);
    for (int i = 0; i < d; i++) {
        rc = lko_e4m3_encode(ldexp(y[i], -j), &codes[i]);
        if (rc != LKO_OK)
            return rc;
    }
    *scale = ldexpf(1.0f, j);
    return LKO_OK;
}

/* Many rows: x is [n_rows][d] bf16, codes [n_rows][d], scales [n_rows]. */
int lko_quantize_rows(const uint16_t *x_bf16, int64_t n_rows, int d,
                      uint8_t *codes, float *scales)
{
    for (int64_t r = 0; r < n_rows; r++) {
        int rc = lko_quantize_row(x_bf16 + r * d, d, codes + r * d, scales + r);
        if (rc != LKO_OK)
            return rc;
    }
    return LKO_OK;
}

/* ------------------------------------------------------------------------- */
/* RoPE on the leading features (reading R12).                                */
/* ------------------------------------------------------------------------- */
int lko_rope_row(const uint16_t *x_bf16, int d, int rope_dim, const float *cos_t,
                 const float *sin_t, uint16_t *y_bf16)
{
    if (rope_dim < 0 || rope_dim > d || (rope_dim & 1)) return LKO_E_ARG;
    const int h = rope_dim / 2;
    for (int i = 0; i < d; i++) y_bf16[i] = x_bf16[i];
    for (int i = 0; i < h; i++) {
        const float a = (float)lko_bf16_decode(x_bf16[i]);
        const float b = (float)lko_bf16_decode(x_bf16[i + h]);
        const float ac = a * cos_t[i], bs = b * sin_t[i];
        const float as = a * sin_t[i], bc = b * cos_t[i];
        const float re = ac - bs, im = as + bc;
        if (lko_bf16_round((double)re, &y_bf16[i]) != LKO_OK) return LKO_E_RANGE;
        if (lko_bf16_round((double)im, &y_bf16[i + h]) != LKO_OK) return LKO_E_RANGE;
    }
    return LKO_OK;
}

/* RoPE then act_quant of many rows: x is [n_rows][d] bf16 and row r uses the cos/sin
 * row (r / rows_per_table_row) of tables [*][rope_dim / 2]. */
int lko_rope_quantize_rows(const uint16_t *x_bf16, int64_t n_rows, int d, int rope_dim,
                           const float *cos_t, const float *sin_t, int64_t rows_per_table_row,
                           uint8_t *codes, float *scales)
{
    uint16_t y[512];
    if (d > 512 || rows_per_table_row < 1) return LKO_E_ARG;
    for (int64_t r = 0; r < n_rows; r++) {
        const int64_t tr = r / rows_per_table_row;
        int rc = lko_rope_row(x_bf16 + r * d, d, rope_dim, cos_t + tr * (rope_dim / 2),
                              sin_t + tr * (rope_dim / 2), y);
        if (rc != LKO_OK) return rc;
        rc = lko_quantize_row(y, d, codes + r * d, scales + r);
        if (rc != LKO_OK) return rc;
    }
    return LKO_OK;
}

/* Weight fold of Indexer.forward (reading R6): the weights times the query's fp8
 * scale, then times softmax_scale = d ** -0.5, both products in float32. */
void lko_fold_weights(const float *w, const float *q_scale, int64_t n, int d,
                      float *w_eff)
{
    const float softmax_scale = (float)pow((double)d, -0.5);
    for (int64_t i = 0; i < n; i++) {
        float a = w[i] * q_scale[i];
        w_eff[i] = a * softmax_scale;
    }
}

/* ------------------------------------------------------------------------- */
/* Mask and index score.                                                      */
/* ------------------------------------------------------------------------- */

/* Valid prefix length L of score row (b, t) (reading R8).  seq_len_b < 0 means
 * "no per-sequence length"; lengths are clamped to [0, T]. */
int64_t lko_valid_len(int64_t T, int64_t seq_len_b, int causal, int64_t start_pos,
                      int64_t t)
{
    int64_t L = T;
    if (seq_len_b >= 0 && seq_len_b < L)
        L = seq_len_b;
    if (causal && start_pos + t + 1 < L)
        L = start_pos + t + 1;
    if (L < 0)
        L = 0;
    return L;
}

/* One score row (page "Index scores", formula and fp8_index docstring):
 *   out[s] = k_scale[s] * sum_h w_eff[h] * max(0, sum_i dec(q8[h][i]) dec(k8[s][i]))
 * for s < L, and -inf for L <= s < T (reading R7).  Each per-head dot product is
 * exact in fp64 (every e4m3fn value times 2^9 is an integer below 2^18, so the
 * products are integers times 2^-18 below 2^36 and the sums stay below 2^43); the
 * head sum is accumulated in fp64.
 *   q8: [H][d] codes of this query token; w_eff: [H];
 *   k8: keys of this sequence, row s at k8 + s * d; k_scale: [T]. */
void lko_score_row(const uint8_t *q8, const float *w_eff, int H, int d,
                   const uint8_t *k8, const float *k_scale, int64_t T, int64_t L,
                   double *out)
{
    double *qd = (double *)malloc(sizeof(double) * (size_t)H * (size_t)d);
    double *kd = (double *)malloc(sizeof(double) * (size_t)d);
    for (int i = 0; i < H * d; i++)
        qd[i] = lko_e4m3_decode(q8[i]);
    for (int64_t s = 0; s < T; s++) {
        double acc = 0.0;
        if (s >= L) {
            out[s] = -INFINITY;
            continue;
        }
        for (int i = 0; i < d; i++)
            kd[i] = lko_e4m3_decode(k8[s * d + i]);
        for (int h = 0; h < H; h++) {
            double dot = 0.0;
            for (int i = 0; i < d; i++)
                dot += qd[h * d + i] * kd[i];
            acc += (double)w_eff[h] * (dot > 0.0 ? dot : 0.0);
        }
        out[s] = acc * (double)k_scale[s];
    }
    free(qd);
    free(kd);
}

/* ------------------------------------------------------------------------- */
/* Top-k (Indexer.forward: index_score.topk(...), NKI page: unordered int32 set). */
/* ------------------------------------------------------------------------- */
typedef struct {
    double v;
    int64_t i;
} lko_item;

static int cmp_desc_then_index(const void *pa, const void *pb)
{
    const lko_item *a = (const lko_item *)pa, *b = (const lko_item *)pb;
    if (a->v > b->v) return -1;    /* larger score first (-0 == +0 here) */
    if (a->v < b->v) return 1;
    if (a->i < b->i) return -1;    /* equal scores: lower index first */
    if (a->i > b->i) return 1;
    return 0;
}

/* Full sort of the valid prefix [0, L) by (score descending, index ascending);
 * out[0..k) receives the first min(k, L) indices, the rest -1 (reading R9). */
static int topk_sorted(lko_item *items, int64_t L, int k, int32_t *out)
{
    int64_t n = L < k ? L : k;
    qsort(items, (size_t)L, sizeof(lko_item), cmp_desc_then_index);
    for (int64_t j = 0; j < k; j++)
        out[j] = j < n ? (int32_t)items[j].i : -1;
    return LKO_OK;
}

int lko_topk_f64(const double *v, int64_t L, int k, int32_t *out)
{
    lko_item *items;
    int rc;
    if (k < 1 || L < 0)
        return LKO_E_ARG;
    items = (lko_item *)malloc(sizeof(lko_item) * (size_t)(L > 0 ? L : 1));
    for (int64_t i = 0; i < L; i++) {
        items[i].v = v[i];
        items[i].i = i;
    }
    rc = topk_sorted(items, L, k, out);
    free(items);
    return rc;
}

int lko_topk_f32(const float *v, int64_t L, int k, int32_t *out)
{
    lko_item *items;
    int rc;
    if (k < 1 || L < 0)
        return LKO_E_ARG;
    items = (lko_item *)malloc(sizeof(lko_item) * (size_t)(L > 0 ? L : 1));
    for (int64_t i = 0; i < L; i++) {
        items[i].v = (double)v[i];
        items[i].i = i;
    }
    rc = topk_sorted(items, L, k, out);
    free(items);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Sparse MLA decode attention over the selected indices (reading R13).       */
/* ------------------------------------------------------------------------- */
/* qc [H][Dc], qr [H][Dr] bf16; kv [T][Dc], pe [T][Dr] bf16 (one sequence); idx [n_idx]
 * int32 (-1 = unused); out [H][Dc] fp64.  Returns LKO_E_ARG for an index outside
 * [0, T). */
int lko_sparse_mla_row(const uint16_t *qc, const uint16_t *qr, int H, int Dc, int Dr,
                       const uint16_t *kv, const uint16_t *pe, int64_t T, const int32_t *idx,
                       int n_idx, double scale, double *out)
{
    for (int i = 0; i < n_idx; i++)
        if (idx[i] >= T || idx[i] < -1) return LKO_E_ARG;
    double *s = (double *)malloc(sizeof(double) * (n_idx > 0 ? n_idx : 1));
    if (!s) return LKO_E_ARG;
    for (int h = 0; h < H; h++) {
        double *o = out + (int64_t)h * Dc;
        for (int c = 0; c < Dc; c++) o[c] = 0.0;
        double m = -INFINITY;
        int any = 0;
        for (int i = 0; i < n_idx; i++) {
            if (idx[i] < 0) continue;
            const uint16_t *kt = kv + (int64_t)idx[i] * Dc;
            const uint16_t *rt = pe + (int64_t)idx[i] * Dr;
            double dot = 0.0;
            for (int c = 0; c < Dc; c++) dot += lko_bf16_decode(qc[(int64_t)h * Dc + c]) * lko_bf16_decode(kt[c]);
            for (int c = 0; c < Dr; c++) dot += lko_bf16_decode(qr[(int64_t)h * Dr + c]) * lko_bf16_decode(rt[c]);
            s[i] = scale * dot;
            if (s[i] > m) m = s[i];
            any = 1;
        }
        if (!any) continue;
        double l = 0.0;
        for (int i = 0; i < n_idx; i++) {
            if (idx[i] < 0) continue;
            const double p = exp(s[i] - m);
            l += p;
            const uint16_t *kt = kv + (int64_t)idx[i] * Dc;
            for (int c = 0; c < Dc; c++) o[c] += p * lko_bf16_decode(kt[c]);
        }
        for (int c = 0; c < Dc; c++) o[c] /= l;
    }
    free(s);
    return LKO_OK;
}

/*
 * Plain CPU oracle for the hot path of DeepSeek-V4.1 compressed sparse
 * attention: the fp8 round trip of kv rows, the window selection, the indexer
 * score, the index top-k and the sparse attention with a per-head sink, and
 * the rotary embedding (its table and the rotation) that the kv rows and the
 * queries go through before the path, the candidate-block selection
 * that produces the block mask the indexer takes, and the grouped output
 * projection after it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * shares no code, header, table or helper with it, and it includes nothing
 * from that library.  It is deliberately slow: scalar loops, one element at a
 * time, in double precision, with a single rounding to the output type.
 *
 * Sources (the pages this follows):
 *  - "deepseek_v41_ref::attn" rustdoc, module description and the function
 *    contracts act_quant_inplace, pow2_ceil, window_topk_idxs, sparse_attn,
 *    apply_rotary, freqs_cis (precision contract; ring-cache example).
 *  - "Compressed sparse attention" layer page (atlas, reindex layer,
 *    p=1000), section "All 25 steps": the FP8(W) step, the indexer score
 *    S^I, the top-512 selection I_t, the window set J^w_t, the join Y/J/G_t,
 *    the sink softmax A and O, and the rotations R_t (queries, window keys)
 *    and R_t^-1 (output); the model code and config shown on that page
 *    (RoPE on the last rope_head_dim = 64 values, rope_theta = 10000 at
 *    ratio 0).
 *  - "attn_v41.rs" source page, module documentation (selection width
 *    limit, -1 = absent, indices offset past the window rows) and the
 *    AttnV41Run struct (q after RoPE, rows_a / rows_b, idx layout).
 *
 * Readings taken where the pages are silent (each is listed with its reason
 * in the design notes of the repository):
 *  - e4m3 is the OCP E4M3FN format (bias 7, 3 fraction bits, subnormals,
 *    largest finite 448, no infinities): the page's 448 rules out E4M3FNUZ.
 *  - The fp8 block is 32 consecutive values along a row.
 *  - A negative value that rounds to zero keeps its sign (-0).
 *  - The top-k breaks ties by the lower position; +0 and -0 are equal;
 *    -inf and NaN scores are excluded; fewer than k valid positions are
 *    padded with -1.  The selection is a set; it is written in ascending
 *    position order.
 *  - The softmax subtracts m = max(sink_h, max_i s_i) before exp: the
 *    result is the same real number, it only avoids overflow of exp.
 *  - Index values outside [0, rows_a_len + rows_b_len) are skipped like -1.
 *  - The RoPE table is cos/sin of p * theta^(-2i/rope_dim), rounded once to
 *    binary32; the rotation's binary32 products are not fused.
 *  - A candidate block's score is the largest valid score of its positions;
 *    the blocks are chosen by the index top-k's rule.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* bf16 <-> double                                                     */
/* ------------------------------------------------------------------ */

/* bf16 is the top 16 bits of an IEEE binary32; widening is exact. */
double ora_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round a double to the nearest bf16, ties to even, in one step.
 * bf16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 * Normal numbers in [2^-126, 2^128) have a quantum of 2^(E-7) where
 * E = floor(log2|x|); below 2^-126 the quantum is the subnormal step
 * 2^-133.  A magnitude that rounds to 2^128 or more overflows to inf.
 */
uint16_t ora_double_to_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7F80;
    int e2;
    frexp(a, &e2);             /* a = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;            /* floor(log2 a) */
    int qexp = (E < -126) ? -133 : E - 7;
    double q = ldexp(1.0, qexp);
    double r = nearbyint(a / q) * q;  /* default mode: to nearest, ties even */
    if (r >= ldexp(1.0, 128))
        return sign | 0x7F80;
    float rf = (float)r;              /* exact: r is on the bf16 grid */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* fp8 round trip (act_quant_inplace; FP8(W) step)                     */
/* ------------------------------------------------------------------ */

/*
 * pow2_ceil: 2^ceil(log2 v) for a positive normal binary32 v, from the IEEE
 * fields: a value whose fraction field is zero is already a power of two;
 * otherwise the result is the power of two one above its exponent.
 */
float ora_pow2_ceil(float v)
{
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    uint32_t exp_field = (u >> 23) & 0xFFu;
    uint32_t frac_field = u & 0x7FFFFFu;
    uint32_t out_exp = exp_field + (frac_field != 0 ? 1u : 0u);
    uint32_t r = out_exp << 23;
    float f;
    memcpy(&f, &r, sizeof f);
    return f;
}

/*
 * Round y (|y| <= 448 after the clamp) to the nearest OCP E4M3FN value, ties
 * to even.  E4M3FN normal numbers are 1.fff * 2^(e-7), e = 1..15, so in the
 * binade [2^E, 2^(E+1)) the quantum is 2^(E-3); below 2^-6 the subnormals
 * 0.fff * 2^-6 have the quantum 2^-9.  The sign of y is kept, zero included.
 */
double ora_e4m3_round(double y)
{
    double a = fabs(y);
    double r;
    if (a == 0.0) {
        r = 0.0;
    } else {
        int e2;
        frexp(a, &e2);
        int E = e2 - 1;
        int qexp = (E < -6) ? -9 : E - 3;
        double q = ldexp(1.0, qexp);
        r = nearbyint(a / q) * q;
    }
    return copysign(r, y);
}

/*
 * One block of n values (n = 32 in the method): amax over the block, floored
 * at 1e-4 (binary32), scale = pow2_ceil(amax / 448) with the division done in
 * binary32, each value divided by the scale, clamped to +-448, rounded to
 * e4m3, multiplied back by the scale and rounded to bf16.
 */
static void fp8_round_block(const uint16_t *in, uint16_t *out, int n)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float v = (float)fabs(ora_bf16_to_double(in[i]));  /* exact */
        if (v > amax)
            amax = v;
    }
    if (amax < 1e-4f)
        amax = 1e-4f;
    float s = ora_pow2_ceil(amax / 448.0f);
    for (int i = 0; i < n; ++i) {
        double x = ora_bf16_to_double(in[i]);
        double y = x / (double)s;           /* exact: s is a power of two */
        if (y > 448.0)
            y = 448.0;
        if (y < -448.0)
            y = -448.0;
        double e = ora_e4m3_round(y);
        out[i] = ora_double_to_bf16(e * (double)s);
    }
}

/*
 * Rows of row_len bf16 values (row_len a multiple of block); in and out may
 * be the same buffer.  Returns 0, or -1 for a row_len that is not a multiple
 * of the block.
 */
int ora_fp8_round_rows(const uint16_t *in, uint16_t *out, int64_t rows,
                       int32_t row_len, int32_t block)
{
    if (block <= 0 || row_len % block != 0)
        return -1;
    uint16_t tmp[4096];
    if (block > 4096)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int32_t c = 0; c < row_len; c += block) {
            const uint16_t *src = in + r * (int64_t)row_len + c;
            fp8_round_block(src, tmp, block);
            memcpy(out + r * (int64_t)row_len + c, tmp,
                   sizeof(uint16_t) * (size_t)block);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* window selection (window_topk_idxs; J^w_t)                          */
/* ------------------------------------------------------------------ */

/*
 * start_pos == 0: one causal window per query into the chunk itself,
 *   cols = min(n_tokens, window); query t sees chunk rows
 *   max(0, t - window + 1) .. t in ascending order, then -1.
 * start_pos > 0: one query (the token at start_pos); the whole ring, oldest
 *   first: slot (start_pos + 1 + c) mod window once the ring has wrapped
 *   (start_pos >= window - 1); before that slots 0..start_pos, then -1.
 * Writes idx[n_tokens][cols] and returns cols, or -1 when start_pos > 0 and
 * n_tokens != 1.
 */
int ora_window_idx(int64_t start_pos, int32_t n_tokens, int32_t window,
                   int32_t *idx)
{
    if (start_pos == 0) {
        int32_t cols = n_tokens < window ? n_tokens : window;
        for (int32_t t = 0; t < n_tokens; ++t) {
            int32_t lo = t - window + 1;
            if (lo < 0)
                lo = 0;
            for (int32_t c = 0; c < cols; ++c) {
                int32_t slot = lo + c;
                idx[(int64_t)t * cols + c] = (slot <= t) ? slot : -1;
            }
        }
        return cols;
    }
    if (n_tokens != 1)
        return -1;
    for (int32_t c = 0; c < window; ++c) {
        if (start_pos >= window - 1)
            idx[c] = (int32_t)((start_pos + 1 + c) % window);
        else
            idx[c] = (c <= start_pos) ? c : -1;
    }
    return window;
}

/* ------------------------------------------------------------------ */
/* indexer score (S^I) for one query                                   */
/* ------------------------------------------------------------------ */

/* Causal count of compressed positions visible to the token at position pos:
 * floor((pos + 1) / ratio), capped at the rows present. */
int64_t ora_causal_count(int64_t pos, int32_t ratio, int64_t n_rows)
{
    int64_t n = (pos + 1) / ratio;
    return n < n_rows ? n : n_rows;
}

/*
 * S[j] = sum_h w[h] * ReLU( sum_d qI[h][d] * kI[j][d] ) for j < n_valid and,
 * when cand is given, cand[j / cand_block] != 0; every other j gets -inf.
 * qI: [n_heads][head_dim] bf16, kI: [n_rows][head_dim] bf16 (one key per
 * compressed position, shared by all heads), w: [n_heads] f32.
 */
void ora_indexer_scores_one(const uint16_t *qI, const uint16_t *kI,
                            const float *w, const uint8_t *cand,
                            int32_t cand_block, int32_t n_heads,
                            int32_t head_dim, int64_t n_rows, int64_t n_valid,
                            double *out)
{
    for (int64_t j = 0; j < n_rows; ++j) {
        int allowed = j < n_valid;
        if (allowed && cand != NULL && cand[j / cand_block] == 0)
            allowed = 0;
        if (!allowed) {
            out[j] = -INFINITY;
            continue;
        }
        double total = 0.0;
        for (int32_t h = 0; h < n_heads; ++h) {
            double dot = 0.0;
            for (int32_t d = 0; d < head_dim; ++d)
                dot += ora_bf16_to_double(qI[(int64_t)h * head_dim + d]) *
                       ora_bf16_to_double(kI[j * head_dim + d]);
            double relu = dot > 0.0 ? dot : 0.0;
            total += (double)w[h] * relu;
        }
        out[j] = total;
    }
}

/* ------------------------------------------------------------------ */
/* index top-k (I_t = top_k(S^I ...))                                  */
/* ------------------------------------------------------------------ */

struct ora_scored {
    double s;
    int64_t j;
};

/* Order: higher score first; equal scores (+0 == -0) by lower position. */
static int cmp_scored(const void *pa, const void *pb)
{
    const struct ora_scored *a = (const struct ora_scored *)pa;
    const struct ora_scored *b = (const struct ora_scored *)pb;
    if (a->s > b->s)
        return -1;
    if (a->s < b->s)
        return 1;
    if (a->j < b->j)
        return -1;
    if (a->j > b->j)
        return 1;
    return 0;
}

static int cmp_position(const void *pa, const void *pb)
{
    int64_t a = ((const struct ora_scored *)pa)->j;
    int64_t b = ((const struct ora_scored *)pb)->j;
    return (a > b) - (a < b);
}

/*
 * Valid positions are those whose score is neither -inf nor NaN.  The m =
 * min(k, #valid) best positions in (score desc, position asc) order form the
 * selection; it is written as positions plus offset in ascending position
 * order, then -1 up to k entries.  Returns m, or -1 on allocation failure.
 */
int64_t ora_topk_one(const double *scores, int64_t n, int32_t k,
                     int32_t offset, int32_t *out)
{
    struct ora_scored *v = (struct ora_scored *)malloc(
        sizeof(struct ora_scored) * (size_t)(n > 0 ? n : 1));
    if (v == NULL)
        return -1;
    int64_t nv = 0;
    for (int64_t j = 0; j < n; ++j) {
        double s = scores[j];
        if (isnan(s) || (isinf(s) && s < 0))
            continue;
        v[nv].s = s;
        v[nv].j = j;
        ++nv;
    }
    qsort(v, (size_t)nv, sizeof(struct ora_scored), cmp_scored);
    int64_t m = nv < k ? nv : k;
    qsort(v, (size_t)m, sizeof(struct ora_scored), cmp_position);
    for (int32_t i = 0; i < k; ++i)
        out[i] = (i < m) ? (int32_t)(v[i].j + offset) : -1;
    free(v);
    return m;
}

/* ------------------------------------------------------------------ */
/* sparse attention with the sink (S, A, O steps; sparse_attn)         */
/* ------------------------------------------------------------------ */

/*
 * The gathered row for joint index ix: rows_a (the window rows) for
 * ix < rows_a_len, rows_b (the compressed rows) for the rest; NULL when ix
 * is -1 or out of range.
 */
static const uint16_t *gather_row(int64_t ix, const uint16_t *rows_a,
                                  int64_t rows_a_len, const uint16_t *rows_b,
                                  int64_t rows_b_len, int32_t head_dim)
{
    if (ix < 0)
        return NULL;
    if (ix < rows_a_len)
        return rows_a + ix * head_dim;
    if (rows_b != NULL && ix - rows_a_len < rows_b_len)
        return rows_b + (ix - rows_a_len) * head_dim;
    return NULL;
}

/*
 * Attention weights of one head of one query: for each idx entry i, A_i =
 * exp(s_i) / (exp(sink) + sum_j exp(s_j)) with s_i = scale * q . g_i, and 0
 * for skipped entries.  Also returns the sink's share exp(sink) / den.
 * Scores are shifted by m = max(sink, max_i s_i) before exp.
 */
double ora_attn_weights_one_head(const uint16_t *q_h, const uint16_t *rows_a,
                                 int64_t rows_a_len, const uint16_t *rows_b,
                                 int64_t rows_b_len, const int32_t *idx,
                                 int32_t width, float sink, double scale,
                                 int32_t head_dim, double *weights)
{
    double m = (double)sink;
    for (int32_t i = 0; i < width; ++i) {
        const uint16_t *g = gather_row(idx[i], rows_a, rows_a_len, rows_b,
                                       rows_b_len, head_dim);
        if (g == NULL) {
            weights[i] = -INFINITY;
            continue;
        }
        double dot = 0.0;
        for (int32_t d = 0; d < head_dim; ++d)
            dot += ora_bf16_to_double(q_h[d]) * ora_bf16_to_double(g[d]);
        weights[i] = dot * scale;
        if (weights[i] > m)
            m = weights[i];
    }
    double den = exp((double)sink - m);
    for (int32_t i = 0; i < width; ++i)
        if (!isinf(weights[i]))
            den += exp(weights[i] - m);
    for (int32_t i = 0; i < width; ++i)
        weights[i] = isinf(weights[i]) ? 0.0 : exp(weights[i] - m) / den;
    return exp((double)sink - m) / den;
}

/*
 * One query, all heads: o[h] = sum_i A_{h,i} g_i, rounded to bf16.
 * q: [n_heads][head_dim], sink: [n_heads], out: [n_heads][head_dim].
 * A query with no valid index gets o = 0.  Returns 0, or -1 on allocation
 * failure.
 */
int ora_sparse_attn_one(const uint16_t *q, const uint16_t *rows_a,
                        int64_t rows_a_len, const uint16_t *rows_b,
                        int64_t rows_b_len, const int32_t *idx, int32_t width,
                        const float *sink, double scale, int32_t n_heads,
                        int32_t head_dim, uint16_t *out)
{
    double *wts = (double *)malloc(sizeof(double) * (size_t)(width > 0 ? width : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)head_dim);
    if (wts == NULL || acc == NULL) {
        free(wts);
        free(acc);
        return -1;
    }
    for (int32_t h = 0; h < n_heads; ++h) {
        const uint16_t *q_h = q + (int64_t)h * head_dim;
        ora_attn_weights_one_head(q_h, rows_a, rows_a_len, rows_b, rows_b_len,
                                  idx, width, sink[h], scale, head_dim, wts);
        for (int32_t d = 0; d < head_dim; ++d)
            acc[d] = 0.0;
        for (int32_t i = 0; i < width; ++i) {
            const uint16_t *g = gather_row(idx[i], rows_a, rows_a_len, rows_b,
                                           rows_b_len, head_dim);
            if (g == NULL)
                continue;
            for (int32_t d = 0; d < head_dim; ++d)
                acc[d] += wts[i] * ora_bf16_to_double(g[d]);
        }
        for (int32_t d = 0; d < head_dim; ++d)
            out[(int64_t)h * head_dim + d] = ora_double_to_bf16(acc[d]);
    }
    free(wts);
    free(acc);
    return 0;
}

/* ------------------------------------------------------------------ */
/* rotary position embedding (apply_rotary, freqs_cis; R_t, R_t^-1)    */
/* ------------------------------------------------------------------ */

/*
 * The RoPE table at ratio 0 ("deepseek_v41_ref::attn" rustdoc, freqs_cis:
 * [seqlen][dim/2] pairs (cos, sin), no YaRN; base rope_theta = 10000 in the
 * config shown on the "Compressed sparse attention" layer page).
 *
 * Reading (the pages name the table and its shape, not its formula): pair i
 * of position p holds the cosine and sine of the angle p * theta^(-2i/dim),
 * the usual rotary frequency ladder, pair 0 turning fastest.  Each entry is
 * the real number rounded once to binary32; it is evaluated in long double
 * (64-bit significand) so that the one rounding to binary32 is the only one
 * that matters.
 *
 * table: [n_pos][rope_dim / 2][2] floats.  Returns 0, or -1 for an odd or
 * non-positive rope_dim or a non-positive theta.
 */
int ora_rope_table(double theta, int32_t rope_dim, int64_t n_pos, float *table)
{
    if (rope_dim <= 0 || rope_dim % 2 != 0 || !(theta > 0.0))
        return -1;
    int32_t half = rope_dim / 2;
    for (int32_t i = 0; i < half; ++i) {
        long double expo = -(long double)(2 * i) / (long double)rope_dim;
        long double freq = powl((long double)theta, expo);
        for (int64_t p = 0; p < n_pos; ++p) {
            long double ang = (long double)p * freq;
            table[(p * half + i) * 2 + 0] = (float)cosl(ang);
            table[(p * half + i) * 2 + 1] = (float)sinl(ang);
        }
    }
    return 0;
}

/*
 * Rotate the last rope_dim values of each row ("deepseek_v41_ref::attn"
 * rustdoc, apply_rotary; "Compressed sparse attention", All 25 steps:
 * Q_{...,448:} <- R_t Q, W_{t,448:} <- R_t w^n, and the inverse R_t^-1 on O).
 *
 * The rotated part is read as rope_dim/2 complex numbers, element 2i the
 * real part and element 2i+1 the imaginary part of number i; number i is
 * multiplied by table[pos][i] = cos + i sin (by cos - i sin when inverse is
 * set: the negated angle).  The product is taken in binary32, as the
 * precision paragraph of the same page fixes:
 *     re = x0*c - x1*s,   im = x0*s + x1*c
 * with each product and each sum rounded to binary32 (no fused
 * multiply-add; reading: the pages fix the precision, not the order), and
 * each result rounded once to bf16.  Values before the rotated part are
 * copied.
 *
 * in, out: [rows][row_len] bf16 (may be the same buffer); row r is at
 * position row_pos[r]; table: [..][rope_dim/2][2].  Returns 0, or -1 for a
 * rope_dim that is odd, non-positive or larger than row_len.
 */
int ora_rope_rows(const uint16_t *in, uint16_t *out, int64_t rows,
                  int32_t row_len, int32_t rope_dim, const float *table,
                  const int64_t *row_pos, int32_t inverse)
{
    if (rope_dim <= 0 || rope_dim % 2 != 0 || rope_dim > row_len)
        return -1;
    int32_t half = rope_dim / 2;
    int32_t start = row_len - rope_dim;
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *x = in + r * (int64_t)row_len;
        uint16_t *y = out + r * (int64_t)row_len;
        for (int32_t d = 0; d < start; ++d)
            y[d] = x[d];
        const float *tab = table + row_pos[r] * (int64_t)half * 2;
        for (int32_t i = 0; i < half; ++i) {
            float c = tab[2 * i + 0];
            float s = tab[2 * i + 1];
            if (inverse)
                s = -s;
            float x0 = (float)ora_bf16_to_double(x[start + 2 * i]);
            float x1 = (float)ora_bf16_to_double(x[start + 2 * i + 1]);
            float a = x0 * c;
            float b = x1 * s;
            float re = a - b;
            float e = x0 * s;
            float f = x1 * c;
            float im = e + f;
            y[start + 2 * i] = ora_double_to_bf16((double)re);
            y[start + 2 * i + 1] = ora_double_to_bf16((double)im);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* candidate blocks (the candidate-source layer's block-level mask)     */
/* ------------------------------------------------------------------ */

/*
 * The candidate-source layer publishes a block-level candidate mask that
 * later index sources apply ("attn_v41" module page and "attn_v41.rs":
 * SharedV41.candidates [queries][cand_width]; a candidate-block top-k
 * selection beside the index top-k; config candidate_topk_blocks = 2048,
 * candidate_block_size = 8 on the "Compressed sparse attention" layer page).
 *
 * Readings (the pages name the selection, not how a block is scored): block
 * b covers compressed positions [b * cand_block, (b + 1) * cand_block) of a
 * score row; its score is the largest score of its positions that is
 * neither -inf nor NaN (-inf when there is none); the mask marks the
 * topk_blocks best blocks under the index top-k's own rule (score
 * descending, equal scores to the lower block, -inf blocks never chosen).
 * Block scores are maxima of the given scores, so no arithmetic enters.
 *
 * scores: [n] doubles; mask: [ceil(n / cand_block)] bytes, 1 = candidate.
 * Returns the number of candidate blocks, or -1 on a bad argument or an
 * allocation failure.
 */
int64_t ora_candidate_blocks_one(const double *scores, int64_t n,
                                 int32_t cand_block, int32_t topk_blocks,
                                 uint8_t *mask)
{
    if (cand_block < 1 || topk_blocks < 1 || n < 0)
        return -1;
    int64_t nb = (n + cand_block - 1) / cand_block;
    double *bs = (double *)malloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1));
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)topk_blocks);
    if (bs == NULL || sel == NULL) {
        free(bs);
        free(sel);
        return -1;
    }
    for (int64_t b = 0; b < nb; ++b) {
        double m = -INFINITY;
        for (int64_t j = b * cand_block; j < n && j < (b + 1) * cand_block; ++j) {
            double s = scores[j];
            if (!isnan(s) && s > m)
                m = s;
        }
        bs[b] = m;
    }
    int64_t got = ora_topk_one(bs, nb, topk_blocks, 0, sel);
    if (got >= 0) {
        memset(mask, 0, (size_t)nb);
        for (int32_t i = 0; i < topk_blocks; ++i)
            if (sel[i] >= 0)
                mask[sel[i]] = 1;
    }
    free(bs);
    free(sel);
    return got;
}

/* ------------------------------------------------------------------ */
/* grouped output projection (o^g = [O_bar_h]_{h in r} W_OA,r; D = o^g W_OB) */
/* ------------------------------------------------------------------ */

/*
 * The output side of the layer ("Compressed sparse attention", All 25 steps,
 * "Grouped output": o^g_{t,r} = [O_bar_{h,t}]_{h in r} W_{OA,r} and
 * Delta = o^g W_{OB}; the model code on that page views o as [T, groups,
 * heads*head_dim/groups] and contracts each group with its own slice of wo_a,
 * then applies wo_b to the flattened groups; "attn_v41.rs": wo_a is
 * [groups * o_rank, gw] and wo_b [dim, groups * o_rank], both [out, in];
 * "deepseek_v41_ref::attn" precision paragraph: every projection accumulates
 * in f32 and returns bf16).
 *
 * o_bar: [T][groups * gw] bf16 (the attention output after the inverse
 * rotation, heads contiguous, so group g holds heads g*H/groups ..);
 * wo_a: [groups * rank][gw]; wo_b: [dim][groups * rank];
 * og: [T][groups * rank] bf16 out; x: [T][dim] bf16 out.
 * og[t][g*rank + r] = sum_d o_bar[t][g*gw + d] * wo_a[g*rank + r][d], and
 * x[t][c] = sum_j og[t][j] * wo_b[c][j] over the bf16 og, each sum taken in
 * double and rounded once to bf16 (the f32 accumulation of the pages is the
 * same real number up to its rounding).
 */
void ora_grouped_output(const uint16_t *o_bar, const uint16_t *wo_a,
                        const uint16_t *wo_b, int64_t T, int32_t groups,
                        int32_t rank, int32_t gw, int32_t dim, uint16_t *og,
                        uint16_t *x)
{
    int64_t width = (int64_t)groups * gw;
    int64_t og_w = (int64_t)groups * rank;
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *ot = o_bar + t * width;
        uint16_t *gt = og + t * og_w;
        for (int32_t g = 0; g < groups; ++g) {
            for (int32_t r = 0; r < rank; ++r) {
                const uint16_t *wr = wo_a + ((int64_t)g * rank + r) * gw;
                double acc = 0.0;
                for (int32_t d = 0; d < gw; ++d)
                    acc += ora_bf16_to_double(ot[(int64_t)g * gw + d]) *
                           ora_bf16_to_double(wr[d]);
                gt[(int64_t)g * rank + r] = ora_double_to_bf16(acc);
            }
        }
        uint16_t *xt = x + t * dim;
        for (int32_t c = 0; c < dim; ++c) {
            const uint16_t *wc = wo_b + (int64_t)c * og_w;
            double acc = 0.0;
            for (int64_t j = 0; j < og_w; ++j)
                acc += ora_bf16_to_double(gt[j]) * ora_bf16_to_double(wc[j]);
            xt[c] = ora_double_to_bf16(acc);
        }
    }
}

/*
 * One projection as the pages' linear_bf16 ("deepseek_v41_ref::attn"
 * precision paragraph: f32 accumulation, bf16 result; weights [out, in]):
 * y[m][n] = sum_k a[m][k] * w[n][k], the sum in double, rounded once to bf16.
 * a: [M][K], w: [N][K], y: [M][N], all bf16.
 */
void ora_linear_bf16(const uint16_t *a, const uint16_t *w, int64_t M,
                     int32_t N, int32_t K, uint16_t *y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int32_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int32_t k = 0; k < K; ++k)
                acc += ora_bf16_to_double(a[m * K + k]) *
                       ora_bf16_to_double(w[(int64_t)n * K + k]);
            y[m * N + n] = ora_double_to_bf16(acc);
        }
}

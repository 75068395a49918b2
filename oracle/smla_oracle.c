/*
 * Plain FP64 CPU oracle for sparse MLA decode and the split-KV LSE merge.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * HIP library; it is written from the pages' statement of the method:
 *
 *   [sparse_mla_cute page]  "What this module computes": per token t and head h,
 *       over the active columns c (c < lens[t] and indices[t,c] >= 0),
 *       s_c = bmm1 * q[t,h].kv[c],  p_c = exp(s_c - m),
 *       out = bmm2 * sum_c p_c kv[c] / (sum_c p_c + exp(sink_h - m)),
 *       m the maximum of the scores and the sink; the first 128 columns index the
 *       sliding-window pool, the others the compressed pool; a token with no
 *       active column gets zeros.
 *   [attn_sparse page]  module docstring: the E4M3-P online-softmax recipe
 *       (P = exp2(s*scale_log2 - max + log2 448) as E4M3, RN, satfinite; FP32
 *       sums of the unquantized P; rescale when the running max rises), the
 *       split merge (weights exp2(max_c - max), BF16(sum*k_scale/total),
 *       LSE = max + log2(total/448)), the "Rows of count 0" rule, and
 *       SparseDcpDecode.kernel's contiguous key split of the clamped count.
 *   [sparse_mla_cute page]  "How.": the chunk-local recipe (one softmax per
 *       128-column chunk at its own maximum, P = 256 exp2(S - m_c) as FP8,
 *       the chunks' partials weighted by exp2(m_c - M) / L over the chunks
 *       and the sink).
 *   [dcp page]  DcpValue.merge: LSE-weighted merge of D sources, weights
 *       exp2(lse - top) / sum, empty sources weighted 0.
 *
 * Everything is computed in double precision, one (token, head) at a time,
 * column by column, with no blocking or reordering beyond what the formula or
 * the recipe states.
 *
 * Parity pins (tests, CPU only): E4M3 decode against torch.float8_e4m3fn for
 * all 256 codes; exact mode against dense float64 scaled-dot-product attention
 * on materialised rows; softmax invariants; the zero-count rule; mimic mode
 * and chunk-local mode reducing to exact mode when P is not quantized;
 * lse_merge split consistency; chunk-local mode equal to lse_merge of its
 * chunks computed one by one, and to a hand-worked two-chunk example.
 * The E4M3-P recipes have no printed worked values on the pages: their
 * quantization steps are pinned only through those reductions, invariants
 * and the hand-worked example ("parity unpinned" for the recipes' rounding
 * details beyond them).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EBADARG 1
#define ORACLE_ERANGE 2   /* an active column's index is >= rows of its pool */
#define ORACLE_ENAN 3     /* an E4M3 NaN code (0x7F / 0xFF) in q or an active row */

#define ORACLE_LSE_LOG2 1u

/* ---------------------------------------------------------------------------
 * Number formats
 * ------------------------------------------------------------------------- */

/* OCP E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; there is no
 * infinity; the largest finite magnitude is 448. */
double oracle_e4m3_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int exponent = (code >> 3) & 0xF;
    int mantissa = code & 0x7;
    double magnitude;
    if (exponent == 0xF && mantissa == 0x7)
        return NAN;
    if (exponent == 0)
        magnitude = ldexp((double)mantissa, -9);
    else
        magnitude = ldexp(1.0 + mantissa / 8.0, exponent - 7);
    return sign ? -magnitude : magnitude;
}

/* E4M3 of x: round to nearest, ties to even, saturating to +-448 ("satfinite,
 * RN" on the attn_sparse page, store_fp8_pair_shared).  Done by searching the
 * 127 non-negative finite codes, which are ordered by value, for the nearest;
 * on a tie the code with an even mantissa (even code) wins. */
uint8_t oracle_e4m3_encode(double x)
{
    double a = fabs(x);
    int best = 0;
    if (isnan(x))
        return 0x7F;
    if (a >= 448.0) {
        best = 0x7E;
    } else {
        int lo = 0;
        int hi;
        while (lo + 1 <= 0x7E && oracle_e4m3_value((uint8_t)(lo + 1)) <= a)
            lo++;
        hi = lo + 1 <= 0x7E ? lo + 1 : lo;
        if (hi == lo) {
            best = lo;
        } else {
            double dlo = a - oracle_e4m3_value((uint8_t)lo);
            double dhi = oracle_e4m3_value((uint8_t)hi) - a;
            if (dlo < dhi)
                best = lo;
            else if (dhi < dlo)
                best = hi;
            else
                best = (lo % 2 == 0) ? lo : hi;
        }
    }
    if (best == 0)
        return (x < 0 || (x == 0 && signbit(x))) ? 0x80 : 0x00;
    return (uint8_t)(x < 0 ? (0x80 | best) : best);
}

/* BF16 is the upper half of an IEEE binary32. */
double oracle_bf16_value(uint16_t bits)
{
    union { uint32_t u; float f; } v;
    v.u = ((uint32_t)bits) << 16;
    return (double)v.f;
}

/* ---------------------------------------------------------------------------
 * Shared argument handling (of the oracle only)
 * ------------------------------------------------------------------------- */

typedef struct {
    const uint8_t *q;
    int64_t q_stride_t, q_stride_h;
    const uint8_t *kv_a;
    int64_t rows_a;
    const uint8_t *kv_b;
    int64_t rows_b;
    int32_t split_col;
    int32_t row_bytes, qk_dim;
    const int32_t *indices, *lens;
    int32_t T, H, W;
    double bmm1, bmm2;
    const float *sinks;
} problem;

/* The row of column c of token t, or NULL (with *status set) when the index is
 * out of range.  Columns below split_col use pool A, the rest pool B; with no
 * pool B every column uses pool A ("the first 128 columns" rule, generalised to
 * split_col). */
static const uint8_t *row_of(const problem *p, int t, int c, int *status)
{
    int32_t idx = p->indices[(int64_t)t * p->W + c];
    int use_b = (p->kv_b != NULL) && (c >= p->split_col);
    int64_t rows = use_b ? p->rows_b : p->rows_a;
    const uint8_t *pool = use_b ? p->kv_b : p->kv_a;
    if (idx < 0 || (int64_t)idx >= rows) {
        *status = ORACLE_ERANGE;
        return NULL;
    }
    return pool + (int64_t)idx * p->row_bytes;
}

/* n = clamp(lens[t], 0, W). */
static int active_count(const problem *p, int t)
{
    int n = p->lens[t];
    if (n < 0)
        n = 0;
    if (n > p->W)
        n = p->W;
    return n;
}

static int is_active(const problem *p, int t, int c, int n)
{
    return c < n && p->indices[(int64_t)t * p->W + c] >= 0;
}

/* Element d of a row: with 576- or 512-byte rows, the E4M3 byte d.  With
 * 656-byte fp8_ds_mla rows (the dsa_indexer page: a 656-byte MLA cache entry
 * holding [kv_c_normed | k_pe], viewed as FP8, FP32 and BF16), read as bytes
 * 0..511 the E4M3 latent, bytes 512..527 four FP32 scales (one per 128 latent
 * elements), bytes 528..655 the 64-element rope in BF16: latent element d is
 * E4M3(byte d) * scale[d / 128], rope element d - 512 is the BF16 value. */
#define DS_MLA_ROW 656

static double kv_value(const problem *p, const uint8_t *row, int d)
{
    if (p->row_bytes != DS_MLA_ROW)
        return oracle_e4m3_value(row[d]);
    if (d < 512) {
        float scale;
        memcpy(&scale, row + 512 + 4 * (d / 128), sizeof scale);
        return oracle_e4m3_value(row[d]) * (double)scale;
    } else {
        uint16_t bits;
        memcpy(&bits, row + 528 + 2 * (d - 512), sizeof bits);
        return oracle_bf16_value(bits);
    }
}

/* q[t,h] . kv_row over the first qk_dim elements, exactly (every E4M3 value and
 * every product is exact in double, and so is a product with a BF16 or an FP32
 * scaled value; the sum of at most 576 of them loses nothing that matters at
 * the tolerances used). */
static double dot_qk(const problem *p, int t, int h, const uint8_t *row, int *status)
{
    const uint8_t *q = p->q + (int64_t)t * p->q_stride_t + (int64_t)h * p->q_stride_h;
    double acc = 0.0;
    for (int d = 0; d < p->qk_dim; d++) {
        double a = oracle_e4m3_value(q[d]);
        double b = kv_value(p, row, d);
        if (isnan(a) || isnan(b) || isinf(b))
            *status = ORACLE_ENAN;
        acc += a * b;
    }
    return acc;
}

static int check_problem(const problem *p)
{
    if (!p->q || !p->kv_a || !p->indices || !p->lens)
        return ORACLE_EBADARG;
    if (p->T < 0 || p->H <= 0 || p->W <= 0)
        return ORACLE_EBADARG;
    if (p->row_bytes < 512 || p->qk_dim < 1 || p->qk_dim > p->row_bytes)
        return ORACLE_EBADARG;
    if (p->row_bytes == DS_MLA_ROW && p->qk_dim != 576)
        return ORACLE_EBADARG;
    if (p->kv_b && (p->split_col < 0 || p->split_col > p->W))
        return ORACLE_EBADARG;
    return ORACLE_OK;
}

#define V_DIM 512 /* V is the first 512 bytes of a row on every page */

/* ---------------------------------------------------------------------------
 * C1: exact mode, the formula of the sparse_mla_cute page, with the LSE
 * ln(sum_c e^{s_c} + e^{sink}) so that out * e^{lse} = bmm2 * sum_c e^{s_c} v_c.
 * units: (t, h) pairs, n_units of them; NULL means every (t, h) in order.
 * out: [n_units, 512] doubles; lse: [n_units] doubles.
 * ------------------------------------------------------------------------- */
int oracle_decode_exact(
    const uint8_t *q, int64_t q_stride_t, int64_t q_stride_h,
    const uint8_t *kv_a, int64_t rows_a,
    const uint8_t *kv_b, int64_t rows_b, int32_t split_col,
    int32_t row_bytes, int32_t qk_dim,
    const int32_t *indices, const int32_t *lens,
    int32_t T, int32_t H, int32_t W,
    double bmm1, double bmm2, const float *sinks, uint32_t flags,
    const int32_t *units, int32_t n_units,
    double *out, double *lse)
{
    problem p = {q, q_stride_t, q_stride_h, kv_a, rows_a, kv_b, rows_b, split_col,
                 row_bytes, qk_dim, indices, lens, T, H, W, bmm1, bmm2, sinks};
    int status = check_problem(&p);
    int count = units ? n_units : T * H;
    double *scores;
    if (status != ORACLE_OK)
        return status;
    scores = (double *)malloc(sizeof(double) * (size_t)(W > 0 ? W : 1));
    if (!scores)
        return ORACLE_EBADARG;
    for (int u = 0; u < count && status == ORACLE_OK; u++) {
        int t = units ? units[2 * u] : u / H;
        int h = units ? units[2 * u + 1] : u % H;
        int n, any = 0;
        double m = -INFINITY, z = 0.0;
        double *o = out + (int64_t)u * V_DIM;
        if (t < 0 || t >= T || h < 0 || h >= H) {
            status = ORACLE_EBADARG;
            break;
        }
        n = active_count(&p, t);
        /* scores s_c of the active columns, and their maximum */
        for (int c = 0; c < n; c++) {
            const uint8_t *row;
            if (!is_active(&p, t, c, n))
                continue;
            row = row_of(&p, t, c, &status);
            if (!row)
                break;
            scores[c] = bmm1 * dot_qk(&p, t, h, row, &status);
            if (scores[c] > m)
                m = scores[c];
            any = 1;
        }
        if (status != ORACLE_OK)
            break;
        for (int j = 0; j < V_DIM; j++)
            o[j] = 0.0;
        if (!any) { /* zero-count rule: zeros and LSE -inf, sink or not */
            lse[u] = -INFINITY;
            continue;
        }
        if (sinks && (double)sinks[h] > m)
            m = (double)sinks[h];
        for (int c = 0; c < n; c++) {
            const uint8_t *row;
            double w;
            if (!is_active(&p, t, c, n))
                continue;
            row = row_of(&p, t, c, &status);
            w = exp(scores[c] - m);
            z += w;
            for (int j = 0; j < V_DIM; j++)
                o[j] += w * kv_value(&p, row, j);
        }
        if (sinks)
            z += exp((double)sinks[h] - m);
        for (int j = 0; j < V_DIM; j++)
            o[j] = bmm2 * o[j] / z;
        lse[u] = m + log(z);
        if (flags & ORACLE_LSE_LOG2)
            lse[u] /= log(2.0);
    }
    free(scores);
    return status;
}

/* ---------------------------------------------------------------------------
 * C2: mimic mode, the attn_sparse page's E4M3-P recipe step by step.
 *
 * Per (t, h): the clamped count n is split into `splits` contiguous ranges
 * (per = ceil(n / splits), first = min(n, s * per), mine = min(n - first, per),
 * as SparseDcpDecode.kernel); each range runs in chunks of `chunk` positions:
 *   s2 = s * log2(e)  (base-2 score; -inf when the column is inactive)
 *   m_new = max(m_run, max s2);  alpha = 2^(m_run - m_new)  (1 if m_run = -inf)
 *   p = 2^(s2 - m_new + log2 anchor)                           (double)
 *   p_hat = E4M3(p)           (terms = 1)
 *   p_hat = E4M3(p) + E4M3(16 (p - E4M3(p))) / 16   (terms = 2)
 *   l = l * alpha + sum p   (the unquantized P);  acc = acc * alpha + sum p_hat v
 * then the ranges merge (the merge method): M = max over ranges of m (and the
 * base-2 sink), w = 2^(m - M), L = sum w l (+ anchor * 2^(sink2 - M)),
 * out = bmm2 * sum w acc / L, LSE2 = M - log2 anchor + log2 L.
 * With `quantize` = 0, p_hat = p (no rounding), which reduces to exact mode.
 * ------------------------------------------------------------------------- */
int oracle_decode_mimic(
    const uint8_t *q, int64_t q_stride_t, int64_t q_stride_h,
    const uint8_t *kv_a, int64_t rows_a,
    const uint8_t *kv_b, int64_t rows_b, int32_t split_col,
    int32_t row_bytes, int32_t qk_dim,
    const int32_t *indices, const int32_t *lens,
    int32_t T, int32_t H, int32_t W,
    double bmm1, double bmm2, const float *sinks, uint32_t flags,
    int32_t splits, int32_t chunk, double anchor, int32_t terms, int32_t quantize,
    const int32_t *units, int32_t n_units,
    double *out, double *lse)
{
    problem p = {q, q_stride_t, q_stride_h, kv_a, rows_a, kv_b, rows_b, split_col,
                 row_bytes, qk_dim, indices, lens, T, H, W, bmm1, bmm2, sinks};
    const double log2e = 1.0 / log(2.0);
    int status = check_problem(&p);
    int count = units ? n_units : T * H;
    double *m_s, *l_s, *acc_s, *s2, *phat;
    if (status != ORACLE_OK)
        return status;
    if (splits < 1 || chunk < 1 || !(anchor > 0) || terms < 1 || terms > 2)
        return ORACLE_EBADARG;
    m_s = (double *)malloc(sizeof(double) * (size_t)splits);
    l_s = (double *)malloc(sizeof(double) * (size_t)splits);
    acc_s = (double *)malloc(sizeof(double) * (size_t)splits * V_DIM);
    s2 = (double *)malloc(sizeof(double) * (size_t)chunk);
    phat = (double *)malloc(sizeof(double) * (size_t)chunk);
    if (!m_s || !l_s || !acc_s || !s2 || !phat) {
        free(m_s); free(l_s); free(acc_s); free(s2); free(phat);
        return ORACLE_EBADARG;
    }
    for (int u = 0; u < count && status == ORACLE_OK; u++) {
        int t = units ? units[2 * u] : u / H;
        int h = units ? units[2 * u + 1] : u % H;
        int n, per, any = 0;
        double big_m = -INFINITY, big_l = 0.0;
        double *o = out + (int64_t)u * V_DIM;
        if (t < 0 || t >= T || h < 0 || h >= H) {
            status = ORACLE_EBADARG;
            break;
        }
        n = active_count(&p, t);
        per = (n + splits - 1) / splits;
        for (int s = 0; s < splits && status == ORACLE_OK; s++) {
            int first = s * per < n ? s * per : n;
            int mine = n - first < per ? n - first : per;
            double m_run = -INFINITY, l_run = 0.0;
            double *acc = acc_s + (int64_t)s * V_DIM;
            for (int j = 0; j < V_DIM; j++)
                acc[j] = 0.0;
            for (int base = first; base < first + mine && status == ORACLE_OK; base += chunk) {
                int cnt = first + mine - base < chunk ? first + mine - base : chunk;
                double chunk_max = -INFINITY, m_new, alpha, bias, sum_p = 0.0;
                for (int i = 0; i < cnt; i++) {
                    int c = base + i;
                    s2[i] = -INFINITY;
                    if (is_active(&p, t, c, n)) {
                        const uint8_t *row = row_of(&p, t, c, &status);
                        if (!row)
                            break;
                        s2[i] = bmm1 * dot_qk(&p, t, h, row, &status) * log2e;
                        any = 1;
                    }
                    if (s2[i] > chunk_max)
                        chunk_max = s2[i];
                }
                if (status != ORACLE_OK)
                    break;
                /* the running maximum and the rescale of what came before it */
                m_new = m_run > chunk_max ? m_run : chunk_max;
                alpha = (m_run == -INFINITY) ? 1.0 : exp2(m_run - m_new);
                bias = (m_new == -INFINITY) ? 0.0 : m_new - log2(anchor);
                for (int i = 0; i < cnt; i++) {
                    double pv = 0.0, hi;
                    if (s2[i] != -INFINITY)
                        pv = exp2(s2[i] - bias);
                    sum_p += pv;
                    if (!quantize) {
                        phat[i] = pv;
                        continue;
                    }
                    hi = oracle_e4m3_value(oracle_e4m3_encode(pv));
                    phat[i] = hi;
                    if (terms == 2)
                        phat[i] += oracle_e4m3_value(oracle_e4m3_encode(16.0 * (pv - hi))) / 16.0;
                }
                l_run = l_run * alpha + sum_p;
                for (int j = 0; j < V_DIM; j++)
                    acc[j] *= alpha;
                for (int i = 0; i < cnt; i++) {
                    const uint8_t *row;
                    if (phat[i] == 0.0)
                        continue; /* inactive, or P rounded to zero */
                    row = row_of(&p, t, base + i, &status);
                    for (int j = 0; j < V_DIM; j++)
                        acc[j] += phat[i] * kv_value(&p, row, j);
                }
                m_run = m_new;
            }
            m_s[s] = m_run;
            l_s[s] = l_run;
        }
        if (status != ORACLE_OK)
            break;
        for (int j = 0; j < V_DIM; j++)
            o[j] = 0.0;
        if (!any) { /* zero-count rule */
            lse[u] = -INFINITY;
            continue;
        }
        /* the merge over ranges (and the sink) */
        for (int s = 0; s < splits; s++)
            if (m_s[s] > big_m)
                big_m = m_s[s];
        if (sinks && (double)sinks[h] * log2e > big_m)
            big_m = (double)sinks[h] * log2e;
        for (int s = 0; s < splits; s++) {
            double w = (m_s[s] == -INFINITY) ? 0.0 : exp2(m_s[s] - big_m);
            big_l += w * l_s[s];
            for (int j = 0; j < V_DIM; j++)
                o[j] += w * acc_s[(int64_t)s * V_DIM + j];
        }
        if (sinks)
            big_l += anchor * exp2((double)sinks[h] * log2e - big_m);
        for (int j = 0; j < V_DIM; j++)
            o[j] = bmm2 * o[j] / big_l;
        lse[u] = big_m - log2(anchor) + log2(big_l); /* base 2 */
        if (!(flags & ORACLE_LSE_LOG2))
            lse[u] *= log(2.0);
    }
    free(m_s); free(l_s); free(acc_s); free(s2); free(phat);
    return status;
}

/* ---------------------------------------------------------------------------
 * C2b: chunk-local mode, the sparse_mla_cute page's "How." recipe.
 *
 * Per (t, h): the clamped count n is cut into chunks of `width` consecutive
 * columns, chunk k = [k * width, min((k + 1) * width, n)) (chunk 0 is the
 * first `width` columns, the sliding-window columns at width 128).  Each
 * chunk runs its own softmax in base 2, with no running maximum:
 *   s2 = s * log2(e)  (-inf when the column is inactive)
 *   m_k = max over the chunk of s2   (-inf when no column of it is active)
 *   p = 2^(s2 - m_k + log2 anchor)   (double; anchor 256 on that page)
 *   p_hat = E4M3(p)      (terms = 1: P as FP8)
 *   p_hat = E4M3(p) + E4M3(16 (p - E4M3(p))) / 16   (terms = 2)
 *   l_k = sum p  (the unquantized P);  acc_k = sum p_hat v
 * then the chunks merge with the sink: M = max(max_k m_k, sink2),
 * w_k = 2^(m_k - M), L = sum w_k l_k (+ anchor * 2^(sink2 - M)),
 * out = bmm2 * sum w_k acc_k / L, LSE2 = M - log2 anchor + log2 L.
 * With `quantize` = 0, p_hat = p, which reduces to exact mode.
 * ------------------------------------------------------------------------- */
int oracle_decode_chunk_local(
    const uint8_t *q, int64_t q_stride_t, int64_t q_stride_h,
    const uint8_t *kv_a, int64_t rows_a,
    const uint8_t *kv_b, int64_t rows_b, int32_t split_col,
    int32_t row_bytes, int32_t qk_dim,
    const int32_t *indices, const int32_t *lens,
    int32_t T, int32_t H, int32_t W,
    double bmm1, double bmm2, const float *sinks, uint32_t flags,
    int32_t width, double anchor, int32_t terms, int32_t quantize,
    const int32_t *units, int32_t n_units,
    double *out, double *lse)
{
    problem p = {q, q_stride_t, q_stride_h, kv_a, rows_a, kv_b, rows_b, split_col,
                 row_bytes, qk_dim, indices, lens, T, H, W, bmm1, bmm2, sinks};
    const double log2e = 1.0 / log(2.0);
    int status = check_problem(&p);
    int count = units ? n_units : T * H;
    double *s2, *acc_k;
    if (status != ORACLE_OK)
        return status;
    if (width < 1 || !(anchor > 0) || terms < 1 || terms > 2)
        return ORACLE_EBADARG;
    s2 = (double *)malloc(sizeof(double) * (size_t)width);
    acc_k = (double *)malloc(sizeof(double) * V_DIM);
    if (!s2 || !acc_k) {
        free(s2); free(acc_k);
        return ORACLE_EBADARG;
    }
    for (int u = 0; u < count && status == ORACLE_OK; u++) {
        int t = units ? units[2 * u] : u / H;
        int h = units ? units[2 * u + 1] : u % H;
        int n, any = 0;
        double big_m = -INFINITY, big_l = 0.0, sink2 = -INFINITY;
        double *o = out + (int64_t)u * V_DIM;
        if (t < 0 || t >= T || h < 0 || h >= H) {
            status = ORACLE_EBADARG;
            break;
        }
        n = active_count(&p, t);
        /* pass 1: every chunk's maximum, hence M (the merge needs it before any weight) */
        for (int base = 0; base < n && status == ORACLE_OK; base += width) {
            int cnt = n - base < width ? n - base : width;
            for (int i = 0; i < cnt; i++) {
                if (is_active(&p, t, base + i, n)) {
                    const uint8_t *row = row_of(&p, t, base + i, &status);
                    double v;
                    if (!row)
                        break;
                    v = bmm1 * dot_qk(&p, t, h, row, &status) * log2e;
                    any = 1;
                    if (v > big_m)
                        big_m = v;
                }
            }
        }
        if (status != ORACLE_OK)
            break;
        for (int j = 0; j < V_DIM; j++)
            o[j] = 0.0;
        if (!any) { /* zero-count rule */
            lse[u] = -INFINITY;
            continue;
        }
        if (sinks) {
            sink2 = (double)sinks[h] * log2e;
            if (sink2 > big_m)
                big_m = sink2;
        }
        /* pass 2: each chunk's softmax at its own maximum, its P.V, and its weighted share */
        for (int base = 0; base < n && status == ORACLE_OK; base += width) {
            int cnt = n - base < width ? n - base : width;
            double m_k = -INFINITY, l_k = 0.0, w_k;
            for (int i = 0; i < cnt; i++) {
                s2[i] = -INFINITY;
                if (is_active(&p, t, base + i, n)) {
                    const uint8_t *row = row_of(&p, t, base + i, &status);
                    if (!row)
                        break;
                    s2[i] = bmm1 * dot_qk(&p, t, h, row, &status) * log2e;
                }
                if (s2[i] > m_k)
                    m_k = s2[i];
            }
            if (status != ORACLE_OK || m_k == -INFINITY)
                continue; /* a chunk with no active column adds nothing */
            for (int j = 0; j < V_DIM; j++)
                acc_k[j] = 0.0;
            for (int i = 0; i < cnt; i++) {
                double pv, ph, hi;
                const uint8_t *row;
                if (s2[i] == -INFINITY)
                    continue;
                pv = exp2(s2[i] - m_k + log2(anchor));
                l_k += pv;
                ph = pv;
                if (quantize) {
                    hi = oracle_e4m3_value(oracle_e4m3_encode(pv));
                    ph = hi;
                    if (terms == 2)
                        ph += oracle_e4m3_value(oracle_e4m3_encode(16.0 * (pv - hi))) / 16.0;
                }
                if (ph == 0.0)
                    continue;
                row = row_of(&p, t, base + i, &status);
                for (int j = 0; j < V_DIM; j++)
                    acc_k[j] += ph * kv_value(&p, row, j);
            }
            w_k = exp2(m_k - big_m);
            big_l += w_k * l_k;
            for (int j = 0; j < V_DIM; j++)
                o[j] += w_k * acc_k[j];
        }
        if (status != ORACLE_OK)
            break;
        if (sinks)
            big_l += anchor * exp2(sink2 - big_m);
        for (int j = 0; j < V_DIM; j++)
            o[j] = bmm2 * o[j] / big_l;
        lse[u] = big_m - log2(anchor) + log2(big_l); /* base 2 */
        if (!(flags & ORACLE_LSE_LOG2))
            lse[u] *= log(2.0);
    }
    free(s2); free(acc_k);
    return status;
}

/* ---------------------------------------------------------------------------
 * C3: LSE merge of S split-KV partials (the dcp page, DcpValue.merge).
 * partials: BF16 bits [S, T, H, D]; lse2: base-2 LSE [S, T, H].
 * A source is empty unless its LSE is finite (NaN, +-inf are empty); empty
 * sources are never read.  No valid source: zeros and LSE -inf.
 * out: [T, H, D] doubles; lse_out: [T, H] doubles (natural log unless
 * ORACLE_LSE_LOG2).
 * ------------------------------------------------------------------------- */
int oracle_lse_merge(const uint16_t *partials, const float *lse2,
                     int32_t S, int32_t T, int32_t H, int32_t D, uint32_t flags,
                     double *out, double *lse_out)
{
    if (!partials || !lse2 || S < 1 || T < 0 || H < 1 || D < 1)
        return ORACLE_EBADARG;
    for (int t = 0; t < T; t++) {
        for (int h = 0; h < H; h++) {
            int64_t th = (int64_t)t * H + h;
            double top = -INFINITY, total = 0.0;
            int any = 0;
            double *o = out + th * D;
            for (int d = 0; d < D; d++)
                o[d] = 0.0;
            for (int s = 0; s < S; s++) {
                double v = (double)lse2[(int64_t)s * T * H + th];
                if (isfinite(v)) {
                    any = 1;
                    if (v > top)
                        top = v;
                }
            }
            if (!any) {
                lse_out[th] = -INFINITY;
                continue;
            }
            for (int s = 0; s < S; s++) {
                double v = (double)lse2[(int64_t)s * T * H + th];
                if (isfinite(v))
                    total += exp2(v - top);
            }
            for (int s = 0; s < S; s++) {
                double v = (double)lse2[(int64_t)s * T * H + th];
                const uint16_t *x = partials + ((int64_t)s * T * H + th) * D;
                double w;
                if (!isfinite(v))
                    continue;
                w = exp2(v - top) / total;
                for (int d = 0; d < D; d++)
                    o[d] += w * oracle_bf16_value(x[d]);
            }
            lse_out[th] = top + log2(total);
            if (!(flags & ORACLE_LSE_LOG2))
                lse_out[th] *= log(2.0);
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * C4: the MLA value tail (the dcp page, DcpValue class docstring and its merge
 * method; "as in MlaValue"): per row t and head h, the S sources' partials are
 * LSE-merged as in C3 and rounded once to BF16 (the merged latent row); W_UV
 * maps it to the head's 128 output values,
 *     acc[v] = sum_{k < 512} latent[k] * W_UV[h][k][v],
 * the product is rounded to BF16, multiplied by sigmoid(gate[t][h*128 + v]) =
 * 1 / (1 + e^{-gate}) and rounded to BF16 again.  A row whose request total
 * totals[t / rows_per_request] is <= 0 (a padded row, whose gate may be NaN)
 * is written as zeros; totals == NULL makes every row live.
 * partials: BF16 bits [S, T, H, 512]; lse2: [S, T, H] base 2; w_uv: BF16 bits,
 * element (h, k, v) at w_uv[h * w_stride_h + v * w_stride_v + k]; gate: BF16
 * bits [T, H * 128]; out: [T, H * 128] doubles, each exactly a BF16 value.
 * ------------------------------------------------------------------------- */

/* BF16 of x, round to nearest even: 8 significant bits for normal values, the fixed quantum
 * 2^-133 below 2^-126; zeros, infinities and NaN pass through. */
static double bf16_round(double x)
{
    int e;
    double m;
    if (x == 0.0 || isnan(x) || isinf(x))
        return x;
    if (fabs(x) < ldexp(1.0, -126))
        return ldexp(nearbyint(ldexp(x, 133)), -133);
    m = frexp(x, &e); /* x = m 2^e, 1/2 <= |m| < 1 */
    return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

int oracle_mla_value(const uint16_t *partials, const float *lse2, int32_t S, int32_t T,
                     int32_t H, const uint16_t *w_uv, int64_t w_stride_h, int64_t w_stride_v,
                     const uint16_t *gate, const int32_t *totals, int32_t rows_per_request,
                     double *out)
{
    double latent[V_DIM];
    if (!partials || !lse2 || !w_uv || !gate || !out || S < 1 || T < 0 || H < 1 ||
        rows_per_request < 1)
        return ORACLE_EBADARG;
    for (int t = 0; t < T; t++) {
        int live = !totals || totals[t / rows_per_request] > 0;
        for (int h = 0; h < H; h++) {
            int64_t th = (int64_t)t * H + h;
            double top = -INFINITY, total = 0.0;
            double *o = out + th * 128;
            for (int j = 0; j < V_DIM; j++)
                latent[j] = 0.0;
            for (int s = 0; s < S; s++) {
                double v = (double)lse2[(int64_t)s * T * H + th];
                if (isfinite(v) && v > top)
                    top = v;
            }
            if (top != -INFINITY) {
                for (int s = 0; s < S; s++) {
                    double v = (double)lse2[(int64_t)s * T * H + th];
                    if (isfinite(v))
                        total += exp2(v - top);
                }
                for (int s = 0; s < S; s++) {
                    double v = (double)lse2[(int64_t)s * T * H + th];
                    const uint16_t *x = partials + ((int64_t)s * T * H + th) * V_DIM;
                    double w;
                    if (!isfinite(v))
                        continue;
                    w = exp2(v - top) / total;
                    for (int j = 0; j < V_DIM; j++)
                        latent[j] += w * oracle_bf16_value(x[j]);
                }
            }
            for (int j = 0; j < V_DIM; j++)
                latent[j] = bf16_round(latent[j]);
            for (int v = 0; v < 128; v++) {
                double acc = 0.0, g, sig;
                if (!live) {
                    o[v] = 0.0;
                    continue;
                }
                for (int k = 0; k < V_DIM; k++)
                    acc += latent[k] * oracle_bf16_value(w_uv[h * w_stride_h + v * w_stride_v + k]);
                g = oracle_bf16_value(gate[(int64_t)t * H * 128 + h * 128 + v]);
                sig = 1.0 / (1.0 + exp(-g));
                o[v] = bf16_round(bf16_round(acc) * sig);
            }
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * C5: dense paged MLA decode (the dcp page, stock_decode: a paged FP8 cache
 * addressed through a block table, the q rows of a request masked causally,
 * caller-owned out and LSE).  Query row t = b * q_len + i (request b, its i-th
 * of q_len rows) attends to the first n_t = clamp(lengths[b] - (q_len - 1 - i),
 * 0, max_pages * page_size) keys of the request's context; key k lives in row
 * k % page_size of page block_table[b][k / page_size], each row 576 bytes (512
 * latent + 64 rope, V the first 512).  The score and the softmax are the
 * sparse_mla_cute formula of C1 (no sink), the LSE natural or base 2; a row
 * with n_t = 0 gives zeros and LSE -inf.
 * q: [B * q_len, H, 576] (strides in bytes); cache: pages of page_stride bytes.
 * out: [n_units, 512]; lse: [n_units]; units as in C1 (NULL: every (t, h)).
 * ------------------------------------------------------------------------- */
int oracle_paged_decode_exact(
    const uint8_t *q, int64_t q_stride_t, int64_t q_stride_h,
    const uint8_t *cache, int64_t num_pages, int32_t page_size, int64_t page_stride,
    const int32_t *block_table, int32_t max_pages, const int32_t *lengths,
    int32_t B, int32_t q_len, int32_t H, double bmm1, double bmm2, uint32_t flags,
    const int32_t *units, int32_t n_units, double *out, double *lse)
{
    const int32_t T = B * q_len;
    const int64_t width = (int64_t)max_pages * page_size;
    int count = units ? n_units : T * H;
    double *scores;
    int status = ORACLE_OK;
    if (!q || !cache || !block_table || !lengths || !out || !lse || B < 0 || q_len < 1 ||
        H < 1 || page_size < 1 || max_pages < 1 || page_stride < (int64_t)page_size * 576)
        return ORACLE_EBADARG;
    scores = (double *)malloc(sizeof(double) * (size_t)(width > 0 ? width : 1));
    if (!scores)
        return ORACLE_EBADARG;
    for (int u = 0; u < count && status == ORACLE_OK; u++) {
        int t = units ? units[2 * u] : u / H;
        int h = units ? units[2 * u + 1] : u % H;
        int b, i;
        int64_t n;
        double m = -INFINITY, z = 0.0;
        double *o = out + (int64_t)u * V_DIM;
        const uint8_t *qr;
        if (t < 0 || t >= T || h < 0 || h >= H) {
            status = ORACLE_EBADARG;
            break;
        }
        b = t / q_len;
        i = t % q_len;
        qr = q + (int64_t)t * q_stride_t + (int64_t)h * q_stride_h;
        n = (int64_t)lengths[b] - (q_len - 1 - i); /* causal: row i sees one key more than i-1 */
        if (n < 0)
            n = 0;
        if (n > width)
            n = width;
        for (int j = 0; j < V_DIM; j++)
            o[j] = 0.0;
        if (n == 0) {
            lse[u] = -INFINITY;
            continue;
        }
        for (int64_t k = 0; k < n; k++) {
            int32_t page = block_table[(int64_t)b * max_pages + k / page_size];
            const uint8_t *row;
            double acc = 0.0;
            if (page < 0 || page >= num_pages) {
                status = ORACLE_ERANGE;
                break;
            }
            row = cache + (int64_t)page * page_stride + (k % page_size) * 576;
            for (int d = 0; d < 576; d++) {
                double a = oracle_e4m3_value(qr[d]);
                double c = oracle_e4m3_value(row[d]);
                if (isnan(a) || isnan(c))
                    status = ORACLE_ENAN;
                acc += a * c;
            }
            scores[k] = bmm1 * acc;
            if (scores[k] > m)
                m = scores[k];
        }
        if (status != ORACLE_OK)
            break;
        for (int64_t k = 0; k < n; k++) {
            int32_t page = block_table[(int64_t)b * max_pages + k / page_size];
            const uint8_t *row = cache + (int64_t)page * page_stride + (k % page_size) * 576;
            double w = exp(scores[k] - m);
            z += w;
            for (int j = 0; j < V_DIM; j++)
                o[j] += w * oracle_e4m3_value(row[j]);
        }
        for (int j = 0; j < V_DIM; j++)
            o[j] = bmm2 * o[j] / z;
        lse[u] = m + log(z);
        if (flags & ORACLE_LSE_LOG2)
            lse[u] /= log(2.0);
    }
    free(scores);
    return status;
}

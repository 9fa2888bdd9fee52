/*
 * dsa_oracle.c -- plain fp64 CPU oracle for the DSA sparse-attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke entry and the
 * bench's cpu_baseline leg may load this file's library.  It shares no code,
 * header, table or helper with the HIP library: it has its own dtype codes,
 * its own bf16 / fp8 decoders and its own layout arithmetic, and it reads the
 * same input bytes the GPU reads.  Everything is computed in double precision,
 * written as the plain definition, with no blocking, fusion or reordering.
 *
 * Sources (pages of the reference, cited by title and section):
 *  - "GLM-5.2 架构解剖" (GLM-5.2 anatomy), section 结构全图 (full structure
 *    diagram), Indexer box: 32 index heads x 128 dims, a single key per token
 *    shared by all index heads, fp8 per-1x128 key quantisation with a
 *    power-of-two scale, index cache of 132 B per token, top-k = 2048 written
 *    as an int32 [tokens x 2048] buffer; sparse MLA with 64 heads that runs
 *    only on the 2048 selected rows of a 576-wide latent cache (512 + 64).
 *  - same page, section 核心机制·层调度 (layer scheduling): "shared" layers
 *    reuse the previous full layer's indices unchanged.
 *  - same page, section ATOM 侧 (ATOM-side optimisations), row stable_topk:
 *    the selection must be deterministic when scores tie.
 *  - same page, section 注意点 (caveats), second box: with fewer than 2048
 *    tokens the selection takes every row and sparse attention is dense.
 *  - ATOM pull request #2980 page, Limitations: the fp8 format is OCP E4M3fn.
 *  - The lightning-indexer score itself is the DeepSeek-V3.2 definition
 *    score_s = sum_h w_h * ReLU(q_h . k_s * scale_s); the anatomy page gives
 *    its shapes (wq_b 2048 -> 32x128, wk 6144 -> 128, weights_proj -> 32)
 *    but prints no formula.
 *
 * Parity pins: every function here is pinned by tests under tests/ that do
 * not reuse this code (closed forms, library routines on special cases,
 * brute force on tiny inputs, invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Oracle-local dtype codes (chosen to match the Python wrapper only). */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2 };

enum {
    ORC_OK = 0,
    ORC_BAD_ARG = -1,
    ORC_BAD_INDEX = -2, /* index out of range or repeated */
};

/* ---------------------------------------------------------------- decoders */

/* bfloat16: the upper half of an IEEE binary32; exact. */
double orc_decode_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP 8-bit E4M3 ("fn": finite, no infinities).  Sign s, exponent e (4 bits,
 * bias 7), mantissa m (3 bits).  e = 15 with m = 7 is the only NaN pattern;
 * e = 0 is subnormal m * 2^-9; otherwise (1 + m/8) * 2^(e-7).  Largest
 * finite magnitude is 1.75 * 2^8 = 448. */
double orc_decode_fp8_e4m3fn(uint8_t b)
{
    int s = b >> 7;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

static double load_elem(int dt, const void *base, int64_t idx)
{
    switch (dt) {
    case ORC_F32:
        return (double)((const float *)base)[idx];
    case ORC_BF16:
        return orc_decode_bf16(((const uint16_t *)base)[idx]);
    case ORC_FP8:
        return orc_decode_fp8_e4m3fn(((const uint8_t *)base)[idx]);
    }
    return NAN;
}

static int elem_size(int dt)
{
    return dt == ORC_F32 ? 4 : dt == ORC_BF16 ? 2 : dt == ORC_FP8 ? 1 : 0;
}

/* ------------------------------------------------------------------ layout */

/*
 * Ragged layout.  Sequence b owns cache rows kv_indptr[b] .. kv_indptr[b+1]-1
 * (ctx_b of them) and query rows q_indptr[b] .. q_indptr[b+1]-1 (q_len_b).
 * Query j of sequence b sits at position p = ctx_b - q_len_b + j and sees the
 * causal prefix s = 0 .. p, i.e. n = p + 1 tokens.  A NULL q_indptr means one
 * query per sequence (decode), so n = ctx_b.
 */
typedef struct {
    int b;
    int64_t kv_base;
    int64_t n;
} orc_row;

static int orc_row_of(int B, const int64_t *kv_indptr, const int32_t *q_indptr, int64_t i,
                      orc_row *out)
{
    int b;
    if (q_indptr == NULL) {
        if (i < 0 || i >= B)
            return ORC_BAD_ARG;
        out->b = (int)i;
        out->kv_base = kv_indptr[i];
        out->n = kv_indptr[i + 1] - kv_indptr[i];
        return ORC_OK;
    }
    for (b = 0; b < B; ++b) {
        if (i >= q_indptr[b] && i < q_indptr[b + 1]) {
            int64_t ctx = kv_indptr[b + 1] - kv_indptr[b];
            int64_t qlen = q_indptr[b + 1] - q_indptr[b];
            int64_t j = i - q_indptr[b];
            out->b = b;
            out->kv_base = kv_indptr[b];
            out->n = ctx - qlen + j + 1;
            return ORC_OK;
        }
    }
    return ORC_BAD_ARG;
}

/*
 * Paged caches.  With a block table, token s of sequence b lives in physical
 * row block_table[b * bt_stride + s / page_size] * page_size + s % page_size
 * of every per-token cache (index keys and latent KV); kv_indptr then only
 * gives the context lengths.  Without one (NULL), the row is kv_base + s.
 */
typedef struct {
    const int32_t *block_table;
    int64_t bt_stride;
    int64_t page_size;
    int64_t cache_rows;
} orc_pages;

static int64_t orc_token_row(const orc_pages *pg, const orc_row *r, int64_t s)
{
    if (!pg || !pg->block_table)
        return r->kv_base + s;
    return (int64_t)pg->block_table[r->b * pg->bt_stride + s / pg->page_size] * pg->page_size +
           s % pg->page_size;
}

/* Visible-token count per query row (exported so tests can check layouts). */
int orc_visible_counts(int B, const int64_t *kv_indptr, const int32_t *q_indptr, int64_t T,
                       int64_t *n_out)
{
    int64_t i;
    for (i = 0; i < T; ++i) {
        orc_row r;
        if (orc_row_of(B, kv_indptr, q_indptr, i, &r) != ORC_OK)
            return ORC_BAD_ARG;
        n_out[i] = r.n;
    }
    return ORC_OK;
}

/* ----------------------------------------------------------------- indexer */

/*
 * Lightning-indexer score for every query row i and visible token s < n_i:
 *
 *   a_h     = sum_d q[i,h,d] * k[s,d]                 (decoded values)
 *   r_h     = max(0, a_h * qs[i,h] * ks[s])
 *   score   = sum_h w[i,h] * r_h
 *
 * q is [T][H][D] of q_dt; q_scale is [T][H] (NULL means 1); w is [T][H];
 * key row `row` starts at byte row * k_row_stride_bytes of k and holds D
 * elements of k_dt; its scale is k_scale[row * k_scale_stride] (NULL means 1).
 * With a block table, key row `row` is the token's physical row (see orc_pages).
 * Scores go to scores[i * ld + s] for s < n_i; other entries are untouched.
 * If mag is not NULL it receives sum_h |w_h| * qs_h * ks_s * sum_d |q_hd k_sd|,
 * the magnitude that bounds the rounding error of any summation order.
 */
int orc_index_scores(int B, const int64_t *kv_indptr, const int32_t *q_indptr, int64_t T,
                     int H, int D, int q_dt, const void *q, const float *q_scale, const float *w,
                     int k_dt, const void *k, int64_t k_row_stride_bytes, const float *k_scale,
                     int64_t k_scale_stride, double *scores, int64_t ld, double *mag,
                     const int32_t *block_table, int64_t bt_stride, int64_t page_size)
{
    int64_t i;
    int bad = 0;
    const orc_pages pg = {block_table, bt_stride, page_size, 0};
    if (block_table && page_size < 1)
        return ORC_BAD_ARG;
    if (B <= 0 || T < 0 || H <= 0 || D <= 0 || !elem_size(q_dt) || !elem_size(k_dt) || !q ||
        !w || !k || !scores || !kv_indptr)
        return ORC_BAD_ARG;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (i = 0; i < T; ++i) {
        orc_row r;
        int64_t s;
        if (orc_row_of(B, kv_indptr, q_indptr, i, &r) != ORC_OK || r.n > ld) {
            bad |= 1;
            continue;
        }
        for (s = 0; s < r.n; ++s) {
            int64_t row = orc_token_row(&pg, &r, s);
            const uint8_t *krow = (const uint8_t *)k + row * k_row_stride_bytes;
            double ks = k_scale ? (double)k_scale[row * k_scale_stride] : 1.0;
            double score = 0.0, m = 0.0;
            int h, d;
            for (h = 0; h < H; ++h) {
                double a = 0.0, am = 0.0;
                double qs = q_scale ? (double)q_scale[i * H + h] : 1.0;
                double wh = (double)w[i * H + h];
                double rh;
                for (d = 0; d < D; ++d) {
                    double qv = load_elem(q_dt, q, (i * H + h) * (int64_t)D + d);
                    double kv = load_elem(k_dt, krow, d);
                    a += qv * kv;
                    am += fabs(qv * kv);
                }
                rh = a * qs * ks;
                if (rh < 0.0)
                    rh = 0.0;
                score += wh * rh;
                m += fabs(wh) * qs * ks * am;
            }
            scores[i * ld + s] = score;
            if (mag)
                mag[i * ld + s] = m;
        }
    }
    return bad ? ORC_BAD_ARG : ORC_OK;
}

/* ------------------------------------------------------------------- top-k */

typedef struct {
    double score;
    int64_t s;
} orc_cand;

/* Strict total order: higher score first; equal scores (IEEE ==, so -0 and
 * +0 tie) are ordered by ascending position. */
static int orc_cand_cmp(const void *pa, const void *pb)
{
    const orc_cand *a = (const orc_cand *)pa, *b = (const orc_cand *)pb;
    if (a->score > b->score)
        return -1;
    if (a->score < b->score)
        return 1;
    return (a->s < b->s) ? -1 : (a->s > b->s) ? 1 : 0;
}

/*
 * Per-row top-k.  Row i has n[i] candidates scores[i * ld + s], s < n[i].
 * The output row holds the first min(k, n[i]) positions in the order above;
 * the remaining slots of the k-wide row hold -1.
 */
int orc_topk(int64_t T, const int64_t *n, const double *scores, int64_t ld, int k,
             int32_t *out)
{
    int64_t i;
    int bad = 0;
    if (T < 0 || k <= 0 || !n || !scores || !out)
        return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (i = 0; i < T; ++i) {
        int64_t m = n[i], s, take;
        orc_cand *c;
        if (m < 0 || m > ld) {
            bad |= 1;
            continue;
        }
        c = (orc_cand *)malloc((size_t)(m > 0 ? m : 1) * sizeof(orc_cand));
        if (!c) {
            bad |= 1;
            continue;
        }
        for (s = 0; s < m; ++s) {
            c[s].score = scores[i * ld + s];
            c[s].s = s;
        }
        qsort(c, (size_t)m, sizeof(orc_cand), orc_cand_cmp);
        take = m < k ? m : k;
        for (s = 0; s < k; ++s)
            out[i * k + s] = s < take ? (int32_t)c[s].s : -1;
        free(c);
    }
    return bad ? ORC_BAD_ARG : ORC_OK;
}

/* -------------------------------------------------------------- sparse MLA */

/*
 * Sparse MLA for every query row i and head h over the selected rows
 * J = the non-negative entries of indices[i * k .. i * k + k - 1] in stored
 * order (each must be < n_i and appear once).  With c_j the decoded latent
 * row kv_base + J_j (times kv_scale), 576 = Dc + Dr wide:
 *
 *   z_j   = sm_scale * sum_{d < Dc+Dr} q[i,h,d] * c_j[d]
 *   m     = max_j z_j ,   l = sum_j exp(z_j - m)
 *   o[e]  = sum_j exp(z_j - m) * c_j[e] / l        for e < Dc
 *   lse   = m + log(l)
 *
 * The key is the whole latent row (latent plus rope part), the value is its
 * first Dc entries: the absorbed form in which the output stays in latent
 * space.  An empty J gives o = 0 and lse = -inf.  q is [T][H][Dc+Dr]; kv is
 * [rows][Dc+Dr]; out is [T][H][Dc]; lse is [T][H] (may be NULL).
 * physical_rows > 0 means the indices are physical cache rows (paged caches:
 * each must be < physical_rows); 0 means positions within the sequence.
 */
int orc_sparse_mla(int B, const int64_t *kv_indptr, const int32_t *q_indptr, int64_t T, int H,
                   int Dc, int Dr, double sm_scale, int q_dt, const void *q, int kv_dt,
                   const void *kv, double kv_scale, const int32_t *indices, int k, double *out,
                   double *lse, int64_t physical_rows)
{
    int64_t i;
    int bad = 0;
    const int Dqk = Dc + Dr;
    if (B <= 0 || T < 0 || H <= 0 || Dc <= 0 || Dr < 0 || k <= 0 || !elem_size(q_dt) ||
        !elem_size(kv_dt) || !q || !kv || !indices || !out || !kv_indptr)
        return ORC_BAD_ARG;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (i = 0; i < T; ++i) {
        orc_row r;
        int nj = 0, j, j2, h, d, e;
        int32_t *J;
        double *z;
        if (orc_row_of(B, kv_indptr, q_indptr, i, &r) != ORC_OK) {
            bad |= 1;
            continue;
        }
        J = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
        z = (double *)malloc(sizeof(double) * (size_t)k);
        if (!J || !z) {
            free(J);
            free(z);
            bad |= 1;
            continue;
        }
        for (j = 0; j < k; ++j) {
            int32_t idx = indices[i * k + j];
            if (idx < 0)
                continue;
            if ((int64_t)idx >= (physical_rows > 0 ? physical_rows : r.n))
                bad |= 2;
            for (j2 = 0; j2 < nj; ++j2)
                if (J[j2] == idx)
                    bad |= 2;
            J[nj++] = idx;
        }
        if (bad & 2) {
            free(J);
            free(z);
            continue;
        }
        for (h = 0; h < H; ++h) {
            int64_t qoff = (i * H + h) * (int64_t)Dqk;
            double m = -INFINITY, l = 0.0;
            double *o = out + (i * H + h) * (int64_t)Dc;
            for (j = 0; j < nj; ++j) {
                int64_t row = physical_rows > 0 ? (int64_t)J[j] : r.kv_base + J[j];
                double acc = 0.0;
                for (d = 0; d < Dqk; ++d)
                    acc += load_elem(q_dt, q, qoff + d) *
                           (load_elem(kv_dt, kv, row * Dqk + d) * kv_scale);
                z[j] = sm_scale * acc;
                if (z[j] > m)
                    m = z[j];
            }
            for (e = 0; e < Dc; ++e)
                o[e] = 0.0;
            for (j = 0; j < nj; ++j) {
                int64_t row = physical_rows > 0 ? (int64_t)J[j] : r.kv_base + J[j];
                double p = exp(z[j] - m);
                l += p;
                for (e = 0; e < Dc; ++e)
                    o[e] += p * (load_elem(kv_dt, kv, row * Dqk + e) * kv_scale);
            }
            if (nj > 0)
                for (e = 0; e < Dc; ++e)
                    o[e] /= l;
            if (lse)
                lse[i * H + h] = nj > 0 ? m + log(l) : -INFINITY;
        }
        free(J);
        free(z);
    }
    return (bad & 2) ? ORC_BAD_INDEX : bad ? ORC_BAD_ARG : ORC_OK;
}

/* ------------------------------------------------------ index-cache writer */

/*
 * The step in front of the indexer ([anatomy], full structure diagram,
 * Indexer box: interleaved rope, then fp8 per-1x128 quantisation with a ue8m0
 * (power-of-two) scale, written into the 132-byte index cache; ATOM-side
 * optimisations, fused indexer kernel: q rope + fp8 quantisation + k-cache
 * write in one pass, for index_head_dim 128 and rope dim 64).
 *
 * Readings (the pages give the format, not the arithmetic):
 *  - one quantisation group is one head's D values (the "1x128" block);
 *  - the scale is the smallest power of two s with amax / s <= 448, where
 *    amax is the group's largest magnitude; an all-zero group takes s = 1,
 *    and s is never taken below 2^-126 so that it stays a normal fp32;
 *  - each code is x / s rounded to the nearest E4M3FN value, ties to the
 *    even code, magnitudes past 448 saturating, the sign kept (so -0 and
 *    small negatives give 0x80);
 *  - rope acts on the D_r values starting at rope_off, in interleaved pairs
 *    (2i, 2i+1), i < D_r / 2, with cos and sin read from a caller-supplied
 *    table row (cos of the D_r / 2 frequencies, then their sin).  Its result
 *    is an fp32 value that the quantiser then rounds to 8 bits, so it is
 *    computed in fp32 with every product and sum rounded on its own (this
 *    file is built without contraction); quantisation itself is exact.
 */

/* Nearest E4M3FN code to v (finite), by search over the 127 non-negative
 * finite codes in value order; on a tie the even code wins. */
uint8_t orc_encode_fp8_e4m3fn(double v)
{
    double a = fabs(v);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 126; ++c) {
        double d = fabs(orc_decode_fp8_e4m3fn((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best_d = d;
            best = c;
        }
    }
    return (uint8_t)(best | (signbit(v) ? 0x80 : 0));
}

/* Smallest power of two s = 2^e, e >= -126, with amax <= 448 * s; 1 if amax == 0. */
double orc_pow2_scale(double amax)
{
    int e = -126;
    if (amax == 0.0)
        return 1.0;
    while (amax > ldexp(448.0, e))
        ++e;
    return ldexp(1.0, e);
}

/* One interleaved rope pair: (x0, x1) -> (x0 c - x1 s, x0 s + x1 c) in fp32. */
void orc_rope_pair_f32(float x0, float x1, float c, float s, float *y0, float *y1)
{
    float a = x0 * c;
    float b = x1 * s;
    float d = x0 * s;
    float e = x1 * c;
    *y0 = a - b;
    *y1 = d + e;
}

/*
 * Quantise rows x[r][h][0..D) (dtype dt) group by group.  When cos_sin is
 * non-NULL, row r first takes rope at position positions[r] (table row
 * positions[r] of rope_rows, D_r floats each).  Group (r, h) is written to
 * codes + dst * code_stride + h * D (bytes) and scales[dst * scale_stride + h]
 * with dst = dst_rows ? dst_rows[r] : r; a negative dst is skipped.
 */
int orc_index_quant(int64_t rows, int H, int D, int dt, const void *x, const int64_t *positions,
                    const float *cos_sin, int64_t rope_rows, int D_r, int rope_off,
                    const int64_t *dst_rows, uint8_t *codes, int64_t code_stride, float *scales,
                    int64_t scale_stride)
{
    int bad = 0;
    if (rows < 0 || H < 1 || D < 1 || !x || !codes || !scales || code_stride < (int64_t)H * D ||
        scale_stride < H)
        return ORC_BAD_ARG;
    if (cos_sin && (!positions || D_r < 2 || (D_r & 1) || rope_off < 0 || rope_off + D_r > D))
        return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t dst = dst_rows ? dst_rows[r] : r;
        float *v = (float *)malloc(sizeof(float) * (size_t)D);
        if (!v) {
            bad |= 1;
            continue;
        }
        if (cos_sin && (positions[r] < 0 || positions[r] >= rope_rows))
            bad |= 2;
        for (int h = 0; h < H && dst >= 0 && !(bad & 2); ++h) {
            double amax = 0.0, s;
            for (int d = 0; d < D; ++d)
                v[d] = (float)load_elem(dt, x, (r * H + h) * (int64_t)D + d);
            if (cos_sin) {
                const float *cs = cos_sin + positions[r] * (int64_t)D_r;
                for (int i = 0; i < D_r / 2; ++i) {
                    float *p = v + rope_off + 2 * i;
                    orc_rope_pair_f32(p[0], p[1], cs[i], cs[D_r / 2 + i], &p[0], &p[1]);
                }
            }
            for (int d = 0; d < D; ++d)
                if (fabs((double)v[d]) > amax)
                    amax = fabs((double)v[d]);
            s = orc_pow2_scale(amax);
            for (int d = 0; d < D; ++d)
                codes[dst * code_stride + (int64_t)h * D + d] = orc_encode_fp8_e4m3fn((double)v[d] / s);
            scales[dst * scale_stride + h] = (float)s;
        }
        free(v);
    }
    return (bad & 2) ? ORC_BAD_INDEX : bad ? ORC_BAD_ARG : ORC_OK;
}

/* Threads the OpenMP runtime will use for the calls above. */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * oracle.c -- plain, slow, fp64 CPU reference for masked (block-sparse)
 * attention.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only code allowed to load this library.
 * It shares no code, header, table or helper with the GPU path, and the GPU
 * path never calls it.
 *
 * What it computes
 * ----------------
 * Tessera (arXiv 2609.25869), abstract: block-sparse attention computes only
 * the query/key interactions a logical mask selects, and the runtime must keep
 * exactly those interactions. For each query row q with kept key set S(q):
 *
 *     s_k  = (sum_c Q[q,c] * K[k,c]) / sqrt(d)          for k in S(q)
 *     O[q] = sum_k exp(s_k - m) V[k] / sum_k exp(s_k - m),  m = max_k s_k
 *
 * and O[q] = 0 when S(q) is empty. Scores of unkept pairs are dropped before
 * the softmax. Everything is evaluated in double precision; bf16 and fp32
 * inputs convert to double exactly.
 *
 * Which pairs are kept (mask kinds)
 * ---------------------------------
 *  BLOCK   : Tessera abstract / FG-Attn (arXiv 2509.16518) abstract -- a
 *            logical mask over bq x bk blocks; every pair of a kept block is
 *            kept. Block i covers positions [i*b, min((i+1)*b, L)).
 *  SLICE   : FG-Attn abstract -- M x 1 slices: all M queries of a query block
 *            share one list of single keys.
 *  VIDEO   : Sparse VideoGen summary ("Sparse VideoGen", "Splash Attention")
 *            -- per-head spatial pattern (key in the query's frame, or in the
 *            anchor frame) or temporal pattern (key pixel within a Chebyshev
 *            radius of the query pixel, any frame), evaluated on exact token
 *            coordinates.
 * Temporal-major heads ("Splash Attention": token layouts permuted into
 * temporal-major order): logical position j = p*T + t of the frame-major token
 * i = t*HW + p. BLOCK and SLICE masks of such a head index logical positions.
 * Tensors and outputs always stay in frame-major token order.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OM_BLOCK = 1, OM_BLOCK_BITS = 2, OM_SLICE = 3, OM_VIDEO = 4 };
enum { OM_DENSE = 0, OM_SPATIAL = 1, OM_TEMPORAL = 2 };
enum { OM_BF16 = 0, OM_F32 = 1, OM_F64 = 2 };

typedef struct {
    int32_t kind, B, H;
    int64_t L;
    int32_t bq, bk;              /* BLOCK: block shape; SLICE: bq = M */
    const uint8_t *block_u8;     /* [B][H][nqb][nkb], nonzero = kept */
    const uint64_t *block_bits;  /* [B][H][nqb][ceil(nkb/64)], bit (j%64) of word j/64 */
    const int64_t *row_ptr;      /* SLICE: [B*H*nqb + 1] */
    const int32_t *col_idx;      /* SLICE: logical key positions */
    const uint8_t *head_pattern; /* VIDEO: [H] */
    int32_t anchor, radius;
    int32_t T, Hg, Wg;
    const uint8_t *head_layout;  /* [H]: 0 frame-major, 1 temporal-major; NULL = all 0 */
} om_mask_t;

static int64_t nblocks(int64_t L, int64_t b) { return (L + b - 1) / b; }

static int is_tm(const om_mask_t *m, int h) { return m->head_layout && m->head_layout[h] == 1; }

/* frame-major token -> logical position of head h */
static int64_t logical_pos(const om_mask_t *m, int h, int64_t i)
{
    if (!is_tm(m, h)) return i;
    int64_t HW = (int64_t)m->Hg * m->Wg;
    int64_t t = i / HW, p = i % HW;
    return p * m->T + t;
}

/* logical position of head h -> frame-major token */
static int64_t token_of(const om_mask_t *m, int h, int64_t j)
{
    if (!is_tm(m, h)) return j;
    int64_t HW = (int64_t)m->Hg * m->Wg;
    int64_t p = j / m->T, t = j % m->T;
    return t * HW + p;
}

/* Is the pair (query token q, key token k) of head (b,h) kept? */
static int kept(const om_mask_t *m, int b, int h, int64_t q, int64_t k)
{
    if (m->kind == OM_VIDEO) {
        int pat = m->head_pattern[h];
        if (pat == OM_DENSE) return 1;
        int64_t HW = (int64_t)m->Hg * m->Wg;
        int64_t tq = q / HW, tk = k / HW;
        if (pat == OM_SPATIAL) return tk == tq || tk == m->anchor;
        int64_t yq = (q % HW) / m->Wg, xq = (q % HW) % m->Wg;
        int64_t yk = (k % HW) / m->Wg, xk = (k % HW) % m->Wg;
        return llabs(yk - yq) <= m->radius && llabs(xk - xq) <= m->radius;
    }
    int64_t jq = logical_pos(m, h, q), jk = logical_pos(m, h, k);
    int64_t nqb = nblocks(m->L, m->bq), nkb = nblocks(m->L, m->bk);
    int64_t bh = (int64_t)b * m->H + h;
    if (m->kind == OM_BLOCK)
        return m->block_u8[(bh * nqb + jq / m->bq) * nkb + jk / m->bk] != 0;
    if (m->kind == OM_BLOCK_BITS) {
        int64_t words = (nkb + 63) / 64;
        int64_t kb = jk / m->bk;
        return (int)((m->block_bits[(bh * nqb + jq / m->bq) * words + kb / 64] >> (kb % 64)) & 1u);
    }
    return 0; /* SLICE is expanded through its list, see row_keys */
}

/* All key tokens kept for query token q of head (b,h); returns the count. */
int64_t om_row_keys(const om_mask_t *m, int32_t b, int32_t h, int64_t q, int32_t *keys)
{
    int64_t n = 0;
    if (m->kind == OM_SLICE) {
        int64_t nqb = nblocks(m->L, m->bq);
        int64_t list = ((int64_t)b * m->H + h) * nqb + logical_pos(m, h, q) / m->bq;
        for (int64_t e = m->row_ptr[list]; e < m->row_ptr[list + 1]; ++e)
            keys[n++] = (int32_t)token_of(m, h, m->col_idx[e]);
        return n;
    }
    for (int64_t k = 0; k < m->L; ++k)
        if (kept(m, b, h, q, k)) keys[n++] = (int32_t)k;
    return n;
}

static double load(const void *p, int dtype, int64_t idx)
{
    if (dtype == OM_F64) return ((const double *)p)[idx];
    if (dtype == OM_F32) return (double)((const float *)p)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)p)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * Attention output for the requested rows. rows[r] is a flat row id
 * (b*H + h)*L + q. Q, K, V are [B][H][L][d] in `dtype`. out is [nrows][d]
 * fp64; kept_count (optional) receives |S(q)| per row.
 */
void om_attend(const om_mask_t *m, int32_t d, int32_t dtype, const void *Q, const void *K,
               const void *V, const int64_t *rows, int64_t nrows, double *out, int64_t *kept_count)
{
    const double scale = 1.0 / sqrt((double)d);
#pragma omp parallel
    {
        int32_t *keys = (int32_t *)malloc(sizeof(int32_t) * (size_t)(m->L > 0 ? m->L : 1));
        double *s = (double *)malloc(sizeof(double) * (size_t)(m->L > 0 ? m->L : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t row = rows[r];
            int64_t bh = row / m->L, q = row % m->L;
            int b = (int)(bh / m->H), h = (int)(bh % m->H);
            int64_t n = om_row_keys(m, b, h, q, keys);
            if (kept_count) kept_count[r] = n;
            double *o = out + r * d;
            for (int c = 0; c < d; ++c) o[c] = 0.0;
            if (n == 0) continue;
            int64_t qbase = (bh * m->L + q) * d;
            double mx = -INFINITY;
            for (int64_t e = 0; e < n; ++e) {
                int64_t kbase = (bh * m->L + keys[e]) * d;
                double acc = 0.0;
                for (int c = 0; c < d; ++c) acc += load(Q, dtype, qbase + c) * load(K, dtype, kbase + c);
                s[e] = acc * scale;
                if (s[e] > mx) mx = s[e];
            }
            double den = 0.0;
            for (int64_t e = 0; e < n; ++e) {
                double w = exp(s[e] - mx);
                den += w;
                int64_t vbase = (bh * m->L + keys[e]) * d;
                for (int c = 0; c < d; ++c) o[c] += w * load(V, dtype, vbase + c);
            }
            for (int c = 0; c < d; ++c) o[c] /= den;
        }
        free(keys);
        free(s);
    }
}

/* Number of kept pairs of head (b,h): the sum of |S(q)| over every query. */
int64_t om_count_pairs(const om_mask_t *m, int32_t b, int32_t h)
{
    int64_t total = 0;
    if (m->kind == OM_BLOCK || m->kind == OM_BLOCK_BITS) {
        /* every pair of a kept block is kept: sum of kept block areas */
        int64_t nqb = nblocks(m->L, m->bq), nkb = nblocks(m->L, m->bk);
        int64_t bh = (int64_t)b * m->H + h;
        int64_t words = (nkb + 63) / 64;
#pragma omp parallel for reduction(+ : total) schedule(static)
        for (int64_t i = 0; i < nqb; ++i) {
            int64_t rq = (i + 1) * m->bq < m->L ? m->bq : m->L - i * m->bq;
            for (int64_t j = 0; j < nkb; ++j) {
                int on = m->kind == OM_BLOCK ? m->block_u8[(bh * nqb + i) * nkb + j] != 0
                                             : (int)((m->block_bits[(bh * nqb + i) * words + j / 64] >> (j % 64)) & 1u);
                if (on) total += rq * ((j + 1) * m->bk < m->L ? m->bk : m->L - j * m->bk);
            }
        }
        return total;
    }
    if (m->kind == OM_SLICE) {
        int64_t nqb = nblocks(m->L, m->bq);
        int64_t bh = (int64_t)b * m->H + h;
        for (int64_t i = 0; i < nqb; ++i) {
            int64_t rq = (i + 1) * m->bq < m->L ? m->bq : m->L - i * m->bq;
            total += rq * (m->row_ptr[bh * nqb + i + 1] - m->row_ptr[bh * nqb + i]);
        }
        return total;
    }
#pragma omp parallel for reduction(+ : total) schedule(dynamic, 64)
    for (int64_t q = 0; q < m->L; ++q) {
        int64_t n = 0;
        for (int64_t k = 0; k < m->L; ++k) n += kept(m, b, h, q, k);
        total += n;
    }
    return total;
}

/* Keys kept by any query of the M-row query block `blk` of head (b,h), as a
 * 0/1 array over key tokens (used to size the mask-defined gather bytes). */
void om_block_union(const om_mask_t *m, int32_t b, int32_t h, int64_t blk, int32_t M, uint8_t *used)
{
    memset(used, 0, (size_t)m->L);
    int32_t *keys = (int32_t *)malloc(sizeof(int32_t) * (size_t)m->L);
    int64_t hi = (blk + 1) * M < m->L ? (blk + 1) * M : m->L;
    for (int64_t j = blk * M; j < hi; ++j) {
        int64_t n = om_row_keys(m, b, h, token_of(m, h, j), keys);
        for (int64_t e = 0; e < n; ++e) used[keys[e]] = 1;
    }
    free(keys);
}

/*
 * Sum over the M-row query blocks of head (b,h), taken in the head's logical
 * order (block beta = logical positions [beta*M, min((beta+1)*M, L))), of
 * |K_beta|: the number of distinct keys kept by at least one query of beta.
 * FG-Attn (arXiv 2509.16518), abstract: a block of queries needs only the keys
 * relevant to it; |K_beta| is the count of key (and value) rows such a block
 * must load at least once, the basis of the mask-defined gather bytes.
 *
 * BLOCK masks are taken at block granularity: the rows of beta fall in the
 * logical query blocks i = floor(j / bq), and a key is kept by some row of
 * beta exactly when its key block is kept by one of those i, so |K_beta| is
 * the summed (cropped) size of the key blocks kept by any such i. SLICE and
 * VIDEO masks take the union of the rows' own key lists (om_block_union).
 */
int64_t om_union_total(const om_mask_t *m, int32_t b, int32_t h, int32_t M)
{
    const int64_t nbeta = nblocks(m->L, M);
    int64_t total = 0;
    if (m->kind == OM_BLOCK || m->kind == OM_BLOCK_BITS) {
        const int64_t nqb = nblocks(m->L, m->bq), nkb = nblocks(m->L, m->bk);
        const int64_t words = (nkb + 63) / 64;
        const int64_t bh = (int64_t)b * m->H + h;
#pragma omp parallel reduction(+ : total)
        {
            uint8_t *any = (uint8_t *)malloc((size_t)nkb);
#pragma omp for schedule(dynamic, 4)
            for (int64_t beta = 0; beta < nbeta; ++beta) {
                const int64_t j0 = beta * M, j1 = (beta + 1) * M < m->L ? (beta + 1) * M : m->L;
                memset(any, 0, (size_t)nkb);
                for (int64_t i = j0 / m->bq; i <= (j1 - 1) / m->bq; ++i)
                    for (int64_t kb = 0; kb < nkb; ++kb) {
                        const int on = m->kind == OM_BLOCK
                                           ? m->block_u8[(bh * nqb + i) * nkb + kb] != 0
                                           : (int)((m->block_bits[(bh * nqb + i) * words + kb / 64] >> (kb % 64)) & 1u);
                        if (on) any[kb] = 1;
                    }
                for (int64_t kb = 0; kb < nkb; ++kb)
                    if (any[kb]) total += (kb + 1) * m->bk < m->L ? m->bk : m->L - kb * m->bk;
            }
            free(any);
        }
        return total;
    }
#pragma omp parallel reduction(+ : total)
    {
        uint8_t *used = (uint8_t *)malloc((size_t)m->L);
#pragma omp for schedule(dynamic, 1)
        for (int64_t beta = 0; beta < nbeta; ++beta) {
            om_block_union(m, b, h, beta, M, used);
            for (int64_t k = 0; k < m->L; ++k) total += used[k];
        }
        free(used);
    }
    return total;
}

/*
 * csa2_oracle.c -- plain, slow CPU reference of CSA2 sparse attention over one
 * global KV cache shared by every decoder layer (Causal Encoder-Decoder).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU library, and the product path never calls it.
 *
 * Sources (cited by page title and section):
 *   [CED]  "CED: Continuing Context with a Causal Encoder and Decoder"
 *          (ai-systems-engineering.com), sections "One Token Sequence and
 *          Causal Access" (Fig. 2), "Shared Global KV and Per-Layer Local KV"
 *          (Fig. 3), "Selecting Positions and Reading Values with Attention"
 *          (Fig. 4), "What Full, Reindex, and Reuse Share" (Fig. 5).
 *   [KVC]  "DeepSeek-V4.1 Flash Pushes KV Cache Compression for Agent
 *          Workloads" (news.puhulab.com), draft article, "Ana Gelisme" and
 *          closing paragraph: the main cache is FP4 with E2M1 elements.
 *
 * Readings taken where the pages are silent (each is listed in the design doc):
 *   - FP4 blocks are 32 elements with one E8M0 (power-of-two) scale, chosen
 *     as floor(log2 amax) - 2 (the microscaling rule for E2M1, whose largest
 *     binade starts at 4), clamped to [-127, 127]; elements round to nearest
 *     with ties to the even code and saturate at 6; the sign bit is kept.
 *   - The indexer score is a plain dot product of 64-dim bf16 vectors, summed
 *     in double and rounded once to fp32.
 *   - Selection order: higher score first, equal scores by lower position.
 *   - Softmax scale is passed in (1/sqrt(128) in every workload); no sinks,
 *     biases or rotary terms.
 *   - The window reads the layer's own local KV for positions
 *     [max(t - W + 1, lo, 0), t]; it is not de-duplicated against the global
 *     selection.
 *
 * All arithmetic on values is in double.  Nothing here is blocked, fused or
 * reordered beyond the definitions above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_H 16
#define ORC_D 128
#define ORC_DI 64
#define ORC_ROW 256

enum { ORC_FULL = 0, ORC_REINDEX = 1, ORC_REUSE = 2 };

/* ------------------------------------------------------------------ bf16 */

static double bf16_val(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------- FP4 */

/* E2M1 magnitudes for the 3-bit magnitude code [KVC]. */
static const double e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Nearest E2M1 magnitude code to y >= 0, ties to the even code. Values above
 * 6 are nearest to 6, so saturation falls out of the search. */
static int e2m1_nearest(double y)
{
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        double d = fabs(y - e2m1_mag[c]);
        double bd = fabs(y - e2m1_mag[best]);
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1))
            best = c;
    }
    return best;
}

/* Shared power-of-two exponent of one 32-element block. */
static int block_exponent(double amax)
{
    if (amax == 0.0)
        return -127;
    int e;
    frexp(amax, &e); /* amax = m * 2^e, m in [0.5, 1): floor(log2 amax) = e-1 */
    int E = (e - 1) - 2;
    if (E < -127) E = -127;
    if (E > 127) E = 127;
    return E;
}

/* x: [rows][dim] bf16, dim % 32 == 0.  codes: [rows][dim/2], low nibble holds
 * the even channel.  scales: [rows][dim/32], byte = E + 127. */
int orc_fp4_pack(const uint16_t *x, int64_t rows, int32_t dim, uint8_t *codes, uint8_t *scales)
{
    if (dim <= 0 || dim % 32 != 0 || rows < 0)
        return 1;
    int64_t nblk = rows * (dim / 32);
    for (int64_t b = 0; b < nblk; ++b) {
        const uint16_t *xb = x + b * 32;
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) {
            double a = fabs(bf16_val(xb[i]));
            if (a > amax) amax = a;
        }
        int E = block_exponent(amax);
        scales[b] = (uint8_t)(E + 127);
        uint8_t *cb = codes + b * 16;
        memset(cb, 0, 16);
        for (int i = 0; i < 32; ++i) {
            double v = bf16_val(xb[i]);
            int mag = e2m1_nearest(ldexp(fabs(v), -E));
            int code = (signbit(v) ? 8 : 0) | mag;
            cb[i / 2] |= (uint8_t)(code << (4 * (i & 1)));
        }
    }
    return 0;
}

static double fp4_value(uint8_t code, uint8_t scale)
{
    double m = e2m1_mag[code & 7] * ldexp(1.0, (int)scale - 127);
    return (code & 8) ? -m : m;
}

int orc_fp4_unpack(const uint8_t *codes, const uint8_t *scales, int64_t rows, int32_t dim, double *out)
{
    if (dim <= 0 || dim % 32 != 0 || rows < 0)
        return 1;
    int64_t n = rows * dim;
    for (int64_t i = 0; i < n; ++i) {
        uint8_t byte = codes[i / 2];
        uint8_t code = (i & 1) ? (byte >> 4) : (byte & 15);
        out[i] = fp4_value(code, scales[i / 32]);
    }
    return 0;
}

/* ------------------------------------------------- FP4 with E4M3 / 16 */

/* The pages' own form of the FP4 cache [KVC, summary and closing paragraph]:
 * E2M1 elements with one E4M3 scale per 16 channels.  E4M3 is the 8-bit
 * float with 1 sign bit, 4 exponent bits (bias 7) and 3 mantissa bits, no
 * infinities, and S.1111.111 as NaN; exponent field 0 holds subnormals
 * m/8 * 2^-6.  Readings (the pages fix neither): the scale of a block is the
 * finite non-negative E4M3 value nearest to amax / 6 (so the block's largest
 * magnitude lands on E2M1's largest, 6), ties to the even code; each element
 * becomes the E2M1 magnitude c whose value c * s is nearest to |x| (ties to
 * the even code, beyond 6 s the nearest is 6 s); the sign bit is kept; a
 * block whose scale is 0 has every magnitude code 0. */
double orc_e4m3_value(uint8_t b)
{
    int e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7)
        return NAN;
    double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
    return (b & 0x80) ? -v : v;
}

/* Scale code of a block: scan the non-negative finite codes 0x00..0x7E and
 * keep the one with the least |6 v - amax|, ties to the even code.  Above
 * 6 * 448 the nearest finite value is 448 itself (taken directly: there the
 * double differences would absorb amax's size and compare equal).  Below it
 * every difference that decides the choice is between numbers of similar
 * size, so it is exact. */
static uint8_t e4m3_block_scale(double amax)
{
    if (amax >= 6.0 * 448.0)
        return 0x7E;
    int best = 0;
    double bd = fabs(amax);
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(6.0 * orc_e4m3_value((uint8_t)c) - amax);
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bd = d;
        }
    }
    return (uint8_t)best;
}

/* E2M1 magnitude code of |x| = a under scale s > 0: the c with the least
 * |e2m1(c) s - a| (exact products), ties to the even code.  From 6 s on the
 * nearest is 6 s (code 7), taken directly since a saturated block's
 * elements can dwarf the grid and absorb the differences. */
static int e2m1_nearest_scaled(double a, double s)
{
    if (a >= 6.0 * s)
        return 7;
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        double d = fabs(e2m1_mag[c] * s - a);
        double bd = fabs(e2m1_mag[best] * s - a);
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1))
            best = c;
    }
    return best;
}

/* x: [rows][dim] bf16, dim % 16 == 0.  codes: [rows][dim/2] (low nibble =
 * even channel); scales: E4M3 bytes [rows][dim/16]. */
int orc_fp4e_pack(const uint16_t *x, int64_t rows, int32_t dim, uint8_t *codes, uint8_t *scales)
{
    if (dim <= 0 || dim % 16 != 0 || rows < 0)
        return 1;
    int64_t nblk = rows * (dim / 16);
    for (int64_t b = 0; b < nblk; ++b) {
        const uint16_t *xb = x + b * 16;
        double amax = 0.0;
        for (int i = 0; i < 16; ++i) {
            double a = fabs(bf16_val(xb[i]));
            if (a > amax) amax = a;
        }
        uint8_t sc = e4m3_block_scale(amax);
        double s = orc_e4m3_value(sc);
        scales[b] = sc;
        uint8_t *cb = codes + b * 8;
        memset(cb, 0, 8);
        for (int i = 0; i < 16; ++i) {
            double v = bf16_val(xb[i]);
            int mag = s > 0.0 ? e2m1_nearest_scaled(fabs(v), s) : 0;
            int code = (signbit(v) ? 8 : 0) | mag;
            cb[i / 2] |= (uint8_t)(code << (4 * (i & 1)));
        }
    }
    return 0;
}

static double fp4e_value(uint8_t code, uint8_t scale)
{
    double m = e2m1_mag[code & 7] * orc_e4m3_value(scale);
    return (code & 8) ? -m : m;
}

int orc_fp4e_unpack(const uint8_t *codes, const uint8_t *scales, int64_t rows, int32_t dim, double *out)
{
    if (dim <= 0 || dim % 16 != 0 || rows < 0)
        return 1;
    int64_t n = rows * dim;
    for (int64_t i = 0; i < n; ++i) {
        uint8_t byte = codes[i / 2];
        uint8_t code = (i & 1) ? (byte >> 4) : (byte & 15);
        out[i] = fp4e_value(code, scales[i / 16]);
    }
    return 0;
}

/* ---------------------------------------------- sequence compression m */

/* Nearest bf16 to a double, ties to even (one rounding; bf16 has fp32's
 * exponent range and 8 significant bits). */
static uint16_t bf16_rne(double v)
{
    double a = fabs(v);
    double r;
    if (a == 0.0) {
        r = 0.0;
    } else if (a < ldexp(1.0, -126)) {   /* subnormal: multiples of 2^-133 */
        r = ldexp(nearbyint(ldexp(a, 133)), -133);
    } else {
        int e;
        frexp(a, &e);                     /* a in [2^(e-1), 2^e) */
        r = ldexp(nearbyint(ldexp(a, 8 - e)), e - 8);
    }
    float f = (float)r;                   /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t h = (uint16_t)(u >> 16);
    return signbit(v) ? (uint16_t)(h | 0x8000u) : h;
}

/* Sequence compression [CED, "What Does the Sequence Compression Rate
 * Reduce?": with rate m, the information of m positions is combined into one
 * entry].  The combine rule is not given; the reading taken here is the
 * element-wise mean of the group's bf16 rows, rounded once to bf16.
 * x: bf16 [groups][m][dim] -> out bf16 [groups][dim]. */
int orc_compress(const uint16_t *x, int64_t groups, int32_t m, int32_t dim, uint16_t *out)
{
    if (m < 1 || dim <= 0 || groups < 0)
        return 1;
    for (int64_t g = 0; g < groups; ++g)
        for (int32_t d = 0; d < dim; ++d) {
            /* the sum starts from the first element, so the mean of
               negative zeros keeps its sign (IEEE: -0 + -0 = -0) */
            double s = bf16_val(x[(g * m) * dim + d]);
            for (int32_t i = 1; i < m; ++i)
                s += bf16_val(x[(g * m + i) * dim + d]);
            out[g * dim + d] = bf16_rne(s / m);
        }
    return 0;
}

/* ---------------------------------------------------------------- scores */

/* s[j] = fl32(sum_d q[d] * k[j][d]) for j < n  [CED, Fig. 4: indexer Q from
 * the layer's h against indexer K of the global cache]. */
void orc_scores(const uint16_t *q_idx, const uint16_t *k_idx, int64_t n, float *s)
{
    for (int64_t j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int d = 0; d < ORC_DI; ++d)
            acc += bf16_val(q_idx[d]) * bf16_val(k_idx[j * ORC_DI + d]);
        s[j] = (float)acc;
    }
}

/* Block score: max of the tokenwise scores in each block of `block` tokens,
 * over the first n tokens.  out has ceil(n / block) entries. */
void orc_block_scores(const float *s, int64_t n, int32_t block, float *out)
{
    int64_t nb = (n + block - 1) / block;
    for (int64_t b = 0; b < nb; ++b) {
        float m = -INFINITY;
        for (int64_t j = b * block; j < (b + 1) * block && j < n; ++j)
            if (s[j] > m) m = s[j];
        out[b] = m;
    }
}

/* ------------------------------------------------------------- selection */

typedef struct {
    float s;
    int32_t id;
} ranked;

/* Higher score first; equal scores (including -0 vs +0) by lower position. */
static int cmp_rank(const void *a, const void *b)
{
    const ranked *x = (const ranked *)a, *y = (const ranked *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->id > y->id) - (x->id < y->id);
}

static int cmp_int(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Top-k [CED, Fig. 4]: the first k candidates under the order above; the
 * chosen positions are written ascending and padded with -1.  ids == NULL
 * means candidate i is position i; ids[i] < 0 marks an empty slot.  Returns
 * the number of positions chosen. */
int32_t orc_topk(const float *s, const int32_t *ids, int64_t n, int32_t k, int32_t *out)
{
    ranked *r = (ranked *)malloc(sizeof(ranked) * (size_t)(n > 0 ? n : 1));
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        int32_t id = ids ? ids[i] : (int32_t)i;
        if (id < 0) continue;
        r[m].s = s[i];
        r[m].id = id;
        ++m;
    }
    qsort(r, (size_t)m, sizeof(ranked), cmp_rank);
    int32_t take = (int32_t)(m < k ? m : k);
    for (int32_t i = 0; i < take; ++i) out[i] = r[i].id;
    qsort(out, (size_t)take, sizeof(int32_t), cmp_int);
    for (int32_t i = take; i < k; ++i) out[i] = -1;
    free(r);
    return take;
}

/* ------------------------------------------------------------- attention */

/* Softmax attention of 16 query heads over n entries [CED, Fig. 4: Main Q
 * scores the concatenated entries and weights their Values]. */
void orc_attention(const uint16_t *q, const double *K, const double *V, int64_t n, double scale, double *out)
{
    double *z = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int h = 0; h < ORC_H; ++h) {
        double *o = out + h * ORC_D;
        for (int d = 0; d < ORC_D; ++d) o[d] = 0.0;
        if (n == 0) continue;
        double m = -INFINITY;
        for (int64_t e = 0; e < n; ++e) {
            double acc = 0.0;
            for (int d = 0; d < ORC_D; ++d)
                acc += bf16_val(q[h * ORC_D + d]) * K[e * ORC_D + d];
            z[e] = acc * scale;
            if (z[e] > m) m = z[e];
        }
        double l = 0.0;
        for (int64_t e = 0; e < n; ++e) {
            double p = exp(z[e] - m);
            l += p;
            for (int d = 0; d < ORC_D; ++d) o[d] += p * V[e * ORC_D + d];
        }
        for (int d = 0; d < ORC_D; ++d) o[d] /= l;
    }
    free(z);
}

/* ------------------------------------------------------- one query, layer */

typedef struct {
    int32_t fp4;             /* 0: bf16 rows; 1: FP4 + E8M0 per 32; 2: FP4 + E4M3 per 16 */
    int64_t t_cap;           /* rows (entries) per sequence */
    int32_t m;               /* positions per entry (sequence compression rate) */
    const uint16_t *kv;      /* bf16 [n_seq][t_cap][256]: K | V */
    const uint8_t *codes;    /* FP4 [n_seq][t_cap][128] */
    const uint8_t *scales;   /* E8M0 [n_seq][t_cap][8], or E4M3 [n_seq][t_cap][16] */
    const uint16_t *k_idx;   /* bf16 [n_seq][t_cap][64] */
} orc_cache;

/* The last entry a query at position t may read: with m positions per entry
 * only complete groups are visible, entry j holding positions m j .. m j +
 * m - 1 [CED, "What Does the Sequence Compression Rate Reduce?"; Fig. 2's
 * causal rule applied to the group's last position].  -1 when none is. */
static int64_t last_entry(const orc_cache *c, int64_t t)
{
    return (t + 1) / c->m - 1;
}

/* Global K and V of entry j of sequence seq, as doubles. */
static void cache_row(const orc_cache *c, int32_t seq, int64_t j, double *K, double *V)
{
    int64_t r = (int64_t)seq * c->t_cap + j;
    if (c->fp4 == 2) {
        double row[ORC_ROW];
        orc_fp4e_unpack(c->codes + r * (ORC_ROW / 2), c->scales + r * (ORC_ROW / 16), 1, ORC_ROW, row);
        memcpy(K, row, sizeof(double) * ORC_D);
        memcpy(V, row + ORC_D, sizeof(double) * ORC_D);
    } else if (c->fp4) {
        double row[ORC_ROW];
        orc_fp4_unpack(c->codes + r * (ORC_ROW / 2), c->scales + r * (ORC_ROW / 32), 1, ORC_ROW, row);
        memcpy(K, row, sizeof(double) * ORC_D);
        memcpy(V, row + ORC_D, sizeof(double) * ORC_D);
    } else {
        for (int d = 0; d < ORC_D; ++d) {
            K[d] = bf16_val(c->kv[r * ORC_ROW + d]);
            V[d] = bf16_val(c->kv[r * ORC_ROW + ORC_D + d]);
        }
    }
}

/* Attention of one query at position t over the global entries in sel (the
 * -1 slots are empty) concatenated with the local window [CED, Fig. 4; the
 * window comes from the layer's own local KV, Fig. 3, and may repeat a
 * position that is also selected]. */
static int attend_one(const orc_cache *c, int32_t seq, int32_t t, const uint16_t *q,
                      const int32_t *sel, int32_t k, const uint16_t *lk, const uint16_t *lv,
                      int32_t cap, int32_t W, int32_t lo, double scale, double *out)
{
    int32_t w0 = t - W + 1;
    if (w0 < lo) w0 = lo;
    if (w0 < 0) w0 = 0;
    int32_t nw = (W > 0 && t >= w0) ? t - w0 + 1 : 0;
    if (nw > cap) return 2;
    double *K = (double *)malloc(sizeof(double) * ORC_D * (size_t)(k + nw + 1));
    double *V = (double *)malloc(sizeof(double) * ORC_D * (size_t)(k + nw + 1));
    int64_t n = 0;
    int rc = 0;
    for (int32_t i = 0; i < k; ++i) {
        int32_t j = sel[i];
        if (j < 0) continue;
        if (j > last_entry(c, t) || j >= c->t_cap) { rc = 3; goto done; } /* causal, Fig. 2 */
        cache_row(c, seq, j, K + n * ORC_D, V + n * ORC_D);
        ++n;
    }
    for (int32_t w = w0; w < w0 + nw; ++w) {
        int64_t slot = (int64_t)seq * cap + (w % cap);
        for (int d = 0; d < ORC_D; ++d) {
            K[n * ORC_D + d] = bf16_val(lk[slot * ORC_D + d]);
            V[n * ORC_D + d] = bf16_val(lv[slot * ORC_D + d]);
        }
        ++n;
    }
    orc_attention(q, K, V, n, scale, out);
done:
    free(K);
    free(V);
    return rc;
}

/* One query of one layer in the given mode [CED, Fig. 5]:
 *   Full    scores every position <= t with its own indexer query and keeps
 *           the top k; with pool > 0 it also keeps the top `pool` positions
 *           as the candidate pool of later Reindex layers.  With block > 1 the
 *           score of a block is the max of its tokenwise scores, the pool is
 *           every position of the top pool/block blocks, and the top k are
 *           chosen tokenwise inside the pool.
 *   Reindex scores only the pool of the most recent Full layer with its own
 *           indexer query and keeps the top k.
 *   Reuse   keeps the selection of the previous layer.
 * Every mode then attends with its own Main Q and local window. */
static int layer_one(const orc_cache *c, int mode, int32_t seq, int32_t t,
                     const uint16_t *q, const uint16_t *q_idx,
                     const uint16_t *lk, const uint16_t *lv, int32_t cap, int32_t W, int32_t lo,
                     int32_t k, int32_t pool, int32_t block, int32_t *pool_io, int32_t *sel_io,
                     double scale, double *out)
{
    if (t < 0 || t >= c->t_cap * c->m) return 4;
    const uint16_t *kseq = c->k_idx + (int64_t)seq * c->t_cap * ORC_DI;
    const int64_t tg = last_entry(c, t);  /* entries 0..tg are causal */
    if (mode == ORC_FULL) {
        int64_t n = tg + 1;
        float *s = (float *)malloc(sizeof(float) * (size_t)n);
        orc_scores(q_idx, kseq, n, s);
        if (block <= 1) {
            if (pool > 0) orc_topk(s, NULL, n, pool, pool_io);
            orc_topk(s, NULL, n, k, sel_io);
        } else {
            int64_t nb = (n + block - 1) / block;
            int32_t nbsel = pool / block;
            float *bs = (float *)malloc(sizeof(float) * (size_t)nb);
            int32_t *blocks = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nbsel > 0 ? nbsel : 1));
            float *ps = (float *)malloc(sizeof(float) * (size_t)(pool > 0 ? pool : 1));
            orc_block_scores(s, n, block, bs);
            orc_topk(bs, NULL, nb, nbsel, blocks);
            for (int32_t i = 0; i < nbsel; ++i)
                for (int32_t r = 0; r < block; ++r) {
                    int64_t j = (int64_t)blocks[i] * block + r;
                    int32_t id = (blocks[i] >= 0 && j <= tg) ? (int32_t)j : -1;
                    pool_io[i * block + r] = id;
                    ps[i * block + r] = id >= 0 ? s[id] : -INFINITY;
                }
            orc_topk(ps, pool_io, pool, k, sel_io);
            free(bs);
            free(blocks);
            free(ps);
        }
        free(s);
    } else if (mode == ORC_REINDEX) {
        float *ps = (float *)malloc(sizeof(float) * (size_t)(pool > 0 ? pool : 1));
        for (int32_t i = 0; i < pool; ++i) {
            int32_t j = pool_io[i];
            if (j >= 0) orc_scores(q_idx, kseq + (int64_t)j * ORC_DI, 1, &ps[i]);
            else ps[i] = -INFINITY;
        }
        orc_topk(ps, pool_io, pool, k, sel_io);
        free(ps);
    } else if (mode != ORC_REUSE) {
        return 5;
    }
    return attend_one(c, seq, t, q, sel_io, k, lk, lv, cap, W, lo, scale, out);
}

/* -------------------------------------------------------- decode append */

/* Decode append [CED, section "Why Prefill Recomputes a Recent Segment":
 * once a token is chosen, its global KV is appended and every layer updates
 * its local state].  For each sequence b with 0 <= pos[b] < t_cap: row pos[b]
 * of kv [n_seq][t_cap][256] takes kv_new[b], row pos[b] of k_idx
 * [n_seq][t_cap][64] takes kidx_new[b] (when kidx_new is given), and for each
 * of the L layers slot pos[b] % cap of lk, lv [L][n_seq][cap][128] takes
 * k_new, v_new [L][n_seq][128].  Other sequences are left alone.  The rows
 * are bf16; an FP4 cache is the packing of the updated kv. */
void orc_append(int32_t n_seq, int64_t t_cap, const int32_t *pos,
                const uint16_t *kv_new, const uint16_t *kidx_new, uint16_t *kv, uint16_t *k_idx,
                int32_t L, int32_t cap, const uint16_t *k_new, const uint16_t *v_new,
                uint16_t *lk, uint16_t *lv)
{
    for (int32_t b = 0; b < n_seq; ++b) {
        int64_t p = pos[b];
        if (p < 0 || p >= t_cap) continue;
        memcpy(kv + ((int64_t)b * t_cap + p) * 2 * ORC_D, kv_new + (int64_t)b * 2 * ORC_D,
               sizeof(uint16_t) * 2 * ORC_D);
        if (kidx_new)
            memcpy(k_idx + ((int64_t)b * t_cap + p) * ORC_DI, kidx_new + (int64_t)b * ORC_DI,
                   sizeof(uint16_t) * ORC_DI);
        for (int32_t l = 0; l < L; ++l) {
            int64_t slot = ((int64_t)l * n_seq + b) * cap + p % cap;
            memcpy(lk + slot * ORC_D, k_new + ((int64_t)l * n_seq + b) * ORC_D,
                   sizeof(uint16_t) * ORC_D);
            memcpy(lv + slot * ORC_D, v_new + ((int64_t)l * n_seq + b) * ORC_D,
                   sizeof(uint16_t) * ORC_D);
        }
    }
}

/* ------------------------------------------------------------ public API */

/* One layer for nq queries.  q [nq][16][128], q_idx [nq][64];
 * local ring lk, lv [n_seq][cap][128] (position p in slot p % cap);
 * pool_io [nq][pool], sel_io [nq][k] (inputs for Reindex / Reuse, outputs
 * otherwise); out [nq][16][128]. */
int orc_layer(int32_t nq, const int32_t *q_pos, const int32_t *q_seq, int32_t mode,
              int32_t fp4, int64_t t_cap, int32_t m, const uint16_t *kv, const uint8_t *codes,
              const uint8_t *scales, const uint16_t *k_idx,
              const uint16_t *q, const uint16_t *q_idx,
              const uint16_t *lk, const uint16_t *lv, int32_t cap, int32_t W, int32_t lo,
              int32_t k, int32_t pool, int32_t block, int32_t *pool_io, int32_t *sel_io,
              double scale, double *out)
{
    orc_cache c = {fp4, t_cap, m > 1 ? m : 1, kv, codes, scales, k_idx};
    if (mode == ORC_REINDEX && pool <= 0) return 6;
    if (mode == ORC_FULL && block > 1 && (pool <= 0 || pool % block)) return 6;
    for (int32_t i = 0; i < nq; ++i) {
        int rc = layer_one(&c, mode, q_seq[i], q_pos[i], q + (int64_t)i * ORC_H * ORC_D,
                           q_idx + (int64_t)i * ORC_DI, lk, lv, cap, W, lo, k, pool, block,
                           pool_io + (int64_t)i * (pool > 0 ? pool : 0),
                           sel_io + (int64_t)i * k, scale, out + (int64_t)i * ORC_H * ORC_D);
        if (rc) return rc;
    }
    return 0;
}

/* Attention only, on a given selection (used to re-run attention on another
 * implementation's indices). */
int orc_attend(int32_t nq, const int32_t *q_pos, const int32_t *q_seq,
               int32_t fp4, int64_t t_cap, int32_t m, const uint16_t *kv, const uint8_t *codes,
               const uint8_t *scales, const uint16_t *q, const int32_t *sel, int32_t k,
               const uint16_t *lk, const uint16_t *lv, int32_t cap, int32_t W, int32_t lo,
               double scale, double *out)
{
    orc_cache c = {fp4, t_cap, m > 1 ? m : 1, kv, codes, scales, NULL};
    for (int32_t i = 0; i < nq; ++i) {
        int rc = attend_one(&c, q_seq[i], q_pos[i], q + (int64_t)i * ORC_H * ORC_D,
                            sel + (int64_t)i * k, k, lk, lv, cap, W, lo, scale,
                            out + (int64_t)i * ORC_H * ORC_D);
        if (rc) return rc;
    }
    return 0;
}

/* A decoder stack of n_layers layers over one shared global cache, one decode
 * query per sequence [CED, Fig. 5: modes are fixed per layer in advance].
 * q [L][n_seq][16][128], q_idx [L][n_seq][64], lk/lv [L][n_seq][cap][128],
 * sel_out [L][n_seq][k], pool_out [n_seq][pool], out [L][n_seq][16][128]. */
int orc_stack(int32_t n_layers, const int32_t *modes, int32_t n_seq, const int32_t *q_pos,
              int32_t fp4, int64_t t_cap, int32_t mrate, const uint16_t *kv, const uint8_t *codes,
              const uint8_t *scales, const uint16_t *k_idx,
              const uint16_t *q, const uint16_t *q_idx, const uint16_t *lk, const uint16_t *lv,
              int32_t cap, int32_t W, int32_t lo, int32_t k, int32_t pool, int32_t block,
              double scale, int32_t *sel_out, int32_t *pool_out, double *out)
{
    int32_t *q_seq = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_seq);
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_seq * k);
    int rc = 0;
    int have_pool = 0;
    for (int32_t b = 0; b < n_seq; ++b) q_seq[b] = b;
    for (int64_t i = 0; i < (int64_t)n_seq * k; ++i) sel[i] = -1;
    for (int32_t l = 0; l < n_layers && !rc; ++l) {
        int32_t m = modes[l];
        if (m == ORC_REUSE && l == 0) { rc = 7; break; }
        if (m == ORC_REINDEX && !have_pool) { rc = 7; break; }
        int64_t qo = (int64_t)l * n_seq;
        rc = orc_layer(n_seq, q_pos, q_seq, m, fp4, t_cap, mrate, kv, codes, scales, k_idx,
                       q + qo * ORC_H * ORC_D, q_idx + qo * ORC_DI,
                       lk + qo * cap * ORC_D, lv + qo * cap * ORC_D, cap, W, lo,
                       k, pool, block, pool_out, sel, scale, out + qo * ORC_H * ORC_D);
        if (m == ORC_FULL && pool > 0) have_pool = 1;
        memcpy(sel_out + qo * k, sel, sizeof(int32_t) * (size_t)n_seq * k);
    }
    free(q_seq);
    free(sel);
    return rc;
}

/* Bounded replay of a prompt's recent segment [CED, section "Why Prefill
 * Recomputes a Recent Segment", Fig. 6]: positions pos[0..n) of sequence seq
 * pass through every decoder layer again so that each layer rebuilds its
 * local state; window references before lo (normally the segment's first
 * position) are cut off, the approximation that section describes.  For each
 * layer l in order: the segment's local rows k_new / v_new [L][n][128] enter
 * the layer's ring (slot p % cap; n <= cap, so no two rows share a slot),
 * then every query of the segment runs the layer's mode (Fig. 5) exactly as
 * orc_layer does.  lk, lv [L][n_seq][cap][128] are updated in place.
 * q [L][n][16][128], q_idx [L][n][64], sel_out [L][n][k], pool_out [n][pool],
 * out [L][n][16][128]. */
int orc_replay(int32_t n_layers, const int32_t *modes, int32_t n_seq, int32_t seq, int32_t n,
               const int32_t *pos, int32_t fp4, int64_t t_cap, int32_t mrate, const uint16_t *kv,
               const uint8_t *codes, const uint8_t *scales, const uint16_t *k_idx,
               const uint16_t *q, const uint16_t *q_idx, uint16_t *lk, uint16_t *lv,
               int32_t cap, int32_t W, int32_t lo, int32_t k, int32_t pool, int32_t block,
               const uint16_t *k_new, const uint16_t *v_new, double scale,
               int32_t *sel_out, int32_t *pool_out, double *out)
{
    if (n < 0 || n > cap || seq < 0 || seq >= n_seq) return 8;
    int32_t *q_seq = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1) * k);
    int rc = 0;
    int have_pool = 0;
    for (int32_t i = 0; i < n; ++i) q_seq[i] = seq;
    for (int64_t i = 0; i < (int64_t)n * k; ++i) sel[i] = -1;
    for (int32_t l = 0; l < n_layers && !rc; ++l) {
        int32_t m = modes[l];
        if (m == ORC_REUSE && l == 0) { rc = 7; break; }
        if (m == ORC_REINDEX && !have_pool) { rc = 7; break; }
        uint16_t *rk = lk + (int64_t)l * n_seq * cap * ORC_D;
        uint16_t *rv = lv + (int64_t)l * n_seq * cap * ORC_D;
        for (int32_t i = 0; i < n; ++i) {
            if (pos[i] < 0 || pos[i] >= t_cap * (mrate > 1 ? mrate : 1)) { rc = 4; break; }
            int64_t slot = (int64_t)seq * cap + pos[i] % cap;
            memcpy(rk + slot * ORC_D, k_new + ((int64_t)l * n + i) * ORC_D, sizeof(uint16_t) * ORC_D);
            memcpy(rv + slot * ORC_D, v_new + ((int64_t)l * n + i) * ORC_D, sizeof(uint16_t) * ORC_D);
        }
        if (rc) break;
        int64_t qo = (int64_t)l * n;
        rc = orc_layer(n, pos, q_seq, m, fp4, t_cap, mrate, kv, codes, scales, k_idx,
                       q + qo * ORC_H * ORC_D, q_idx + qo * ORC_DI, rk, rv, cap, W, lo,
                       k, pool, block, pool_out, sel, scale, out + qo * ORC_H * ORC_D);
        if (m == ORC_FULL && pool > 0) have_pool = 1;
        memcpy(sel_out + qo * k, sel, sizeof(int32_t) * (size_t)n * k);
    }
    free(q_seq);
    free(sel);
    return rc;
}

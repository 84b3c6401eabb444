/*
 * csa2.h -- C ABI of an MI355X (gfx950) library for CSA2 sparse attention of
 * decoder queries over one global KV cache shared by every decoder layer, as
 * used by a Causal Encoder-Decoder (YOCO-style) model.
 *
 * Source of the operations: "CED: Continuing Context with a Causal Encoder and
 * Decoder" (ai-systems-engineering.com):
 *   - "One Token Sequence and Causal Access", Fig. 2: a query at position t
 *     may read positions <= t (its own included), never later ones;
 *   - "Shared Global KV and Per-Layer Local KV", Fig. 3: the global main KV
 *     and indexer keys are produced once and read by every decoder layer;
 *     Main Q, indexer Q and the local KV are per layer;
 *   - "Selecting Positions and Reading Values with Attention", Fig. 4: the
 *     indexer (indexer Q against indexer K) picks top-k positions; their
 *     global entries are gathered, joined with the local sliding window and
 *     attended by Main Q in one softmax; a position may appear in both parts;
 *   - "What Full, Reindex, and Reuse Share", Fig. 5: per-layer modes fixed in
 *     advance; Full scores every causal position, Reindex rescores only the
 *     candidate pool built by the first Full layer, Reuse takes the previous
 *     layer's selection; every layer recomputes attention with its own Main Q
 *     and local KV.
 * FP4 main cache: E2M1 elements ("DeepSeek-V4.1 Flash Pushes KV Cache
 * Compression for Agent Workloads", draft article), here with one E8M0
 * (power-of-two) scale per 32 elements.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns and
 *     allocates every buffer (inputs, outputs and workspace); the library
 *     allocates nothing except inside a stack plan object.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns; nothing synchronises and no device
 *     data is read on the host.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error nothing is enqueued.  Kernel faults surface at the caller's
 *     next synchronisation.  No C++ exception crosses this ABI.
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Shapes: 16 query heads share one KV head (MQA); head_dim 128 for K and
 *     V; indexer vectors have 64 elements.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_VERSION 100
#define CSA2_HEADS 16
#define CSA2_HEAD_DIM 128
#define CSA2_INDEX_DIM 64

typedef enum {
    CSA2_OK = 0,
    CSA2_ERR_INVALID_ARG = 1, /* null pointer, negative size, unknown enum, misaligned pointer */
    CSA2_ERR_SHAPE = 2,       /* sizes that do not fit together */
    CSA2_ERR_SCHEDULE = 3,    /* a layer schedule the modes do not allow */
    CSA2_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the size query returned */
    CSA2_ERR_UNSUPPORTED = 5, /* current device is not gfx950 */
    CSA2_ERR_NO_DEVICE = 6,   /* no HIP device visible */
    CSA2_ERR_HIP = 7,         /* the HIP runtime refused a launch */
    CSA2_ERR_TOO_LARGE = 8    /* beyond the fixed scratch of csa2_sparse_attn_noalloc */
} csa2_status;

typedef enum { CSA2_MODE_FULL = 0, CSA2_MODE_REINDEX = 1, CSA2_MODE_REUSE = 2 } csa2_mode;

typedef enum { CSA2_KV_BF16 = 0, CSA2_KV_FP4 = 1, CSA2_KV_FP4_E4M3 = 2 } csa2_kv_format;

/* The global cache shared by all decoder layers (Fig. 3).
 *   BF16: data = uint16 [n_seq][t_cap][256]; channels 0..127 are K, 128..255 V.
 *   FP4:  data = uint8 codes [n_seq][t_cap][128]: bytes 0..63 hold K, 64..127
 *         hold V, two elements per byte, low nibble = even channel;
 *         scales = uint8 E8M0 [n_seq][t_cap][8]: bytes 0..3 scale the four
 *         32-channel blocks of K, bytes 4..7 those of V.
 *         This is exactly what csa2_pack_fp4 writes for rows of 256 (K | V).
 *   FP4_E4M3: the pages' own form ("DeepSeek-V4.1 Flash ...", summary: E2M1
 *         with an E4M3 scale per 16 channels): codes as for FP4; scales =
 *         uint8 E4M3 [n_seq][t_cap][16]: bytes 0..7 scale the eight
 *         16-channel blocks of K, bytes 8..15 those of V (144 B per token).
 *         This is exactly what csa2_pack_fp4_e4m3 writes for rows of 256.
 *   k_idx = indexer keys, bf16 [n_seq][t_cap][64].
 * data, scales and k_idx must be 16-byte aligned; t_cap <= 2^24.
 * m: positions per global entry ("CED", section "What Does the Sequence
 * Compression Rate Reduce?"): 0 or 1 — one entry per position (the
 * decoder's cache); 2 — entry j combines positions 2j and 2j + 1 (the
 * encoder's rate; see csa2_compress), and a query at position t reads only
 * entries whose whole group is at or before t, i.e. j <= (t + 1) / 2 - 1.
 * q_pos arguments stay token positions (the window reads positions); every
 * call, the prefill-chunk calls and the bounded replay included, applies
 * that entry bound. */
typedef struct {
    int32_t format;           /* csa2_kv_format */
    int32_t n_seq;
    int64_t t_cap;            /* rows (entries) per sequence */
    const void *data;
    const uint8_t *scales;    /* FP4 only; NULL for BF16 */
    const uint16_t *k_idx;
    int32_t m;                /* positions per entry: 0 or 1, or 2 */
} csa2_cache;

/* A layer's local (sliding-window) KV, a ring of `cap` slots per sequence:
 * position p is held in slot p % cap.  k, v: bf16 [n_seq][cap][128].
 * The window of a query at t is positions [max(t - window + 1, lo, 0), t]
 * (Fig. 4: the recent positions including t).  0 <= window <= cap. */
typedef struct {
    const uint16_t *k;
    const uint16_t *v;
    int32_t cap;
    int32_t window;
    int32_t lo;
} csa2_local;

int csa2_version(void);
const char *csa2_status_str(csa2_status s);

/* CSA2_OK when a HIP device is current and it is gfx950. */
csa2_status csa2_device_check(void);

/* ------------------------------------------------------------------ FP4 */

/* Quantise rows of bf16 to FP4 (E2M1 + E8M0 per 32 elements).
 * x: bf16 [rows][dim], dim % 32 == 0; codes: [rows][dim/2] (low nibble =
 * even channel); scales: [rows][dim/32].  For each 32-element block with
 * largest magnitude a: E = clamp(floor(log2 a) - 2, -127, 127) (E = -127
 * when a = 0), scale byte = E + 127, and each element x becomes the E2M1
 * value nearest to x * 2^-E (ties to the even code, magnitudes above 6 give
 * 6, the sign bit is kept, so -0 gives code 8).  x and codes 16-byte aligned.
 * Also used for the decode append of one row per sequence. */
csa2_status csa2_pack_fp4(const uint16_t *x, int64_t rows, int32_t dim, uint8_t *codes,
                          uint8_t *scales, void *stream);

/* Exact dequantisation: out[i] = (-1)^s * e2m1(c) * 2^(byte - 127) as fp32
 * (exact for scale bytes 0..253).  out: float [rows][dim], 16-byte aligned. */
csa2_status csa2_unpack_fp4(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                            int32_t dim, float *out, void *stream);

/* Quantise rows of bf16 to FP4 with one E4M3 scale per 16 elements (the
 * pages' own form).  x: bf16 [rows][dim], dim % 16 == 0; codes [rows][dim/2]
 * (low nibble = even channel); scales: E4M3 bytes [rows][dim/16].  For each
 * block with largest magnitude a, the scale s is the E4M3 value (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits) nearest to a / 6, ties to the
 * even code, saturating at 448 (0x7E); each element x becomes the E2M1
 * magnitude c for which c * s is nearest to |x| (ties to the even code,
 * beyond 6 s: 6), keeping the sign bit; when s is 0 every magnitude is 0.
 * x 16-byte aligned, codes 8-byte aligned. */
csa2_status csa2_pack_fp4_e4m3(const uint16_t *x, int64_t rows, int32_t dim, uint8_t *codes,
                               uint8_t *scales, void *stream);

/* Exact dequantisation of that form: out[i] = (-1)^s * e2m1(c) * e4m3(scale)
 * as fp32.  out 16-byte aligned, codes 8-byte aligned. */
csa2_status csa2_unpack_fp4_e4m3(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                                 int32_t dim, float *out, void *stream);

/* ------------------------------------------------- sequence compression */

/* Sequence compression ("CED", section "What Does the Sequence Compression
 * Rate Reduce?": with rate m the information of m positions is combined into
 * one entry).  The pages do not give the combine rule; this library's
 * reading is the element-wise mean of the group's rows, rounded once to bf16
 * (nearest, ties to even).  x: bf16 [groups][m][dim] (m consecutive
 * positions per group); out: bf16 [groups][dim]; m in {1, 2}; dim % 8 == 0;
 * x and out 16-byte aligned.  Apply it to the K | V rows and to the indexer
 * keys, then pack the entries as usual. */
csa2_status csa2_compress(const uint16_t *x, int64_t groups, int32_t m, int32_t dim,
                          uint16_t *out, void *stream);

/* --------------------------------------------------------------- append */

/* Decode append ("CED", section "Why Prefill Recomputes a Recent Segment":
 * once a token is chosen, the global KV of its position is appended and every
 * decoder layer updates its local state).  For every sequence b with
 * 0 <= pos[b] < t_cap, row pos[b] of the global cache receives kv[b] (K | V,
 * bf16 [n_seq][256]; FP4-packed exactly as csa2_pack_fp4 or
 * csa2_pack_fp4_e4m3 does for the cache's format, or copied for a BF16 cache) and, when kidx is not NULL, its indexer key kidx[b] (bf16
 * [n_seq][64]); with m = 2 the global row is the new entry's (already
 * combined) row and is written to entry (pos[b] + 1) / 2 - 1 only when
 * pos[b] completes its group (pos[b] odd).  Then, for each of the n_local
 * layers l, slot pos[b] %
 * local[l].cap of that layer's ring receives k_new[l][b] and v_new[l][b]
 * (bf16 [n_seq][128] each).  Sequences with pos[b] outside [0, m t_cap)
 * are skipped.  The call WRITES through cache->data, cache->scales,
 * cache->k_idx and local[l].k / .v (the const of those structs is for the
 * read-only calls).  kv may be NULL to update the local rings only.
 *   pos: int32 [cache->n_seq]; local, k_new, v_new: host arrays [n_local]
 *   (n_local may be 0 and then they may be NULL); every row pointer and ring
 *   16-byte aligned, every local[l].cap > 0.  Rows written here are read by
 *   later calls on the same stream. */
csa2_status csa2_append(const csa2_cache *cache, const int32_t *pos, const uint16_t *kv,
                        const uint16_t *kidx, int32_t n_local, const csa2_local *local,
                        const uint16_t *const *k_new, const uint16_t *const *v_new,
                        void *stream);

/* -------------------------------------------------------------- indexer */

/* Indexer scores (Fig. 4: indexer Q of the layer against indexer K of the
 * global cache), a plain 64-element dot product accumulated in fp32.
 *   q_idx: bf16 [nq][64]; q_pos, q_seq: int32 [nq] (position and sequence of
 *   each query; q_seq may be NULL, then query i reads sequence i).  A query
 *   whose sequence id is out of range reads nothing (all scores -inf).
 *   nq <= 65535.
 * Dense (cand == NULL): scores[i][b] for b < ceil(t_cap / block): with block
 *   1 the score of position b; with block > 1 the max of the scores of the
 *   positions of block b (positions [b*block, b*block + block)).  Positions
 *   after q_pos[i] are masked (Fig. 2): their score is -inf and a block with
 *   none left is -inf.
 * Candidates (cand != NULL, block must be 1): scores[i][c] = score of
 *   position cand[i][c] (cand: int32 [nq][n_cand]); -inf for slots < 0 or
 *   after q_pos[i].
 * scores: float with row stride ld_scores (elements). */
csa2_status csa2_index_score(const csa2_cache *cache, const uint16_t *q_idx, const int32_t *q_pos,
                             const int32_t *q_seq, int32_t nq, const int32_t *cand, int64_t n_cand,
                             int32_t block, float *scores, int64_t ld_scores, void *stream);

/* Dense indexer scores of a prefill chunk: nq queries, all on sequence `seq`,
 * each at its own position q_pos[i] ("CED...", "Why Prefill Recomputes a
 * Recent Segment", Fig. 6: the recent positions pass through the decoder
 * again; each one selects like a decode query).  scores[i][t] for entries
 * t < t_cap, -inf past the query's last readable entry (t > q_pos[i] when
 * m <= 1; t > (q_pos[i] + 1) / 2 - 1 when m = 2).  The product Q_I K_I^T runs on MFMA (bf16 in, fp32
 * accumulation); q_idx: bf16 [nq][64]; scores: float, row stride ld_scores
 * >= t_cap. */
csa2_status csa2_prefill_score(const csa2_cache *cache, int32_t seq, const uint16_t *q_idx,
                               const int32_t *q_pos, int32_t nq, float *scores, int64_t ld_scores,
                               void *stream);

/* Indexer top-k of a prefill chunk ("CED...", "Why Prefill Recomputes a
 * Recent Segment", Fig. 6, with the selection of "Selecting Positions and
 * Reading Values with Attention", Fig. 4): nq queries on sequence `seq`, query
 * i at position q_pos[i], choose the k entries p it may read (p <= q_pos[i], or
 * with m = 2 p <= (q_pos[i] + 1) / 2 - 1) with the largest
 * q_idx[i] . k_idx[seq][p] (ties: lower entry first), written ascending to
 * sel[i][0..k), -1 padded.  The same selection as csa2_index_score followed by
 * csa2_topk on each row, computed without materialising the score rows: the
 * product runs on MFMA and only a candidate superset of the top-k is kept.
 * Limits: 1 <= k <= 2048, t_cap <= 262144 (else CSA2_ERR_SHAPE).  ws: at least
 * csa2_prefill_topk_workspace() bytes, no initial contents needed; q_pos
 * outside [0, t_cap) is clamped to t_cap - 1, negative gives an all -1 row. */
csa2_status csa2_prefill_topk_workspace(int32_t nq, int64_t t_cap, int32_t k, size_t *bytes);
csa2_status csa2_prefill_topk(const csa2_cache *cache, int32_t seq, const uint16_t *q_idx,
                              const int32_t *q_pos, int32_t nq, int32_t k, int32_t *sel, void *ws,
                              size_t ws_bytes, void *stream);

/* Top-k selection (Fig. 4) of each row of scores: float [nq][n] with row
 * stride ld.  Order: higher score first, equal scores by lower position
 * (-0 equals +0).  Entries equal to -inf, and slots whose id is < 0, are
 * never chosen.  ids (nullable, int32 [nq][n]) maps slot c to its position;
 * its non-negative entries must be ascending within a row (every pool this
 * library writes is).  out: int32 [nq][k], the chosen positions ascending,
 * padded with -1 when fewer than k can be chosen.  When out2 != NULL the
 * first k2 >= k under the same order are also written to out2 [nq][k2]
 * (the Full layer's candidate pool, Fig. 5).  n <= 2^24.  ws: at least the
 * size returned by csa2_topk_workspace (may be 0).  Rows longer than 32768
 * slots keep per-row counters in fixed records at the start of ws (max(nq, 64)
 * of them, addressed by row index only) that every call leaves zero, so a
 * workspace zero-filled once serves any later calls with nq <= 64 (any n, k,
 * k2), or with the same nq; zero-fill it again before a call with a
 * different nq above 64.  Calls sharing a workspace must not overlap. */
csa2_status csa2_topk(const float *scores, int32_t nq, int64_t n, int64_t ld, const int32_t *ids,
                      int32_t k, int32_t *out, int32_t k2, int32_t *out2, void *ws,
                      size_t ws_bytes, void *stream);
csa2_status csa2_topk_workspace(int32_t nq, int64_t n, int32_t k, int32_t k2, size_t *bytes);

/* Positions of chosen blocks: tokens[i][c*block + r] = blocks[i][c]*block + r
 * when blocks[i][c] >= 0 and that position is <= q_pos[i], else -1.
 * blocks: int32 [nq][nb] ascending (as csa2_topk writes them). */
csa2_status csa2_expand_blocks(const int32_t *blocks, int32_t nq, int32_t nb, int32_t block,
                               const int32_t *q_pos, int32_t *tokens, void *stream);

/* ------------------------------------------------------------ attention */

/* Sparse attention (Fig. 4): for each query i and head h, one softmax over
 * the global entries listed in sel[i] (int32 [nq][k]; slots < 0 or after
 * q_pos[i] are skipped) followed by the local window of q_pos[i]; logits are
 * sm_scale * (q . K); entries are not de-duplicated.  FP4 entries are
 * dequantised exactly.  q: bf16 [nq][16][128]; out: bf16 [nq][16][128]
 * (fp32 accumulation, rounded to nearest even).  A query with no entry at
 * all gets zeros.  q_seq may be NULL (query i reads sequence i).  nq <= 65535.
 * ws: at least csa2_sparse_attn_workspace bytes: 0 when one workgroup covers
 * a query (k <= 256 and window <= 32, or nq >= 20, where each query gets one
 * workgroup of its own); otherwise a fixed 16 KiB block of per-query counters
 * (at the start, addressed by query index only, left zero by every call)
 * followed by per-chunk partials.  It must be zero-filled before its first
 * use; after that it serves calls of any shape.  Calls sharing it must not
 * overlap. */
csa2_status csa2_sparse_attn(const csa2_cache *cache, const uint16_t *q, const int32_t *q_pos,
                             const int32_t *q_seq, int32_t nq, const int32_t *sel, int32_t k,
                             const csa2_local *local, float sm_scale, uint16_t *out, void *ws,
                             size_t ws_bytes, void *stream);
csa2_status csa2_sparse_attn_workspace(int32_t nq, int32_t k, int32_t window, size_t *bytes);

/* csa2_sparse_attn without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation).  It allocates nothing and calls no allocating
 * routine: the split form's counters and partials live in one fixed device
 * array per GPU inside the library (4 MiB + 16 KiB, held until the process
 * ends), whose counters each call clears with a small kernel on `stream`
 * before using them.  Same arguments, results and rules as csa2_sparse_attn
 * otherwise (bit-identical outputs).  Limit: the partials of nq queries times
 * chunks-per-query must fit 4 MiB -- nq * max(ceil(k / 256), ceil(window /
 * 32)) <= 504 when nq < 20 (e.g. 19 queries at k = 6656, window 128: 26
 * chunks each); from 20 queries on no scratch is used and any size is accepted.  Larger calls
 * return CSA2_ERR_TOO_LARGE and enqueue nothing.  Every call on a GPU shares
 * its array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller. */
csa2_status csa2_sparse_attn_noalloc(const csa2_cache *cache, const uint16_t *q,
                                     const int32_t *q_pos, const int32_t *q_seq, int32_t nq,
                                     const int32_t *sel, int32_t k, const csa2_local *local,
                                     float sm_scale, uint16_t *out, void *stream);

/* ------------------------------------------------------------ layer stack */

/* A decoder stack over one shared global cache with one decode query per
 * sequence (query b belongs to sequence b), modes fixed per layer (Fig. 5):
 *   Full    dense indexer scores, top-k selection and, with pool > 0, the
 *           candidate pool of the top `pool` positions (layer 0 is Full; a
 *           later Full layer builds a new pool).  With
 *           block > 1 the pool is every position of the top pool/block
 *           blocks by block score (max of its tokenwise scores) and the top-k
 *           is chosen tokenwise inside it.
 *   Reindex: its own indexer query rescores the pool; top-k inside it.
 *   Reuse:  the previous layer's selection, unchanged.
 * Every layer then runs csa2_sparse_attn with its own q and local KV.
 * All per-layer arrays are HOST arrays of n_layers device pointers. */
typedef struct {
    int32_t n_layers;
    const int32_t *modes;              /* host [n_layers], csa2_mode */
    const csa2_cache *cache;           /* host pointer */
    const int32_t *q_pos;              /* device int32 [n_seq] */
    int32_t k;                         /* selected global entries per layer */
    int32_t pool;                      /* pool size in positions (0: no Reindex layers) */
    int32_t block;                     /* 1: tokenwise Full scoring; 64: blockwise */
    float sm_scale;
    const uint16_t *const *q;          /* [l] -> bf16 [n_seq][16][128] */
    const uint16_t *const *q_idx;      /* [l] -> bf16 [n_seq][64]; unused (may be NULL) for Reuse */
    const csa2_local *local;           /* host [n_layers] */
    uint16_t *const *out;              /* [l] -> bf16 [n_seq][16][128] */
    int32_t *const *sel_out;           /* NULL, or [l] -> int32 [n_seq][k] (entries may be NULL) */
    int32_t *pool_out;                 /* NULL, or int32 [n_seq][pool] */
    void *scan_events[2];              /* optional timing hook: two hipEvent_t the caller
                                          created (with timing).  csa2_stack_run stores the
                                          start and end of layer 0's indexer scan kernel in
                                          them (the kernel's own times); a plan records them
                                          on the stream right before and after that kernel.
                                          NULL skips */
    /* Decode append (optional; see csa2_append).  When append_kv is not NULL
     * the stack first writes position q_pos[b] of every sequence: the global
     * row append_kv (bf16 [n_seq][256]), the indexer key append_kidx (bf16
     * [n_seq][64], may be NULL) and, when append_k and append_v are not NULL,
     * layer l's local ring slot from append_k[l] / append_v[l] (bf16
     * [n_seq][128]; a NULL pair skips that layer).  Layer 0's scan then sees
     * the new position.  In a plan the append is recorded with the layers, so
     * a launch appends whatever the buffers hold at that time. */
    const uint16_t *append_kv;
    const uint16_t *append_kidx;
    const uint16_t *const *append_k;   /* host [n_layers], or NULL */
    const uint16_t *const *append_v;   /* host [n_layers], or NULL */
    void *const *attn_events;          /* optional timing hook: NULL, or a host array of
                                          2 * n_layers hipEvent_t the caller created (with
                                          timing); csa2_stack_run stores the start and end of
                                          layer l's attention kernel (its own times) in
                                          entries 2l and 2l + 1.  Ignored by a plan */
} csa2_stack_desc;

/* Workspace of csa2_stack_run.  Its counters sit at the start at offsets
 * that depend only on n_seq (and on nothing up to 64 sequences) and every run
 * leaves them zero: zero-fill the workspace before its first use, and again
 * only before reusing it for a stack with a different n_seq above 64. */
csa2_status csa2_stack_workspace(const csa2_stack_desc *desc, size_t *bytes);
/* Run every layer in order on `stream`.  Validates the schedule: layer 0 must
 * be Full and Reindex needs pool > 0; k <= pool when pool > 0; block is 1 or
 * 64, and with 64, pool > 0 and pool % 64 == 0.  With block 64 and a pool of
 * at most 16384 positions, pool_out is written only when given (the layers
 * score the pool from its block ids). */
csa2_status csa2_stack_run(const csa2_stack_desc *desc, void *ws, size_t ws_bytes, void *stream);

/* A stack plan records what csa2_stack_run would enqueue, once, into a HIP
 * graph; each launch replays it on `stream`.  Every pointer of `desc` and `ws`
 * is fixed at creation: the caller keeps those buffers alive for the plan's
 * life and may change their contents between launches (new queries, new
 * cache rows).  The workspace follows the csa2_stack_workspace rules (zero
 * before the first launch, left zero by each); launches of plans sharing a
 * workspace must not overlap.  With scan_events set, the event records are
 * part of the graph.  Creation validates like csa2_stack_run and returns its
 * codes (CSA2_ERR_HIP if the runtime cannot record or instantiate the graph);
 * the plan object and its graph are the only memory the library allocates,
 * released by csa2_stack_plan_destroy. */
typedef struct csa2_stack_plan csa2_stack_plan;
csa2_status csa2_stack_plan_create(const csa2_stack_desc *desc, void *ws, size_t ws_bytes,
                                   csa2_stack_plan **plan);
csa2_status csa2_stack_plan_launch(const csa2_stack_plan *plan, void *stream);
csa2_status csa2_stack_plan_destroy(csa2_stack_plan *plan);

/* ------------------------------------------------------- bounded replay */

/* Bounded replay of a prompt's recent segment ("CED", section "Why Prefill
 * Recomputes a Recent Segment", Fig. 6): once the global KV of the whole
 * prompt is in the cache, only the last positions pass through the decoder
 * again, so that every layer rebuilds its local state; window references
 * before the segment are cut off (set each layer's local.lo to the segment's
 * first position for the section's approximation; a smaller lo lets the
 * window read older ring slots).
 * The n queries at q_pos (device int32 [n], each in [0, t_cap); normally
 * consecutive) all belong to sequence `seq`.  Layer by layer, in the
 * schedule's order: when local_k and local_v are set, the segment's local
 * rows local_k[l] / local_v[l] (bf16 [n][128]; a NULL pair skips the layer)
 * enter slot q_pos[i] % cap of the layer's ring (n <= cap, so no two rows
 * share a slot); then every query runs the layer's mode exactly as a decode
 * query at its position would (Full: its own top-k over [0, t] and, with
 * pool > 0, its pool; Reindex: top-k of its pool; Reuse: the previous
 * layer's picks) and attends with the layer's q and window.  All ring rows
 * are written before layer 0 runs (each layer reads only its own ring).
 *   q [l] -> bf16 [n][16][128]; q_idx [l] -> bf16 [n][64] (unused on Reuse);
 *   out [l] -> bf16 [n][16][128]; sel_out NULL or [l] -> int32 [n][k];
 *   pool_out NULL or int32 [n][pool].  1 <= n <= 65535.
 * Workspace rules as csa2_stack_workspace, with n in place of n_seq
 * (zero-filled before first use; again before a different n above 64; calls
 * sharing one must not overlap).  A Full layer with block 1, no
 * pool, k <= 2048 and t_cap <= 2^18 uses the fused top-k of
 * csa2_prefill_topk; otherwise the segment's score rows are materialised
 * (n * t_cap floats of workspace). */
typedef struct {
    int32_t n_layers;
    const int32_t *modes;              /* host [n_layers], csa2_mode */
    const csa2_cache *cache;           /* host pointer */
    int32_t seq;                       /* the sequence replayed */
    int32_t n;                         /* queries in the segment */
    const int32_t *q_pos;              /* device int32 [n] */
    int32_t k;
    int32_t pool;
    int32_t block;                     /* 1, or 64 (blockwise Full) */
    float sm_scale;
    const uint16_t *const *q;          /* host [n_layers] of device pointers */
    const uint16_t *const *q_idx;
    const csa2_local *local;           /* host [n_layers] */
    const uint16_t *const *local_k;    /* host [n_layers], or NULL */
    const uint16_t *const *local_v;    /* host [n_layers], or NULL */
    uint16_t *const *out;
    int32_t *const *sel_out;
    int32_t *pool_out;
} csa2_replay_desc;

csa2_status csa2_replay_workspace(const csa2_replay_desc *desc, size_t *bytes);
csa2_status csa2_replay_run(const csa2_replay_desc *desc, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */

// csa2_kernels.h -- host-side launchers of the gfx950 kernels (internal).
// Each launcher only enqueues on `s`; shapes are validated by the caller
// (csa2_api.cpp) before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

struct CacheView {
    int32_t fp4;            // 0: bf16 rows; 1: FP4 + E8M0 per 32; 2: FP4 + E4M3 per 16
    int32_t n_seq;
    int64_t t_cap;          // entries per sequence
    int32_t msh;            // log2 of positions per entry (0, or 1 for m = 2)
    const void* data;       // bf16 [n_seq][t_cap][256] or codes [n_seq][t_cap][128]
    const uint8_t* scales;  // [n_seq][t_cap][8] (E8M0) or [n_seq][t_cap][16] (E4M3)
    const uint16_t* k_idx;  // [n_seq][t_cap][64]
};

struct LocalView {
    const uint16_t* k;
    const uint16_t* v;
    int32_t cap, window, lo;
};

hipError_t launch_pack_fp4(const uint16_t* x, int64_t nblk, uint8_t* codes, uint8_t* scales,
                           hipStream_t s);
hipError_t launch_unpack_fp4(const uint8_t* codes, const uint8_t* scales, int64_t nblk, float* out,
                             hipStream_t s);
// FP4 with one E4M3 scale per 16 elements: nblk blocks of 16.
hipError_t launch_pack_fp4e(const uint16_t* x, int64_t nblk, uint8_t* codes, uint8_t* scales,
                            hipStream_t s);
hipError_t launch_unpack_fp4e(const uint8_t* codes, const uint8_t* scales, int64_t nblk, float* out,
                              hipStream_t s);

// Sequence compression: out[g] = bf16 mean of x[g][0..m), m in {1, 2}; dim % 8 == 0.
hipError_t launch_compress(const uint16_t* x, int64_t groups, int32_t m, int32_t dim, uint16_t* out,
                           hipStream_t s);

// Dense indexer scores: scores[i][b], b < ceil(t_cap / block), block in {1, 64}.
// Decode append: the new position's global row (FP4-packed or copied),
// indexer key and every listed layer's local K/V ring slot, per sequence.
constexpr int kMaxAppendLayers = 32;  // layers per launch (kernel argument size)
struct AppendLocal {
    uint16_t* k;
    uint16_t* v;
    const uint16_t* k_new;  // bf16 [n rows][128]
    const uint16_t* v_new;
    int32_t cap;
};
struct AppendArgs {
    const int32_t* pos;  // [n rows] positions; rows outside [0, t_cap << msh) are skipped
    int32_t seq;         // -1: row b belongs to sequence b; else every row to `seq`
    int32_t* q_seq_out;  // null, or [n rows]: receives each row's sequence
    int64_t t_cap;         // entries per sequence
    int32_t msh;           // log2 of positions per entry: the global row of a
                           // position completing its group goes to that entry
    int32_t fp4;           // the cache's format code (CacheView::fp4)
    const uint16_t* kv;    // bf16 [n rows][256] or null
    const uint16_t* kidx;  // bf16 [n rows][64] or null
    uint8_t* codes;        // FP4 cache
    uint8_t* scales;
    uint16_t* bf16;        // bf16 cache
    uint16_t* k_idx;
    int32_t n_local;
    AppendLocal local[kMaxAppendLayers];
};
hipError_t launch_append(const AppendArgs& a, int32_t n_rows, hipStream_t s);

// With ev0/ev1 set, the kernel's own start and end times are recorded in them.
hipError_t launch_score_dense(const CacheView& c, const uint16_t* q_idx, const int32_t* q_pos,
                              const int32_t* q_seq, int32_t nq, int32_t block, float* scores,
                              int64_t ld, hipStream_t s, hipEvent_t ev0 = nullptr,
                              hipEvent_t ev1 = nullptr);
// The decode step's first tokenwise scan (query b on sequence b, one per
// sequence) with the step's append (one launch's worth of layers) in the same
// launch: the scan reads each query's new key from the append rows.
hipError_t launch_score_dense_append(const CacheView& c, const uint16_t* q_idx,
                                     const int32_t* q_pos, int32_t nq, float* scores, int64_t ld,
                                     const AppendArgs& a, hipStream_t s, hipEvent_t ev0 = nullptr,
                                     hipEvent_t ev1 = nullptr);
// Candidate scores: scores[i][j] = score of position cand[i][j].
hipError_t launch_score_cand(const CacheView& c, const uint16_t* q_idx, const int32_t* q_pos,
                             const int32_t* q_seq, int32_t nq, const int32_t* cand, int64_t n_cand,
                             float* scores, int64_t ld, hipStream_t s);

// Dense scores of many queries on one sequence (prefill chunk), on MFMA.
hipError_t launch_score_mq(const CacheView& c, int32_t seq, const uint16_t* q_idx,
                           const int32_t* q_pos, int32_t nq, float* scores, int64_t ld,
                           hipStream_t s);

// Fused indexer top-k of a prefill chunk on one sequence (MFMA scores, never
// written out).  Limits: k <= kPfMaxK, t_cap <= kPfMaxT.  The workspace needs
// no initial contents.
constexpr int kPfCap = 4096;
constexpr int32_t kPfMaxK = 2048;
constexpr int64_t kPfMaxT = int64_t(1) << 18;
size_t prefill_topk_ws_bytes(int32_t nq, int64_t t_cap);
hipError_t launch_prefill_topk(const CacheView& c, int32_t seq, const uint16_t* q_idx,
                               const int32_t* q_pos, int32_t nq, int32_t k, int32_t* sel, void* ws,
                               hipStream_t s);

// Candidate scores + top-k among them (n_cand <= 16384); with block_shift
// b > 0, `cand` holds n_cand >> b block ids per query and candidate c is
// position cand[c >> b] * 2^b + c % 2^b (n_cand a multiple of 2^b); `scores` holds nq
// rows of score_select_ld(n_cand) floats (whole 128-byte lines per row, so no
// line is written by two workgroups); `ctr` holds nq counters kCtrStride words
// apart that must be zero and are left zero.
__host__ __device__ inline int64_t score_select_ld(int64_t n_cand) { return (n_cand + 31) / 32 * 32; }
hipError_t launch_score_select(const CacheView& c, const uint16_t* q_idx, const int32_t* q_pos,
                               const int32_t* q_seq, int32_t nq, const int32_t* cand,
                               int64_t n_cand, float* scores, uint32_t* ctr, int32_t k,
                               int32_t* sel, hipStream_t s, int32_t block_shift = 0);
constexpr int64_t kFusedSelectMax = 16384;

size_t topk_ws_bytes(int32_t nq, int64_t n, int32_t k, int32_t k2);
hipError_t launch_topk(const float* scores, int32_t nq, int64_t n, int64_t ld, const int32_t* ids,
                       int32_t k, int32_t* out, int32_t k2, int32_t* out2, void* ws, hipStream_t s);

// msh: the positions are those of entries of 2^msh positions (q_pos stays a
// token position).
hipError_t launch_expand_blocks(const int32_t* blocks, int32_t nq, int32_t nb, int32_t block,
                                const int32_t* q_pos, int32_t* tokens, hipStream_t s,
                                int32_t msh = 0);

// From this many queries on, attention runs one workgroup per query (no
// workspace); below it, each query is split over several workgroups.  The
// split kernel holds ~105 KB of LDS (one workgroup per CU) and its last
// chunk of each query merges the others, so its time grows with the queries
// while the one-per-query loop stays flat until the queries fill the CUs.
// Measured per call, each build in its own process (k = 2048, W = 128: 8
// chunks a query), split vs loop: 16 queries 22.8 / 25.6 us, 24: 25.5 /
// 25.3, 32: 28.4 / 25.4, 48: 40.0 / 25.7, 128: 71.8 / 27.1; with k = 512 (4
// chunks): 8 queries 17.8 / 18.8, 16: 19.1 / 18.3, 32: 21.3 / 18.2.
constexpr int32_t kManyQueries = 20;
// Queries a block of per-query counters covers (the split attention's, the
// stack's Reindex select's): the blocks keep this size for any call, so a
// workspace's layout does not depend on the number of queries up to it.
constexpr int32_t kCtrBlockQueries = 64;
static_assert(kCtrBlockQueries >= kManyQueries, "every split call's counters fit the block");

// Per-query arrival counters sit 256 bytes apart, so the workgroups of
// different queries never contend for one cache line.
constexpr int64_t kCtrStride = 64;
// The split form's workspace: a fixed block of per-query counters (one for
// each query a split call can have), then the per-chunk partials.  The
// counters' addresses depend on nothing but the query index, so a workspace
// serves calls of any shape without being cleared again (every call leaves
// its counters zero).
constexpr size_t kAttnCtrBytes = (size_t)kCtrBlockQueries * kCtrStride * sizeof(uint32_t);
size_t attn_part_bytes(int32_t nq, int32_t k, int32_t window);
size_t attn_ws_bytes(int32_t nq, int32_t k, int32_t window);  // 0, or kAttnCtrBytes + partials
// ctr: kAttnCtrBytes (zero, left zero); part: attn_part_bytes.
hipError_t launch_sparse_attn_parts(const CacheView& c, const uint16_t* q, const int32_t* q_pos,
                                    const int32_t* q_seq, int32_t nq, const int32_t* sel, int32_t k,
                                    const LocalView& loc, float sm_scale, uint16_t* out,
                                    uint32_t* ctr, float* part, hipStream_t s,
                                    hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
// The allocation-free form: counters and partials in a fixed device array of
// kStaticScratchBytes (partials of up to 504 query-chunks, e.g. 19 queries of
// 26 chunks); a larger call returns hipErrorInvalidValue.
constexpr size_t kStaticScratchBytes = kAttnCtrBytes + ((size_t)4 << 20);
hipError_t launch_sparse_attn_static(const CacheView& c, const uint16_t* q, const int32_t* q_pos,
                                     const int32_t* q_seq, int32_t nq, const int32_t* sel, int32_t k,
                                     const LocalView& loc, float sm_scale, uint16_t* out,
                                     hipStream_t s);
hipError_t launch_sparse_attn(const CacheView& c, const uint16_t* q, const int32_t* q_pos,
                              const int32_t* q_seq, int32_t nq, const int32_t* sel, int32_t k,
                              const LocalView& loc, float sm_scale, uint16_t* out, void* ws,
                              hipStream_t s);

}  // namespace csa2

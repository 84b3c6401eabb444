// k_score.hip -- indexer scores: the layer's 64-element indexer query against
// the indexer keys of the shared global cache ("CED: Continuing Context with a
// Causal Encoder and Decoder", section "Selecting Positions and Reading Values
// with Attention", Fig. 4), causally masked (same page, Fig. 2: a query at t
// reads positions <= t only).
//
// Decode scoring is a GEMV over T keys of 128 B each: pure HBM streaming at
// about one flop per byte, so it runs on the vector ALUs, not MFMA.  Eight
// lanes share one key: each lane loads 16 contiguous bytes, so every load
// instruction of a wave reads 1 KB of consecutive memory (8 keys), and the
// eight partial dots are summed with three lane exchanges.
#include <hip/hip_ext.h>

#include <algorithm>

#include "csa2_dev.h"
#include "csa2_kernels.h"
#include "csa2_pack.h"
#include "csa2_select.h"

namespace csa2 {

constexpr int kScoreTile = 256;  // keys per workgroup (4 waves x 64)

__device__ __forceinline__ float dot8(const float* q, uint4 k) {
    float a = q[0] * bf16_lo(k.x);
    a = fmaf(q[1], bf16_hi(k.x), a);
    a = fmaf(q[2], bf16_lo(k.y), a);
    a = fmaf(q[3], bf16_hi(k.y), a);
    a = fmaf(q[4], bf16_lo(k.z), a);
    a = fmaf(q[5], bf16_hi(k.z), a);
    a = fmaf(q[6], bf16_lo(k.w), a);
    a = fmaf(q[7], bf16_hi(k.w), a);
    return a;
}

__device__ __forceinline__ void load_q8(const uint16_t* q, float* qf) {
    const uint4 v = *reinterpret_cast<const uint4*>(q);
    qf[0] = bf16_lo(v.x); qf[1] = bf16_hi(v.x);
    qf[2] = bf16_lo(v.y); qf[3] = bf16_hi(v.y);
    qf[4] = bf16_lo(v.z); qf[5] = bf16_hi(v.z);
    qf[6] = bf16_lo(v.w); qf[7] = bf16_hi(v.w);
}

// One 256-key tile of query qi's dense scores (tile index bx).  Lane (grp,
// sub) of a wave handles bytes [16 sub, 16 sub + 16) of key base + 8 r + grp
// in round r.  app_kidx (or null): the decode append's new indexer keys
// ([nq][64]); entry te of query qi -- the one its own position completes, which
// the append writes in the same launch -- is read from there instead of the
// cache.
template <int BLOCK>
__device__ __forceinline__ void score_dense_tile(const uint16_t* __restrict__ k_idx, int32_t n_seq,
                                                 int64_t t_cap, int32_t msh,
                                                 const uint16_t* __restrict__ q_idx,
                                                 const int32_t* __restrict__ q_pos,
                                                 const int32_t* __restrict__ q_seq,
                                                 float* __restrict__ scores, int64_t ld, int qi,
                                                 int bx, const uint16_t* __restrict__ app_kidx) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane & 7, grp = lane >> 3;
    const int64_t base = (int64_t)bx * kScoreTile + wave * 64;
    float* srow = scores + (int64_t)qi * ld;
    const int32_t seq = q_seq ? q_seq[qi] : qi;
    // the last entry the query may read: entries of 2^msh positions count
    // once their whole group is at or before the query's position
    int64_t t = (((int64_t)q_pos[qi] + 1) >> msh) - 1;
    if (seq < 0 || seq >= n_seq) t = -1;  // a bad sequence id reads nothing
    if (t >= t_cap) t = t_cap - 1;
    if (base >= t_cap) return;
    const float NEG = -__builtin_inff();
    if (base > t) {  // the whole wave is after the query: masked
        if (BLOCK == 1) {
            if (base + lane < t_cap) srow[base + lane] = NEG;
        } else if (lane == 0) {
            srow[base / 64] = NEG;
        }
        return;
    }
    float qf[8];
    load_q8(q_idx + (int64_t)qi * kIdxDim + sub * 8, qf);
    const uint4* kb = reinterpret_cast<const uint4*>(k_idx) + (int64_t)seq * t_cap * 8;
    int64_t te = -1;  // the entry the append writes for this query, if any
    if (app_kidx) {
        const int32_t p = q_pos[qi];
        if (p >= 0 && p < (t_cap << msh) && ((p + 1) & ((1 << msh) - 1)) == 0) te = ((p + 1) >> msh) - 1;
    }
    uint4 kv[8];
    if (te >= base && te < base + 64) {  // wave-uniform: this wave holds the new entry
        const uint4* ka = reinterpret_cast<const uint4*>(app_kidx + (int64_t)qi * kIdxDim);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t tok = base + r * 8 + grp;
            kv[r] = tok == te ? ka[sub] : (tok <= t ? kb[tok * 8 + sub] : make_uint4(0, 0, 0, 0));
        }
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t tok = base + r * 8 + grp;
            kv[r] = (tok <= t) ? kb[tok * 8 + sub] : make_uint4(0, 0, 0, 0);
        }
    }
    float s[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) s[r] = sum8(dot8(qf, kv[r]));
    if (BLOCK == 1) {
        // lane (grp, sub) stores key base + 8 sub + grp: one 256 B coalesced store
        float v = s[0];
#pragma unroll
        for (int r = 1; r < 8; ++r) v = (sub == r) ? s[r] : v;
        const int64_t tok = base + sub * 8 + grp;
        if (tok < t_cap) srow[tok] = (tok <= t) ? v : NEG;
    } else {
        float m = NEG;
#pragma unroll
        for (int r = 0; r < 8; ++r)
            if (base + r * 8 + grp <= t) m = fmaxf(m, s[r]);
        m = fmaxf(m, __shfl_xor(m, 8, 64));
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        if (lane == 0) srow[base / 64] = m;
    }
}

// grid: (ceil(t_cap / 256), nq).
template <int BLOCK>
__global__ __launch_bounds__(256) void k_score_dense(const uint16_t* __restrict__ k_idx,
                                                     int32_t n_seq, int64_t t_cap, int32_t msh,
                                                     const uint16_t* __restrict__ q_idx,
                                                     const int32_t* __restrict__ q_pos,
                                                     const int32_t* __restrict__ q_seq,
                                                     float* __restrict__ scores, int64_t ld) {
    score_dense_tile<BLOCK>(k_idx, n_seq, t_cap, msh, q_idx, q_pos, q_seq, scores, ld, blockIdx.y,
                            blockIdx.x, nullptr);
}

// The decode step's first indexer scan and its append in one launch ("CED",
// section "Why Prefill Recomputes a Recent Segment": the new position's global
// KV and every layer's local row are appended before the layers read them).
// grid: (max(tiles, nq (1 + groups)), nq + 1): rows 0 .. nq-1 are the scan
// (query b reads sequence b); in row nq, workgroup x < nq (1 + groups) does
// the append's workgroup (x % nq, x / nq).  The scan takes query b's new key
// from the append's rows, so it needs no order against the append's writes;
// later launches read the appended rows.
__global__ __launch_bounds__(256) void k_score_dense_append(const uint16_t* __restrict__ k_idx,
                                                            int32_t n_seq, int64_t t_cap, int32_t msh,
                                                            const uint16_t* __restrict__ q_idx,
                                                            const int32_t* __restrict__ q_pos,
                                                            float* __restrict__ scores, int64_t ld,
                                                            AppendArgs a, int32_t groups) {
    const int nq = (int)gridDim.y - 1;
    if ((int)blockIdx.y == nq) {
        const int x = blockIdx.x;
        if (x < nq * (1 + groups)) append_rows(a, x % nq, x / nq);
        return;
    }
    score_dense_tile<1>(k_idx, n_seq, t_cap, msh, q_idx, q_pos, nullptr, scores, ld, blockIdx.y,
                        blockIdx.x, a.kidx);
}

// grid: (ceil(n_cand / 256), nq).  Same lane layout; key c of the tile is
// position cand[qi][c].
__global__ __launch_bounds__(256) void k_score_cand(const uint16_t* __restrict__ k_idx,
                                                    int32_t n_seq, int64_t t_cap, int32_t msh,
                                                    const uint16_t* __restrict__ q_idx,
                                                    const int32_t* __restrict__ q_pos,
                                                    const int32_t* __restrict__ q_seq,
                                                    const int32_t* __restrict__ cand,
                                                    int64_t n_cand, float* __restrict__ scores,
                                                    int64_t ld) {
    const int qi = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane & 7, grp = lane >> 3;
    const int64_t base = (int64_t)blockIdx.x * kScoreTile + wave * 64;
    if (base >= n_cand) return;
    float* srow = scores + (int64_t)qi * ld;
    const int32_t* crow = cand + (int64_t)qi * n_cand;
    const int32_t seq = q_seq ? q_seq[qi] : qi;
    // the last entry the query may read: entries of 2^msh positions count
    // once their whole group is at or before the query's position
    int64_t t = (((int64_t)q_pos[qi] + 1) >> msh) - 1;
    if (seq < 0 || seq >= n_seq) t = -1;
    if (t >= t_cap) t = t_cap - 1;
    float qf[8];
    load_q8(q_idx + (int64_t)qi * kIdxDim + sub * 8, qf);
    const uint4* kb = reinterpret_cast<const uint4*>(k_idx) + (int64_t)(seq < 0 ? 0 : seq) * t_cap * 8;
    uint4 kv[8];
    bool ok[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int64_t c = base + r * 8 + grp;
        const int64_t tok = (c < n_cand) ? crow[c] : -1;
        ok[r] = tok >= 0 && tok <= t;
        kv[r] = ok[r] ? kb[tok * 8 + sub] : make_uint4(0, 0, 0, 0);
    }
    float s[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) s[r] = ok[r] ? sum8(dot8(qf, kv[r])) : -__builtin_inff();
    float v = s[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) v = (sub == r) ? s[r] : v;
    const int64_t c = base + sub * 8 + grp;
    if (c < n_cand) srow[c] = v;
}

// Candidate scoring fused with the selection among the candidates, for the
// Reindex layers (rescore the Full layer's pool with the layer's own indexer
// query and keep the top k, "What Full, Reindex, and Reuse Share", Fig. 5).
// MODE 0, grid (ceil(n_cand / sel_keys<R>()), nq): every workgroup scores
// sel_keys<R>() candidates into `scores` (agent-scope atomic stores, read back
// with agent-scope atomic loads); every arrival on the per-query counter `ctr`
// (reset on exit) is a release and the last one, after an acquire fence,
// selects the top k of all n_cand <= kSelMaxCand candidates.  For a handful of
// queries (decode).
// MODE 1, same grid: the scores alone (plain stores); MODE 2, grid (1, nq),
// launched after it: one workgroup per query selects.  For many queries, where
// leaving the selections to the last arrivals would pile them onto whichever
// XCD falls behind (as in the long-row top-k).
constexpr int kSelMaxCand = 16384;
constexpr int kSelNT = 1024;

// A workgroup scores (kSelNT / 64) * 8 * R candidates (R per lane group of 8
// lanes, one 128-byte key each): R = 8 when the queries alone give enough
// workgroups to fill the GPU, R = 2 for a handful of queries (decode), where
// spreading the gather over 4x the workgroups shortens it.
template <int R>
constexpr int sel_keys() { return (kSelNT / 64) * 8 * R; }

template <int R, int MODE>
__global__ __launch_bounds__(kSelNT) void k_score_select(const uint16_t* __restrict__ k_idx,
                                                         int32_t n_seq, int64_t t_cap, int32_t msh,
                                                         const uint16_t* __restrict__ q_idx,
                                                         const int32_t* __restrict__ q_pos,
                                                         const int32_t* __restrict__ q_seq,
                                                         const int32_t* __restrict__ cand,
                                                         int64_t n_cand, float* __restrict__ scores,
                                                         uint32_t* __restrict__ ctr, int32_t k,
                                                         int32_t* __restrict__ sel, int32_t bs) {
    __shared__ WaveSelShared<kSelNT> sh;
    __shared__ int last;
    const int qi = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane & 7, grp = lane >> 3;
    const int64_t base = (int64_t)blockIdx.x * sel_keys<R>() + wave * 8 * R;
    float* srow = scores + (int64_t)qi * score_select_ld(n_cand);
    // bs > 0: cand holds n_cand >> bs block ids per query, candidate c being
    // position cand[c >> bs] * 2^bs + c % 2^bs (-1 for an empty block)
    const int32_t* crow = cand + (int64_t)qi * (n_cand >> bs);
    const int32_t seq = q_seq ? q_seq[qi] : qi;
    // the last entry the query may read: entries of 2^msh positions count
    // once their whole group is at or before the query's position
    int64_t t = (((int64_t)q_pos[qi] + 1) >> msh) - 1;
    if (seq < 0 || seq >= n_seq) t = -1;
    if (t >= t_cap) t = t_cap - 1;
    if (MODE != 2 && base < n_cand) {
        float qf[8];
        load_q8(q_idx + (int64_t)qi * kIdxDim + sub * 8, qf);
        const uint4* kb =
            reinterpret_cast<const uint4*>(k_idx) + (int64_t)(seq < 0 ? 0 : seq) * t_cap * 8;
        uint4 kv[R];
        bool ok[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t c = base + r * 8 + grp;
            int64_t tok = -1;
            if (c < n_cand) {
                const int32_t id = crow[c >> bs];
                tok = bs ? (id >= 0 ? (int64_t)id * (1 << bs) + (c & ((1 << bs) - 1)) : -1) : id;
            }
            ok[r] = tok >= 0 && tok <= t;
            kv[r] = ok[r] ? kb[tok * 8 + sub] : make_uint4(0, 0, 0, 0);
        }
        float my = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float sc = ok[r] ? sum8(dot8(qf, kv[r])) : -__builtin_inff();
            if (sub == r) my = sc;
        }
        const int64_t c = base + sub * 8 + grp;
        if (sub < R && c < n_cand) {
            if (MODE == 0) store_coherent(&srow[c], my);
            else srow[c] = my;
        }
    }
    if (MODE == 1) return;
    if (MODE == 0) {
        hand_off_wait();  // this thread's score stores are complete
        __syncthreads();
        if (threadIdx.x == 0) last = arrive_last_release(&ctr[qi * kCtrStride], gridDim.x);
        __syncthreads();
        if (!last) return;
    }
    if (n_cand <= kSelNT * 8)  // every wave holds keys
        wave_select<kSelNT, 8, MODE == 0>(srow, crow, (int)n_cand, k, sel + (int64_t)qi * k, sh, bs);
    else
        wave_select<kSelNT, kSelMaxCand / kSelNT, MODE == 0>(srow, crow, (int)n_cand, k, sel + (int64_t)qi * k, sh,
                                                            bs);
    if (MODE == 0 && threadIdx.x == 0) ctr[qi * kCtrStride] = 0u;
}

hipError_t launch_score_select(const CacheView& c, const uint16_t* q_idx, const int32_t* q_pos,
                               const int32_t* q_seq, int32_t nq, const int32_t* cand,
                               int64_t n_cand, float* scores, uint32_t* ctr, int32_t k,
                               int32_t* sel, hipStream_t s, int32_t block_shift) {
    if (nq == 0 || n_cand == 0) return hipSuccess;
    if (n_cand > kSelMaxCand) return hipErrorInvalidValue;
    if (block_shift < 0 || block_shift > 16 || (n_cand & ((1 << block_shift) - 1))) return hipErrorInvalidValue;
    const int64_t wide = (n_cand + sel_keys<8>() - 1) / sel_keys<8>();
    if (wide * nq >= 256) {  // the queries fill the GPU
        hipLaunchKernelGGL((k_score_select<8, 1>), dim3((uint32_t)wide, (uint32_t)nq), dim3(kSelNT), 0, s,
                           c.k_idx, c.n_seq, c.t_cap, c.msh, q_idx, q_pos, q_seq, cand, n_cand,
                           scores, ctr, k, sel, block_shift);
        hipLaunchKernelGGL((k_score_select<8, 2>), dim3(1u, (uint32_t)nq), dim3(kSelNT), 0, s,
                           c.k_idx, c.n_seq, c.t_cap, c.msh, q_idx, q_pos, q_seq, cand, n_cand,
                           scores, ctr, k, sel, block_shift);
    } else {
        const int64_t nb = (n_cand + sel_keys<2>() - 1) / sel_keys<2>();
        hipLaunchKernelGGL((k_score_select<2, 0>), dim3((uint32_t)nb, (uint32_t)nq), dim3(kSelNT), 0, s,
                           c.k_idx, c.n_seq, c.t_cap, c.msh, q_idx, q_pos, q_seq, cand, n_cand,
                           scores, ctr, k, sel, block_shift);
    }
    return hipGetLastError();
}

hipError_t launch_score_dense(const CacheView& c, const uint16_t* q_idx, const int32_t* q_pos,
                              const int32_t* q_seq, int32_t nq, int32_t block, float* scores,
                              int64_t ld, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (nq == 0 || c.t_cap == 0) return hipSuccess;
    dim3 grid((uint32_t)((c.t_cap + kScoreTile - 1) / kScoreTile), (uint32_t)nq);
    if (block == 1)
        hipExtLaunchKernelGGL(k_score_dense<1>, grid, dim3(256), 0, s, ev0, ev1, 0, c.k_idx, c.n_seq,
                              c.t_cap, c.msh, q_idx, q_pos, q_seq, scores, ld);
    else
        hipExtLaunchKernelGGL(k_score_dense<64>, grid, dim3(256), 0, s, ev0, ev1, 0, c.k_idx, c.n_seq,
                              c.t_cap, c.msh, q_idx, q_pos, q_seq, scores, ld);
    return hipGetLastError();
}

hipError_t launch_score_dense_append(const CacheView& c, const uint16_t* q_idx,
                                     const int32_t* q_pos, int32_t nq, float* scores, int64_t ld,
                                     const AppendArgs& a, hipStream_t s, hipEvent_t ev0,
                                     hipEvent_t ev1) {
    if (nq == 0 || c.t_cap == 0) return hipSuccess;
    const int32_t groups = (a.n_local + kAppendLayersPerWg - 1) / kAppendLayersPerWg;
    const int64_t tiles = (c.t_cap + kScoreTile - 1) / kScoreTile;
    dim3 grid((uint32_t)std::max<int64_t>(tiles, (int64_t)nq * (1 + groups)), (uint32_t)nq + 1);
    hipExtLaunchKernelGGL(k_score_dense_append, grid, dim3(256), 0, s, ev0, ev1, 0, c.k_idx, c.n_seq,
                          c.t_cap, c.msh, q_idx, q_pos, scores, ld, a, groups);
    return hipGetLastError();
}

hipError_t launch_score_cand(const CacheView& c, const uint16_t* q_idx, const int32_t* q_pos,
                             const int32_t* q_seq, int32_t nq, const int32_t* cand, int64_t n_cand,
                             float* scores, int64_t ld, hipStream_t s) {
    if (nq == 0 || n_cand == 0) return hipSuccess;
    dim3 grid((uint32_t)((n_cand + kScoreTile - 1) / kScoreTile), (uint32_t)nq);
    hipLaunchKernelGGL(k_score_cand, grid, dim3(256), 0, s, c.k_idx, c.n_seq, c.t_cap, c.msh, q_idx,
                       q_pos, q_seq, cand, n_cand, scores, ld);
    return hipGetLastError();
}

}  // namespace csa2

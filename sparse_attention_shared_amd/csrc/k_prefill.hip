// k_prefill.hip -- indexer top-k of a prefill chunk: many queries on one
// sequence, each at its own position, select their k best positions by
// q_I . k_I over the causal range ("CED: Continuing Context with a Causal
// Encoder and Decoder", section "Why Prefill Recomputes a Recent Segment",
// Fig. 6: the recent positions pass through the decoder again and each one
// selects as a decode query does, section "Selecting Positions and Reading
// Values with Attention", Fig. 4).
//
// The score matrix (queries x positions x 64 dims) is a dense contraction; it
// runs on v_mfma_f32_16x16x32_bf16 and is never written out.  Four launches:
//   1. cmax:   scores on MFMA over a sample -- every eighth 64-position step;
//              per query, the maximum key of every 16-position chunk of the
//              sample goes to the workspace.
//   2. thresh: per query, thr = the m-th largest sampled chunk maximum, m =
//              1.3 k / 8: about 1.3 k scores of the whole row reach it.
//   3. filter: all the scores on MFMA; positions with key >= thr are
//              appended, with their keys, to the query's candidate list.
//   4. select: per query, candidates are put in position order through an
//              LDS bitmap, then the exact (score desc, position asc) top-k is
//              taken and written ascending.  The list certifies itself: when
//              it holds at least k positions, the k-th best score is >= thr,
//              so every top-k position is on it.  A query with fewer (an
//              unlucky sample) or with more than the list holds (ties) is
//              resolved exactly by recomputing its scores.
#include <algorithm>

#include "csa2_dev.h"
#include "csa2_kernels.h"
#include "csa2_select.h"

namespace csa2 {

typedef __attribute__((ext_vector_type(8))) __bf16 pf_bf16x8;
typedef __attribute__((ext_vector_type(4))) float pf_f32x4;

constexpr int kPfQB = 4;        // 16-query blocks per wave
constexpr int kPfQ = 16 * kPfQB; // queries per workgroup tile (every wave takes all of them)
// 64 queries a tile keep the filter within 128 VGPRs and its LDS within a
// quarter of the CU's, so four of its workgroups (four waves per SIMD) share
// a CU: the latency of the candidate hand-offs is hidden by the other waves.
constexpr int kPfCStride = 512; // positions between sampled 64-position steps
constexpr int kPfCSteps = 4;    // sampled steps per chunk-maximum workgroup
constexpr int kPfFiltSpan = 4096;  // positions per filter workgroup
constexpr int kPfFiltSeg = 512;    // positions per LDS list flush (about 11 candidates per query)
constexpr int kPfChunk = 16;    // positions per chunk maximum
constexpr int kPfLB = 24;       // LDS candidate slots per query in the filter
constexpr int kPfSelNT = 512;

__device__ __forceinline__ int64_t pf_clamp_pos(int64_t p, int64_t t_cap) {
    return p < 0 ? -1 : (p >= t_cap ? t_cap - 1 : p);
}

// The last entry a query at position p may read: an entry of 2^msh positions
// counts once its whole group is at or before p (msh 0: the position itself);
// -1 for a negative position.  Every kernel below works on entries.
__device__ __forceinline__ int64_t pf_last_entry(int64_t p, int32_t msh) {
    return p < 0 ? -1 : ((p + 1) >> msh) - 1;
}

// Query fragments of the tile's kPfQ queries (B operand): lane column n16 of
// block i is query q0 + 16 i + n16, dims 32 kb + 8 g .. + 8.
__device__ __forceinline__ void pf_load_q(const uint16_t* __restrict__ q_idx, int32_t nq,
                                          int64_t q0, int n16, int g, pf_bf16x8 (&a)[kPfQB][2]) {
#pragma unroll
    for (int i = 0; i < kPfQB; ++i) {
        const int64_t qq = q0 + 16 * i + n16;
        // a query past nq repeats the last one; its scores are never used
        const uint4* row = reinterpret_cast<const uint4*>(q_idx + (qq < nq ? qq : nq - 1) * kIdxDim + 8 * g);
        a[i][0] = __builtin_bit_cast(pf_bf16x8, row[0]);
        a[i][1] = __builtin_bit_cast(pf_bf16x8, row[4]);
    }
}

// Key fragments of positions t0 .. t0 + 63 (A operand): lane row n16 of block
// j is position t0 + 16 j + n16.  Rows past t_cap repeat the last row: every
// query masks those positions, so no branch guards the loads.
__device__ __forceinline__ void pf_load_k(const uint16_t* __restrict__ kseq, int32_t t_cap,
                                          int32_t t0, int n16, int g, pf_bf16x8 (&b)[4][2]) {
    // byte offsets stay 32-bit (t_cap <= 2^24 rows of 128 B) over the
    // wave-uniform base
    const char* base = reinterpret_cast<const char*>(kseq);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t tt = (uint32_t)min(t0 + 16 * j + n16, t_cap - 1);
        const uint4* row = reinterpret_cast<const uint4*>(base + (tt * 128u + 16u * (uint32_t)g));
        b[j][0] = __builtin_bit_cast(pf_bf16x8, row[0]);
        b[j][1] = __builtin_bit_cast(pf_bf16x8, row[4]);
    }
}

// Scores of position block j against query block i: lane holds query
// q0 + 16 i + n16 at positions t0 + 16 j + 4 g + r, r = 0..3.  The cmax and
// filter kernels both call this, so their scores agree bit for bit.
__device__ __forceinline__ pf_f32x4 pf_tile(const pf_bf16x8 (&kf)[2], const pf_bf16x8 (&qf)[2]) {
    pf_f32x4 c = {0.f, 0.f, 0.f, 0.f};
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0], qf[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1], qf[1], c, 0, 0, 0);
    return c;
}

// Clamped position of the lane's query of each block (-1 past nq), and the
// largest and smallest of them over the tile (wave-uniform).  The loads are
// unconditional (index clamped to nq - 1), so all of them are in flight at once.
__device__ __forceinline__ void pf_tile_pos(const int32_t* __restrict__ q_pos, int32_t nq,
                                            int64_t t_cap, int32_t msh, int64_t q0, int n16,
                                            int32_t (&pos)[kPfQB], int32_t& tmax, int32_t& tmin) {
    int32_t raw[kPfQB];
#pragma unroll
    for (int i = 0; i < kPfQB; ++i) {
        const int64_t qq = q0 + 16 * i + n16;
        raw[i] = q_pos[qq < nq ? qq : nq - 1];
    }
    tmax = -1;
    tmin = INT32_MAX;
#pragma unroll
    for (int i = 0; i < kPfQB; ++i) {
        const int64_t qq = q0 + 16 * i + n16;
        pos[i] = qq < nq ? (int32_t)pf_clamp_pos(pf_last_entry(raw[i], msh), t_cap) : -1;
        tmax = max(tmax, pos[i]);
        tmin = min(tmin, pos[i]);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        tmax = max(tmax, __shfl_xor(tmax, o, 64));
        tmin = min(tmin, __shfl_xor(tmin, o, 64));
    }
    tmax = __builtin_amdgcn_readfirstlane(tmax);  // wave-uniform: scalar registers
    tmin = __builtin_amdgcn_readfirstlane(tmin);
}

// ---- 1. sampled chunk maxima -------------------------------------------
// A chunk is the 16 positions one lane holds for one query in a 64-position
// step: t0 + 16 j + 4 g + r (j, r = 0..3), so its maximum needs no
// cross-lane traffic.  Sampled chunk c holds a position <= t exactly when
// c < pf_nchunks(t).
template <bool MASK>
__device__ __forceinline__ void pf_cmax_step(const pf_bf16x8 (&kf)[4][2],
                                             const pf_bf16x8 (&qf)[kPfQB][2], int32_t t0, int g,
                                             const int32_t (&pos)[kPfQB], float (&m)[kPfQB]) {
    const float NEG = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        pf_f32x4 c[kPfQB];
#pragma unroll
        for (int i = 0; i < kPfQB; ++i) c[i] = pf_tile(kf[j], qf[i]);
        const int32_t tt = t0 + 16 * j + 4 * g;
#pragma unroll
        for (int i = 0; i < kPfQB; ++i) {
            if (MASK) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (tt + r > pos[i]) c[i][r] = NEG;
            }
            // chained from the running maximum (already canonical): two
            // v_max3_f32, no quieting of the MFMA results
            m[i] = fmaxf(fmaxf(m[i], c[i][0]), c[i][1]);
            m[i] = fmaxf(fmaxf(m[i], c[i][2]), c[i][3]);
        }
    }
}

// The cmax workgroup's four waves take different query tiles (4 x kPfQ
// queries) over the same sampled positions, so each 64-position key tile is
// loaded from global memory once and read by all four waves from LDS.  Rows are
// padded to 144 bytes: the 16 lanes of a lane group read 16 rows at one
// column, and the padding puts them in 16 different bank groups.
constexpr int kPfWQ = 4 * kPfQ;      // queries per cmax workgroup
constexpr int kPfTileRow = 36;       // LDS words per key row (128 B + 16 B)
constexpr int kPfTileWords = 64 * kPfTileRow;

// The two 16-byte pieces thread tid (of 256) loads of the key tile at t0:
// rows tid / 8 and 32 + tid / 8, dims 8 (tid % 8) .. + 8.  Rows past t_cap
// repeat the last row (masked by every query).
__device__ __forceinline__ void pf_tile_load(const uint16_t* __restrict__ kseq, int32_t t_cap,
                                             int32_t t0, int tid, uint4& r0, uint4& r1) {
    const int32_t ta = min(t0 + (tid >> 3), t_cap - 1), tb = min(t0 + 32 + (tid >> 3), t_cap - 1);
    r0 = *reinterpret_cast<const uint4*>(kseq + (int64_t)ta * kIdxDim + 8 * (tid & 7));
    r1 = *reinterpret_cast<const uint4*>(kseq + (int64_t)tb * kIdxDim + 8 * (tid & 7));
}

__device__ __forceinline__ void pf_tile_store(uint32_t* buf, int tid, const uint4& r0, const uint4& r1) {
    *reinterpret_cast<uint4*>(buf + (tid >> 3) * kPfTileRow + 4 * (tid & 7)) = r0;
    *reinterpret_cast<uint4*>(buf + (32 + (tid >> 3)) * kPfTileRow + 4 * (tid & 7)) = r1;
}

// Key fragments of the tile's position blocks (the layout pf_load_k gives).
__device__ __forceinline__ void pf_tile_frag(const uint32_t* buf, int n16, int g, pf_bf16x8 (&kf)[4][2]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t* row = buf + (16 * j + n16) * kPfTileRow;
        kf[j][0] = __builtin_bit_cast(pf_bf16x8, *reinterpret_cast<const uint4*>(row + 4 * g));
        kf[j][1] = __builtin_bit_cast(pf_bf16x8, *reinterpret_cast<const uint4*>(row + 16 + 4 * g));
    }
}

// grid (ceil(nq / kPfWQ), ceil(t_cap / (kPfCStride kPfCSteps))), 256 threads.
// Sampled step i starts at position kPfCStride i; its chunk g (of 4) is
// written to cmax[q][4 i + g] (ldc words per query).
__global__ __launch_bounds__(256) void k_pf_cmax(const uint16_t* __restrict__ kseq, int32_t t_cap,
                                                 const uint16_t* __restrict__ q_idx,
                                                 const int32_t* __restrict__ q_pos, int32_t nq,
                                                 int32_t msh, uint32_t* __restrict__ cmax,
                                                 int64_t ldc) {
    __shared__ uint32_t tile[2][kPfTileWords];
    __shared__ int32_t wmax[4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g = lane >> 4;
    const int64_t q0 = (int64_t)blockIdx.x * kPfWQ + wave * kPfQ;  // this wave's queries
    const int32_t span0 = (int32_t)blockIdx.y * (kPfCStride * kPfCSteps);
    int32_t tmax, tmin, pos[kPfQB];
    pf_tile_pos(q_pos, nq, t_cap, msh, min(q0, (int64_t)nq - 1), n16, pos, tmax, tmin);
    if (q0 >= nq) tmax = -1;  // a wave past the last query computes nothing
    if (lane == 0) wmax[wave] = tmax;
    __syncthreads();
    const int32_t T = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    if (span0 > T) return;  // uniform over the workgroup
    const int nsteps = min(kPfCSteps, (min(T, t_cap - 1) - span0) / kPfCStride + 1);
    pf_bf16x8 qf[kPfQB][2];
    pf_load_q(q_idx, nq, q0 < nq ? q0 : 0, n16, g, qf);
    const float NEG = -__builtin_inff();
    auto step = [&](const uint32_t* buf, int32_t t0) {
        if (t0 > tmax) return;  // wave-uniform
        pf_bf16x8 kf[4][2];
        pf_tile_frag(buf, n16, g, kf);
        float m[kPfQB];
#pragma unroll
        for (int i = 0; i < kPfQB; ++i) m[i] = NEG;
        if (t0 + 63 <= tmin)  // no query of the wave masks these positions
            pf_cmax_step<false>(kf, qf, t0, g, pos, m);
        else
            pf_cmax_step<true>(kf, qf, t0, g, pos, m);
        const int64_t c0 = 4 * (t0 / kPfCStride) + g;
#pragma unroll
        for (int i = 0; i < kPfQB; ++i) {
            const int64_t qq = q0 + 16 * i + n16;
            if (qq < nq) cmax[qq * ldc + c0] = score_key(m[i]);
        }
    };
    // tile s is read from LDS while tiles s + 1 and s + 2 wait in registers.
    // After a step its successor goes to the other buffer (whose readers
    // finished with it before the previous barrier) and the freed registers
    // request the tile three steps ahead.  Step 0 is peeled: it is where the
    // query fragments are first used, so inside the loop the only loads in
    // flight are tiles and the compiler's waits count only those.
    constexpr int D = kPfCStride;
    uint4 a0, a1, b0, b1, c0, c1;
    pf_tile_load(kseq, t_cap, span0, tid, a0, a1);
    pf_tile_load(kseq, t_cap, span0 + D, tid, b0, b1);
    pf_tile_load(kseq, t_cap, span0 + 2 * D, tid, c0, c1);
    pf_tile_store(tile[0], tid, a0, a1);
    lds_barrier();
    step(tile[0], span0);
    pf_tile_store(tile[1], tid, b0, b1);                    // tile 1
    pf_tile_load(kseq, t_cap, span0 + 3 * D, tid, b0, b1);  // tile 3
    lds_barrier();
    for (int s = 1; s < nsteps; s += 2) {  // tile[1] holds tile s, c tile s + 1, b tile s + 2
        const int32_t t0 = span0 + D * s;
        step(tile[1], t0);
        pf_tile_store(tile[0], tid, c0, c1);                  // tile s + 1
        pf_tile_load(kseq, t_cap, t0 + 3 * D, tid, c0, c1);  // tile s + 3
        lds_barrier();
        if (s + 1 >= nsteps) break;
        step(tile[0], t0 + D);
        pf_tile_store(tile[1], tid, b0, b1);                  // tile s + 2
        pf_tile_load(kseq, t_cap, t0 + 4 * D, tid, b0, b1);  // tile s + 4
        lds_barrier();
    }
}

// Sampled chunks holding at least one position <= t: step i (positions
// kPfCStride i ..) has chunk g's first position at kPfCStride i + 4 g.
__device__ __forceinline__ int64_t pf_nchunks(int64_t t) {
    if (t < 0) return 0;
    const int64_t g = (t % kPfCStride) >> 2;
    return 4 * (t / kPfCStride) + (g < 3 ? g : 3) + 1;
}

// Sampled chunk maxima whose m-th largest is the threshold: about 1.3 k
// scores of the row reach it (the sample is 1/8 of the positions and a
// chunk's maximum stands for one score), so a list shorter than k -- which
// sends the query to the exact recompute -- is a rare event for scores
// without structure.
__device__ __forceinline__ int32_t pf_sample_rank(int32_t k) {
    return (13 * k + 79) / 80;
}

// ---- 2. thresholds -----------------------------------------------------------
// key -> the float with that key (keys below that of -inf give a NaN, which
// lets every score through the float pre-filter of the filter kernel).
__device__ __forceinline__ float key_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

struct PfThrLds {
    alignas(16) int hist[kHistWords];
    int res[4];
};

// grid nq, 256 threads, dynamic LDS ldc keys.
__global__ __launch_bounds__(256) void k_pf_thresh(const uint32_t* __restrict__ cmax, int64_t ldc,
                                                   const int32_t* __restrict__ q_pos,
                                                   int32_t msh, int64_t t_cap, int32_t k,
                                                   float* __restrict__ thr_f,
                                                   uint32_t* __restrict__ thr_k,
                                                   uint32_t* __restrict__ cnt) {
    extern __shared__ uint32_t pf_keys[];
    __shared__ PfThrLds sh;
    const int q = blockIdx.x, tid = threadIdx.x;
    const int64_t t = pf_clamp_pos(pf_last_entry(q_pos[q], msh), t_cap);
    const int64_t nc = pf_nchunks(t);
    const int32_t m = pf_sample_rank(k);
    uint32_t thr = 1u;  // fewer sampled chunks than m: every valid position is a candidate
    if (nc >= m) {
        // ldc is a multiple of 4 and the row is 16-byte aligned: stage whole
        // uint4s (keys past nc are never read), eight loads in flight per thread
        const uint4* src = reinterpret_cast<const uint4*>(cmax + (int64_t)q * ldc);
        uint4* dst = reinterpret_cast<uint4*>(pf_keys);
        const int nv = (int)((nc + 3) / 4);
        for (int i0 = tid; i0 < nv; i0 += 8 * 256) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = (i0 + u * 256 < nv) ? src[i0 + u * 256] : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (i0 + u * 256 < nv) dst[i0 + u * 256] = v[u];
        }
        __syncthreads();
        uint32_t tau;
        int need;
        lds_kth<256>(pf_keys, (int)nc, m, 0, sh.hist, sh.res, tau, need);
        thr = need > 0 ? tau : tau + 1u;
        if (thr < 1u) thr = 1u;
    }
    if (tid == 0) {
        thr_k[q] = thr;
        thr_f[q] = key_float(thr);
        cnt[q] = 0u;
    }
}

// ---- 3. filter ---------------------------------------------------------------
// Pre-filter granularity: a lane's four scores of one tile (one query, four
// consecutive positions) are queued together when any of them passes, so one
// wave-wide compaction (a ballot) serves four compares.
constexpr int kPfQueue = kPfQB * 64 + 64;  // per-wave queue: one tile row's entries at most, plus < 64 left by a drain
constexpr int kPfFiltMinWaves = kPfQB <= 4 ? 4 : (kPfQB <= 6 ? 3 : 2);  // per SIMD (VGPR budget)

constexpr int kPfCopyT = 256 / kPfQ;  // threads copying one query's list at a flush
static_assert(kPfCopyT * kPfQ == 256 && kPfLB % kPfCopyT == 0, "the list copy splits evenly");

struct PfFiltLds {
    uint2 buf[kPfQ][kPfLB];          // per-query candidates of this workgroup
    uint4 qscore[4][kPfQueue];       // per-wave queue: the four scores of an entry
    uint32_t qtag[4][kPfQueue];      // and (first position << 7 | query in tile)
    int n[kPfQ];
    int base[kPfQ];
    int32_t pos[kPfQ];
    float thf[kPfQ];
};

// Exact test of the first `count` queued entries (causal mask, key >= thr);
// the scores that pass go to their query's list.
__device__ __forceinline__ void pf_drain(PfFiltLds& sh, int wave, int lane, int count,
                                         int64_t q0, uint32_t* __restrict__ cnt,
                                         uint2* __restrict__ cand, int32_t cap) {
    for (int e = lane; e < count; e += 64) {
        const uint4 sc = sh.qscore[wave][e];
        const uint32_t tag = sh.qtag[wave][e];
        const int ql = (int)(tag & 127u);
        const int32_t t0 = (int32_t)(tag >> 7);
        const int32_t lim = sh.pos[ql];
        // key(s) >= thr is s >= key_float(thr) for every score that is not a
        // NaN (the keys order scores as floats do, -0 and +0 alike)
        const float thf = sh.thf[ql];
        const float v[4] = {__uint_as_float(sc.x), __uint_as_float(sc.y), __uint_as_float(sc.z),
                            __uint_as_float(sc.w)};
        uint32_t okm = 0u;
#pragma unroll
        for (int r = 0; r < 4; ++r) okm |= (uint32_t)(t0 + r <= lim && v[r] >= thf) << r;
        if (okm == 0u) continue;
        // one list reservation for all of the entry's passing positions, then
        // one pass per passing position (most entries have one)
        int slot = atomicAdd(&sh.n[ql], __popc(okm));
        do {
            const int r = __builtin_ctz(okm);
            okm &= okm - 1u;
            const float vr = r == 0 ? v[0] : (r == 1 ? v[1] : (r == 2 ? v[2] : v[3]));
            const uint2 ent = make_uint2((uint32_t)(t0 + r), score_key(vr));
            if (slot < kPfLB) {
                sh.buf[ql][slot] = ent;
            } else {  // this workgroup's list of the query is full: straight to its global list
                const uint32_t gs = atomicAdd(&cnt[q0 + ql], 1u);
                if (gs < (uint32_t)cap) cand[(q0 + ql) * cap + gs] = ent;
            }
            ++slot;
        } while (okm != 0u);
    }
}

// grid (ceil(nq / kPfQ), ceil(t_cap / kPfFiltSpan)), 256 threads.  cand: [nq][cap]
// (position, key); cnt: [nq].
__global__ __launch_bounds__(256, kPfFiltMinWaves) void k_pf_filter(const uint16_t* __restrict__ kseq, int32_t t_cap,
                                                   const uint16_t* __restrict__ q_idx,
                                                   const int32_t* __restrict__ q_pos, int32_t nq,
                                                   int32_t msh, const float* __restrict__ thr_f,
                                                   uint32_t* __restrict__ cnt,
                                                   uint2* __restrict__ cand, int32_t cap) {
    __shared__ PfFiltLds sh;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g = lane >> 4;
    const int64_t q0 = (int64_t)blockIdx.x * kPfQ;
    const int32_t span0 = (int32_t)blockIdx.y * kPfFiltSpan;
    int32_t tmax, tmin, pos[kPfQB];
    pf_tile_pos(q_pos, nq, t_cap, msh, q0, n16, pos, tmax, tmin);
    if (span0 > tmax) return;  // uniform over the workgroup
    if (tid < kPfQ) {
        const int64_t qq = q0 + tid;
        sh.pos[tid] = qq < nq ? (int32_t)pf_clamp_pos(pf_last_entry(q_pos[qq], msh), t_cap) : -1;
        sh.thf[tid] = qq < nq ? thr_f[qq] : __builtin_inff();
        sh.n[tid] = 0;
    }
    float th[kPfQB];
#pragma unroll
    for (int i = 0; i < kPfQB; ++i) {
        const int64_t qq = q0 + 16 * i + n16;
        const float tv = thr_f[qq < nq ? qq : nq - 1];
        th[i] = qq < nq ? tv : __builtin_inff();
    }
    pf_bf16x8 qf[kPfQB][2];
    pf_load_q(q_idx, nq, q0, n16, g, qf);
    __syncthreads();
    // One pass over the span, the next step's key fragments in flight while
    // a step computes.  Every kPfFiltSeg positions (two steps of the four
    // waves) the per-query LDS lists go to the global lists, so their
    // capacity covers a segment while the workgroup's set-up covers the whole
    // span.  Every wave runs the same number of steps (the barriers of the
    // flush), computing only the steps that hold a position <= tmax.
    constexpr int kSegSteps = kPfFiltSeg / 256;
    const int nsteps = min(kPfFiltSpan / 256, (min(tmax, t_cap - 1) - span0) / 256 + 1);
    // the wave's queue holds qn entries from slot 0 (wave-uniform); drains
    // take whole batches of 64, one entry a lane, and move the rest to the front
    int qn = 0;
    pf_bf16x8 kn[4][2];
    pf_load_k(kseq, t_cap, span0 + wave * 64, n16, g, kn);
    for (int s = 0; s < nsteps; ++s) {
        const int32_t t0 = span0 + wave * 64 + 256 * s;
        pf_bf16x8 kf[4][2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            kf[j][0] = kn[j][0];
            kf[j][1] = kn[j][1];
        }
        pf_load_k(kseq, t_cap, t0 + 256, n16, g, kn);  // rows clamped: always in bounds
        if (t0 <= tmax && t0 < t_cap) {                 // wave-uniform
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pf_f32x4 c[kPfQB];
#pragma unroll
                for (int i = 0; i < kPfQB; ++i) c[i] = pf_tile(kf[j], qf[i]);
                const uint32_t tag = (((uint32_t)t0 + 16u * j + 4u * g) << 7) | (uint32_t)n16;
                // float pre-filter (passes every finite key >= thr: the largest
                // of the four scores against the threshold's float), one query
                // block at a time: a ballot of the passing lanes, and each
                // passing lane's queue slot is qn + the number of passing
                // lanes below it (qn < 64 before the first block, so every
                // slot is below kPfQueue)
#pragma unroll
                for (int i = 0; i < kPfQB; ++i) {
                    // max3 chains from a canonical value (no canonicalising
                    // of the MFMA results)
                    float mx = fmaxf(fmaxf(-__builtin_inff(), c[i][0]), c[i][1]);
                    mx = fmaxf(fmaxf(mx, c[i][2]), c[i][3]);
                    const bool pass = mx >= th[i];
                    const uint64_t pm = __ballot(pass);
                    if (pm != 0ull) {  // wave-uniform
                        if (pass) {
                            const int below = (int)__builtin_amdgcn_mbcnt_hi(
                                (uint32_t)(pm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)pm, 0u));
                            const int r = qn + below;
                            sh.qscore[wave][r] =
                                make_uint4(__float_as_uint(c[i][0]), __float_as_uint(c[i][1]),
                                           __float_as_uint(c[i][2]), __float_as_uint(c[i][3]));
                            sh.qtag[wave][r] = tag + 16u * i;
                        }
                        qn += (int)__popcll(pm);
                    }
                }
                if (qn >= 64) {  // whole batches; fewer than 64 entries stay, so
                                 // the next tile row's (at most kPfQB * 64) still fit
                    const int nb = qn & ~63;
                    pf_drain(sh, wave, lane, nb, q0, cnt, cand, cap);
                    qn -= nb;
                    // the rest to the front: lane l reads slot nb + l and
                    // writes slot l, which only lane l read in the drain (the
                    // wave's LDS accesses complete in order)
                    if (lane < qn) {
                        const uint4 a = sh.qscore[wave][nb + lane];
                        const uint32_t tg = sh.qtag[wave][nb + lane];
                        sh.qscore[wave][lane] = a;
                        sh.qtag[wave][lane] = tg;
                    }
                }
            }
        }
        if (s % kSegSteps == kSegSteps - 1 || s == nsteps - 1) {  // uniform: flush the lists
            // the barriers order LDS only (lds_barrier): the next step's key
            // fragments stay in flight, and the list stores to global memory
            // need no order within the launch.  Queued entries wait for the
            // next segment's lists, except at the end of the span.
            if (s == nsteps - 1) {
                pf_drain(sh, wave, lane, qn, q0, cnt, cand, cap);
                qn = 0;
            }
            lds_barrier();
            if (tid < kPfQ) {
                const int m = min(sh.n[tid], kPfLB);
                // the tile's counters through a uniform base (scalar registers)
                uint32_t* cq = cnt + __builtin_amdgcn_readfirstlane((int)q0);
                sh.base[tid] = m > 0 ? (int)atomicAdd(cq + tid, (uint32_t)m) : 0;
            }
            lds_barrier();
            {  // kPfCopyT threads a query, slots tid % kPfCopyT + kPfCopyT u
                const int ql = tid / kPfCopyT;
                const int m = min(sh.n[ql], kPfLB), b = sh.base[ql];
#pragma unroll
                for (int u = 0; u < kPfLB / kPfCopyT; ++u) {
                    const int j = tid % kPfCopyT + kPfCopyT * u;
                    if (j < m && b + j < cap) cand[(q0 + ql) * cap + b + j] = sh.buf[ql][j];
                }
            }
            lds_barrier();
            if (tid < kPfQ) sh.n[tid] = 0;
            lds_barrier();
        }
    }
}

// ---- 4. select ---------------------------------------------------------------
// Per query: the candidates' keys stay in registers for the exact radix
// select of (tau, need); then two bitmaps over the query's positions put the
// chosen ones in order -- A marks keys above tau, B keys equal to it, of
// which the `need` lowest positions are taken -- and one scan over the words
// writes them ascending.  The radix histogram and the bitmaps share the
// dynamic LDS (the histogram is dead once tau is known).
struct PfSelLds {
    alignas(16) uint32_t small[64];
    int tmp[2 * (kPfSelNT / 64 + 1)];
    int wtmp[2 * kPfSelNT / 64];
    int res[8];
};

// Exact top-k of one query by recomputing its scores (VALU dot products): the
// path of a query whose candidate list overflowed.
__device__ void pf_select_recompute(const uint16_t* __restrict__ kseq, const uint16_t* __restrict__ qr,
                                    int64_t t, int32_t k, int32_t* __restrict__ dst, int* hist,
                                    PfSelLds& sh) {
    // the query stays packed (two bf16 a word): half the registers of fp32,
    // the same products
    uint32_t qw[kIdxDim / 2];
#pragma unroll
    for (int d = 0; d < kIdxDim; d += 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(qr + d);
        qw[d / 2 + 0] = v.x;
        qw[d / 2 + 1] = v.y;
        qw[d / 2 + 2] = v.z;
        qw[d / 2 + 3] = v.w;
    }
    auto K = [&](int64_t i) -> uint32_t {
        if (i > t) return 0u;
        const uint4* row = reinterpret_cast<const uint4*>(kseq + i * kIdxDim);
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const uint4 v = row[w];
            const uint32_t kw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                s = fmaf(bf16_lo(qw[4 * w + h]), bf16_lo(kw[h]), s);
                s = fmaf(bf16_hi(qw[4 * w + h]), bf16_hi(kw[h]), s);
            }
        }
        return score_key(s);
    };
    uint32_t tau;
    int need;
    kth_fn<kPfSelNT>(K, t + 1, k, 0, 0u, hist, sh.res, tau, need);
    ordered_write<kPfSelNT>(K, t + 1, tau, need, nullptr, k, dst, sh.wtmp);
}

// Dynamic LDS of k_pf_select: the radix histogram or the two bitmaps.
size_t pf_select_lds_bytes(int64_t t_cap) {
    const size_t nw = (size_t)((t_cap + 31) / 32);
    return std::max((size_t)kHistWords, 2 * nw) * sizeof(uint32_t);
}

// grid nq, 512 threads, dynamic LDS pf_select_lds_bytes(t_cap).
__global__ __launch_bounds__(kPfSelNT, 6) void k_pf_select(const uint16_t* __restrict__ kseq,
                                                        int64_t t_cap,
                                                        const uint16_t* __restrict__ q_idx,
                                                        const int32_t* __restrict__ q_pos,
                                                        int32_t msh, int32_t k,
                                                        const uint32_t* __restrict__ cnt,
                                                        const uint2* __restrict__ cand, int32_t cap,
                                                        int32_t* __restrict__ sel) {
    extern __shared__ uint32_t pf_dyn[];
    __shared__ PfSelLds sh;
    int* hist = reinterpret_cast<int*>(pf_dyn);
    const int q = blockIdx.x, tid = threadIdx.x;
    int32_t* dst = sel + (int64_t)q * k;
    const int64_t t = pf_clamp_pos(pf_last_entry(q_pos[q], msh), t_cap);
    if (t < 0) {
        for (int i = tid; i < k; i += kPfSelNT) dst[i] = -1;
        return;
    }
    const uint32_t n = cnt[q];
    // too many candidates for the list, or too few to certify the selection
    if (n > (uint32_t)cap || ((int64_t)n < k && (int64_t)n < t + 1)) {
        pf_select_recompute(kseq, q_idx + (int64_t)q * kIdxDim, t, k, dst, hist, sh);
        return;
    }
    constexpr int PER = kPfCap / kPfSelNT;
    uint2 cv[PER];
    const uint2* src = cand + (int64_t)q * cap;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int i = tid + u * kPfSelNT;
        cv[u] = i < (int)n ? src[i] : make_uint2(0xFFFFFFFFu, 0u);
    }
    // every candidate is at or above the threshold, so their keys share
    // their top bits; the radix works on the bits below that common prefix
    // (shifted up; the set low bit keeps every key nonzero and the order
    // unchanged; with no common bit the keys stay as they are, never 0),
    // so its first digit spreads over the whole histogram
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int u = 0; u < PER; ++u)
        if (cv[u].x != 0xFFFFFFFFu) {
            kmin = min(kmin, cv[u].y);
            kmax = max(kmax, cv[u].y);
        }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
    }
    if ((tid & 63) == 0) {
        sh.wtmp[tid >> 6] = (int)kmin;
        sh.wtmp[kPfSelNT / 64 + (tid >> 6)] = (int)kmax;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kPfSelNT / 64; ++w) {
        kmin = min(kmin, (uint32_t)sh.wtmp[w]);
        kmax = max(kmax, (uint32_t)sh.wtmp[kPfSelNT / 64 + w]);
    }
    const int sp = kmin <= kmax ? min(31, __clz((int)(kmin ^ kmax))) : 0;
    uint32_t kv[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) kv[u] = cv[u].x != 0xFFFFFFFFu ? (sp ? (cv[u].y << sp) | 1u : cv[u].y) : 0u;
    uint32_t tau;
    int need;
    kth_regs<kPfSelNT, PER>(kv, k, hist, sh.res, sh.small, tau, need);
    // bitmap A (positions 0..t) of the chosen keys takes the histogram's
    // place; aux holds the keys equal to tau (ties, taken lowest position
    // first), then A's word prefixes
    const int nw = (int)(t / 32 + 1);
    uint32_t* bma = pf_dyn;
    uint32_t* aux = pf_dyn + nw;
    for (int w = tid; w < (need > 0 ? 2 * nw : nw); w += kPfSelNT) pf_dyn[w] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const uint32_t p = cv[u].x;  // a candidate's position is <= t
        if (kv[u] > tau)
            atomicOr(&bma[p >> 5], 1u << (p & 31));
        else if (need > 0 && kv[u] == tau && kv[u] != 0u)
            atomicOr(&aux[p >> 5], 1u << (p & 31));
    }
    __syncthreads();
    // contiguous words per thread, so one scan orders them
    const int wpt = (nw + kPfSelNT - 1) / kPfSelNT;
    const int w0 = min(nw, tid * wpt), w1 = min(nw, w0 + wpt);
    if (need > 0) {  // uniform: the `need` lowest tied positions join A
        int cb = 0;
        for (int w = w0; w < w1; ++w) cb += __popc(aux[w]);
        int tb;
        int eq = block_excl_scan<kPfSelNT>(cb, sh.tmp, &tb);
        for (int w = w0; w < w1 && eq < need; ++w) {
            uint32_t e = aux[w], m = bma[w];
            while (e != 0u && eq < need) {
                const uint32_t low = e & (0u - e);
                m |= low;
                e ^= low;
                ++eq;
            }
            bma[w] = m;
        }
        __syncthreads();
    }
    int ca = 0;
    for (int w = w0; w < w1; ++w) ca += __popc(bma[w]);
    int chosen;
    int run = block_excl_scan<kPfSelNT>(ca, sh.tmp, &chosen);
    for (int w = w0; w < w1; ++w) {  // aux: chosen positions before word w
        const uint32_t m = bma[w];
        aux[w] = (uint32_t)run;
        run += __popc(m);
    }
    __syncthreads();
    // each chosen candidate's place is its rank among the chosen positions
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const uint32_t p = cv[u].x;
        if (kv[u] > tau || (need > 0 && kv[u] == tau && kv[u] != 0u)) {
            const uint32_t m = bma[p >> 5];
            if ((m >> (p & 31)) & 1u) {
                const int rank = (int)aux[p >> 5] + __popc(m & ((1u << (p & 31)) - 1u));
                if (rank < k) dst[rank] = (int32_t)p;
            }
        }
    }
    for (int i = min(chosen, k) + tid; i < k; i += kPfSelNT) dst[i] = -1;
}

// Multi-query scores of a prefill chunk on one sequence: S = Q_I K_I^T, a
// dense contraction (queries x positions x 64), on v_mfma_f32_16x16x32_bf16.
// Both operands come straight from global memory in MFMA layout: lane l holds
// 8 consecutive dims of query row l%16 (A) or of key l%16 (B), so every load
// is 16 contiguous bytes.  Workgroup tile: 64 queries x 256 positions; wave w
// takes positions [64w, 64w + 64).  Positions after a query are -inf.
__global__ __launch_bounds__(256) void k_score_mq(const uint16_t* __restrict__ kseq, int64_t t_cap,
                                                  const uint16_t* __restrict__ q_idx,
                                                  const int32_t* __restrict__ q_pos, int32_t nq,
                                                  int32_t msh, float* __restrict__ scores,
                                                  int64_t ld) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n16 = lane & 15, g = lane >> 4;
    const int64_t q0 = (int64_t)blockIdx.y * 64;
    const int64_t t0 = (int64_t)blockIdx.x * 256 + wave * 64;
    if (t0 >= t_cap) return;
    // the largest position any query of the tile may read
    int64_t tmax = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t qq = q0 + 16 * i + n16;
        const int64_t p = qq < nq ? pf_last_entry(q_pos[qq], msh) : -1;
        tmax = p > tmax ? p : tmax;
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        const int64_t other = __shfl_xor(tmax, o, 64);
        tmax = other > tmax ? other : tmax;
    }
    const float NEG = -__builtin_inff();
    if (t0 > tmax) {  // every position of this wave is after every query: masked
        for (int i = 0; i < 64; ++i) {
            const int64_t qq = q0 + i;
            if (qq < nq && t0 + lane < t_cap) scores[qq * ld + t0 + lane] = NEG;
        }
        return;
    }
    pf_bf16x8 a[4][2], b[4][2];
    int32_t pos[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t qq = q0 + 16 * i + n16;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (qq < nq) v = *reinterpret_cast<const uint4*>(q_idx + qq * kIdxDim + 32 * kb + 8 * g);
            a[i][kb] = __builtin_bit_cast(pf_bf16x8, v);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t qr = q0 + 16 * i + 4 * g + r;
            pos[i][r] = qr < nq ? (int32_t)pf_last_entry(q_pos[qr], msh) : -1;
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t tt = t0 + 16 * j + n16;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (tt < t_cap) v = *reinterpret_cast<const uint4*>(kseq + tt * kIdxDim + 32 * kb + 8 * g);
            b[j][kb] = __builtin_bit_cast(pf_bf16x8, v);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pf_f32x4 c = {0.f, 0.f, 0.f, 0.f};
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][0], b[j][0], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][1], b[j][1], c, 0, 0, 0);
            // lane holds position t0 + 16j + n16 for queries q0 + 16i + 4g + r
            const int64_t tt = t0 + 16 * j + n16;
            if (tt < t_cap) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t qr = q0 + 16 * i + 4 * g + r;
                    if (qr < nq) scores[qr * ld + tt] = (tt <= pos[i][r]) ? c[r] : NEG;
                }
            }
        }
}

hipError_t launch_score_mq(const CacheView& c, int32_t seq, const uint16_t* q_idx,
                           const int32_t* q_pos, int32_t nq, float* scores, int64_t ld,
                           hipStream_t s) {
    if (nq == 0) return hipSuccess;
    const uint16_t* kseq = c.k_idx + (int64_t)seq * c.t_cap * kIdxDim;
    dim3 grid((uint32_t)((c.t_cap + 255) / 256), (uint32_t)((nq + 63) / 64));
    hipLaunchKernelGGL(k_score_mq, grid, dim3(256), 0, s, kseq, c.t_cap, q_idx, q_pos, nq, c.msh,
                       scores, ld);
    return hipGetLastError();
}

size_t prefill_topk_ws_bytes(int32_t nq, int64_t t_cap) {
    const int64_t ldc = 4 * ((t_cap + kPfCStride - 1) / kPfCStride);
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    return al((size_t)nq * ldc * 4) + 3 * al((size_t)nq * 4) + al((size_t)nq * kPfCap * 8);
}

hipError_t launch_prefill_topk(const CacheView& c, int32_t seq, const uint16_t* q_idx,
                               const int32_t* q_pos, int32_t nq, int32_t k, int32_t* sel, void* ws,
                               hipStream_t s) {
    if (nq == 0) return hipSuccess;
    const int64_t ldc = 4 * ((c.t_cap + kPfCStride - 1) / kPfCStride);
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    char* p = static_cast<char*>(ws);
    uint32_t* cmax = reinterpret_cast<uint32_t*>(p);
    p += al((size_t)nq * ldc * 4);
    float* thr_f = reinterpret_cast<float*>(p);
    p += al((size_t)nq * 4);
    uint32_t* thr_k = reinterpret_cast<uint32_t*>(p);
    p += al((size_t)nq * 4);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(p);
    p += al((size_t)nq * 4);
    uint2* cand = reinterpret_cast<uint2*>(p);
    const uint16_t* kseq = c.k_idx + (int64_t)seq * c.t_cap * kIdxDim;
    const dim3 grid((uint32_t)((nq + kPfWQ - 1) / kPfWQ),
                    (uint32_t)((c.t_cap + kPfCStride * kPfCSteps - 1) / (kPfCStride * kPfCSteps)));
    hipLaunchKernelGGL(k_pf_cmax, grid, dim3(256), 0, s, kseq, (int32_t)c.t_cap, q_idx, q_pos, nq, c.msh,
                       cmax, ldc);
    hipLaunchKernelGGL(k_pf_thresh, dim3(nq), dim3(256), (size_t)ldc * 4, s, cmax, ldc, q_pos,
                       c.msh, c.t_cap, k, thr_f, thr_k, cnt);
    const dim3 fgrid((uint32_t)((nq + kPfQ - 1) / kPfQ), (uint32_t)((c.t_cap + kPfFiltSpan - 1) / kPfFiltSpan));
    hipLaunchKernelGGL(k_pf_filter, fgrid, dim3(256), 0, s, kseq, (int32_t)c.t_cap, q_idx, q_pos, nq, c.msh,
                       thr_f, cnt, cand, kPfCap);
    hipLaunchKernelGGL(k_pf_select, dim3(nq), dim3(kPfSelNT), pf_select_lds_bytes(c.t_cap), s, kseq, c.t_cap,
                       q_idx, q_pos, c.msh, k, cnt, cand, kPfCap, sel);
    return hipGetLastError();
}

}  // namespace csa2

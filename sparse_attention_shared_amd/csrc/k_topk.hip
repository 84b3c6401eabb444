// k_topk.hip -- top-k selection of indexer scores ("CED: Continuing Context with
// a Causal Encoder and Decoder", section "Selecting Positions and Reading
// Values with Attention", Fig. 4: the indexer keeps the positions with the
// highest scores), with the Full layer's wider candidate pool taken from the
// same ranking (section "What Full, Reindex, and Reuse Share", Fig. 5).
//
// Order: higher score first, equal scores by lower slot.  Scores become
// order-preserving 32-bit keys (key 0 = not selectable).  A selection is the
// pair (tau, need): every key > tau is chosen, plus the first `need` keys equal
// to tau in slot order; an ordered compaction then writes the chosen slots
// ascending.  tau is found by an exact radix select on 12 + 12 + 8 bit digits
// that stops as soon as a whole bucket is taken.
//
// Short rows (<= 32768 slots): one 1024-thread workgroup per row, keys in LDS.
// Long rows: three multi-workgroup kernels per row set --
//   hist:  12-bit histogram of the top digit (LDS, then device atomics); the
//          last workgroup of a row picks the boundary bucket of each target;
//   cand:  every chunk counts its keys above the bucket and appends the keys of
//          the bucket to a small candidate list; the last workgroup resolves
//          (tau, need) exactly on the candidates and turns per-chunk counts
//          into output offsets;
//   write: each chunk writes its chosen slots at its offset, in order.
// The workspace's counters and histogram reset themselves, so it must be
// zero-filled before its first use and is left zero-filled by every call.
#include "csa2_dev.h"
#include "csa2_kernels.h"
#include "csa2_select.h"

namespace csa2 {

constexpr int kSmallNT = 1024;
constexpr int kSmallMax = 32768;  // slots kept in LDS by the one-workgroup path
constexpr int kLongNT = 1024;
constexpr int kChunk = 8192;      // slots per workgroup on the long path
constexpr int kCandCap = 4096;    // candidates per row and target
constexpr int kMaxTargets = 2;

// ---------------------------------------------------------------- short rows
template <bool IDS, int PER>
__global__ __launch_bounds__(kSmallNT) void k_topk_small(const float* __restrict__ scores,
                                                         int64_t n, int64_t ld,
                                                         const int32_t* __restrict__ ids,
                                                         int32_t k, int32_t* __restrict__ out,
                                                         int32_t k2, int32_t* __restrict__ out2) {
    __shared__ RegSelShared<kSmallNT> sh;
    const int64_t row = blockIdx.x;
    const float* s = scores + row * ld;
    const int32_t* irow = IDS ? ids + row * n : nullptr;
#pragma unroll 1
    for (int t = 0; t < (out2 ? 2 : 1); ++t) {
        if (t) __syncthreads();
        const int32_t kk = t ? k2 : k;
        int32_t* dst = t ? out2 + row * k2 : out + row * k;
        reg_select<kSmallNT, PER, IDS>(s, irow, (int)n, kk, dst, sh);
    }
}

// ----------------------------------------------------------------- long rows
// Per-row workspace of the long path.
struct RowState {
    uint32_t hist[kHistBins];
    uint32_t ctr_hist, ctr_cand;
    uint32_t bucket[kMaxTargets];  // top digit of the boundary bucket
    int32_t rem[kMaxTargets];      // rank still needed inside that bucket
    uint32_t ncand[kMaxTargets];
    uint32_t tau[kMaxTargets];
    int32_t need[kMaxTargets];
    int32_t total[kMaxTargets];
    int32_t pad[2];
};
struct Cand {
    uint32_t key;
    int32_t slot;
};
// chunk records: [row][target][chunk] {above-bucket count, output offset, tau-equal keys before}
struct ChunkRec {
    int32_t gt, off, eq_before, pad;
};

struct LongWs {
    RowState* st;   // [nq]
    Cand* cand;     // [nq][targets][kCandCap]
    ChunkRec* rec;  // [nq][targets][n_chunk]
};

__device__ __forceinline__ int64_t chunk_begin(int c) { return (int64_t)c * kChunk; }

// grid (n_chunk, nq)
__global__ __launch_bounds__(kLongNT) void k_topk_hist(const float* __restrict__ scores, int64_t n,
                                                       int64_t ld, const int32_t* __restrict__ ids,
                                                       int32_t k, int32_t k2, LongWs ws) {
    __shared__ alignas(16) int hist[kHistWords];
    __shared__ int res[4];
    __shared__ int last;
    const int c = blockIdx.x, nc = gridDim.x;
    const int64_t row = blockIdx.y;
    const int tid = threadIdx.x;
    const float* s = scores + row * ld;
    const int32_t* irow = ids ? ids + row * n : nullptr;
    RowState* st = ws.st + row;
    for (int i = tid; i < kHistWords; i += kLongNT) hist[i] = 0;
    __syncthreads();
    constexpr int kPer = kChunk / kLongNT;
    const int64_t b0 = chunk_begin(c);
    uint32_t kr[kPer];
    load_keys<kPer, kLongNT>(s, irow, n, b0 + tid, kr);
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        if (kr[j]) atomicAdd(&hist[hidx((int)(kr[j] >> 20))], 1);
    __syncthreads();
    for (int i = tid; i < kHistBins; i += kLongNT) {
        const int v = hist[hidx(i)];
        if (v) atomicAdd(&st->hist[i], (uint32_t)v);
    }
    __syncthreads();  // the workgroup's stores are ordered before thread 0's release
    if (tid == 0) last = arrive_last(&st->ctr_hist, (uint32_t)nc);
    __syncthreads();  // thread 0's acquire covers the workgroup
    if (!last) return;
    // the last workgroup of the row: boundary bucket of each target
    {
        constexpr int kB = kHistBins / kLongNT;
        uint32_t hv[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u)
            hv[u] = __hip_atomic_load(&st->hist[tid + u * kLongNT], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            hist[hidx(tid + u * kLongNT)] = (int)hv[u];
            st->hist[tid + u * kLongNT] = 0u;
        }
    }
    __syncthreads();
    for (int t = 0; t < kMaxTargets; ++t) {
        const int kk = t ? k2 : k;
        if (kk <= 0) continue;
        if (tid < 64) wave_find_bucket(hist, kHistBins, kk, res);
        __syncthreads();
        if (tid == 0) {
            if (res[3] <= kk) {  // every selectable key is taken
                st->bucket[t] = 0u;
                st->rem[t] = -1;
            } else {
                st->bucket[t] = (uint32_t)res[0];
                st->rem[t] = kk - res[1];
            }
        }
        __syncthreads();
    }
    if (tid == 0) st->ctr_hist = 0u;
}

// grid (n_chunk, nq)
__global__ __launch_bounds__(kLongNT) void k_topk_cand(const float* __restrict__ scores, int64_t n,
                                                       int64_t ld, const int32_t* __restrict__ ids,
                                                       int32_t k, int32_t k2, LongWs ws) {
    __shared__ uint32_t ckeys[kCandCap];
    __shared__ int32_t cslot[kCandCap];
    __shared__ alignas(16) int hist[kHistWords];
    __shared__ int tmp[kLongNT / 64 + 1];
    __shared__ int res[4];
    __shared__ int cnt_gt[kMaxTargets], cnt_cand[kMaxTargets], cbase[kMaxTargets];
    __shared__ int last;
    const int c = blockIdx.x, nc = gridDim.x;
    const int64_t row = blockIdx.y;
    const int tid = threadIdx.x;
    const float* s = scores + row * ld;
    const int32_t* irow = ids ? ids + row * n : nullptr;
    RowState* st = ws.st + row;
    const int nt = k2 > 0 ? 2 : 1;
    uint32_t bucket[kMaxTargets] = {0u, 0u};
    int rem[kMaxTargets] = {0, 0};
    for (int t = 0; t < nt; ++t) {
        bucket[t] = st->bucket[t];
        rem[t] = st->rem[t];
    }
    if (tid < kMaxTargets) {
        cnt_gt[tid] = 0;
        cnt_cand[tid] = 0;
    }
    __syncthreads();
    // this chunk's keys stay in registers for the two passes below
    constexpr int kPer = kChunk / kLongNT;
    const int64_t b0 = chunk_begin(c);
    uint32_t kr[kPer];
    load_keys<kPer, kLongNT>(s, irow, n, b0 + tid, kr);
    // per target: keys above the boundary bucket and keys inside it
    int gt[kMaxTargets] = {0, 0}, nca[kMaxTargets] = {0, 0};
#pragma unroll
    for (int t = 0; t < kMaxTargets; ++t) {
        const bool all = rem[t] < 0;
        const uint32_t bk = bucket[t];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint32_t d = kr[j] >> 20;
            gt[t] += kr[j] && (all || d > bk);
            nca[t] += kr[j] && !all && d == bk;
        }
    }
    // wave totals, one LDS atomic per wave: the wave's base in the chunk's
    // range of the candidate list, and the chunk's count of keys above it
    const int lane = tid & 63;
    int wbase[kMaxTargets] = {0, 0};
#pragma unroll
    for (int t = 0; t < kMaxTargets; ++t) {
        if (t >= nt) break;
        const int wn = wave_sum_dpp(nca[t]), wg = wave_sum_dpp(gt[t]);
        int b = 0;
        if (lane == 0) {
            if (wn) b = atomicAdd(&cnt_cand[t], wn);
            if (wg) atomicAdd(&cnt_gt[t], wg);
        }
        wbase[t] = __builtin_amdgcn_readfirstlane(b);
    }
    __syncthreads();
    if (tid < nt) {
        // one device atomic per chunk reserves its range of the candidate list
        cbase[tid] = (int)atomicAdd(&st->ncand[tid], (uint32_t)cnt_cand[tid]);
    }
    __syncthreads();
    // candidates go to their place by ballots: no atomics per key
#pragma unroll
    for (int t = 0; t < kMaxTargets; ++t) {
        if (t >= nt || rem[t] < 0) continue;
        Cand* cb = ws.cand + ((int64_t)row * kMaxTargets + t) * kCandCap;
        int pos0 = cbase[t] + wbase[t];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const bool is = kr[j] && (kr[j] >> 20) == bucket[t];
            const uint64_t m = __ballot(is);
            if (is) {
                const int pos = pos0 + lanes_below(m);
                if (pos < kCandCap) {
                    cb[pos].key = kr[j];
                    cb[pos].slot = (int32_t)(tid + (int64_t)j * kLongNT + b0);
                }
            }
            pos0 += __popcll(m);
        }
    }
    if (tid < nt) ws.rec[((int64_t)row * kMaxTargets + tid) * nc + c].gt = cnt_gt[tid];
    __syncthreads();  // the workgroup's stores are ordered before thread 0's release
    if (tid == 0) last = arrive_last(&st->ctr_cand, (uint32_t)nc);
    __syncthreads();  // thread 0's acquire covers the workgroup
    if (!last) return;
    // ---- last workgroup of the row: exact (tau, need) and chunk offsets.
    // Every load it needs is issued first: both targets' candidate lists
    // (whole buffers: slots past the count are read but not used) and the
    // per-chunk counts of keys above the bucket.
    constexpr int kCpt = kCandCap / kLongNT;  // candidates per thread
    static_assert(kCandCap == kCpt * kLongNT, "whole candidates per thread");
    const int cper = (nc + kLongNT - 1) / kLongNT;  // nc <= 2048 chunks: at most 4
    const int cc0 = min(nc, tid * cper), cc1 = min(nc, cc0 + cper);
    Cand cpre[kMaxTargets][kCpt];
    int gpre[kMaxTargets][4];
    uint32_t mpre[kMaxTargets];
#pragma unroll
    for (int t = 0; t < kMaxTargets; ++t) {
        mpre[t] = t < nt ? __hip_atomic_load(&st->ncand[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
        const Cand* cb = ws.cand + ((int64_t)row * kMaxTargets + t) * kCandCap;
        const ChunkRec* rec = ws.rec + ((int64_t)row * kMaxTargets + t) * nc;
#pragma unroll
        for (int u = 0; u < kCpt; ++u) cpre[t][u] = t < nt ? cb[tid + u * kLongNT] : Cand{0u, 0};
#pragma unroll
        for (int u = 0; u < 4; ++u) gpre[t][u] = (t < nt && cc0 + u < cc1) ? rec[cc0 + u].gt : 0;
    }
#pragma unroll
    for (int t = 0; t < kMaxTargets; ++t) {
        if (t >= nt) break;
        const int kk = t ? k2 : k;
        ChunkRec* rec = ws.rec + ((int64_t)row * kMaxTargets + t) * nc;
        const uint32_t m = mpre[t];
        uint32_t tau;
        int need;
        bool exact = true;
        if (rem[t] < 0) {
            tau = 0u;  // all selectable keys
            need = 0;
        } else if (m <= (uint32_t)kCandCap) {
#pragma unroll
            for (int u = 0; u < kCpt; ++u) {
                const int i = tid + u * kLongNT;
                if (i < (int)m) {
                    ckeys[i] = cpre[t][u].key;
                    cslot[i] = cpre[t][u].slot;
                }
            }
            __syncthreads();
            lds_kth<kLongNT>(ckeys, (int)m, rem[t], 12, hist, res, tau, need);
        } else {
            exact = false;  // bucket too large for LDS: resolve below over the row
            tau = 0u;
            need = 0;
        }
        if (!exact) {
            // Radix over the whole row (rare): prefix = bucket, three more digits.
            uint32_t prefix = bucket[t] << 20, mask = 0xFFF00000u;
            int r = rem[t];
            for (int shift = 8; shift >= 0; shift -= 8) {
                const int bits = shift == 8 ? 12 : 8;
                const int nb = 1 << bits;
                const uint32_t bm = (uint32_t)nb - 1u;
                for (int i = tid; i < nb; i += kLongNT) hist[i] = 0;
                __syncthreads();
                for (int64_t i = tid; i < n; i += kLongNT) {
                    const uint32_t key = load_key(s, irow, i);
                    if (key && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & bm], 1);
                }
                __syncthreads();
                if (tid == 0) {
                    int acc = 0;
                    for (int b = nb - 1; b >= 0; --b) {
                        if (acc + hist[b] >= r) {
                            res[0] = b;
                            res[1] = acc;
                            break;
                        }
                        acc += hist[b];
                    }
                }
                __syncthreads();
                prefix |= (uint32_t)res[0] << shift;
                mask |= bm << shift;
                r -= res[1];
                __syncthreads();
            }
            tau = prefix;
            need = r;
        }
        // per-chunk counts of keys > tau inside the bucket and of keys == tau
        // (reuse hist as two int arrays of nc entries)
        int* cgt = hist;
        int* ceq = hist + 2048;
        for (int i = tid; i < nc; i += kLongNT) {
            cgt[i] = 0;
            ceq[i] = 0;
        }
        __syncthreads();
        if (rem[t] >= 0) {
            if (exact) {
                // a chunk's candidates are contiguous in the list, so a wave's
                // 64 usually share one chunk: then one atomic per wave
                const int lane = tid & 63;
                for (int i0 = tid - lane; i0 < (int)m; i0 += kLongNT) {
                    const int i = i0 + lane;
                    const bool in = i < (int)m;
                    const int ch = in ? cslot[i] / kChunk : -1;
                    const int g1 = in && ckeys[i] > tau;
                    const int e1 = in && ckeys[i] == tau && need > 0;
                    const int ch0 = __builtin_amdgcn_readfirstlane(ch);
                    if (__ballot(in && ch != ch0) == 0) {
                        const int sg = wave_sum_dpp(g1), se = wave_sum_dpp(e1);
                        if (lane == 0) {
                            if (sg) atomicAdd(&cgt[ch0], sg);
                            if (se) atomicAdd(&ceq[ch0], se);
                        }
                    } else if (in) {
                        if (g1) atomicAdd(&cgt[ch], 1);
                        else if (e1) atomicAdd(&ceq[ch], 1);
                    }
                }
            } else {
                for (int64_t i = tid; i < n; i += kLongNT) {
                    const uint32_t key = load_key(s, irow, i);
                    if ((key >> 20) != bucket[t]) continue;
                    if (key > tau) atomicAdd(&cgt[i / kChunk], 1);
                    else if (key == tau && need > 0) atomicAdd(&ceq[i / kChunk], 1);
                }
            }
        }
        __syncthreads();
        {
            // chunk offsets: each thread owns a run of consecutive chunks
            const int c0 = cc0, c1 = cc1;
            int gtv[4], eqsum = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) gtv[u] = gpre[t][u];
            for (int ch = c0; ch < c1; ++ch) eqsum += ceq[ch];
            int tot;
            int eqb = block_excl_scan<kLongNT>(eqsum, tmp, &tot);
            int selsum = 0, e2 = eqb;
            for (int ch = c0; ch < c1; ++ch) {
                selsum += gtv[ch - c0] + cgt[ch] + min(max(need - e2, 0), ceq[ch]);
                e2 += ceq[ch];
            }
            int total;
            int off = block_excl_scan<kLongNT>(selsum, tmp, &total);
            for (int ch = c0; ch < c1; ++ch) {
                rec[ch].off = off;
                rec[ch].eq_before = eqb;
                off += gtv[ch - c0] + cgt[ch] + min(max(need - eqb, 0), ceq[ch]);
                eqb += ceq[ch];
            }
            if (tid == 0) {
                st->tau[t] = tau;
                st->need[t] = need;
                st->total[t] = total;
                st->ncand[t] = 0u;
            }
        }
        __syncthreads();
    }
    if (tid == 0) st->ctr_cand = 0u;
}

// grid (n_chunk, nq)
__global__ __launch_bounds__(kLongNT) void k_topk_write(const float* __restrict__ scores, int64_t n,
                                                        int64_t ld, const int32_t* __restrict__ ids,
                                                        int32_t k, int32_t* __restrict__ out,
                                                        int32_t k2, int32_t* __restrict__ out2,
                                                        LongWs ws) {
    __shared__ uint32_t keys[kChunk];
    __shared__ int wtmp[2 * kLongNT / 64];
    const int c = blockIdx.x, nc = gridDim.x;
    const int64_t row = blockIdx.y;
    const int tid = threadIdx.x;
    const float* s = scores + row * ld;
    const int32_t* irow = ids ? ids + row * n : nullptr;
    const RowState* st = ws.st + row;
    const int64_t b0 = chunk_begin(c), b1 = min(n, b0 + kChunk);
    const int64_t len = b1 - b0;
    stage_keys<kLongNT>(s + b0, irow ? irow + b0 : nullptr, len, keys);
    __syncthreads();
    const int nt = out2 ? 2 : 1;
    for (int t = 0; t < nt; ++t) {
        const int32_t kk = t ? k2 : k;
        int32_t* dst = (t ? out2 + row * k2 : out + row * k);
        const ChunkRec r = ws.rec[((int64_t)row * kMaxTargets + t) * nc + c];
        const uint32_t tau = st->tau[t];
        const int need = st->need[t];
        const int32_t* ich = irow ? irow + b0 : nullptr;
        ordered_write<kLongNT>([&](int64_t i) { return keys[i]; }, len, tau, need, ich, kk, dst,
                               wtmp, r.off, r.eq_before, false, b0);
        if (c == nc - 1)
            for (int i = st->total[t] + tid; i < kk; i += kLongNT) dst[i] = -1;
        __syncthreads();
    }
}

static int32_t long_chunks(int64_t n) { return (int32_t)((n + kChunk - 1) / kChunk); }

size_t topk_ws_bytes(int32_t nq, int64_t n, int32_t, int32_t) {
    if (n <= kSmallMax) return 0;
    const size_t nc = (size_t)long_chunks(n);
    return (size_t)nq * (sizeof(RowState) + kMaxTargets * kCandCap * sizeof(Cand) +
                         kMaxTargets * nc * sizeof(ChunkRec)) + 256;
}

hipError_t launch_topk(const float* scores, int32_t nq, int64_t n, int64_t ld, const int32_t* ids,
                       int32_t k, int32_t* out, int32_t k2, int32_t* out2, void* ws, hipStream_t s) {
    if (nq == 0) return hipSuccess;
    if (n <= kSmallMax) {
        const dim3 g((uint32_t)nq), b(kSmallNT);
        if (n <= 16 * kSmallNT) {
            if (ids) hipLaunchKernelGGL((k_topk_small<true, 16>), g, b, 0, s, scores, n, ld, ids, k, out, k2, out2);
            else hipLaunchKernelGGL((k_topk_small<false, 16>), g, b, 0, s, scores, n, ld, ids, k, out, k2, out2);
        } else {
            if (ids) hipLaunchKernelGGL((k_topk_small<true, 32>), g, b, 0, s, scores, n, ld, ids, k, out, k2, out2);
            else hipLaunchKernelGGL((k_topk_small<false, 32>), g, b, 0, s, scores, n, ld, ids, k, out, k2, out2);
        }
        return hipGetLastError();
    }
    const int32_t nc = long_chunks(n);
    char* base = static_cast<char*>(ws);
    LongWs w;
    w.st = reinterpret_cast<RowState*>(base);
    w.cand = reinterpret_cast<Cand*>(base + (size_t)nq * sizeof(RowState));
    w.rec = reinterpret_cast<ChunkRec*>(reinterpret_cast<char*>(w.cand) +
                                        (size_t)nq * kMaxTargets * kCandCap * sizeof(Cand));
    const int32_t kk2 = out2 ? k2 : 0;
    dim3 grid((uint32_t)nc, (uint32_t)nq);
    hipLaunchKernelGGL(k_topk_hist, grid, dim3(kLongNT), 0, s, scores, n, ld, ids, k, kk2, w);
    hipLaunchKernelGGL(k_topk_cand, grid, dim3(kLongNT), 0, s, scores, n, ld, ids, k, kk2, w);
    hipLaunchKernelGGL(k_topk_write, grid, dim3(kLongNT), 0, s, scores, n, ld, ids, k, out, kk2,
                       out2, w);
    return hipGetLastError();
}

// tokens[i][c*block + r] = blocks[i][c]*block + r when the block is chosen and
// the position is <= q_pos[i], else -1.
__global__ __launch_bounds__(256) void k_expand_blocks(const int32_t* __restrict__ blocks, int32_t nb,
                                                       int32_t block, const int32_t* __restrict__ q_pos,
                                                       int32_t* __restrict__ tokens) {
    const int32_t qi = blockIdx.y;
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = (int64_t)nb * block;
    if (j >= n) return;
    const int32_t b = blocks[(int64_t)qi * nb + j / block];
    const int64_t pos = (int64_t)b * block + j % block;
    tokens[(int64_t)qi * n + j] = (b >= 0 && pos <= q_pos[qi]) ? (int32_t)pos : -1;
}

hipError_t launch_expand_blocks(const int32_t* blocks, int32_t nq, int32_t nb, int32_t block,
                                const int32_t* q_pos, int32_t* tokens, hipStream_t s) {
    const int64_t n = (int64_t)nb * block;
    if (nq == 0 || n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_expand_blocks, dim3((uint32_t)((n + 255) / 256), (uint32_t)nq), dim3(256),
                       0, s, blocks, nb, block, q_pos, tokens);
    return hipGetLastError();
}

}  // namespace csa2

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
// Long rows: two multi-workgroup kernels per row set --
//   hist:  12-bit histogram of the top digit (LDS, then device atomics); one
//          workgroup per row picks the boundary bucket of each target;
//   keep:  every chunk compacts, in slot order, the keys any target can still
//          take (those at or above the lowest boundary bucket) into its own
//          region; one workgroup per row holds the row's kept keys (about k
//          plus one bucket) in registers, resolves (tau, need) of each target
//          exactly on them and writes both selections in order.
// For a handful of rows the per-row step is done by the row's last chunk
// workgroup to arrive; for rows enough to fill the GPU each kernel is two
// launches, chunks then one workgroup per row.
// The workspace's counters and histogram reset themselves, so it must be
// zero-filled before its first use and is left zero-filled by every call.
#include <algorithm>

#include "csa2_dev.h"
#include "csa2_kernels.h"
#include "csa2_select.h"

namespace csa2 {

constexpr int kSmallNT = 1024;
constexpr int kSmallMax = 32768;  // slots kept in LDS by the one-workgroup path
constexpr int kLongNT = 1024;
constexpr int kChunk = 8192;      // slots per workgroup on the long path
constexpr int kMaxTargets = 2;
constexpr int kStage = 12288;     // kept keys of a row the last workgroup holds in registers
constexpr int kMaxChunks = 2048;  // rows of up to 2^24 slots

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
    uint32_t ctr_hist, ctr_keep;
    uint32_t bucket[kMaxTargets];  // top digit of the boundary bucket
    int32_t rem[kMaxTargets];      // rank still needed inside that bucket (-1: take all)
    int32_t pad[2];
};
struct Cand {
    uint32_t key;
    int32_t val;  // the slot's output value (its id, or the slot)
};

struct LongWs {
    RowState* st;    // [nq]
    Cand* keep;      // [nq][n_chunk][kChunk]: each chunk's kept keys, slot order
    int32_t* nkeep;  // [nq][n_chunk]
};

__device__ __forceinline__ int64_t chunk_begin(int c) { return (int64_t)c * kChunk; }

// MODE 0, grid (n_chunk, nq): every workgroup adds its chunk to the row
// histogram and the last one of a row finds the boundary buckets; MODE 1, the
// chunks alone, then MODE 2, grid (1, nq): one workgroup per row finds them
// (many rows: see k_topk_keep).
template <int MODE>
__global__ __launch_bounds__(kLongNT) void k_topk_hist(const float* __restrict__ scores, int64_t n,
                                                       int64_t ld, const int32_t* __restrict__ ids,
                                                       int32_t k, int32_t k2, LongWs ws) {
    __shared__ alignas(16) int hist[kHistWords];
    __shared__ int res[4];
    __shared__ int last;
    const int c = blockIdx.x, nc = (int)((n + kChunk - 1) / kChunk);
    const int64_t row = blockIdx.y;
    const int tid = threadIdx.x;
    const float* s = scores + row * ld;
    const int32_t* irow = ids ? ids + row * n : nullptr;
    RowState* st = ws.st + row;
    if (MODE != 2) {
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
        if (MODE == 1) return;
        // the row histogram is built and read by device atomics; the
        // release of every arrival and the acquire of the last order them
        hand_off_wait();
        __syncthreads();
        if (tid == 0) last = arrive_last_release(&st->ctr_hist, (uint32_t)nc);
        __syncthreads();
        if (!last) return;
    }
    // the row's resolving workgroup: boundary bucket of each target
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

struct KeepLds {
    union {
        struct {  // a chunk: keys and output values of its slots
            uint32_t key[kChunk];
            int32_t val[kChunk];
        } c;
    } u;
    alignas(16) int hist[kHistWords];
    int koff[kMaxChunks + 1];
    int tmp[kLongNT / 64 + 1];
    int tmp2[2 * (kLongNT / 64 + 1)];
    int wtmp[2 * kLongNT / 64];
    int res[4];
    int res2[kMaxTargets][4];
    int last;
};

// MODE 0, grid (n_chunk, nq): every workgroup compacts its chunk and the last
// one of a row to finish (acquire-release arrival) resolves the row.  For a
// handful of rows (decode).
// MODE 1, grid (n_chunk, nq): the chunks alone; MODE 2, grid (1, nq), launched
// after it: one workgroup per row resolves it.  For many rows (a replayed
// segment, a prefill chunk): with the rows' resolution left to whichever
// workgroup arrives last, an XCD that falls behind receives the late arrivals
// and with them the 13 us resolutions, so it falls further behind (128 rows of
// 131072: one XCD still starting chunk workgroups at 150 us while the other
// seven were done by 60 us); a launch of its own deals them out evenly.
template <int MODE>
__global__ __launch_bounds__(kLongNT) void k_topk_keep(const float* __restrict__ scores, int64_t n,
                                                       int64_t ld, const int32_t* __restrict__ ids,
                                                       int32_t k, int32_t* __restrict__ out,
                                                       int32_t k2, int32_t* __restrict__ out2,
                                                       LongWs ws) {
    __shared__ KeepLds sh;
    const int c = blockIdx.x, nc = (int)((n + kChunk - 1) / kChunk);
    const int64_t row = blockIdx.y;
    const int tid = threadIdx.x;
    const float* s = scores + row * ld;
    const int32_t* irow = ids ? ids + row * n : nullptr;
    RowState* st = ws.st + row;
    const int nt = out2 ? 2 : 1;
    uint32_t bucket[kMaxTargets] = {0u, 0u};
    int rem[kMaxTargets] = {0, 0};
    uint32_t low = 0xFFFFFFFFu;  // the lowest key any target can take
    for (int t = 0; t < nt; ++t) {
        bucket[t] = st->bucket[t];
        rem[t] = st->rem[t];
        low = min(low, rem[t] < 0 ? 1u : bucket[t] << 20);
    }
    if (MODE != 2) {
        // ---- the chunk: stage keys and output values (loads all issued first)
        const int64_t b0 = chunk_begin(c);
        const int len = (int)min((int64_t)kChunk, n - b0);
        {
            constexpr int kPer = kChunk / kLongNT;
            float v[kPer];
            int32_t id[kPer];
#pragma unroll
            for (int u = 0; u < kPer; ++u) v[u] = s[b0 + min(tid + u * kLongNT, len - 1)];
#pragma unroll
            for (int u = 0; u < kPer; ++u) id[u] = irow ? irow[b0 + min(tid + u * kLongNT, len - 1)] : 0;
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int i = tid + u * kLongNT;
                const uint32_t key = score_key(v[u]);
                sh.u.c.key[i] = (i < len && id[u] >= 0 && key != kNegInfKey) ? key : 0u;
                sh.u.c.val[i] = irow ? id[u] : (int32_t)(b0 + i);
            }
        }
        __syncthreads();
        // thread t owns slots 8 t .. 8 t + 7: kept ones go to the chunk's region in order
        uint32_t kk8[8];
        {
            const uint4 a = *reinterpret_cast<const uint4*>(&sh.u.c.key[8 * tid]);
            const uint4 b = *reinterpret_cast<const uint4*>(&sh.u.c.key[8 * tid + 4]);
            kk8[0] = a.x; kk8[1] = a.y; kk8[2] = a.z; kk8[3] = a.w;
            kk8[4] = b.x; kk8[5] = b.y; kk8[6] = b.z; kk8[7] = b.w;
        }
        int mine = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) mine += kk8[u] >= low;  // key 0 (past len too) is below low
        int tot;
        int pos = block_excl_scan<kLongNT>(mine, sh.tmp, &tot);
        // kept keys (a key and its value as one 8-byte word) and counts
        uint64_t* reg = reinterpret_cast<uint64_t*>(ws.keep + ((int64_t)row * nc + c) * kChunk);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (kk8[u] >= low)
                reg[pos++] = (uint64_t)kk8[u] | ((uint64_t)(uint32_t)sh.u.c.val[8 * tid + u] << 32);
        if (tid == 0) ws.nkeep[row * nc + c] = tot;
        if (MODE == 1) return;
        __syncthreads();  // the workgroup's stores are ordered before thread 0's release
        if (tid == 0) sh.last = arrive_last(&st->ctr_keep, (uint32_t)nc);
        __syncthreads();  // thread 0's acquire covers the workgroup
        if (!sh.last) return;
    }

    // ---- the last workgroup of the row: chunk offsets of the kept keys
    {
        const int c0 = 2 * tid;  // nc <= 2048: two chunks per thread
        const int32_t* nk = ws.nkeep + row * nc;
        const int a = c0 < nc ? nk[c0] : 0;
        const int b = c0 + 1 < nc ? nk[c0 + 1] : 0;
        int all;
        const int pre = block_excl_scan<kLongNT>(a + b, sh.tmp, &all);
        if (c0 < nc) sh.koff[c0] = pre;
        if (c0 + 1 < nc) sh.koff[c0 + 1] = pre + a;
        if (tid == 0) sh.koff[nc] = all;
    }
    __syncthreads();
    const int m = sh.koff[nc];
    const Cand* kb = ws.keep + (int64_t)row * nc * kChunk;
    // kept key i of the row: chunk = the last one whose offset is <= i
    auto at = [&](int64_t i) -> Cand {
        int lo = 0, hi = nc - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sh.koff[mid] <= i) lo = mid;
            else hi = mid - 1;
        }
        const uint64_t w = *reinterpret_cast<const uint64_t*>(kb + (int64_t)lo * kChunk + (i - sh.koff[lo]));
        return Cand{(uint32_t)w, (int32_t)(uint32_t)(w >> 32)};
    };
    if (m <= kStage) {
        // thread t holds kept keys [E t, E t + E) of the row in registers
        // (the row order is chunk-major, each chunk in slot order)
        constexpr int kE = kStage / kLongNT;
        static_assert(kStage == kE * kLongNT, "whole entries per thread");
        const int E = (m + kLongNT - 1) / kLongNT;
        const int i0 = min(tid * E, m);
        int ch = 0;  // the chunk holding entry i0: the last one whose offset is <= i0
        {
            int lo = 0, hi = nc - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sh.koff[mid] <= i0) lo = mid;
                else hi = mid - 1;
            }
            ch = lo;
        }
        int64_t addr[kE];
        int off = i0 - sh.koff[ch];
#pragma unroll
        for (int u = 0; u < kE; ++u) {
            const bool in = u < E && i0 + u < m;
            while (in && ch < nc - 1 && i0 + u >= sh.koff[ch + 1]) {  // past this chunk's keys
                ++ch;
                off = i0 + u - sh.koff[ch];
            }
            addr[u] = in ? (int64_t)ch * kChunk + off : 0;
            off += in;
        }
        Cand e[kE];
#pragma unroll
        for (int u = 0; u < kE; ++u) {  // every load issued before any use
            const uint64_t w = *reinterpret_cast<const uint64_t*>(kb + addr[u]);
            e[u] = Cand{(uint32_t)w, (int32_t)(uint32_t)(w >> 32)};
        }
        uint32_t key[kE];
#pragma unroll
        for (int u = 0; u < kE; ++u) key[u] = (u < E && i0 + u < m) ? e[u].key : 0u;
        // (tau, need) of both targets at once: the top 12 bits are the
        // bucket's; two more 10-bit digits, each target stopping as soon as a
        // whole sub-bucket completes its selection
        uint32_t tau[kMaxTargets] = {0u, 0u};  // rem < 0: every selectable key
        int need[kMaxTargets] = {0, 0};
        {
            uint32_t prefix[kMaxTargets], mask[kMaxTargets];
            int r[kMaxTargets];
            bool done[kMaxTargets];
#pragma unroll
            for (int t = 0; t < kMaxTargets; ++t) {
                done[t] = t >= nt || rem[t] < 0;
                prefix[t] = bucket[t] << 20;
                mask[t] = 0xFFF00000u;
                r[t] = rem[t];
            }
            constexpr int kBits = 10;
            constexpr uint32_t kDm = (1u << kBits) - 1u;
            constexpr int kW = (1 << kBits) + (1 << kBits) / 16;  // hidx(1 << kBits)
            for (int shift = 20 - kBits; shift >= 0 && !(done[0] && done[1]); shift -= kBits) {
                for (int i = tid; i < kMaxTargets * kW; i += kLongNT) sh.hist[i] = 0;
                __syncthreads();
#pragma unroll
                for (int u = 0; u < kE; ++u)
#pragma unroll
                    for (int t = 0; t < kMaxTargets; ++t)
                        if (!done[t] && key[u] && (key[u] & mask[t]) == prefix[t])
                            atomicAdd(&sh.hist[t * kW + hidx((int)((key[u] >> shift) & kDm))], 1);
                __syncthreads();
                const int w = tid >> 6;
                if (w < kMaxTargets && !done[w]) wave_find_bucket(sh.hist + w * kW, 1 << kBits, r[w], sh.res2[w]);
                __syncthreads();
#pragma unroll
                for (int t = 0; t < kMaxTargets; ++t) {
                    if (done[t]) continue;
                    prefix[t] |= (uint32_t)sh.res2[t][0] << shift;
                    mask[t] |= kDm << shift;
                    r[t] -= sh.res2[t][1];
                    if (sh.res2[t][2] == r[t]) {  // the whole sub-bucket is taken
                        done[t] = true;
                        tau[t] = prefix[t] - 1u;  // every key >= prefix
                    } else if (shift == 0) {
                        tau[t] = prefix[t];
                        need[t] = r[t];
                    }
                }
            }
        }
        // ordered writes: one scan of packed (greater, equal) counts per
        // target (m <= kStage < 2^16, so the halves never carry)
        int packed[kMaxTargets] = {0, 0};
#pragma unroll
        for (int u = 0; u < kE; ++u)
#pragma unroll
            for (int t = 0; t < kMaxTargets; ++t) {
                packed[t] += key[u] > tau[t];
                packed[t] += ((need[t] > 0) & (key[u] == tau[t])) << 16;
            }
        int total[kMaxTargets];
        int before[kMaxTargets];
        block_excl_scan2<kLongNT>(packed[0], packed[1], sh.tmp2, before, total);
        for (int t = 0; t < nt; ++t) {
            const int32_t kk = t ? k2 : k;
            int32_t* dst = t ? out2 + row * k2 : out + row * k;
            int eq = (int)((uint32_t)before[t] >> 16);
            int pos = (int)((uint32_t)before[t] & 0xFFFFu) + min(need[t], eq);
#pragma unroll
            for (int u = 0; u < kE; ++u) {
                bool take = key[u] > tau[t];
                if (need[t] > 0 && key[u] == tau[t]) {
                    take = eq < need[t];
                    ++eq;
                }
                if (take && pos < kk) dst[pos++] = e[u].val;
            }
            const int chosen = (int)((uint32_t)total[t] & 0xFFFFu) +
                               min(need[t], (int)((uint32_t)total[t] >> 16));
            for (int i = min(chosen, kk) + tid; i < kk; i += kLongNT) dst[i] = -1;
        }
    } else {
        // a row with many keys tied around the boundary: read them in place
        auto K = [&](int64_t i) { return at(i).key; };
        auto V = [&](int64_t i) { return at(i).val; };
        for (int t = 0; t < nt; ++t) {
            const int32_t kk = t ? k2 : k;
            int32_t* dst = t ? out2 + row * k2 : out + row * k;
            uint32_t tau = 0u;
            int need = 0;
            if (rem[t] >= 0) kth_fn<kLongNT>(K, m, rem[t], 12, bucket[t] << 20, sh.hist, sh.res, tau, need);
            ordered_write_v<kLongNT>(K, V, m, tau, need, kk, dst, sh.wtmp);
        }
    }
    if (tid == 0) st->ctr_keep = 0u;
}

static int32_t long_chunks(int64_t n) { return (int32_t)((n + kChunk - 1) / kChunk); }

// Row records first, at least kMinRowStates of them, so their addresses
// depend only on the row index: a workspace cleared once serves calls of any
// row length with up to kMinRowStates rows (each call leaves its records
// zero); the chunks' kept keys follow, as scratch.
constexpr int32_t kMinRowStates = 64;
static size_t row_state_bytes(int32_t nq) {
    return (size_t)std::max(nq, kMinRowStates) * sizeof(RowState);
}

size_t topk_ws_bytes(int32_t nq, int64_t n, int32_t, int32_t) {
    if (n <= kSmallMax) return 0;
    const size_t nc = (size_t)long_chunks(n);
    return row_state_bytes(nq) + (size_t)nq * (nc * kChunk * sizeof(Cand) + nc * sizeof(int32_t)) + 256;
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
    if (nc > kMaxChunks) return hipErrorInvalidValue;
    char* base = static_cast<char*>(ws);
    LongWs w;
    w.st = reinterpret_cast<RowState*>(base);
    w.keep = reinterpret_cast<Cand*>(base + row_state_bytes(nq));
    w.nkeep = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(w.keep) +
                                         (size_t)nq * nc * kChunk * sizeof(Cand));
    const int32_t kk2 = out2 ? k2 : 0;
    dim3 grid((uint32_t)nc, (uint32_t)nq);
    if ((int64_t)nc * nq >= 256) {  // the rows fill the GPU
        hipLaunchKernelGGL(k_topk_hist<1>, grid, dim3(kLongNT), 0, s, scores, n, ld, ids, k, kk2, w);
        hipLaunchKernelGGL(k_topk_hist<2>, dim3(1u, (uint32_t)nq), dim3(kLongNT), 0, s, scores, n, ld, ids, k,
                           kk2, w);
        hipLaunchKernelGGL(k_topk_keep<1>, grid, dim3(kLongNT), 0, s, scores, n, ld, ids, k, out, kk2,
                           out2, w);
        hipLaunchKernelGGL(k_topk_keep<2>, dim3(1u, (uint32_t)nq), dim3(kLongNT), 0, s, scores, n, ld, ids, k,
                           out, kk2, out2, w);
    } else {
        hipLaunchKernelGGL(k_topk_hist<0>, grid, dim3(kLongNT), 0, s, scores, n, ld, ids, k, kk2, w);
        hipLaunchKernelGGL(k_topk_keep<0>, grid, dim3(kLongNT), 0, s, scores, n, ld, ids, k, out, kk2,
                           out2, w);
    }
    return hipGetLastError();
}

// tokens[i][c*block + r] = blocks[i][c]*block + r when the block is chosen and
// the entry is readable by query i (entries of 2^msh positions: the whole
// group at or before q_pos[i]), else -1.
__global__ __launch_bounds__(256) void k_expand_blocks(const int32_t* __restrict__ blocks, int32_t nb,
                                                       int32_t block, const int32_t* __restrict__ q_pos,
                                                       int32_t msh, int32_t* __restrict__ tokens) {
    const int32_t qi = blockIdx.y;
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = (int64_t)nb * block;
    if (j >= n) return;
    const int32_t b = blocks[(int64_t)qi * nb + j / block];
    const int64_t pos = (int64_t)b * block + j % block;
    const int64_t last = (((int64_t)q_pos[qi] + 1) >> msh) - 1;
    tokens[(int64_t)qi * n + j] = (b >= 0 && pos <= last) ? (int32_t)pos : -1;
}

hipError_t launch_expand_blocks(const int32_t* blocks, int32_t nq, int32_t nb, int32_t block,
                                const int32_t* q_pos, int32_t* tokens, hipStream_t s, int32_t msh) {
    const int64_t n = (int64_t)nb * block;
    if (nq == 0 || n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_expand_blocks, dim3((uint32_t)((n + 255) / 256), (uint32_t)nq), dim3(256),
                       0, s, blocks, nb, block, q_pos, msh, tokens);
    return hipGetLastError();
}

}  // namespace csa2

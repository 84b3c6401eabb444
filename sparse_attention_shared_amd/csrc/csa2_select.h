// csa2_select.h -- device routines of the exact top-k selection (internal):
// order-preserving keys, the (tau, need) radix select over keys held in LDS,
// and the ordered compaction that writes chosen slots ascending.
// Order: higher score first, equal scores by lower slot ("CED: Continuing
// Context with a Causal Encoder and Decoder", section "Selecting Positions and
// Reading Values with Attention", Fig. 4: the indexer keeps the best-scoring
// positions).
//
// A selection of kk slots is the pair (tau, need): every key > tau is chosen,
// plus the first `need` keys equal to tau in slot order (need = 0 when whole
// buckets are taken).  Key 0 marks a slot that can never be chosen.
#pragma once

#include "csa2_dev.h"

namespace csa2 {

constexpr int kHistBins = 4096;  // 12-bit top digit of the multi-workgroup path

__device__ __forceinline__ uint32_t load_key(const float* s, const int32_t* ids, int64_t i) {
    if (ids && ids[i] < 0) return 0u;
    const uint32_t k = score_key(s[i]);
    return k == kNegInfKey ? 0u : k;
}

__device__ __forceinline__ int wave_sum_dpp(int x) {
    return __builtin_amdgcn_readlane(wave_scan_dpp(x), 63);
}

// Set bits of a 64-bit lane mask below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exact (tau, need) of the kk-th key among the selectable keys keys[0..m) in
// LDS.  The top `known` bits (0 or 12) are shared by every key that can reach
// the kk-th place (the caller already resolved them); the remaining bits are
// resolved 8 at a time, highest first.  hist needs 256 ints, res 4 ints of
// LDS.  NT threads; every thread returns the same result.
template <int NT>
__device__ void lds_kth(const uint32_t* keys, int m, int kk, int known, int* hist, int* res,
                        uint32_t& tau, int& need) {
    const int tid = threadIdx.x, lane = tid & 63;
    tau = 0u;
    need = 0;
    if (m <= 0 || kk <= 0) return;
    uint32_t prefix = 0u, mask = 0u;
    if (known > 0) {
        mask = 0xFFFFFFFFu << (32 - known);
        prefix = keys[0] & mask;
    }
    int rem = kk;
    for (int hi_bit = 32 - known; hi_bit > 0; hi_bit -= 8) {
        const int bits = hi_bit >= 8 ? 8 : hi_bit;
        const int shift = hi_bit - bits;
        const uint32_t dm = (1u << bits) - 1u;
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < m; i += NT) {
            const uint32_t key = keys[i];
            if (key && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dm], 1);
        }
        __syncthreads();
        if (tid < 64) {
            // lane l holds bins 255-4l .. 252-4l (highest bins first)
            const int b0 = 255 - 4 * lane;
            const int c0 = hist[b0], c1 = hist[b0 - 1], c2 = hist[b0 - 2], c3 = hist[b0 - 3];
            const int s = c0 + c1 + c2 + c3;
            const int incl = wave_scan_dpp(s);
            const int total = __builtin_amdgcn_readlane(incl, 63);
            const int excl = incl - s;
            if (lane == 0) res[3] = total;
            if (excl < rem && incl >= rem) {
                int acc = excl, b = b0, c = c0;
                if (acc + c0 < rem) { acc += c0; b = b0 - 1; c = c1;
                    if (acc + c1 < rem) { acc += c1; b = b0 - 2; c = c2;
                        if (acc + c2 < rem) { acc += c2; b = b0 - 3; c = c3; } } }
                res[0] = b;
                res[1] = acc;
                res[2] = c;
            }
        }
        __syncthreads();
        const int total = res[3];
        if (total < rem) {  // fewer selectable keys than kk under this prefix: take all
            tau = prefix ? prefix - 1u : 0u;
            need = 0;
            __syncthreads();
            return;
        }
        const uint32_t bucket = (uint32_t)res[0];
        const int above = res[1], cnt = res[2];
        __syncthreads();
        prefix |= bucket << shift;
        mask |= dm << shift;
        rem -= above;
        if (cnt == rem) {  // the whole bucket is taken: every key >= prefix
            tau = prefix - 1u;
            need = 0;
            return;
        }
    }
    tau = prefix;
    need = rem;
}

// Ordered compaction of slots [0, n) with keys K(i): writes the chosen slots
// (through ids when given) ascending at dst[off0 + ...], counting the keys
// equal to tau from eq0 (the equal keys of earlier slots outside this range).
// Wave w owns a contiguous range of slots; within it, lanes take consecutive
// slots and ballots give every chosen slot its place.  Slot i is written as
// ids[i], or slot0 + i without ids.  Returns the number of slots this range
// chose.  wtmp needs 2 * NT/64 ints of LDS.  When pad is set, dst[total .. kk)
// is filled with -1.
template <int NT, class KeyFn>
__device__ int ordered_write(KeyFn K, int64_t n, uint32_t tau, int need, const int32_t* ids,
                             int32_t kk, int32_t* dst, int* wtmp, int off0 = 0, int eq0 = 0,
                             bool pad = true, int64_t slot0 = 0) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t per = ((n + NW - 1) / NW + 63) / 64 * 64;
    const int64_t r0 = min(n, (int64_t)w * per), r1 = min(n, r0 + per);
    int gt = 0, eq = 0;
    for (int64_t i = r0 + lane; i < r1; i += 64) {
        const uint32_t key = K(i);
        gt += key > tau;
        eq += (key == tau) & (need > 0);
    }
    gt = wave_sum_dpp(gt);
    eq = wave_sum_dpp(eq);
    if (lane == 0) {
        wtmp[w] = gt;
        wtmp[NW + w] = eq;
    }
    __syncthreads();
    // places before this wave: slots chosen by earlier waves and the keys
    // equal to tau they hold
    int eqb = eq0, selb = off0, total = 0, eqrun = eq0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        const int g = wtmp[v], e = wtmp[NW + v];
        const int take = g + min(max(need - eqrun, 0), e);
        if (v < w) selb += take;
        if (v == w) eqb = eqrun;
        total += take;
        eqrun += e;
    }
    for (int64_t i0 = r0; i0 < r1; i0 += 64) {
        const int64_t i = i0 + lane;
        const uint32_t key = i < r1 ? K(i) : 0u;
        const bool eqf = i < r1 && need > 0 && key == tau;
        const uint64_t em = __ballot(eqf);
        const int er = eqb + lanes_below(em);
        const bool take = i < r1 && (key > tau || (eqf && er < need));
        const uint64_t sm = __ballot(take);
        const int pos = selb + lanes_below(sm);
        if (take && pos < kk) dst[pos] = ids ? ids[i] : (int32_t)(slot0 + i);
        eqb += __popcll(em);
        selb += __popcll(sm);
    }
    if (pad)
        for (int i = off0 + total + tid; i < kk; i += NT) dst[i] = -1;
    __syncthreads();
    return total;
}

// Stage the keys of slots [0, n) of a row into LDS; global loads are issued
// eight per thread before any of them is used.
template <int NT>
__device__ void stage_keys(const float* s, const int32_t* ids, int64_t n, uint32_t* keys) {
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += 8 * NT) {
        float v[8];
        int32_t id[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t i = i0 + (int64_t)u * NT;
            v[u] = i < n ? s[i] : -__builtin_inff();
            id[u] = (ids && i < n) ? ids[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t i = i0 + (int64_t)u * NT;
            if (i < n) {
                const uint32_t k = score_key(v[u]);
                keys[i] = (id[u] < 0 || k == kNegInfKey) ? 0u : k;
            }
        }
    }
}

}  // namespace csa2

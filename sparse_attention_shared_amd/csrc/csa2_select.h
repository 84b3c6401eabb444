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

// Keys of slots first + j * STRIDE (j < PER) of a row of n >= 1 slots; slots
// past n give key 0.  Every load is issued before any is used (indices are
// clamped, so no branch guards them).
template <int PER, int STRIDE>
__device__ __forceinline__ void load_keys(const float* s, const int32_t* ids, int64_t n,
                                          int64_t first, uint32_t (&kr)[PER]) {
    float v[PER];
    int32_t w[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = s[min(first + (int64_t)j * STRIDE, n - 1)];
    if (ids) {
#pragma unroll
        for (int j = 0; j < PER; ++j) w[j] = ids[min(first + (int64_t)j * STRIDE, n - 1)];
    } else {
#pragma unroll
        for (int j = 0; j < PER; ++j) w[j] = 0;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const uint32_t k = score_key(v[j]);
        const bool ok = first + (int64_t)j * STRIDE < n && w[j] >= 0 && k != kNegInfKey;
        kr[j] = ok ? k : 0u;
    }
}

__device__ __forceinline__ int wave_sum_dpp(int x) {
    return __builtin_amdgcn_readlane(wave_scan_dpp(x), 63);
}

// Set bits of a 64-bit lane mask below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Padded histogram index: four spare words every 64 bins, so that 64 lanes
// adding to 64 consecutive bins hit 64 different LDS banks, and every run of
// 64 bins starts 16-byte aligned (the bucket search reads them as int4).
__device__ __forceinline__ int hidx(int b) { return b + 4 * (b >> 6); }
constexpr int kHistWords = 4096 + 256;  // LDS ints a 12-bit digit needs

// Bucket search by one wave over nb bins (descending): finds the bin where the
// running count from the top first reaches rem.  Phase A: lane l sums bins
// [nb - per(l+1), nb - per l); a DPP scan finds the lane of the crossing.
// Phase B: that lane's bins are spread over the wave and scanned again.
// Writes res[0] = bin, res[1] = keys in higher bins, res[2] = keys in the
// bin, res[3] = total keys.  Call from all 64 lanes of one wave.
__device__ __forceinline__ void wave_find_bucket(const int* hist, int nb, int rem, int* res) {
    const int lane = threadIdx.x & 63;
    const int per = nb >> 6;  // 64 bins per lane for 12-bit digits, 4 for 8-bit
    // lane l sums bins [nb - per (l + 1), nb - per l): contiguous, 16-byte aligned
    const int4* blk = reinterpret_cast<const int4*>(hist + hidx(nb - per * (lane + 1)));
    int sa = 0;
    if (per == 64) {
        int4 v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = blk[j];
#pragma unroll
        for (int j = 0; j < 16; ++j) sa += v[j].x + v[j].y + v[j].z + v[j].w;
    } else {
        for (int j = 0; j < per / 4; ++j) {
            const int4 v = blk[j];
            sa += v.x + v.y + v.z + v.w;
        }
    }
    const int incl = wave_scan_dpp(sa);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    const uint64_t hit = __ballot(incl >= rem);
    if (total < rem || hit == 0) {
        if (lane == 0) {
            res[0] = 0;
            res[1] = 0;
            res[2] = 0;
            res[3] = total;
        }
        return;
    }
    const int L = __builtin_ctzll(hit);
    const int above_l = __builtin_amdgcn_readlane(incl - sa, L);
    const int topL = nb - 1 - per * L;
    const int c = lane < per ? hist[hidx(topL - lane)] : 0;
    const int ib = wave_scan_dpp(c);
    const uint64_t hit2 = __ballot(lane < per && above_l + ib >= rem);
    const int J = __builtin_ctzll(hit2);
    if (lane == J) {
        res[0] = topL - J;
        res[1] = above_l + ib - c;
        res[2] = c;
        res[3] = total;
    }
}

// Exact (tau, need) of the kk-th key among a workgroup's selectable keys.
// The top `known` bits (0 or 12) are shared by every key that can reach the
// kk-th place (the caller already resolved them, `prefix` holds them).  The
// remaining bits are resolved in digits of 12, 12 and 8 bits, highest first,
// stopping as soon as a whole bucket is taken.  add(mask, prefix, shift, dm)
// adds this thread's keys k with k != 0 and (k & mask) == prefix to
// hist[hidx((k >> shift) & dm)]; it runs once per digit.  hist needs
// kHistWords ints, res 4 ints of LDS.  NT threads; every thread returns the
// same result.
template <int NT, class AddFn>
__device__ void kth_core(AddFn add, int kk, int known, uint32_t prefix, int* hist, int* res,
                         uint32_t& tau, int& need) {
    const int tid = threadIdx.x;
    uint32_t mask = 0u;
    if (known > 0) {
        mask = 0xFFFFFFFFu << (32 - known);
        prefix &= mask;
    } else {
        prefix = 0u;
    }
    int rem = kk;
    for (int hi_bit = 32 - known; hi_bit > 0;) {
        const int bits = hi_bit > 8 ? 12 : 8;
        const int shift = hi_bit - bits;
        const int nb = 1 << bits;
        const uint32_t dm = (uint32_t)nb - 1u;
        for (int i = tid; i < hidx(nb); i += NT) hist[i] = 0;
        __syncthreads();
        add(mask, prefix, shift, dm);
        __syncthreads();
        if (tid < 64) wave_find_bucket(hist, nb, rem, res);
        __syncthreads();
        const int total = res[3];
        const uint32_t bucket = (uint32_t)res[0];
        const int above = res[1], cnt = res[2];
        __syncthreads();
        if (total < rem) {  // fewer selectable keys than kk under this prefix: take all
            tau = prefix ? prefix - 1u : 0u;
            need = 0;
            return;
        }
        prefix |= bucket << shift;
        mask |= dm << shift;
        rem -= above;
        if (cnt == rem) {  // the whole bucket is taken: every key >= prefix
            tau = prefix ? prefix - 1u : 0u;  // prefix 0: every selectable (nonzero) key
            need = 0;
            return;
        }
        hi_bit = shift;
    }
    tau = prefix;
    need = rem;
}

// kth_core over the keys K(0..m): K is called once per slot and digit pass,
// so it may recompute keys.
template <int NT, class KeyFn>
__device__ void kth_fn(KeyFn K, int64_t m, int kk, int known, uint32_t prefix, int* hist, int* res,
                       uint32_t& tau, int& need) {
    tau = 0u;
    need = 0;
    if (m <= 0 || kk <= 0) return;
    const int tid = threadIdx.x;
    kth_core<NT>(
        [&](uint32_t mask, uint32_t pre, int shift, uint32_t dm) {
            for (int64_t i0 = tid; i0 < m; i0 += 4 * NT) {
                uint32_t kv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) kv[u] = (i0 + u * NT < m) ? K(i0 + u * NT) : 0u;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (kv[u] && (kv[u] & mask) == pre)
                        atomicAdd(&hist[hidx((int)((kv[u] >> shift) & dm))], 1);
            }
        },
        kk, known, prefix, hist, res, tau, need);
}

// kth_core over PER keys a thread holds in registers (0 = not selectable),
// with a short cut after the first 12-bit digit: when the bucket holding the
// kk-th key has at most 64 keys, one wave ranks them directly instead of
// running the remaining digits.  small needs 64 words and res 5 ints of LDS
// (besides hist).  NT threads; every thread returns the same result.
template <int NT, int PER>
__device__ void kth_regs(const uint32_t (&kv)[PER], int kk, int* hist, int* res, uint32_t* small,
                         uint32_t& tau, int& need) {
    const int tid = threadIdx.x;
    tau = 0u;
    need = 0;
    if (kk <= 0) return;
    for (int i = tid; i < hidx(4096); i += NT) hist[i] = 0;
    if (tid < 64) small[tid] = 0u;
    if (tid == 0) res[4] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u)
        if (kv[u]) atomicAdd(&hist[hidx((int)(kv[u] >> 20))], 1);
    __syncthreads();
    if (tid < 64) wave_find_bucket(hist, 4096, kk, res);
    __syncthreads();
    const int total = res[3], above = res[1], cnt = res[2];
    const uint32_t bucket = (uint32_t)res[0];
    if (total < kk) return;  // fewer selectable keys than kk: every one (tau 0)
    const int rem = kk - above;
    const uint32_t prefix = bucket << 20;
    if (cnt == rem) {  // the whole bucket is taken
        tau = prefix ? prefix - 1u : 0u;
        return;
    }
    if (cnt > 64) {  // many keys share the bucket: the remaining digits
        __syncthreads();  // every thread has read res
        kth_core<NT>(
            [&](uint32_t mask, uint32_t pre, int shift, uint32_t dm) {
#pragma unroll
                for (int u = 0; u < PER; ++u)
                    if (kv[u] && (kv[u] & mask) == pre) atomicAdd(&hist[hidx((int)((kv[u] >> shift) & dm))], 1);
            },
            rem, 12, prefix, hist, res, tau, need);
        return;
    }
    // the bucket's keys into `small`: one reservation per wave (a wave scan
    // of the lanes' counts), not one LDS atomic per key
    int mine = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) mine += (kv[u] && (kv[u] >> 20) == bucket) ? 1 : 0;
    const int incl = wave_scan_dpp(mine);
    const int wtot = __builtin_amdgcn_readlane(incl, 63);
    if (wtot) {  // wave-uniform
        int base = 0;
        if ((tid & 63) == 63) base = atomicAdd(&res[4], wtot);
        int at = __builtin_amdgcn_readlane(base, 63) + incl - mine;
#pragma unroll
        for (int u = 0; u < PER; ++u)
            if (kv[u] && (kv[u] >> 20) == bucket) small[at++] = kv[u];
    }
    __syncthreads();
    if (tid < 64) {
        // the rem-th largest key of the bucket, one bit at a time from the
        // top of the 20 bits below the bucket's digit: `act` holds the lanes
        // still matching the prefix v; when fewer than r of them have the
        // bit set, all of those are larger than the answer (r drops by
        // their count), else the answer has the bit.  At the end `act` holds
        // the keys equal to v and rem - r keys are larger.  When every key
        // equal to v is taken, tau = v - 1 and need = 0.
        const uint32_t x = small[tid];  // 0 past the bucket's keys
        uint64_t act = __ballot(x != 0u);
        uint32_t v = bucket << 20;
        int r = rem;
        for (int b = 19; b >= 0; --b) {
            const uint64_t ones = __ballot((x >> b) & 1u) & act;
            const int c = __popcll(ones);
            if (c >= r) {
                act = ones;
                v |= 1u << b;
            } else {
                r -= c;
                act &= ~ones;
            }
        }
        if (tid == 0) {
            const int eq = __popcll(act);
            res[0] = (int)(r == eq ? v - 1u : v);
            res[1] = r == eq ? 0 : r;
        }
    }
    __syncthreads();
    tau = (uint32_t)res[0];
    need = res[1];
}

// kth_fn over keys held in LDS.
template <int NT>
__device__ void lds_kth(const uint32_t* keys, int m, int kk, int known, int* hist, int* res,
                        uint32_t& tau, int& need) {
    kth_fn<NT>([&](int64_t i) { return keys[i]; }, m, kk, known, m > 0 ? keys[0] : 0u, hist, res,
               tau, need);
}

// Ordered compaction of slots [0, n) with keys K(i): writes the chosen slots
// ascending as V(i) at dst[off0 + ...], counting the keys equal to tau from
// eq0 (the equal keys of earlier slots outside this range).  Wave w owns a
// contiguous range of slots; within it, lanes take consecutive slots and
// ballots give every chosen slot its place.  Returns the number of slots this
// range chose.  wtmp needs 2 * NT/64 ints of LDS.  When pad is set,
// dst[total .. kk) is filled with -1.
template <int NT, class KeyFn, class ValFn>
__device__ int ordered_write_v(KeyFn K, ValFn V, int64_t n, uint32_t tau, int need, int32_t kk,
                               int32_t* dst, int* wtmp, int off0 = 0, int eq0 = 0, bool pad = true) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t per = ((n + NW - 1) / NW + 63) / 64 * 64;
    const int64_t r0 = min(n, (int64_t)w * per), r1 = min(n, r0 + per);
    int gt = 0, eq = 0;
    for (int64_t i0 = r0 + lane; i0 < r1; i0 += 4 * 64) {
        uint32_t kv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) kv[u] = (i0 + u * 64 < r1) ? K(i0 + u * 64) : 0u;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            gt += kv[u] > tau;
            eq += (kv[u] == tau) & (need > 0) & (i0 + u * 64 < r1);
        }
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
    for (int64_t j0 = r0; j0 < r1; j0 += 4 * 64) {
        uint32_t kv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = j0 + u * 64 + lane;
            kv[u] = i < r1 ? K(i) : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = j0 + u * 64 + lane;
            const bool in = i < r1;
            const bool eqf = in && need > 0 && kv[u] == tau;
            const uint64_t em = __ballot(eqf);
            const int er = eqb + lanes_below(em);
            const bool take = in && (kv[u] > tau || (eqf && er < need));
            const uint64_t sm = __ballot(take);
            const int pos = selb + lanes_below(sm);
            if (take && pos < kk) dst[pos] = V(i);
            eqb += __popcll(em);
            selb += __popcll(sm);
        }
    }
    if (pad)
        for (int i = off0 + total + tid; i < kk; i += NT) dst[i] = -1;
    __syncthreads();
    return total;
}

// ordered_write_v writing slot i as ids[i], or slot0 + i without ids.
template <int NT, class KeyFn>
__device__ int ordered_write(KeyFn K, int64_t n, uint32_t tau, int need, const int32_t* ids,
                             int32_t kk, int32_t* dst, int* wtmp, int off0 = 0, int eq0 = 0,
                             bool pad = true, int64_t slot0 = 0) {
    return ordered_write_v<NT>(
        K, [&](int64_t i) { return ids ? ids[i] : (int32_t)(slot0 + i); }, n, tau, need, kk, dst,
        wtmp, off0, eq0, pad);
}

// LDS of reg_select.
template <int NT>
struct RegSelShared {
    alignas(16) int hist[kHistWords];
    int tmp[NT / 64 + 1];
    int res[4];
};

// Top-kk of one row of n <= NT * PER slots by one workgroup, keys in
// registers: thread t owns slots [t*PER, t*PER + PER); slot i is written as
// ids[i] when IDS (ids non-null, 16-byte aligned rows), else as i.  A 12-bit histogram
// finds the boundary bucket; further 12- and 8-bit histograms of the register
// keys inside it resolve the exact (tau, need), stopping as soon as a whole
// sub-bucket completes the selection; one block scan of packed (greater,
// equal) counts then places every chosen slot, ascending.  Writes dst[0..kk),
// -1 padded.
template <int NT, int PER, bool IDS>
__device__ void reg_select(const float* s, const int32_t* ids, int n, int kk, int32_t* dst,
                           RegSelShared<NT>& sh) {
    static_assert(PER % 4 == 0, "PER must be a multiple of 4");
    const int tid = threadIdx.x;
    const int s0 = tid * PER;
    uint32_t key[PER];
    int32_t id[PER];
    // every load of the row is issued before any is used
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
        float4 f = make_float4(-__builtin_inff(), -__builtin_inff(), -__builtin_inff(),
                               -__builtin_inff());
        int4 iv = make_int4(s0 + j, s0 + j + 1, s0 + j + 2, s0 + j + 3);
        if (s0 + j + 3 < n) {
            f = *reinterpret_cast<const float4*>(s + s0 + j);
            if (IDS) iv = *reinterpret_cast<const int4*>(ids + s0 + j);
        } else {
            if (s0 + j < n) { f.x = s[s0 + j]; if (IDS) iv.x = ids[s0 + j]; }
            if (s0 + j + 1 < n) { f.y = s[s0 + j + 1]; if (IDS) iv.y = ids[s0 + j + 1]; }
            if (s0 + j + 2 < n) { f.z = s[s0 + j + 2]; if (IDS) iv.z = ids[s0 + j + 2]; }
        }
        const float v[4] = {f.x, f.y, f.z, f.w};
        const int32_t w[4] = {iv.x, iv.y, iv.z, iv.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t k = score_key(v[u]);
            key[j + u] = (k == kNegInfKey || (IDS && w[u] < 0)) ? 0u : k;
            if (IDS) id[j + u] = w[u];
        }
    }
    // A long row with a small kk first histograms a 1/8 sample (every eighth
    // key a thread holds): the bucket of the sample's ceil(1.3 kk / 8) + 8-th
    // largest key gives a floor `lo` that about 1.3 kk keys of the row reach,
    // and only those go through the full histogram and the refining passes
    // (top 256 of 16384 blocks: 11.0 -> 9.9 us).  At kk = n / 16 (2048 of
    // 32768) the extra pass costs more than the atomics it saves, so such rows
    // go whole.  The result is exact whatever the sample: if fewer than kk
    // keys reach lo, the row is histogrammed whole.
    uint32_t lo = 1u;
    if (PER >= 16 && n >= 8 * 1024 && kk * 16 < n) {  // uniform
        for (int i = tid; i < kHistWords; i += NT) sh.hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < PER; j += 8)
            if (key[j]) atomicAdd(&sh.hist[hidx((int)(key[j] >> 20))], 1);
        __syncthreads();
        if (tid < 64) wave_find_bucket(sh.hist, kHistBins, (13 * kk + 79) / 80 + 8, sh.res);
        __syncthreads();
        if (sh.res[3] >= (13 * kk + 79) / 80 + 8) lo = max((uint32_t)sh.res[0] << 20, 1u);
        __syncthreads();  // every thread has read res before the next pass writes it
    }
    for (int pass = 0; pass < 2; ++pass) {  // the second only when the floor was too high
        for (int i = tid; i < kHistWords; i += NT) sh.hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (key[j] >= lo) atomicAdd(&sh.hist[hidx((int)(key[j] >> 20))], 1);
        __syncthreads();
        if (tid < 64) wave_find_bucket(sh.hist, kHistBins, kk, sh.res);
        __syncthreads();
        if (lo == 1u || sh.res[3] >= kk) break;  // uniform
        lo = 1u;
        __syncthreads();
    }
    // keys below lo are below the kk-th key: the passes below never take them
    const int total_valid = sh.res[3];
    const uint32_t b1 = (uint32_t)sh.res[0];
    const int rem = kk - sh.res[1], cnt = sh.res[2];
    uint32_t tau = 0u;
    int need = 0;
    if (total_valid > kk && cnt != rem) {
        // resolve the boundary bucket on the register keys: 12 more bits, then
        // the last 8 unless a whole sub-bucket completes the selection
        uint32_t prefix = b1 << 20, mask = 0xFFF00000u;
        int r = rem;
        bool done = false;
        for (int shift = 8; shift >= 0 && !done; shift -= 8) {
            const int bits = shift ? 12 : 8;
            const uint32_t dm = (1u << bits) - 1u;
            for (int i = tid; i < kHistWords; i += NT) sh.hist[i] = 0;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < PER; ++j)
                if (key[j] && (key[j] & mask) == prefix)
                    atomicAdd(&sh.hist[hidx((int)((key[j] >> shift) & dm))], 1);
            __syncthreads();
            if (tid < 64) wave_find_bucket(sh.hist, 1 << bits, r, sh.res);
            __syncthreads();
            prefix |= (uint32_t)sh.res[0] << shift;
            mask |= dm << shift;
            r -= sh.res[1];
            done = sh.res[2] == r;  // the whole sub-bucket is taken
            __syncthreads();
        }
        if (done) {
            tau = prefix - 1u;  // every key >= prefix (the remaining bits are free)
            need = 0;
        } else {
            tau = prefix;
            need = r;
        }
    } else if (total_valid > kk) {
        tau = (b1 << 20) - 1u;  // the whole boundary bucket is taken
    } else {
        tau = lo - 1u;  // every key at or above the floor (every valid key when lo = 1)
    }
    // ordered write: packed counts (greater in the low 16 bits, equal in the high)
    int packed = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        packed += key[j] > tau;
        packed += ((need > 0) & (key[j] == tau)) << 16;
    }
    int total;
    const int before = block_excl_scan<NT>(packed, sh.tmp, &total);
    int e = (int)((uint32_t)before >> 16);  // packed sums wrap like unsigned
    int pos = (int)((uint32_t)before & 0xFFFFu) + min(need, e);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        bool take = key[j] > tau;
        if (need > 0 && key[j] == tau) {
            take = e < need;
            ++e;
        }
        if (take && pos < kk) dst[pos++] = IDS ? id[j] : s0 + j;
    }
    const int chosen = (int)((uint32_t)total & 0xFFFFu) + min(need, (int)((uint32_t)total >> 16));
    for (int i = chosen + tid; i < kk; i += NT) dst[i] = -1;
}

// LDS of wave_select.
template <int NT>
struct WaveSelShared {
    alignas(16) int hist[kHistWords];
    int wcnt[2 * (NT / 64)];
    int res[4];
};

// Top-kk of one row of n <= NT * PER scores by one workgroup, keys in
// registers, slot i written as ids[i] (bs > 0: as the position of slot i
// within block ids[i >> bs] of 2^bs positions).  Wave w owns slots [64 PER w,
// 64 PER (w + 1)); lane l holds slots 64 PER w + 64 j + l, so every wave has
// keys when n is near NT * PER and a wave's slots ascend in (j, l).  Scores of
// slots that can never be chosen must be -inf (key 0).
//  1. loads: scores, then ids (only the write needs them: the barriers below
//     order LDS alone, so the id loads stay in flight until then);
//  2. a 12-bit histogram of the top digit finds the boundary bucket, and
//     12- then 8-bit histograms of the register keys inside it resolve the
//     exact (tau, need), stopping as soon as a whole sub-bucket completes the
//     selection;
//  3. per-wave counts and ballots place every chosen slot, ascending.
// Writes dst[0..kk), -1 padded.  COH: the scores were handed over with
// agent-coherent stores (read with load_coherent).
template <int NT, int PER, bool COH = false>
__device__ __forceinline__ void wave_select(const float* s, const int32_t* ids, int n, int kk, int32_t* dst,
                            WaveSelShared<NT>& sh, int bs = 0) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int s0 = w * 64 * PER + lane;
    float v[PER];
    int32_t id[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j)
        v[j] = COH ? load_coherent(&s[min(s0 + 64 * j, n - 1)]) : s[min(s0 + 64 * j, n - 1)];
    // bs > 0: ids holds one block id per 2^bs slots, slot i being position
    // ids[i >> bs] * 2^bs + i % 2^bs (only slots with a finite score are
    // ever written, so an empty block's slots need no check here)
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int sl = min(s0 + 64 * j, n - 1);
        id[j] = bs ? ids[sl >> bs] * (1 << bs) + (sl & ((1 << bs) - 1)) : ids[sl];
    }
    for (int i = tid; i < kHistWords; i += NT) sh.hist[i] = 0;
    uint32_t key[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const uint32_t k = score_key(v[j]);
        key[j] = (s0 + 64 * j < n && k != kNegInfKey) ? k : 0u;
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (key[j]) atomicAdd(&sh.hist[hidx((int)(key[j] >> 20))], 1);
    lds_barrier();
    if (w == 0) wave_find_bucket(sh.hist, kHistBins, kk, sh.res);
    lds_barrier();
    const int total_valid = sh.res[3];
    const uint32_t b1 = (uint32_t)sh.res[0];
    const int rem = kk - sh.res[1], cnt = sh.res[2];
    uint32_t tau = 0u;  // total_valid <= kk: every valid key (key > 0)
    int need = 0;
    if (total_valid > kk && cnt == rem) {
        tau = (b1 << 20) - 1u;  // the whole boundary bucket is taken
    } else if (total_valid > kk) {
        // 12 more bits, then the last 8 unless a whole sub-bucket completes
        // the selection
        uint32_t prefix = b1 << 20, mask = 0xFFF00000u;
        int r = rem;
        bool done = false;
        for (int shift = 8; shift >= 0 && !done; shift -= 8) {
            const int bits = shift ? 12 : 8;
            const uint32_t dm = (1u << bits) - 1u;
            for (int i = tid; i < kHistWords; i += NT) sh.hist[i] = 0;
            lds_barrier();
#pragma unroll
            for (int j = 0; j < PER; ++j)
                if (key[j] && (key[j] & mask) == prefix)
                    atomicAdd(&sh.hist[hidx((int)((key[j] >> shift) & dm))], 1);
            lds_barrier();
            if (w == 0) wave_find_bucket(sh.hist, 1 << bits, r, sh.res);
            lds_barrier();
            prefix |= (uint32_t)sh.res[0] << shift;
            mask |= dm << shift;
            r -= sh.res[1];
            done = sh.res[2] == r;  // the whole sub-bucket is taken
            lds_barrier();
        }
        if (done) {
            tau = prefix - 1u;  // every key >= prefix (the remaining bits are free)
        } else {
            tau = prefix;
            need = r;
        }
    }
    // ordered write: per-wave (greater, equal) counts, then ballots per j
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        gt += key[j] > tau;
        eq += (need > 0) & (key[j] == tau);
    }
    gt = wave_sum_dpp(gt);
    eq = wave_sum_dpp(eq);
    if (lane == 0) {
        sh.wcnt[w] = gt;
        sh.wcnt[NW + w] = eq;
    }
    lds_barrier();
    int eqb = 0, selb = 0, total = 0, eqrun = 0;
#pragma unroll
    for (int u = 0; u < NW; ++u) {
        const int g = sh.wcnt[u], e = sh.wcnt[NW + u];
        const int take = g + min(max(need - eqrun, 0), e);
        if (u < w) selb += take;
        if (u == w) eqb = eqrun;
        total += take;
        eqrun += e;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const bool eqf = need > 0 && key[j] == tau;
        const uint64_t em = __ballot(eqf);
        const bool take = key[j] > tau || (eqf && eqb + lanes_below(em) < need);
        const uint64_t sm = __ballot(take);
        const int pos = selb + lanes_below(sm);
        if (take && pos < kk) dst[pos] = id[j];
        eqb += __popcll(em);
        selb += __popcll(sm);
    }
    for (int i = min(total, kk) + tid; i < kk; i += NT) dst[i] = -1;
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

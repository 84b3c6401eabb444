// csa2_dev.h -- device helpers shared by the gfx950 kernels of libcsa2.
// Internal header: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kHeads = 16;
constexpr int kHeadDim = 128;
constexpr int kIdxDim = 64;
constexpr int kRowBf16 = 256;   // K | V channels of one global row
constexpr int kRowCodes = 128;  // FP4 code bytes of one global row
constexpr int kRowScales = 8;   // E8M0 bytes of one global row

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Exact fp32 value of code c under block exponent E, built from bits.
// Magnitude codes 1..7 are (1 + f/2) * 2^ec with (ec, f) = (-1,0) (0,0) (0,1)
// (1,0) (1,1) (2,0) (2,1).
__device__ __forceinline__ float fp4_exact(uint32_t c, int E) {
    const uint32_t mag = c & 7u, sign = (c & 8u) << 28;
    if (mag == 0) return __uint_as_float(sign);
    const int ec = (mag == 1) ? -1 : (int)(mag >> 1) - 1;
    const uint32_t f = (mag == 1) ? 0u : (mag & 1u);
    const int be = ec + E + 127;
    uint32_t bits;
    if (be >= 255) bits = 0x7F800000u;
    else if (be >= 1) bits = ((uint32_t)be << 23) | (f << 22);
    else bits = (2u + f) << (ec + E + 148);  // subnormal
    return __uint_as_float(bits | sign);
}

// Order-preserving unsigned key of a score: a larger score gives a larger key;
// -0 and +0 give the same key.  Finite scores and +inf give keys >= 0x00800000;
// -inf gives 0x007FFFFF.  Key 0 is kept free to mark "not selectable".
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
constexpr uint32_t kNegInfKey = 0x007FFFFFu;

// Sum over groups of 8 consecutive lanes (every lane of the group gets it),
// with DPP: swap neighbours, swap pairs, then mirror within the half-row.
__device__ __forceinline__ float sum8(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
    return v;
}

// Lane l combined with lane l ^ 16 (or l ^ 32) without going through LDS:
// v_permlane16_swap / v_permlane32_swap of a value with itself leave x[l] in
// one result and x[l ^ 16] (x[l ^ 32]) in the other, in an order that
// depends on the row; max and + take them in either order.  Every lane of
// the wave must be active.  (In the prefill loop these beat an LDS
// shuffle; in the latency-bound decode kernel the shuffle measured faster.)
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS traffic).
__device__ __forceinline__ int wave_scan_dpp(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) { return wave_scan_dpp(v); }

// Exclusive scan over a whole workgroup of NT threads (NT % 64 == 0, NT <= 4096).
// `tmp` needs NT/64 + 1 ints of LDS.  Returns the exclusive prefix; *total gets
// the sum.  Contains barriers: every thread must call it.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int inc = wave_incl_scan(v);
    if (lane == 63) tmp[w] = inc;
    __syncthreads();
    if (w == 0) {
        int x = lane < NW ? tmp[lane] : 0;
        int xi = wave_incl_scan(x);
        if (lane < NW) tmp[lane] = xi - x;
        if (lane == NW - 1) tmp[NW] = xi;
    }
    __syncthreads();
    int r = tmp[w] + inc - v;
    *total = tmp[NW];
    __syncthreads();
    return r;
}

// Two exclusive scans over a whole workgroup at once (same rules as
// block_excl_scan; `tmp` needs 2 (NT/64 + 1) ints of LDS).
template <int NT>
__device__ __forceinline__ void block_excl_scan2(int a, int b, int* tmp, int (&before)[2],
                                                 int (&total)[2]) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
    if (lane == 63) {
        tmp[w] = ia;
        tmp[NW + 1 + w] = ib;
    }
    __syncthreads();
    if (w == 0) {
        const int xa = lane < NW ? tmp[lane] : 0, xb = lane < NW ? tmp[NW + 1 + lane] : 0;
        const int ya = wave_incl_scan(xa), yb = wave_incl_scan(xb);
        if (lane < NW) {
            tmp[lane] = ya - xa;
            tmp[NW + 1 + lane] = yb - xb;
        }
        if (lane == NW - 1) {
            tmp[NW] = ya;
            tmp[2 * NW + 1] = yb;
        }
    }
    __syncthreads();
    before[0] = tmp[w] + ia - a;
    before[1] = tmp[NW + 1 + w] + ib - b;
    total[0] = tmp[NW];
    total[1] = tmp[2 * NW + 1];
    __syncthreads();
}

// Workgroup barrier that orders LDS only: unlike __syncthreads it does not
// wait for the caller's global loads, so loads issued before it stay in
// flight.  For barriers that publish LDS data alone.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Last-arrival counter of a group of n workgroups, called by thread 0 after a
// barrier that follows the workgroup's stores.  The agent-scope acquire-release
// add publishes those stores (one L2 write-back on the way in) and, for the
// arrival that returns true, makes every other member's visible (one L2
// invalidate on the way out); a barrier after the call extends that to the
// whole workgroup.  The counter is reset by the last arrival's owner.
__device__ __forceinline__ bool arrive_last(uint32_t* ctr, uint32_t n) {
    return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
}

// Agent-scope relaxed atomic stores and loads: the data handed over through
// arrive_last_release is written and read with them (sc1 accesses, which
// neither leave dirty lines in a per-XCD L2 nor read a stale one); the
// release and acquire of the arrival order them.
template <typename T>
__device__ __forceinline__ void store_coherent(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ T load_coherent(const T* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until this thread's memory operations have completed.
__device__ __forceinline__ void hand_off_wait() { __builtin_amdgcn_s_waitcnt(0); }

// Last-arrival counter with the release on every arrival and the acquire
// only where it is needed: each add is a release, so it heads a release
// sequence (every later add on the counter continues it); the arrival that
// returns true has read the value of the add before it, so its acquire fence
// synchronises with every member's release.  Called by thread 0 after a
// barrier that follows the workgroup's stores; a barrier after the call
// extends the acquire to the workgroup.
__device__ __forceinline__ bool arrive_last_release(uint32_t* ctr, uint32_t n) {
    const bool last =
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return last;
}


// XCD-aware remap of a flat workgroup id: the hardware deals consecutive ids
// round-robin over the 8 XCDs; this makes each XCD own a contiguous range of
// logical ids, so neighbouring tiles share an L2.  `n` is the grid size.
__device__ __forceinline__ uint32_t xcd_swizzle(uint32_t id, uint32_t n) {
    constexpr uint32_t X = 8;
    uint32_t per = n / X;
    if (id >= per * X) return id;  // ragged tail keeps its id
    return (id % X) * per + id / X;
}

}  // namespace csa2

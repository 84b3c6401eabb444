// csa2_pack.h -- device routines of the FP4 pack and of the decode append,
// shared by the pack kernels and by the indexer scan, which can run the
// append's workgroups inside its launch.  Internal header: not part of the C
// ABI.
#pragma once

#include "csa2_dev.h"
#include "csa2_kernels.h"

namespace csa2 {

// floor(log2 |x|) of a non-zero bf16 magnitude (bits without the sign).
__device__ __forceinline__ int floor_log2_bf16(uint32_t a) {
    uint32_t e = a >> 7;
    if (e) return (int)e - 127;
    return (31 - __clz(a & 0x7Fu)) - 133;  // subnormal: m * 2^-133
}

// E2M1 magnitude code of bf16 magnitude bits `a` under block exponent E.
// With M the 8-bit significand, Y = 4 * |x| * 2^-E = M * 2^s exactly; the
// round-to-nearest-even decision points of the E2M1 grid {0, .5, 1, 1.5, 2, 3,
// 4, 6} are Y = 1, 3, 5, 7, 10, 14, 20, taken with '>' where the lower code is
// even (the tie goes down) and '>=' where the upper code is even.
__device__ __forceinline__ uint32_t e2m1_mag_code(uint32_t a, int E) {
    if (a == 0) return 0;
    uint32_t ex = a >> 7;
    uint32_t M = ex ? ((a & 0x7Fu) | 0x80u) : (a & 0x7Fu);
    int s = (ex ? (int)ex : 1) - 132 - E;
    uint32_t lhs, sh;
    if (s >= 0) {
        lhs = M << s;  // s <= 4: Y < 32
        sh = 0;
    } else {
        if (s < -8) return 0;  // Y < 1
        lhs = M;
        sh = (uint32_t)(-s);
    }
    return (uint32_t)(lhs > (1u << sh)) + (uint32_t)(lhs >= (3u << sh)) +
           (uint32_t)(lhs > (5u << sh)) + (uint32_t)(lhs >= (7u << sh)) +
           (uint32_t)(lhs > (10u << sh)) + (uint32_t)(lhs >= (14u << sh)) +
           (uint32_t)(lhs > (20u << sh));
}

// Scale: the E4M3 value (1 sign, 4 exponent bits with bias 7, 3 mantissa
// bits) nearest to amax / 6, ties to the even code, saturating at 448.
// amax / 6 is formed as a correctly rounded fp32 quotient: an exact tie of
// the E4M3 rounding needs amax = 6 h with h of 5 significant bits, and then
// the quotient is exact; otherwise amax / 6 lies at least 2^-11 (relative)
// from every E4M3 rounding boundary, far beyond fp32's rounding, so rounding
// the quotient decides as rounding the exact value would.
__device__ __forceinline__ uint32_t e4m3_code_of(float x) {  // x >= 0, finite
    const uint32_t b = __float_as_uint(x);
    if (x < 0.015625f) {  // below 2^-6: multiples of 2^-9, round to nearest even
        const float m = __builtin_rintf(x * 512.0f);  // exact scaling
        return (uint32_t)m;                           // 8 gives 0x08 = 2^-6
    }
    // keep 3 mantissa bits, round to nearest even, rebias 127 -> 7
    const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
    const uint32_t code = (r >> 20) - (120u << 3);
    return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
    const uint32_t e = (code >> 3) & 15u, m = code & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// Scale code of a 16-element block from the bf16 magnitude bits of its amax.
__device__ __forceinline__ uint32_t e4m3_block_scale(uint32_t amax_bits) {
    const float a = __uint_as_float(amax_bits << 16);
    return e4m3_code_of(__fdiv_rn(a, 6.0f));
}

// E2M1 magnitude code of bf16 magnitude bits `a` under scale s: the nearest
// grid value c * s, ties to the even code.  The decision points are 0.25,
// 0.75, 1.25, 1.75, 2.5, 3.5 and 5 times s; each product has at most 7
// significant bits, so the fp32 comparisons are exact.  s = 0 gives 0.
__device__ __forceinline__ uint32_t e2m1_code_scaled(uint32_t a, float s) {
    if (s == 0.f) return 0u;
    const float y = __uint_as_float(a << 16);
    return (uint32_t)(y > 0.25f * s) + (uint32_t)(y >= 0.75f * s) + (uint32_t)(y > 1.25f * s) +
           (uint32_t)(y >= 1.75f * s) + (uint32_t)(y > 2.5f * s) + (uint32_t)(y >= 3.5f * s) +
           (uint32_t)(y > 5.f * s);
}

// ---- decode append ("CED", section "Why Prefill Recomputes a Recent
// Segment": after a token is chosen, every layer updates its local state and
// the global KV of the new position is appended); also the ring rows of a
// replayed segment ("Why Prefill Recomputes a Recent Segment"), where every
// row belongs to one sequence.  Work items (rows, 1 + layer groups), one
// workgroup each: (b, 0) packs (or copies) row b's global K | V, one element
// per thread, and copies its indexer key; in (b, g > 0) each wave copies one
// 256-byte local row (K or V of one layer), 4 bytes per lane, so the ring
// descriptor is wave-uniform.  Every thread issues the position load and its
// source load before it waits for either (`hold`), so the work costs about
// two memory round trips.
constexpr int kAppendLayersPerWg = 2;

template <typename T>
__device__ __forceinline__ void hold(T& x) {
    static_assert(sizeof(T) % 4 == 0, "32-bit words");
    uint32_t* w = reinterpret_cast<uint32_t*>(&x);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) asm volatile("" : "+v"(w[i]));
}

__device__ __forceinline__ void append_rows(const AppendArgs& a, int b, int g) {
    const int tid = threadIdx.x;
    const int64_t sb = a.seq >= 0 ? a.seq : b;  // the row's sequence
    if (g == 0) {
        if (a.q_seq_out && tid == 0) a.q_seq_out[b] = (int32_t)sb;
        // one element of the K | V row per thread: the 32 lanes of a block
        // reduce its largest magnitude and OR their nibbles into code words,
        // so the pack costs a few dozen instructions of latency
        int32_t p = a.pos[b];
        uint32_t x = 0;
        uint4 ki = make_uint4(0u, 0u, 0u, 0u);
        // entries of 2^msh positions: only a position completing its group
        // writes the group's entry
        if (a.kv) x = a.kv[(int64_t)b * 256 + tid];
        if (a.kidx && tid < 8) ki = reinterpret_cast<const uint4*>(a.kidx + (int64_t)b * 64)[tid];
        hold(x);
        hold(ki);
        hold(p);
        if (p < 0 || p >= (a.t_cap << a.msh) || ((p + 1) & ((1 << a.msh) - 1)) != 0) return;
        const int64_t row = sb * a.t_cap + ((p + 1) >> a.msh) - 1;
        if (a.kidx && tid < 8) reinterpret_cast<uint4*>(a.k_idx + row * 64)[tid] = ki;
        if (!a.kv) return;
        if (!a.fp4) {
            a.bf16[row * 256 + tid] = (uint16_t)x;
            return;
        }
        const uint32_t mag = x & 0x7FFFu;
        uint32_t code;
        if (a.fp4 == 2) {  // E4M3 per 16: 16-lane blocks
            uint32_t amax = mag;
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, m, 16));
            const uint32_t sc = e4m3_block_scale(amax);
            code = e2m1_code_scaled(mag, e4m3_to_f32(sc));
            if ((tid & 15) == 0) a.scales[row * 16 + (tid >> 4)] = (uint8_t)sc;
        } else {  // E8M0 per 32
            uint32_t amax = mag;
#pragma unroll
            for (int m = 1; m < 32; m <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, m, 32));
            int E = -127;
            if (amax) E = min(max(floor_log2_bf16(amax) - 2, -127), 127);
            code = e2m1_mag_code(mag, E);
            if ((tid & 31) == 0) a.scales[row * 8 + (tid >> 5)] = (uint8_t)(E + 127);
        }
        // channel 8m + c of the row sits in nibble c of code word m
        uint32_t word = (code | ((x >> 15) << 3)) << (4 * (tid & 7));
#pragma unroll
        for (int m = 1; m < 8; m <<= 1) word |= (uint32_t)__shfl_xor((int)word, m, 32);
        if ((tid & 7) == 0) reinterpret_cast<uint32_t*>(a.codes + row * 128)[tid >> 3] = word;
        return;
    }
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = (g - 1) * kAppendLayersPerWg + (wave >> 1);
    if (l >= a.n_local) return;
    const AppendLocal& L = a.local[l];
    const bool isv = wave & 1;
    const uint32_t* src = reinterpret_cast<const uint32_t*>((isv ? L.v_new : L.k_new) + (int64_t)b * 128);
    uint32_t* dst = reinterpret_cast<uint32_t*>(isv ? L.v : L.k);
    const int32_t cap = L.cap;
    const int lane = tid & 63;
    int32_t p = a.pos[b];
    uint32_t v = src[lane];
    hold(v);
    hold(p);
    if (p < 0 || p >= (a.t_cap << a.msh)) return;
    const int64_t slot = sb * cap + p % cap;
    dst[slot * 64 + lane] = v;
}

}  // namespace csa2

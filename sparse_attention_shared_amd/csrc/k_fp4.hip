// k_fp4.hip -- FP4 (E2M1 elements, one E8M0 scale per 32) pack and exact unpack.
//
// Format: the main cache is FP4 with E2M1 elements ("DeepSeek-V4.1 Flash Pushes
// KV Cache Compression for Agent Workloads", draft article); the scale of each
// 32-element block is a power of two stored as a biased 8-bit exponent.
// Pack rule: E = clamp(floor(log2 amax) - 2, -127, 127), so the block's largest
// magnitude lands in E2M1's top binade [4, 8); each element becomes the nearest
// E2M1 magnitude of |x| * 2^-E, ties to the even code, saturating at 6; the
// sign bit is kept.  All of it is done in integer arithmetic on the bf16 bits,
// so no float rounding mode or denormal setting can change a code.
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

// One 32-element block: 16 words of bf16 pairs in, 16 B of codes and the
// scale byte out.
__device__ __forceinline__ void pack_block(const uint32_t (&w)[16], uint4& codes, uint8_t& scale) {
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        amax = max(amax, w[i] & 0x7FFFu);
        amax = max(amax, (w[i] >> 16) & 0x7FFFu);
    }
    int E = -127;
    if (amax) E = min(max(floor_log2_bf16(amax) - 2, -127), 127);
    uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        uint32_t lo = w[i] & 0xFFFFu, hi = w[i] >> 16;
        uint32_t c0 = e2m1_mag_code(lo & 0x7FFFu, E) | ((lo >> 15) << 3);
        uint32_t c1 = e2m1_mag_code(hi & 0x7FFFu, E) | ((hi >> 15) << 3);
        out[i >> 2] |= (c0 | (c1 << 4)) << (8 * (i & 3));
    }
    codes = make_uint4(out[0], out[1], out[2], out[3]);
    scale = (uint8_t)(E + 127);
}

__device__ __forceinline__ void load_block(const uint16_t* x, uint32_t (&w)[16]) {
    const uint4* src = reinterpret_cast<const uint4*>(x);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 v = src[i];
        w[4 * i + 0] = v.x;
        w[4 * i + 1] = v.y;
        w[4 * i + 2] = v.z;
        w[4 * i + 3] = v.w;
    }
}

// One thread per 32-element block: 64 B of bf16 in, 16 B of codes + 1 scale out.
__global__ __launch_bounds__(256) void k_pack_fp4(const uint16_t* __restrict__ x, int64_t nblk,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblk) return;
    uint32_t w[16];
    load_block(x + b * 32, w);
    uint4 c;
    uint8_t sc;
    pack_block(w, c, sc);
    reinterpret_cast<uint4*>(codes)[b] = c;
    scales[b] = sc;
}

// ---- FP4 with one E4M3 scale per 16 channels (the pages' own cache form,
// "DeepSeek-V4.1 Flash Pushes KV Cache Compression for Agent Workloads").
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

// One thread per 16-element block: 32 B of bf16 in, 8 B of codes + 1 scale out.
__global__ __launch_bounds__(256) void k_pack_fp4e(const uint16_t* __restrict__ x, int64_t nblk,
                                                   uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblk) return;
    const uint4* src = reinterpret_cast<const uint4*>(x + b * 16);
    const uint4 v0 = src[0], v1 = src[1];
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        amax = max(amax, w[i] & 0x7FFFu);
        amax = max(amax, (w[i] >> 16) & 0x7FFFu);
    }
    const uint32_t sc = e4m3_block_scale(amax);
    const float s = e4m3_to_f32(sc);
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t lo = w[i] & 0xFFFFu, hi = w[i] >> 16;
        const uint32_t c0 = e2m1_code_scaled(lo & 0x7FFFu, s) | ((lo >> 15) << 3);
        const uint32_t c1 = e2m1_code_scaled(hi & 0x7FFFu, s) | ((hi >> 15) << 3);
        out[i >> 2] |= (c0 | (c1 << 4)) << (8 * (i & 3));
    }
    reinterpret_cast<uint2*>(codes)[b] = make_uint2(out[0], out[1]);
    scales[b] = (uint8_t)sc;
}

// Exact: an E2M1 value (2 significant bits) times an E4M3 scale (4) is an
// fp32 product without rounding.
__global__ __launch_bounds__(256) void k_unpack_fp4e(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales,
                                                     int64_t nblk, float* __restrict__ out) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblk) return;
    const uint2 c = reinterpret_cast<const uint2*>(codes)[b];
    const float s = e4m3_to_f32(scales[b]);
    const uint32_t w[2] = {c.x, c.y};
    const float mag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
    float4* dst = reinterpret_cast<float4*>(out) + b * 4;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t q = (w[i] >> (4 * j)) & 15u;
            const float m = mag[q & 7u] * s;
            v[j] = (q & 8u) ? -m : m;
        }
        dst[2 * i] = make_float4(v[0], v[1], v[2], v[3]);
        dst[2 * i + 1] = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// ---- decode append ("CED", section "Why Prefill Recomputes a Recent
// Segment": after a token is chosen, every layer updates its local state and
// the global KV of the new position is appended); also the ring rows of a
// replayed segment ("Why Prefill Recomputes a Recent Segment"), where every
// row belongs to one sequence.  Grid (rows, 1 + layer groups): workgroup
// (b, 0) packs (or copies) row b's global K | V, one element per thread, and
// copies its indexer key; in workgroup (b, g > 0) each wave copies one
// 256-byte local row (K or V of one layer), 4 bytes per lane, so the ring
// descriptor is wave-uniform.  Every thread issues the position load and its source load
// before it waits for either (`hold`), so a launch costs about two memory
// round trips.
constexpr int kAppendLayersPerWg = 2;

template <typename T>
__device__ __forceinline__ void hold(T& x) {
    static_assert(sizeof(T) % 4 == 0, "32-bit words");
    uint32_t* w = reinterpret_cast<uint32_t*>(&x);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) asm volatile("" : "+v"(w[i]));
}

__global__ __launch_bounds__(256) void k_append(AppendArgs a) {
    const int b = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
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

hipError_t launch_append(const AppendArgs& a, int32_t n_rows, hipStream_t s) {
    if (n_rows == 0) return hipSuccess;
    const uint32_t groups = (uint32_t)((a.n_local + kAppendLayersPerWg - 1) / kAppendLayersPerWg);
    hipLaunchKernelGGL(k_append, dim3((uint32_t)n_rows, 1 + groups), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---- sequence compression ("CED", section "What Does the Sequence
// Compression Rate Reduce?": with rate m the information of m positions is
// combined into one entry; the combine rule is not given, the element-wise
// mean is the reading taken).  One thread per 8 channels of a group.  For
// m = 2: a + b in fp32 is exact unless the exponents differ by more than 15,
// and then the sum lies within 2^-16 (relative) of a value bf16 represents,
// far from any bf16 rounding tie, so halving and rounding to bf16 once gives
// the correctly rounded mean.
__global__ __launch_bounds__(256) void k_compress(const uint16_t* __restrict__ x, int64_t n8,
                                                  int32_t m, int32_t dim, uint16_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 8-channel piece of the output
    if (i >= n8) return;
    const int64_t per = dim / 8;
    const int64_t g = i / per, c = i % per;
    const uint4* src = reinterpret_cast<const uint4*>(x + g * m * dim) + c;
    uint4 a = src[0];
    if (m == 2) {
        const uint4 b = src[per];
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
        uint32_t r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float lo = (__uint_as_float(aw[j] << 16) + __uint_as_float(bw[j] << 16)) * 0.5f;
            const float hi = (__uint_as_float(aw[j] & 0xFFFF0000u) + __uint_as_float(bw[j] & 0xFFFF0000u)) * 0.5f;
            r[j] = (uint32_t)f_to_bf16(lo) | ((uint32_t)f_to_bf16(hi) << 16);
        }
        a = make_uint4(r[0], r[1], r[2], r[3]);
    }
    reinterpret_cast<uint4*>(out + g * dim)[c] = a;
}

hipError_t launch_compress(const uint16_t* x, int64_t groups, int32_t m, int32_t dim, uint16_t* out,
                           hipStream_t s) {
    const int64_t n8 = groups * (dim / 8);
    if (n8 == 0) return hipSuccess;
    hipLaunchKernelGGL(k_compress, dim3((uint32_t)((n8 + 255) / 256)), dim3(256), 0, s, x, n8, m, dim,
                       out);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_unpack_fp4(const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ scales,
                                                    int64_t nblk, float* __restrict__ out) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblk) return;
    const uint4 c = reinterpret_cast<const uint4*>(codes)[b];
    const int E = (int)scales[b] - 127;
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float4* dst = reinterpret_cast<float4*>(out) + b * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = fp4_exact((w[i] >> (4 * j)) & 15u, E);
        dst[2 * i] = make_float4(v[0], v[1], v[2], v[3]);
        dst[2 * i + 1] = make_float4(v[4], v[5], v[6], v[7]);
    }
}

hipError_t launch_pack_fp4(const uint16_t* x, int64_t nblk, uint8_t* codes, uint8_t* scales,
                           hipStream_t s) {
    if (nblk == 0) return hipSuccess;
    const int64_t grid = (nblk + 255) / 256;
    hipLaunchKernelGGL(k_pack_fp4, dim3((uint32_t)grid), dim3(256), 0, s, x, nblk, codes, scales);
    return hipGetLastError();
}

hipError_t launch_pack_fp4e(const uint16_t* x, int64_t nblk, uint8_t* codes, uint8_t* scales,
                            hipStream_t s) {
    if (nblk == 0) return hipSuccess;
    const int64_t grid = (nblk + 255) / 256;
    hipLaunchKernelGGL(k_pack_fp4e, dim3((uint32_t)grid), dim3(256), 0, s, x, nblk, codes, scales);
    return hipGetLastError();
}

hipError_t launch_unpack_fp4e(const uint8_t* codes, const uint8_t* scales, int64_t nblk, float* out,
                              hipStream_t s) {
    if (nblk == 0) return hipSuccess;
    const int64_t grid = (nblk + 255) / 256;
    hipLaunchKernelGGL(k_unpack_fp4e, dim3((uint32_t)grid), dim3(256), 0, s, codes, scales, nblk,
                       out);
    return hipGetLastError();
}

hipError_t launch_unpack_fp4(const uint8_t* codes, const uint8_t* scales, int64_t nblk, float* out,
                             hipStream_t s) {
    if (nblk == 0) return hipSuccess;
    const int64_t grid = (nblk + 255) / 256;
    hipLaunchKernelGGL(k_unpack_fp4, dim3((uint32_t)grid), dim3(256), 0, s, codes, scales, nblk,
                       out);
    return hipGetLastError();
}

}  // namespace csa2

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
        if (a.kv) x = a.kv[(int64_t)b * 256 + tid];
        if (a.kidx && tid < 8) ki = reinterpret_cast<const uint4*>(a.kidx + (int64_t)b * 64)[tid];
        hold(x);
        hold(ki);
        hold(p);
        if (p < 0 || p >= a.t_cap) return;
        const int64_t row = sb * a.t_cap + p;
        if (a.kidx && tid < 8) reinterpret_cast<uint4*>(a.k_idx + row * 64)[tid] = ki;
        if (!a.kv) return;
        if (!a.fp4) {
            a.bf16[row * 256 + tid] = (uint16_t)x;
            return;
        }
        const uint32_t mag = x & 0x7FFFu;
        uint32_t amax = mag;
#pragma unroll
        for (int m = 1; m < 32; m <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, m, 32));
        int E = -127;
        if (amax) E = min(max(floor_log2_bf16(amax) - 2, -127), 127);
        // channel 8m + c of the block sits in nibble c of code word m
        uint32_t word = (e2m1_mag_code(mag, E) | ((x >> 15) << 3)) << (4 * (tid & 7));
#pragma unroll
        for (int m = 1; m < 8; m <<= 1) word |= (uint32_t)__shfl_xor((int)word, m, 32);
        if ((tid & 7) == 0) reinterpret_cast<uint32_t*>(a.codes + row * 128)[tid >> 3] = word;
        if ((tid & 31) == 0) a.scales[row * 8 + (tid >> 5)] = (uint8_t)(E + 127);
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
    if (p < 0 || p >= a.t_cap) return;
    const int64_t slot = sb * cap + p % cap;
    dst[slot * 64 + lane] = v;
}

hipError_t launch_append(const AppendArgs& a, int32_t n_rows, hipStream_t s) {
    if (n_rows == 0) return hipSuccess;
    const uint32_t groups = (uint32_t)((a.n_local + kAppendLayersPerWg - 1) / kAppendLayersPerWg);
    hipLaunchKernelGGL(k_append, dim3((uint32_t)n_rows, 1 + groups), dim3(256), 0, s, a);
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

hipError_t launch_unpack_fp4(const uint8_t* codes, const uint8_t* scales, int64_t nblk, float* out,
                             hipStream_t s) {
    if (nblk == 0) return hipSuccess;
    const int64_t grid = (nblk + 255) / 256;
    hipLaunchKernelGGL(k_unpack_fp4, dim3((uint32_t)grid), dim3(256), 0, s, codes, scales, nblk,
                       out);
    return hipGetLastError();
}

}  // namespace csa2

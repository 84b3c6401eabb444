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

// One thread per 32-element block: 64 B of bf16 in, 16 B of codes + 1 scale out.
__global__ __launch_bounds__(256) void k_pack_fp4(const uint16_t* __restrict__ x, int64_t nblk,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblk) return;
    const uint4* src = reinterpret_cast<const uint4*>(x) + b * 4;
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint4 v = src[i];
        w[4 * i + 0] = v.x;
        w[4 * i + 1] = v.y;
        w[4 * i + 2] = v.z;
        w[4 * i + 3] = v.w;
    }
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
    reinterpret_cast<uint4*>(codes)[b] = make_uint4(out[0], out[1], out[2], out[3]);
    scales[b] = (uint8_t)(E + 127);
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

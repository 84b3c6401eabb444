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
#include "csa2_pack.h"

namespace csa2 {

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

// ---- decode append: the work itself (append_rows) is in csa2_pack.h, shared
// with the indexer scan that can run it in the same launch.
__global__ __launch_bounds__(256) void k_append(AppendArgs a) { append_rows(a, blockIdx.x, blockIdx.y); }

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

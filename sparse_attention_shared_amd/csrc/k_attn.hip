// k_attn.hip -- sparse attention of 16 query heads over the selected global
// entries joined with the layer's local window, in one softmax ("CED:
// Continuing Context with a Causal Encoder and Decoder", section "Selecting
// Positions and Reading Values with Attention", Fig. 4; global entries come
// from the shared cache, window entries from the layer's own local KV,
// section "Shared Global KV and Per-Layer Local KV", Fig. 3).
//
// Split-K: the entry list of a query (k selected slots, then the window) is
// cut into chunks of 64; one workgroup per (chunk, query) gathers its rows,
// dequantises FP4 exactly into LDS, and writes an unnormalised partial
// (max, sum, P.V) per head; a merge kernel combines the chunks in a fixed
// order, so results do not depend on scheduling.
#include "csa2_dev.h"
#include "csa2_kernels.h"

namespace csa2 {

constexpr int kAttnChunk = 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void store32(float* dst, const float* v) {
#pragma unroll
    for (int i = 0; i < 32; i += 4)
        *reinterpret_cast<float4*>(dst + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
}

// 32 bf16 (64 B) -> 32 floats
__device__ __forceinline__ void bf16x32(const uint16_t* src, float* v) {
    const uint4* p = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 w = p[i];
        v[8 * i + 0] = bf16_lo(w.x); v[8 * i + 1] = bf16_hi(w.x);
        v[8 * i + 2] = bf16_lo(w.y); v[8 * i + 3] = bf16_hi(w.y);
        v[8 * i + 4] = bf16_lo(w.z); v[8 * i + 5] = bf16_hi(w.z);
        v[8 * i + 6] = bf16_lo(w.w); v[8 * i + 7] = bf16_hi(w.w);
    }
}

// 32 FP4 codes (16 B) under one E8M0 scale -> 32 floats, exact
__device__ __forceinline__ void fp4x32(const uint8_t* codes, uint8_t scale, float* v) {
    const uint4 c = *reinterpret_cast<const uint4*>(codes);
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    const int E = (int)scale - 127;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[8 * i + j] = fp4_exact((w[i] >> (4 * j)) & 15u, E);
}

// grid: (n_split, nq), 256 threads.
__global__ __launch_bounds__(256) void k_attn_split(CacheView c, const uint16_t* __restrict__ q,
                                                    const int32_t* __restrict__ q_pos,
                                                    const int32_t* __restrict__ q_seq,
                                                    const int32_t* __restrict__ sel, int32_t k,
                                                    LocalView loc, float sm_scale, int32_t n_split,
                                                    float* __restrict__ ws_o,
                                                    float* __restrict__ ws_ml) {
    __shared__ float qs[kHeads][kHeadDim];
    __shared__ float Ks[kAttnChunk][kHeadDim + 1];
    __shared__ float Vs[kAttnChunk][kHeadDim];
    __shared__ float P[kHeads][kAttnChunk];
    __shared__ int valid[kAttnChunk];

    const int qi = blockIdx.y, split = blockIdx.x, tid = threadIdx.x;
    const int32_t seq = q_seq ? q_seq[qi] : qi;
    int64_t t = q_pos[qi];
    if (seq < 0 || seq >= c.n_seq) t = -1;
    if (t >= c.t_cap) t = c.t_cap - 1;
    int64_t w0 = t - loc.window + 1;
    if (w0 < loc.lo) w0 = loc.lo;
    if (w0 < 0) w0 = 0;
    const int64_t nw = (loc.window > 0 && t >= w0) ? t - w0 + 1 : 0;

    // Main Q of this query -> LDS
    {
        const uint16_t* qrow = q + (int64_t)qi * kHeads * kHeadDim;
        const uint4 w = reinterpret_cast<const uint4*>(qrow)[tid];
        float* d = &qs[0][0] + tid * 8;
        d[0] = bf16_lo(w.x); d[1] = bf16_hi(w.x); d[2] = bf16_lo(w.y); d[3] = bf16_hi(w.y);
        d[4] = bf16_lo(w.z); d[5] = bf16_hi(w.z); d[6] = bf16_lo(w.w); d[7] = bf16_hi(w.w);
    }
    // Gather + dequantise: thread -> (entry e, 32-channel part p) of K and V
    {
        const int e = tid >> 2, p = tid & 3;
        const int64_t ge = (int64_t)split * kAttnChunk + e;
        float kv[32], vv[32];
        bool ok = false;
        if (ge < k) {
            const int64_t j = sel[(int64_t)qi * k + ge];
            if (j >= 0 && j <= t) {
                ok = true;
                const int64_t row = (int64_t)seq * c.t_cap + j;
                if (c.fp4) {
                    const uint8_t* cr = static_cast<const uint8_t*>(c.data) + row * kRowCodes;
                    const uint8_t* sr = c.scales + row * kRowScales;
                    fp4x32(cr + 16 * p, sr[p], kv);
                    fp4x32(cr + 64 + 16 * p, sr[4 + p], vv);
                } else {
                    const uint16_t* br = static_cast<const uint16_t*>(c.data) + row * kRowBf16;
                    bf16x32(br + 32 * p, kv);
                    bf16x32(br + kHeadDim + 32 * p, vv);
                }
            }
        } else if (ge - k < nw) {
            ok = true;
            const int64_t pos = w0 + (ge - k);
            const int64_t slot = (int64_t)seq * loc.cap + pos % loc.cap;
            bf16x32(loc.k + slot * kHeadDim + 32 * p, kv);
            bf16x32(loc.v + slot * kHeadDim + 32 * p, vv);
        }
        if (!ok) {
#pragma unroll
            for (int i = 0; i < 32; ++i) kv[i] = vv[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) Ks[e][32 * p + i] = kv[i];
        store32(&Vs[e][32 * p], vv);
        if (p == 0) valid[e] = ok;
    }
    __syncthreads();

    // Logits and chunk softmax: wave hg owns heads 4hg..4hg+3, lane = entry.
    const int lane = tid & 63, hg = tid >> 6;
    const float zs = sm_scale * kLog2e;
    float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int d = 0; d < kHeadDim; ++d) {
        const float kd = Ks[lane][d];
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = fmaf(qs[4 * hg + i][d], kd, z[i]);
    }
    const bool ok = valid[lane];
    float mh[4], lh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float zi = ok ? z[i] * zs : -__builtin_inff();
        float m = zi;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        const float pi = (ok && m != -__builtin_inff()) ? exp2f(zi - m) : 0.f;
        float l = pi;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
        P[4 * hg + i][lane] = pi;
        mh[i] = m;
        lh[i] = l;
    }
    if (lane == 0) {
        float* ml = ws_ml + (((int64_t)qi * n_split + split) * kHeads + 4 * hg) * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ml[2 * i] = mh[i];
            ml[2 * i + 1] = lh[i];
        }
    }
    __syncthreads();

    // P.V: thread -> channel d, heads 8hh..8hh+7
    const int d = tid & 127, hh = tid >> 7;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int e = 0; e < kAttnChunk; ++e) {
        const float v = Vs[e][d];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(P[8 * hh + i][e], v, acc[i]);
    }
    float* o = ws_o + (((int64_t)qi * n_split + split) * kHeads + 8 * hh) * kHeadDim + d;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i * kHeadDim] = acc[i];
}

// grid: (8, nq), 256 threads: two heads per workgroup, one channel per thread.
__global__ __launch_bounds__(256) void k_attn_merge(const float* __restrict__ ws_o,
                                                    const float* __restrict__ ws_ml,
                                                    int32_t n_split, uint16_t* __restrict__ out) {
    const int qi = blockIdx.y, h = blockIdx.x * 2 + (threadIdx.x >> 7), d = threadIdx.x & 127;
    const float* ml = ws_ml + (int64_t)qi * n_split * kHeads * 2;
    float M = -__builtin_inff();
    for (int s = 0; s < n_split; ++s) M = fmaxf(M, ml[(s * kHeads + h) * 2]);
    float L = 0.f, O = 0.f;
    if (M != -__builtin_inff()) {
        for (int s = 0; s < n_split; ++s) {
            const float m = ml[(s * kHeads + h) * 2];
            if (m == -__builtin_inff()) continue;
            const float f = exp2f(m - M);
            L = fmaf(ml[(s * kHeads + h) * 2 + 1], f, L);
            O = fmaf(ws_o[(((int64_t)qi * n_split + s) * kHeads + h) * kHeadDim + d], f, O);
        }
    }
    const float r = L > 0.f ? O / L : 0.f;
    out[((int64_t)qi * kHeads + h) * kHeadDim + d] = f_to_bf16(r);
}

static int32_t attn_splits(int32_t k, int32_t window) {
    return (k + window + kAttnChunk - 1) / kAttnChunk;
}

size_t attn_ws_bytes(int32_t nq, int32_t k, int32_t window) {
    const int64_t ns = attn_splits(k, window);
    return (size_t)nq * ns * kHeads * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_sparse_attn(const CacheView& c, const uint16_t* q, const int32_t* q_pos,
                              const int32_t* q_seq, int32_t nq, const int32_t* sel, int32_t k,
                              const LocalView& loc, float sm_scale, uint16_t* out, void* ws,
                              hipStream_t s) {
    if (nq == 0) return hipSuccess;
    const int32_t ns = attn_splits(k, loc.window);
    float* ws_o = static_cast<float*>(ws);
    float* ws_ml = ws_o + (size_t)nq * ns * kHeads * kHeadDim;
    if (ns > 0)
        hipLaunchKernelGGL(k_attn_split, dim3((uint32_t)ns, (uint32_t)nq), dim3(256), 0, s, c, q,
                           q_pos, q_seq, sel, k, loc, sm_scale, ns, ws_o, ws_ml);
    hipLaunchKernelGGL(k_attn_merge, dim3(8, (uint32_t)nq), dim3(256), 0, s, ws_o, ws_ml, ns, out);
    return hipGetLastError();
}

}  // namespace csa2

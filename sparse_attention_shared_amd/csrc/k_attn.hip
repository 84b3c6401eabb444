// k_attn.hip -- sparse attention of 16 query heads over the selected global
// entries joined with the layer's local window, in one softmax ("CED:
// Continuing Context with a Causal Encoder and Decoder", section "Selecting
// Positions and Reading Values with Attention", Fig. 4; global entries come
// from the shared cache, window entries from the layer's own local KV,
// section "Shared Global KV and Per-Layer Local KV", Fig. 3).
//
// All 16 heads read the same K/V row (one KV head), so per entry block the
// work is two small dense products: S = K Q^T (16 entries x 16 heads, K = 128
// dims) and O += P V (16 heads x 16 dims, K = 32 entries).  Both run on
// v_mfma_f32_16x16x32_bf16.  FP4 rows are dequantised with their E8M0 scale by
// v_cvt_scalef32_pk_bf16_fp4: an E2M1 value times a power of two is exact in
// bf16 (every scale a 32-channel block can carry keeps the result in range),
// so both products take plain bf16 operands.
//
// Work split (few queries): a query's selected entries are cut into chunks of
// 256 and its window entries spread evenly over the same chunks (at most 32
// each), one workgroup per chunk: 8 waves on 32 selected entries each plus a
// ninth on the chunk's window entries.  Each wave loads, dequantises and
// scores its entries (S and its V^T tile); the softmax uses the workgroup's
// maximum per head, and P^T goes through LDS so that each of the 8 selection
// waves forms O for 16 of the 128 dims over all of the chunk's entries -- no
// wave ever holds a full 16 x 128 O that would have to be summed across
// waves.  Every chunk writes its partial (max, sum, unnormalised O per head)
// to the workspace and the last chunk to finish (a per-query counter)
// combines all of them in chunk order, so results do not depend on
// scheduling.
#include <hip/hip_ext.h>

#include <atomic>

#include "csa2_dev.h"
#include "csa2_kernels.h"

namespace csa2 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kSelWaves = 8;                  // waves on selected entries
constexpr int kWaves = kSelWaves + 1;         // + one wave on the chunk's window entries
constexpr int kThreads = kWaves * 64;
constexpr int kBlk = 32;                      // entries per wave
constexpr int kWgEntries = kSelWaves * kBlk;  // selected entries per workgroup
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
    u32x4_t v = {a, b, c, d};
    return __builtin_bit_cast(bf16x8_t, v);
}

// 2^(byte - 127) as fp32 (exact; byte 0 gives the subnormal 2^-127, kept
// since fp32 denormals are not flushed).
__device__ __forceinline__ float e8m0_value(uint32_t byte) {
    return __builtin_amdgcn_ldexpf(1.0f, (int)byte - 127);
}

// A decode scale split for the hardware conversion, which applies only the
// power-of-two part of its fp32 scale (it is built for E8M0 blocks): codes
// are converted with p2 and the rest of the scale, mult, is applied after.
struct DqScale {
    float p2, mult;
};

// An E4M3 byte (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
// exponent field 0: m/8 * 2^-6) as p2 * mult: 2^(e-7) * (1 + m/8), or
// 2^-9 * m for the subnormals.  Scales are never negative or NaN (the packer
// writes 0x00..0x7E).
__device__ __forceinline__ DqScale e4m3_split(uint32_t byte) {
    const uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
    DqScale d;
    d.p2 = __uint_as_float(e ? (e + 120u) << 23 : (118u << 23));  // 2^(e-7), or 2^-9
    d.mult = e ? 1.f + 0.125f * (float)m : (float)m;
    return d;
}

// An E4M3 byte as fp32 (exact).
__device__ __forceinline__ float e4m3_value(uint32_t byte) {
    const DqScale d = e4m3_split(byte);
    return d.p2 * d.mult;
}

// Scale formats of an FP4 cache (template parameter SF): 0 = one E8M0 byte
// per 32 channels (8 bytes a row), 1 = one E4M3 byte per 16 channels (16
// bytes a row).  Lane group g decodes dims 32 g .. + 32 of K and of V, i.e.
// one E8M0 block or two E4M3 blocks; row_scales gives the lane's scale bits
// (one byte, or two bytes: dims 32 g .. + 16 in the low one) and dw_scale the
// multiplier of code dword kb (dims 32 g + 8 kb .. + 8).
template <int SF>
__device__ __forceinline__ constexpr int row_scale_bytes() { return SF ? 16 : 8; }

template <int SF>
__device__ __forceinline__ constexpr uint32_t unit_scale_bits() { return SF ? 0x3838u : 127u; }

template <int SF>
__device__ __forceinline__ void row_scales(const uint8_t* sp, int g, uint32_t& sk, uint32_t& sv) {
    if (SF == 0) {
        const uint2 sc = *reinterpret_cast<const uint2*>(sp);
        sk = (sc.x >> (8 * g)) & 0xFFu;
        sv = (sc.y >> (8 * g)) & 0xFFu;
    } else {
        const uint4 sc = *reinterpret_cast<const uint4*>(sp);
        sk = ((g < 2 ? sc.x : sc.y) >> (16 * (g & 1))) & 0xFFFFu;
        sv = ((g < 2 ? sc.z : sc.w) >> (16 * (g & 1))) & 0xFFFFu;
    }
}

// The dwords of a row's scales that hold the lane's K and V blocks, loaded
// as they are (row_scale_bits takes the lane's bits out of them).
template <int SF>
__device__ __forceinline__ void row_scale_words(const uint8_t* sp, int g, uint32_t& wk, uint32_t& wv) {
    if (SF == 0) {
        const uint2 sc = *reinterpret_cast<const uint2*>(sp);
        wk = sc.x;
        wv = sc.y;
    } else {
        wk = *reinterpret_cast<const uint32_t*>(sp + 4 * (g >> 1));
        wv = *reinterpret_cast<const uint32_t*>(sp + 8 + 4 * (g >> 1));
    }
}

template <int SF>
__device__ __forceinline__ uint32_t row_scale_bits(uint32_t w, int g) {
    return SF ? (w >> (16 * (g & 1))) & 0xFFFFu : (w >> (8 * g)) & 0xFFu;
}

template <int SF>
__device__ __forceinline__ DqScale dw_scale(uint32_t bits, int kb) {
    if (SF == 0) return DqScale{e8m0_value(bits), 1.f};
    return e4m3_split(kb < 2 ? (bits & 0xFFu) : (bits >> 8));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return (uint32_t)f_to_bf16(a) | ((uint32_t)f_to_bf16(b) << 16);
}

// ---- shared by both attention kernels --------------------------------------
// V^T tile of one wave: 128 dim rows of 32 entry slots (bf16 pairs, 16
// dwords) on a 20-dword pitch, rows skewed by 16 dwords every 32 rows.  The
// pitch puts the 16 rows a lane group reads (one 16-byte read each) on 16
// disjoint groups of 4 banks; the skew puts the four lane groups of a
// transposing store (rows 32 g + ..) on disjoint banks.
constexpr int kVtRow = 20;
constexpr int kVtWave = kHeadDim * kVtRow + 4 * 16;

__device__ __forceinline__ int vt_addr(int d) { return d * kVtRow + (d >> 5) * 16; }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t w, float sc, int sel) {
    bf16x2_t r;
    switch (sel) {
        case 0: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0); break;
        case 1: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1); break;
        case 2: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2); break;
        default: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3); break;
    }
    return __builtin_bit_cast(uint32_t, r);
}

// Codes sel (byte) of w times a split scale -> a bf16 pair.  E8M0 (SF 0):
// the conversion alone.  E4M3 (SF 1): converted to fp32 with p2, times mult
// (exact: an E2M1 value times an E4M3 scale has at most 6 significant
// bits), and the high halves kept (exact values need no rounding).
template <int SF>
__device__ __forceinline__ uint32_t dq_pair(uint32_t w, DqScale d, int sel) {
    if (SF == 0) return cvt_fp4x2(w, d.p2, sel);
    typedef __attribute__((ext_vector_type(2))) float f32x2_t;
    f32x2_t r;
    switch (sel) {
        case 0: r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, d.p2, 0); break;
        case 1: r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, d.p2, 1); break;
        case 2: r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, d.p2, 2); break;
        default: r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, d.p2, 3); break;
    }
    return __builtin_amdgcn_perm(__float_as_uint(r.y * d.mult), __float_as_uint(r.x * d.mult),
                                 0x07060302u);
}

struct RowRaw {  // the FP4 data one lane loads for one entry
    uint4 k, v;
    uint32_t sk, sv;  // scale bits of the lane's K and V blocks, or the dwords holding them
};

struct AttnLds {
    uint32_t vt[kWaves][kVtWave];  // V^T of each wave's 32 entries
    uint4 p[kWaves][64];           // P^T fragments (bf16) of each wave's 32 entries
    float m[kWaves][kHeads];
    float l[kWaves][kHeads];
    int last;
};

// grid: (n_chunk, nq), kThreads threads, n_chunk >= ceil(window / 32).  Wave
// w < 8 of chunk c takes selected entries 256 c + 32 w .. + 32, wave 8 window
// entries wpc c .. + wpc (wpc = ceil(window / n_chunk) <= 32): lane row n16
// loads entries 2 n16 and 2 n16 + 1 of the wave's block (MFMA tiles 0 and 1),
// lane group g dims 32 g .. + 32 of K and of V.  After the second barrier
// wave w < 8 forms dims 16 w .. + 16 of O for the whole chunk.
template <int SF>
__global__ __launch_bounds__(kThreads) void k_attn_chunk(CacheView c, const uint16_t* __restrict__ q,
                                                         const int32_t* __restrict__ q_pos,
                                                         const int32_t* __restrict__ q_seq,
                                                         const int32_t* __restrict__ sel, int32_t k,
                                                         LocalView loc, float sm_scale,
                                                         int32_t n_chunk, float* __restrict__ ws_o,
                                                         float* __restrict__ ws_ml,
                                                         uint32_t* __restrict__ ctr,
                                                         uint16_t* __restrict__ out) {
    __shared__ AttnLds sh;

    const int qi = blockIdx.y, chunk = blockIdx.x;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n16 = lane & 15, g = lane >> 4;
    uint32_t* vt = sh.vt[wave];
    const float NEG = -__builtin_inff();

    const int32_t seq = q_seq ? q_seq[qi] : qi;
    int64_t t = q_pos[qi];  // the query's position (window)
    if (seq < 0 || seq >= c.n_seq) t = -1;
    if (t >= (c.t_cap << c.msh)) t = (c.t_cap << c.msh) - 1;
    // the last global entry it may read: entries of 2^msh positions count
    // once their whole group is at or before t
    const int64_t tg = ((t + 1) >> c.msh) - 1;
    int64_t w0 = t - loc.window + 1;
    if (w0 < loc.lo) w0 = loc.lo;
    if (w0 < 0) w0 = 0;
    const int64_t nw = (loc.window > 0 && t >= w0) ? t - w0 + 1 : 0;

    // ---- slots first, then every row load of both tiles, then the decode
    int kind[2];     // 0 none, 1 global FP4, 2 global bf16, 3 local bf16
    int64_t row[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        kind[u] = 0;
        row[u] = 0;
        if (wave < kSelWaves) {
            const int64_t e = (int64_t)chunk * kWgEntries + wave * kBlk + 2 * n16 + u;
            if (e < k) {
                const int64_t j = sel[(int64_t)qi * k + e];
                if (j >= 0 && j <= tg) {
                    kind[u] = c.fp4 ? 1 : 2;
                    row[u] = (int64_t)seq * c.t_cap + j;
                }
            }
        } else {
            const int wpc = (loc.window + n_chunk - 1) / n_chunk;
            const int sl = 2 * n16 + u;
            const int64_t ew = (int64_t)chunk * wpc + sl;
            if (sl < wpc && ew < nw) {
                kind[u] = 3;
                row[u] = (int64_t)seq * loc.cap + (w0 + ew) % loc.cap;
            }
        }
    }
    // Q^T as the B operand of S: head n16, dims 32 g + 8 kb .. + 8 at step kb
    bf16x8_t qf[4];
    {
        const uint4* qr = reinterpret_cast<const uint4*>(q + ((int64_t)qi * kHeads + n16) * kHeadDim + 32 * g);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const uint4 v = qr[kb];
            qf[kb] = as_bf16x8(v.x, v.y, v.z, v.w);
        }
    }
    uint4 rk[2][4], rv[2][4];  // K and V dims 32 g .. + 32: FP4 uses [0], bf16 all four
    uint32_t rsk[2], rsv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        rsk[u] = rsv[u] = unit_scale_bits<SF>();
        if (kind[u] == 1) {
            const uint8_t* cr = static_cast<const uint8_t*>(c.data) + row[u] * kRowCodes;
            rk[u][0] = *reinterpret_cast<const uint4*>(cr + 16 * g);
            rv[u][0] = *reinterpret_cast<const uint4*>(cr + 64 + 16 * g);
            row_scales<SF>(c.scales + row[u] * row_scale_bytes<SF>(), g, rsk[u], rsv[u]);
        } else if (kind[u] >= 2) {
            const uint16_t* kr = kind[u] == 2 ? static_cast<const uint16_t*>(c.data) + row[u] * kRowBf16
                                              : loc.k + row[u] * kHeadDim;
            const uint16_t* vr = kind[u] == 2 ? kr + kHeadDim : loc.v + row[u] * kHeadDim;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                rk[u][i] = *reinterpret_cast<const uint4*>(kr + 32 * g + 8 * i);
                rv[u][i] = *reinterpret_cast<const uint4*>(vr + 32 * g + 8 * i);
            }
        } else {
            rk[u][0] = rv[u][0] = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int i = 1; i < 4; ++i) rk[u][i] = rv[u][i] = make_uint4(0, 0, 0, 0);
        }
    }
    // ---- decode: K fragments (FP4 scaled exactly by v_cvt_scalef32_pk_bf16_fp4),
    // V dims d, d + 1 of slots 2 n16, 2 n16 + 1 -> two dwords of V^T
    bf16x8_t kf[2][4];
    uint32_t vd[2][16];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (kind[u] == 1) {
            const uint32_t wk[4] = {rk[u][0].x, rk[u][0].y, rk[u][0].z, rk[u][0].w};
            const uint32_t wv[4] = {rv[u][0].x, rv[u][0].y, rv[u][0].z, rv[u][0].w};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const DqScale sk = dw_scale<SF>(rsk[u], kb), sv = dw_scale<SF>(rsv[u], kb);
                kf[u][kb] = as_bf16x8(dq_pair<SF>(wk[kb], sk, 0), dq_pair<SF>(wk[kb], sk, 1),
                                      dq_pair<SF>(wk[kb], sk, 2), dq_pair<SF>(wk[kb], sk, 3));
                vd[u][4 * kb + 0] = dq_pair<SF>(wv[kb], sv, 0);
                vd[u][4 * kb + 1] = dq_pair<SF>(wv[kb], sv, 1);
                vd[u][4 * kb + 2] = dq_pair<SF>(wv[kb], sv, 2);
                vd[u][4 * kb + 3] = dq_pair<SF>(wv[kb], sv, 3);
            }
        } else {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                kf[u][kb] = as_bf16x8(rk[u][kb].x, rk[u][kb].y, rk[u][kb].z, rk[u][kb].w);
                vd[u][4 * kb + 0] = rv[u][kb].x;
                vd[u][4 * kb + 1] = rv[u][kb].y;
                vd[u][4 * kb + 2] = rv[u][kb].z;
                vd[u][4 * kb + 3] = rv[u][kb].w;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int d = 32 * g + 2 * i;
        vt[vt_addr(d) + n16] = __builtin_amdgcn_perm(vd[1][i], vd[0][i], 0x05040100u);
        vt[vt_addr(d + 1) + n16] = __builtin_amdgcn_perm(vd[1][i], vd[0][i], 0x07060302u);
    }
    const uint64_t vm0 = __ballot(kind[0] != 0) & 0xFFFFull;  // bit n16: slot row valid
    const uint64_t vm1 = __ballot(kind[1] != 0) & 0xFFFFull;

    // ---- S^T = K Q^T: lane holds head n16, rows 4 g + r of tile u = slot 8 g + 2 r + u
    const float zs = sm_scale * kLog2e;
    float s[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u][kb], qf[kb], z, 0, 0, 0);
        const uint64_t vm = u ? vm1 : vm0;
#pragma unroll
        for (int r = 0; r < 4; ++r) s[u][r] = ((vm >> (4 * g + r)) & 1) ? z[r] * zs : NEG;
    }
    // ---- softmax over the workgroup's 256 entries: wave maxima -> LDS, then
    // every wave takes the workgroup maximum per head
    // chained from -inf (canonical), so it compiles to v_max3_f32 only
    float m = fmaxf(fmaxf(NEG, s[0][0]), s[0][1]);
    m = fmaxf(fmaxf(m, s[0][2]), s[0][3]);
    m = fmaxf(fmaxf(m, s[1][0]), s[1][1]);
    m = fmaxf(fmaxf(m, s[1][2]), s[1][3]);
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    if (g == 0) sh.m[wave][n16] = m;
    __syncthreads();  // every wave's maxima and V^T tile are in LDS
    float M = NEG;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sh.m[w][n16]);
    const float m_use = M == NEG ? 0.f : M;  // no valid entry: every p is 0
    float p[2][4];
    float lsum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[u][r] = __builtin_amdgcn_exp2f(s[u][r] - m_use);  // 2^-inf = 0
            lsum += p[u][r];
        }
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    if (g == 0) sh.l[wave][n16] = lsum;
    // P^T as the B operand of O^T (slots 8 g + j, head n16): the lane's own
    // slots, so the fragment is built in registers and shared through LDS
    sh.p[wave][lane] = make_uint4(__builtin_bit_cast(uint32_t, (bf16x2_t){(__bf16)p[0][0], (__bf16)p[1][0]}),
                                  __builtin_bit_cast(uint32_t, (bf16x2_t){(__bf16)p[0][1], (__bf16)p[1][1]}),
                                  __builtin_bit_cast(uint32_t, (bf16x2_t){(__bf16)p[0][2], (__bf16)p[1][2]}),
                                  __builtin_bit_cast(uint32_t, (bf16x2_t){(__bf16)p[0][3], (__bf16)p[1][3]}));
    __syncthreads();

    // ---- O^T for dims 16 wave .. + 16 over all 256 entries: A = V^T (dim
    // 16 wave + n16, slots 8 g + j of wave block b), B = P^T of block b; the
    // lane ends with head n16, dims 16 wave + 4 g + r
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) L += sh.l[w][n16];
    const int64_t part0 = (int64_t)qi * n_chunk;
    if (wave < kSelWaves) {  // the window wave has no dims of O
        f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < kWaves; ++b) {
            const uint4 vv = *reinterpret_cast<const uint4*>(&sh.vt[b][vt_addr(16 * wave + n16) + 4 * g]);
            const uint4 pb = sh.p[b][lane];
            o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vv.x, vv.y, vv.z, vv.w),
                                                        as_bf16x8(pb.x, pb.y, pb.z, pb.w), o, 0, 0, 0);
        }
        const int dq = 16 * wave + 4 * g;
        if (n_chunk == 1) {  // the whole query in one workgroup
            const float inv = L > 0.f ? 1.f / L : 0.f;
            *reinterpret_cast<uint2*>(out + ((int64_t)qi * kHeads + n16) * kHeadDim + dq) =
                make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv));
        } else {
            *reinterpret_cast<float4*>(ws_o + ((part0 + chunk) * kHeads + n16) * kHeadDim + dq) =
                make_float4(o[0], o[1], o[2], o[3]);
            if (wave == 0 && g == 0)
                *reinterpret_cast<float2*>(ws_ml + ((part0 + chunk) * kHeads + n16) * 2) = make_float2(M, L);
        }
    }
    if (n_chunk == 1) return;
    __syncthreads();  // the workgroup's stores are ordered before thread 0's release
    if (tid == 0) sh.last = arrive_last(&ctr[qi * kCtrStride], (uint32_t)n_chunk);
    __syncthreads();  // thread 0's acquire covers the workgroup
    if (!sh.last || wave >= kSelWaves) return;
    // ---- the last chunk of the query merges all chunks in order: thread of
    // the 8 selection waves -> head h, kDpt dims
    constexpr int kMergeThreads = kSelWaves * 64;
    constexpr int kDpt = kHeads * kHeadDim / kMergeThreads;
    static_assert(kDpt % 4 == 0, "whole float4s per thread");
    const int h = tid / (kHeadDim / kDpt), d0 = (tid % (kHeadDim / kDpt)) * kDpt;
    float Mq = -__builtin_inff(), Lq = 0.f, aq[kDpt];
#pragma unroll
    for (int i = 0; i < kDpt; ++i) aq[i] = 0.f;
    constexpr int kMB = 64 / kDpt;  // chunks per batch: every load of a batch in flight at once
    for (int j0 = 0; j0 < n_chunk; j0 += kMB) {
        float2 ml[kMB];
        float4 ov[kMB][kDpt / 4];
#pragma unroll
        for (int u = 0; u < kMB; ++u) {
            const int64_t pj = part0 + j0 + u;
            const bool in = j0 + u < n_chunk;
            ml[u] = in ? *reinterpret_cast<const float2*>(ws_ml + (pj * kHeads + h) * 2)
                       : make_float2(-__builtin_inff(), 0.f);
#pragma unroll
            for (int v = 0; v < kDpt / 4; ++v)
                ov[u][v] = in ? *reinterpret_cast<const float4*>(ws_o + (pj * kHeads + h) * kHeadDim + d0 + 4 * v)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float Mn = Mq;
#pragma unroll
        for (int u = 0; u < kMB; ++u) Mn = fmaxf(Mn, ml[u].x);
        if (Mn == -__builtin_inff()) continue;
        const float rs = __builtin_amdgcn_exp2f(Mq - Mn);  // Mq = -inf: 0
        Lq *= rs;
#pragma unroll
        for (int i = 0; i < kDpt; ++i) aq[i] *= rs;
#pragma unroll
        for (int u = 0; u < kMB; ++u) {
            const float f = __builtin_amdgcn_exp2f(ml[u].x - Mn);  // an empty chunk: 0
            Lq = fmaf(ml[u].y, f, Lq);
#pragma unroll
            for (int v = 0; v < kDpt / 4; ++v) {
                aq[4 * v + 0] = fmaf(ov[u][v].x, f, aq[4 * v + 0]);
                aq[4 * v + 1] = fmaf(ov[u][v].y, f, aq[4 * v + 1]);
                aq[4 * v + 2] = fmaf(ov[u][v].z, f, aq[4 * v + 2]);
                aq[4 * v + 3] = fmaf(ov[u][v].w, f, aq[4 * v + 3]);
            }
        }
        Mq = Mn;
    }
    const float inv = Lq > 0.f ? 1.f / Lq : 0.f;
    uint16_t* orow = out + ((int64_t)qi * kHeads + h) * kHeadDim + d0;
#pragma unroll
    for (int v = 0; v < kDpt / 4; ++v)
        *reinterpret_cast<uint2*>(orow + 4 * v) = make_uint2(pack_bf16x2(aq[4 * v] * inv, aq[4 * v + 1] * inv),
                                                             pack_bf16x2(aq[4 * v + 2] * inv, aq[4 * v + 3] * inv));
    if (tid == 0) ctr[qi * kCtrStride] = 0u;  // ready for the next call
}

// ---------------------------------------------------------------------------
// Many queries (a prefill chunk): one workgroup of 4 waves per query, no
// workspace.  Each wave walks its share of the entries in tiles of 32 with an
// online softmax (running max, sum and unnormalised O per head, kept in
// registers) and loads the next tile's rows while the current one computes;
// the 4 waves are combined at the end.  FP4 rows are dequantised with their
// E8M0 scale by v_cvt_scalef32_pk_bf16_fp4 (exact: an E2M1 value times a power
// of two fits bf16), so both products take plain bf16 operands.
//
// Entry slots of a tile: lane row n16 loads entries 2 n16 and 2 n16 + 1 of the
// tile (MFMA tiles 0 and 1), so a lane holds two neighbouring slots of every V
// dim and writes V^T with one dword per dim.  Lane group g loads dims
// 32 g .. 32 g + 31 of K and of V (one scale block each).  The K fragment of
// k-step kb is dims 32 g + 8 kb .. + 8 (the Q fragment uses the same map).
constexpr int kLW = 4;                       // waves per workgroup (many queries)
constexpr int kLWFew = 8;                    // fewer queries than CUs: 8 waves share a query

// V of one wave's 32 entries, row-major (128 bf16 dims a row) on a 72-dword
// (288-byte) pitch, slot s in row 16 (s % 2) + s / 2, so the 8 lanes of one
// 16-byte store (slots 2 n16 + u) write consecutive rows: 8 rows apart in
// banks instead of 16.  The PV product reads it transposed with
// ds_read_b64_tr_b16: within a 16-lane group, lane i receives element i % 4
// of the 8-byte blocks addressed by lanes 4 k + i / 4 (k = 0..3), so lane
// (n16, g) addressing row 16 h + 4 g + n16 / 4 at dims 16 t8 + 4 (n16 % 4)
// receives dim 16 t8 + n16 of slots 8 g + 2 k + h (k = 0..3): the V^T
// operand of the MFMA, whose contraction index then runs over slots 8 g + 0,
// 2, 4, 6, 1, 3, 5, 7 (the P^T operand follows the same order).  The pitch
// puts the four rows a group reads on disjoint banks.
constexpr int kVrRow = 72;
constexpr int kVrWave = 32 * kVrRow;
typedef short i16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void vr_store_row(uint32_t* vr, int slot, int g, const uint32_t (&d)[16]) {
    uint32_t* row = vr + (16 * (slot & 1) + (slot >> 1)) * kVrRow + 16 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        *reinterpret_cast<uint4*>(row + 4 * c) = make_uint4(d[4 * c], d[4 * c + 1], d[4 * c + 2], d[4 * c + 3]);
}

// The V^T operand of dims 16 t8 .. + 16 (A of O^T += V^T P^T).
__device__ __forceinline__ bf16x8_t vr_frag(const uint32_t* vr, int t8, int n16, int g) {
    const uint32_t* p0 = vr + (4 * g + (n16 >> 2)) * kVrRow + 8 * t8 + 2 * (n16 & 3);
    typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
    const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
    const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 16 * kVrRow));
    const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
    return as_bf16x8(ua.x, ua.y, ub.x, ub.y);
}

template <int LW>
struct LoopLds {
    union {
        uint32_t vr[LW][kVrWave];
        float obuf[LW][kHeads][kHeadDim + 4];
    } u;
    float m[LW][kHeads];
    float l[LW][kHeads];
};

// grid nq, LW * 64 threads (LW = 4, or 8 when the queries are fewer than
// the CUs, so that each CU runs two waves per SIMD instead of one).
template <int SF, int LW>
__global__ __launch_bounds__(LW * 64) void k_attn_loop(CacheView c, const uint16_t* __restrict__ q,
                                                        const int32_t* __restrict__ q_pos,
                                                        const int32_t* __restrict__ q_seq,
                                                        const int32_t* __restrict__ sel, int32_t k,
                                                        LocalView loc, float sm_scale,
                                                        uint16_t* __restrict__ out) {
    __shared__ LoopLds<LW> sh;
    const int qi = blockIdx.x, tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n16 = lane & 15, g = lane >> 4;
    uint32_t* vr = sh.u.vr[wave];

    const int32_t seq = q_seq ? q_seq[qi] : qi;
    int64_t t = q_pos[qi];  // the query's position (window)
    if (seq < 0 || seq >= c.n_seq) t = -1;
    if (t >= (c.t_cap << c.msh)) t = (c.t_cap << c.msh) - 1;
    // the last global entry it may read: entries of 2^msh positions count
    // once their whole group is at or before t
    const int64_t tg = ((t + 1) >> c.msh) - 1;
    int64_t w0 = t - loc.window + 1;
    if (w0 < loc.lo) w0 = loc.lo;
    if (w0 < 0) w0 = 0;
    const int64_t nw = (loc.window > 0 && t >= w0) ? t - w0 + 1 : 0;
    const int64_t n_ent = t >= 0 ? (int64_t)k + nw : 0;
    const int n_tiles = (int)((n_ent + 31) / 32);

    // Q^T as the B operand of S: head n16, dims 32 g + 8 kb .. + 8 at step kb
    bf16x8_t qf[4];
    {
        const uint4* qr = reinterpret_cast<const uint4*>(q + ((int64_t)qi * kHeads + n16) * kHeadDim + 32 * g);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const uint4 v = qr[kb];
            qf[kb] = as_bf16x8(v.x, v.y, v.z, v.w);
        }
    }
    const float zs = sm_scale * kLog2e;
    const float NEG = -__builtin_inff();

    // Entry e of the query: a selected position (e < k) or a window position.
    // sel_of(e) reads the selection slot (-1 past the selection); locate()
    // turns it into a kind (0 none, 1 global FP4, 2 global bf16, 3 local
    // bf16) and a row index.
    auto sel_of = [&](int64_t e) -> int32_t { return e < k ? sel[(int64_t)qi * k + e] : -1; };
    auto locate = [&](int64_t e, int64_t j, int& kind, int64_t& row) {
        kind = 0;
        row = 0;
        if (e < k) {
            if (j >= 0 && j <= tg) {
                kind = c.fp4 ? 1 : 2;
                row = (int64_t)seq * c.t_cap + j;
            }
        } else if (e - k < nw) {
            kind = 3;
            row = (int64_t)seq * loc.cap + (w0 + (e - k)) % loc.cap;
        }
    };
    auto load_fp4 = [&](int64_t row, RowRaw& r) {
        const uint8_t* cr = static_cast<const uint8_t*>(c.data) + row * kRowCodes;
        r.k = *reinterpret_cast<const uint4*>(cr + 16 * g);
        r.v = *reinterpret_cast<const uint4*>(cr + 64 + 16 * g);
        row_scales<SF>(c.scales + row * row_scale_bytes<SF>(), g, r.sk, r.sv);
    };

    float m_run = NEG, l_part = 0.f;
    f32x4_t o[8];
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) o[t8] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    // One tile once its K fragments are in kf and its V^T is in LDS: S^T = K
    // Q^T (lane: head n16, rows 4 g + r of MFMA tile u = slot 8 g + 2 r + u),
    // the online softmax, and O^T += V^T P^T (lane: head n16, dims
    // 16 t8 + 4 g + r, so the rescale by alpha is lane-local).  The reference
    // maximum m_run (scaled, log2 units) moves only when a head's tile
    // maximum passes it by more than 8, so most tiles skip the rescale and
    // p = 2^(s zs - m_run) stays below 2^8 (exact up to bf16/fp32 rounding:
    // the softmax does not depend on the reference).
    auto scores = [&](const bf16x8_t (&kf)[2][4], float (&sv)[2][4]) {  // raw scores
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u][kb], qf[kb], z, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[u][r] = z[r];
        }
    };
    auto consume = [&](float (&sv)[2][4], uint64_t vm0, uint64_t vm1) {
        if ((vm0 & vm1) != 0xFFFFull) {  // some slot of the tile is empty: -inf
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (!((vm0 >> (4 * g + r)) & 1)) sv[0][r] = NEG;
                if (!((vm1 >> (4 * g + r)) & 1)) sv[1][r] = NEG;
            }
        }
        float mt = fmaxf(fmaxf(NEG, sv[0][0]), sv[0][1]);  // v_max3_f32 chain
        mt = fmaxf(fmaxf(mt, sv[0][2]), sv[0][3]);
        mt = fmaxf(fmaxf(mt, sv[1][0]), sv[1][1]);
        mt = fmaxf(fmaxf(mt, sv[1][2]), sv[1][3]);
        mt = max_xor32(max_xor16(mt));
        const float ms = mt * zs;            // zs > 0: the scaled tile maximum
        const bool bump = ms > m_run + 8.f;  // m_run = -inf: any valid slot
        if (__ballot(bump)) {
            // v_exp_f32: 2^-inf = 0 (the first valid tile of a head)
            const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - ms) : 1.f;
            if (bump) m_run = ms;
            l_part *= alpha;
#pragma unroll
            for (int t8 = 0; t8 < 8; ++t8) {
                o[t8][0] *= alpha;
                o[t8][1] *= alpha;
                o[t8][2] *= alpha;
                o[t8][3] *= alpha;
            }
        }
        const float nm = m_run == NEG ? 0.f : -m_run;  // no valid slot yet: every p is 0
        float p[2][4];
        float ps = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[u][r] = __builtin_amdgcn_exp2f(fmaf(sv[u][r], zs, nm));  // 2^-inf = 0
                ps += p[u][r];
            }
        l_part += ps;
        // P^T in the contraction order of vr_frag: slots 8 g + 0, 2, 4, 6 (MFMA
        // tile 0, rows 4 g .. + 3), then 8 g + 1, 3, 5, 7 (tile 1)
        const bf16x8_t pf = as_bf16x8(__builtin_bit_cast(uint32_t, (bf16x2_t){(__bf16)p[0][0], (__bf16)p[0][1]}),
                                      __builtin_bit_cast(uint32_t, (bf16x2_t){(__bf16)p[0][2], (__bf16)p[0][3]}),
                                      __builtin_bit_cast(uint32_t, (bf16x2_t){(__bf16)p[1][0], (__bf16)p[1][1]}),
                                      __builtin_bit_cast(uint32_t, (bf16x2_t){(__bf16)p[1][2], (__bf16)p[1][3]}));
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8)
            o[t8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr_frag(vr, t8, n16, g), pf, o[t8], 0, 0, 0);
    };

    // ---- tiles inside the selection of an FP4 cache: every slot is a global
    // FP4 row or empty.  While tile i computes, the rows of tile i + 1 and the
    // selection slots of tile i + 2 are in flight.  An empty slot loads zero
    // codes, so its V is zero.
    const int n_fast = (c.fp4 && t >= 0) ? k / 32 : 0;
    const uint8_t* codes = static_cast<const uint8_t*>(c.data) + (int64_t)max(seq, 0) * c.t_cap * kRowCodes;
    const uint8_t* scl =
        c.scales ? c.scales + (int64_t)max(seq, 0) * c.t_cap * row_scale_bytes<SF>() : nullptr;
    // An empty slot reads row 0 (no branch around the loads) with scale 1:
    // its codes are finite and its p is 0, so it adds nothing.
    const int32_t t32 = (int32_t)tg;  // entries fit 32 bits (t_cap <= 2^24)
    // Row offsets stay 32-bit (entries < 2^24, so entry * 128 < 2^31) over a
    // uniform base, which the loads take as scalar base + vector offset.  The
    // scale dwords are kept as loaded (sk, sv hold whole words here) and
    // their bits taken out only when the tile is decoded: touching a load's
    // result makes the wave wait for it and, the counter being in order, for
    // every load before it, so doing it here would wait out the prefetch.
    auto fetch = [&](int32_t j, RowRaw& r) {
        const bool ok = j >= 0 && j <= t32;
        const uint32_t jj = ok ? (uint32_t)j : 0u;
        const uint32_t off = jj * (uint32_t)kRowCodes + 16u * (uint32_t)g;
        r.k = *reinterpret_cast<const uint4*>(codes + off);
        r.v = *reinterpret_cast<const uint4*>(codes + off + 64u);
        row_scale_words<SF>(scl + jj * (uint32_t)row_scale_bytes<SF>(), g, r.sk, r.sv);
    };
    {
        // two row buffers, used alternately (the loop is unrolled by two), so
        // the rows in flight never have to be copied into the decode registers
        RowRaw ra[2], rb[2];
        int32_t jc[2] = {-1, -1}, jn[2] = {-1, -1};
        // every slot of these tiles is below k: the selection row is read
        // through a uniform base and a 32-bit slot index, with no check
        const int32_t* selq = sel + (int64_t)qi * k;
        int tile = wave;
        if (tile < n_fast) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                jc[u] = selq[tile * 32 + 2 * n16 + u];
                fetch(jc[u], ra[u]);
            }
            if (tile + LW < n_fast) {
#pragma unroll
                for (int u = 0; u < 2; ++u) jn[u] = selq[(tile + LW) * 32 + 2 * n16 + u];
            }
        }
        // one tile from cur; the next tile's rows go to nxt
        auto step = [&](const RowRaw (&cur)[2], RowRaw (&nxt)[2], int tl) {
            const uint64_t vm0 = __ballot(jc[0] >= 0 && jc[0] <= t32) & 0xFFFFull;
            const uint64_t vm1 = __ballot(jc[1] >= 0 && jc[1] <= t32) & 0xFFFFull;
            uint32_t sk[2], sv[2];  // the lane's scale bits; 1 for an empty slot
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bool ok = jc[u] >= 0 && jc[u] <= t32;
                sk[u] = ok ? row_scale_bits<SF>(cur[u].sk, g) : unit_scale_bits<SF>();
                sv[u] = ok ? row_scale_bits<SF>(cur[u].sv, g) : unit_scale_bits<SF>();
            }
            bf16x8_t kf[2][4];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t w[4] = {cur[u].k.x, cur[u].k.y, cur[u].k.z, cur[u].k.w};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const DqScale sc = dw_scale<SF>(sk[u], kb);
                    kf[u][kb] = as_bf16x8(dq_pair<SF>(w[kb], sc, 0), dq_pair<SF>(w[kb], sc, 1),
                                          dq_pair<SF>(w[kb], sc, 2), dq_pair<SF>(w[kb], sc, 3));
                }
            }
            float sc4[2][4];
            scores(kf, sc4);  // K is dead from here on
#pragma unroll
            for (int u = 0; u < 2; ++u) {  // V rows of slots 2 n16 + u, dims 32 g .. + 32
                const uint32_t wv[4] = {cur[u].v.x, cur[u].v.y, cur[u].v.z, cur[u].v.w};
                uint32_t d[16];
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    d[i] = dq_pair<SF>(wv[i >> 2], dw_scale<SF>(sv[u], i >> 2), i & 3);
                vr_store_row(vr, 2 * n16 + u, g, d);
            }
            const int next = tl + LW;
            if (next < n_fast) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    jc[u] = jn[u];
                    fetch(jc[u], nxt[u]);
                }
                if (next + LW < n_fast) {
#pragma unroll
                    for (int u = 0; u < 2; ++u) jn[u] = selq[(next + LW) * 32 + 2 * n16 + u];
                }
            }
            consume(sc4, vm0, vm1);
        };
        for (; tile < n_fast; tile += 2 * LW) {
            step(ra, rb, tile);
            if (tile + LW >= n_fast) break;
            step(rb, ra, tile + LW);
        }
    }

    // ---- the other tiles (window rows, a bf16 cache, a tile across the end of
    // the selection): rows loaded when the tile starts
    for (int tile = n_fast + wave; tile < n_tiles; tile += LW) {
        int kind[2];
        int64_t row[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t e = (int64_t)tile * 32 + 2 * n16 + u;
            locate(e, sel_of(e), kind[u], row[u]);
        }
        const uint64_t vm0 = __ballot(kind[0] != 0) & 0xFFFFull;
        const uint64_t vm1 = __ballot(kind[1] != 0) & 0xFFFFull;
        bf16x8_t kf[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (kind[u] == 1) {
                RowRaw r;
                load_fp4(row[u], r);
                const uint32_t w[4] = {r.k.x, r.k.y, r.k.z, r.k.w};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const DqScale sc = dw_scale<SF>(r.sk, kb);
                    kf[u][kb] = as_bf16x8(dq_pair<SF>(w[kb], sc, 0), dq_pair<SF>(w[kb], sc, 1),
                                          dq_pair<SF>(w[kb], sc, 2), dq_pair<SF>(w[kb], sc, 3));
                }
            } else if (kind[u] >= 2) {
                const uint16_t* kr = kind[u] == 2 ? static_cast<const uint16_t*>(c.data) + row[u] * kRowBf16
                                                  : loc.k + row[u] * kHeadDim;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const uint4 av = *reinterpret_cast<const uint4*>(kr + 32 * g + 8 * kb);
                    kf[u][kb] = as_bf16x8(av.x, av.y, av.z, av.w);
                }
            } else {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) kf[u][kb] = as_bf16x8(0u, 0u, 0u, 0u);
            }
        }
        // V rows eight dims at a time
        uint32_t vd[2][16];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            uint32_t vv[2][4];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (kind[u] == 1) {
                    const uint8_t* cr = static_cast<const uint8_t*>(c.data) + row[u] * kRowCodes;
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(cr + 64 + 16 * g + 4 * i4);
                    // V scale of dims 32 g + 8 i4 .. + 8
                    const DqScale sc =
                        SF ? e4m3_split(c.scales[row[u] * 16 + 8 + 2 * g + (i4 >> 1)])
                           : DqScale{e8m0_value(c.scales[row[u] * kRowScales + 4 + g]), 1.f};
                    vv[u][0] = dq_pair<SF>(w, sc, 0);
                    vv[u][1] = dq_pair<SF>(w, sc, 1);
                    vv[u][2] = dq_pair<SF>(w, sc, 2);
                    vv[u][3] = dq_pair<SF>(w, sc, 3);
                } else if (kind[u] >= 2) {
                    const uint16_t* vr = kind[u] == 2
                                             ? static_cast<const uint16_t*>(c.data) + row[u] * kRowBf16 + kHeadDim
                                             : loc.v + row[u] * kHeadDim;
                    const uint4 bq = *reinterpret_cast<const uint4*>(vr + 32 * g + 8 * i4);
                    vv[u][0] = bq.x; vv[u][1] = bq.y; vv[u][2] = bq.z; vv[u][3] = bq.w;
                } else {
                    vv[u][0] = vv[u][1] = vv[u][2] = vv[u][3] = 0u;
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) vd[u][4 * i4 + i] = vv[u][i];
        }
        vr_store_row(vr, 2 * n16, g, vd[0]);
        vr_store_row(vr, 2 * n16 + 1, g, vd[1]);
        float sc4[2][4];
        scores(kf, sc4);
        consume(sc4, vm0, vm1);
    }
    // ---- combine the waves
    l_part = sum_xor32(sum_xor16(l_part));
    if (g == 0) {
        sh.m[wave][n16] = m_run;
        sh.l[wave][n16] = l_part;
    }
    __syncthreads();  // every wave is done with its V^T tile
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8)
        *reinterpret_cast<float4*>(&sh.u.obuf[wave][n16][16 * t8 + 4 * g]) =
            make_float4(o[t8][0], o[t8][1], o[t8][2], o[t8][3]);
    __syncthreads();
    constexpr int tph = LW * 64 / kHeads;  // threads per head
    constexpr int dpt = kHeadDim / tph;    // dims per thread: 8 (LW 4) or 4 (LW 8)
    const int h = tid / tph, d0 = (tid % tph) * dpt;
    float M = NEG;
#pragma unroll
    for (int w = 0; w < LW; ++w) M = fmaxf(M, sh.m[w][h]);
    float L = 0.f, acc[dpt];
#pragma unroll
    for (int i = 0; i < dpt; ++i) acc[i] = 0.f;
    if (M != NEG) {
#pragma unroll
        for (int w = 0; w < LW; ++w) {
            const float mw = sh.m[w][h];
            const float f = (mw == NEG) ? 0.f : exp2f(mw - M);
            L = fmaf(sh.l[w][h], f, L);
#pragma unroll
            for (int i = 0; i < dpt; ++i) acc[i] = fmaf(sh.u.obuf[w][h][d0 + i], f, acc[i]);
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t* orow = out + ((int64_t)qi * kHeads + h) * kHeadDim + d0;
#pragma unroll
    for (int i = 0; i < dpt; i += 4)
        *reinterpret_cast<uint2*>(orow + i) =
            make_uint2(pack_bf16x2(acc[i] * inv, acc[i + 1] * inv), pack_bf16x2(acc[i + 2] * inv, acc[i + 3] * inv));
}

// Chunks of a query: 256 selected entries each, and enough of them that the
// window spreads at most 32 entries over each.
static int32_t attn_chunks(int32_t k, int32_t window) {
    return std::max(std::max((k + kWgEntries - 1) / kWgEntries, (window + kBlk - 1) / kBlk), 1);
}

size_t attn_part_bytes(int32_t nq, int32_t k, int32_t window) {
    const int64_t nc = attn_chunks(k, window);
    if (nc <= 1 || nq >= kManyQueries) return 0;
    return (size_t)nq * nc * kHeads * (kHeadDim + 2) * sizeof(float);
}

size_t attn_ws_bytes(int32_t nq, int32_t k, int32_t window) {
    const size_t part = attn_part_bytes(nq, k, window);
    return part ? kAttnCtrBytes + part : 0;
}

hipError_t launch_sparse_attn(const CacheView& c, const uint16_t* q, const int32_t* q_pos,
                              const int32_t* q_seq, int32_t nq, const int32_t* sel, int32_t k,
                              const LocalView& loc, float sm_scale, uint16_t* out, void* ws,
                              hipStream_t s) {
    char* base = static_cast<char*>(ws);
    return launch_sparse_attn_parts(c, q, q_pos, q_seq, nq, sel, k, loc, sm_scale, out,
                                    reinterpret_cast<uint32_t*>(base),
                                    base ? reinterpret_cast<float*>(base + kAttnCtrBytes) : nullptr, s);
}

hipError_t launch_sparse_attn_parts(const CacheView& c, const uint16_t* q, const int32_t* q_pos,
                                    const int32_t* q_seq, int32_t nq, const int32_t* sel, int32_t k,
                                    const LocalView& loc, float sm_scale, uint16_t* out,
                                    uint32_t* ctr, float* part, hipStream_t s, hipEvent_t ev0,
                                    hipEvent_t ev1) {
    if (nq == 0) return hipSuccess;
    if (nq >= kManyQueries) {  // one workgroup per query (see kManyQueries)
        const bool few = nq < 256;  // fewer queries than CUs
        if (c.fp4 == 2 && few)
            hipExtLaunchKernelGGL((k_attn_loop<1, kLWFew>), dim3((uint32_t)nq), dim3(kLWFew * 64), 0, s, ev0, ev1, 0, c, q,
                               q_pos, q_seq, sel, k, loc, sm_scale, out);
        else if (c.fp4 == 2)
            hipExtLaunchKernelGGL((k_attn_loop<1, kLW>), dim3((uint32_t)nq), dim3(kLW * 64), 0, s, ev0, ev1, 0, c, q, q_pos,
                               q_seq, sel, k, loc, sm_scale, out);
        else if (few)
            hipExtLaunchKernelGGL((k_attn_loop<0, kLWFew>), dim3((uint32_t)nq), dim3(kLWFew * 64), 0, s, ev0, ev1, 0, c, q,
                               q_pos, q_seq, sel, k, loc, sm_scale, out);
        else
            hipExtLaunchKernelGGL((k_attn_loop<0, kLW>), dim3((uint32_t)nq), dim3(kLW * 64), 0, s, ev0, ev1, 0, c, q, q_pos,
                               q_seq, sel, k, loc, sm_scale, out);
        return hipGetLastError();
    }
    int32_t nc = attn_chunks(k, loc.window);
    if (nc < 1) nc = 1;
    float* ws_o = nc > 1 ? part : nullptr;
    float* ws_ml = nc > 1 ? ws_o + (size_t)nq * nc * kHeads * kHeadDim : nullptr;
    if (nc <= 1) ctr = nullptr;
    if (c.fp4 == 2)
        hipExtLaunchKernelGGL(k_attn_chunk<1>, dim3((uint32_t)nc, (uint32_t)nq), dim3(kThreads), 0, s, ev0, ev1, 0, c,
                           q, q_pos, q_seq, sel, k, loc, sm_scale, nc, ws_o, ws_ml, ctr, out);
    else
        hipExtLaunchKernelGGL(k_attn_chunk<0>, dim3((uint32_t)nc, (uint32_t)nq), dim3(kThreads), 0, s, ev0, ev1, 0, c,
                           q, q_pos, q_seq, sel, k, loc, sm_scale, nc, ws_o, ws_ml, ctr, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Allocation-free form (for callers that cannot allocate: code under graph
// capture, serving loops): the split kernel's counters and partials live in
// one file-scope device array per GPU, held until the process ends.  Its
// address is looked up once per device with hipGetSymbolAddress (the array's
// name in host code is not a device address) and passed to the kernels like
// a caller's workspace.  Every call on a GPU uses the same array, so calls
// that overlap on one GPU race.
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];

// The scratch array's device address on the current device.
hipError_t scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

// Zero n words (a kernel, so that a captured graph holds no memset node).
__global__ __launch_bounds__(256) void k_zero_words(uint32_t* __restrict__ p, int32_t n) {
    const int32_t i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}
}  // namespace

hipError_t launch_sparse_attn_static(const CacheView& c, const uint16_t* q, const int32_t* q_pos,
                                     const int32_t* q_seq, int32_t nq, const int32_t* sel, int32_t k,
                                     const LocalView& loc, float sm_scale, uint16_t* out,
                                     hipStream_t s) {
    if (attn_part_bytes(nq, k, loc.window) > kStaticScratchBytes - kAttnCtrBytes)
        return hipErrorInvalidValue;  // the caller checks this first
    void* base = nullptr;
    if (hipError_t e = scratch_ptr(&base)) return e;
    uint32_t* ctr = static_cast<uint32_t*>(base);
    float* part = reinterpret_cast<float*>(static_cast<char*>(base) + kAttnCtrBytes);
    if (attn_part_bytes(nq, k, loc.window) > 0) {
        // the counters must start at zero whatever an earlier call left
        constexpr int32_t nw = (int32_t)(kAttnCtrBytes / sizeof(uint32_t));
        hipLaunchKernelGGL(k_zero_words, dim3((nw + 255) / 256), dim3(256), 0, s, ctr, nw);
        if (hipError_t e = hipGetLastError()) return e;
    }
    return launch_sparse_attn_parts(c, q, q_pos, q_seq, nq, sel, k, loc, sm_scale, out, ctr, part, s);
}

}  // namespace csa2

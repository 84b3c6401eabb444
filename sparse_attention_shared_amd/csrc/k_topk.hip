// k_topk.hip -- top-k selection of indexer scores ("CED: Continuing Context with
// a Causal Encoder and Decoder", section "Selecting Positions and Reading
// Values with Attention", Fig. 4: the indexer keeps the positions with the
// highest scores), with the Full layer's wider candidate pool from the same
// ranking (section "What Full, Reindex, and Reuse Share", Fig. 5).
//
// Order: higher score first, equal scores by lower slot.  Scores become
// order-preserving 32-bit keys; an exact radix select (four 8-bit digits, most
// significant first) finds the k-th key tau and how many keys equal to tau
// are taken; an ordered compaction then writes the chosen slots ascending.
// One 1024-thread workgroup per row; rows of up to 32768 slots keep their keys
// in LDS, longer rows re-read their scores for each pass.
#include "csa2_dev.h"
#include "csa2_kernels.h"

namespace csa2 {

constexpr int kTkThreads = 1024;
constexpr int kTkLdsKeys = 32768;

struct RowKeys {
    const float* s;
    const int32_t* ids;
    const uint32_t* lds;  // non-null: keys already staged in LDS
    __device__ __forceinline__ uint32_t from_global(int64_t i) const {
        if (ids && ids[i] < 0) return 0u;
        const uint32_t k = score_key(s[i]);
        return k == kNegInfKey ? 0u : k;
    }
    __device__ __forceinline__ uint32_t operator()(int64_t i) const {
        return lds ? lds[i] : from_global(i);
    }
};

struct TkShared {
    int hist[256];
    int scan[kTkThreads / 64 + 1];
    uint32_t bucket;
    int above;
};

// Writes the first kk slots of the row under the order (ascending slots,
// mapped through ids, -1 padded) to dst.
__device__ void select_row(const RowKeys& K, int64_t n, int n_valid, const int32_t* ids,
                           int32_t kk, int32_t* dst, TkShared& sh) {
    const int tid = threadIdx.x;
    uint32_t tau = 0;
    int need = 0;
    if (n_valid > kk) {
        uint32_t prefix = 0, mask = 0;
        int rem = kk;
        for (int shift = 24; shift >= 0; shift -= 8) {
            if (tid < 256) sh.hist[tid] = 0;
            __syncthreads();
            for (int64_t i = tid; i < n; i += kTkThreads) {
                const uint32_t key = K(i);
                if (key && (key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1);
            }
            __syncthreads();
            const int v = tid < 256 ? sh.hist[255 - tid] : 0;
            int tot;
            const int ex = block_excl_scan<kTkThreads>(v, sh.scan, &tot);
            if (tid < 256 && ex < rem && ex + v >= rem) {
                sh.bucket = 255u - (uint32_t)tid;
                sh.above = ex;
            }
            __syncthreads();
            prefix |= sh.bucket << shift;
            mask |= 0xFFu << shift;
            rem -= sh.above;
            __syncthreads();
        }
        tau = prefix;
        need = rem;
    }
    // ordered compaction over contiguous per-thread chunks
    const int64_t chunk = (n + kTkThreads - 1) / kTkThreads;
    const int64_t i0 = min(n, (int64_t)tid * chunk), i1 = min(n, i0 + chunk);
    int gt = 0, eq = 0;
    for (int64_t i = i0; i < i1; ++i) {
        const uint32_t key = K(i);
        gt += key > tau;
        eq += key == tau;
    }
    int tot;
    const int eq_before = block_excl_scan<kTkThreads>(eq, sh.scan, &tot);
    const int take_eq = min(max(need - eq_before, 0), eq);
    int total;
    int off = block_excl_scan<kTkThreads>(gt + take_eq, sh.scan, &total);
    int e = eq_before;
    for (int64_t i = i0; i < i1; ++i) {
        const uint32_t key = K(i);
        bool take = key > tau;
        if (key == tau) {
            take = e < need;
            ++e;
        }
        if (take && off < kk) dst[off++] = ids ? ids[i] : (int32_t)i;
    }
    for (int i = total + tid; i < kk; i += kTkThreads) dst[i] = -1;
    __syncthreads();
}

template <bool IN_LDS>
__global__ __launch_bounds__(kTkThreads) void k_topk(const float* __restrict__ scores, int64_t n,
                                                     int64_t ld, const int32_t* __restrict__ ids,
                                                     int32_t k, int32_t* __restrict__ out,
                                                     int32_t k2, int32_t* __restrict__ out2) {
    __shared__ TkShared sh;
    __shared__ uint32_t keys[IN_LDS ? kTkLdsKeys : 1];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    RowKeys K{scores + row * ld, ids ? ids + row * n : nullptr, nullptr};
    int nv = 0;
    for (int64_t i = tid; i < n; i += kTkThreads) {
        const uint32_t key = K.from_global(i);
        if (IN_LDS) keys[i] = key;
        nv += key != 0u;
    }
    if (IN_LDS) K.lds = keys;
    int n_valid;
    block_excl_scan<kTkThreads>(nv, sh.scan, &n_valid);
    const int32_t* irow = ids ? ids + row * n : nullptr;
    select_row(K, n, n_valid, irow, k, out + row * k, sh);
    if (out2) select_row(K, n, n_valid, irow, k2, out2 + row * k2, sh);
}

size_t topk_ws_bytes(int32_t, int64_t, int32_t, int32_t) { return 0; }

hipError_t launch_topk(const float* scores, int32_t nq, int64_t n, int64_t ld, const int32_t* ids,
                       int32_t k, int32_t* out, int32_t k2, int32_t* out2, void*, hipStream_t s) {
    if (nq == 0) return hipSuccess;
    if (n <= kTkLdsKeys)
        hipLaunchKernelGGL(k_topk<true>, dim3((uint32_t)nq), dim3(kTkThreads), 0, s, scores, n, ld,
                           ids, k, out, k2, out2);
    else
        hipLaunchKernelGGL(k_topk<false>, dim3((uint32_t)nq), dim3(kTkThreads), 0, s, scores, n,
                           ld, ids, k, out, k2, out2);
    return hipGetLastError();
}

// tokens[i][c*block + r] = blocks[i][c]*block + r when the block is chosen and
// the position is <= q_pos[i], else -1.
__global__ __launch_bounds__(256) void k_expand_blocks(const int32_t* __restrict__ blocks, int32_t nb,
                                                       int32_t block, const int32_t* __restrict__ q_pos,
                                                       int32_t* __restrict__ tokens) {
    const int32_t qi = blockIdx.y;
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = (int64_t)nb * block;
    if (j >= n) return;
    const int32_t b = blocks[(int64_t)qi * nb + j / block];
    const int64_t pos = (int64_t)b * block + j % block;
    tokens[(int64_t)qi * n + j] = (b >= 0 && pos <= q_pos[qi]) ? (int32_t)pos : -1;
}

hipError_t launch_expand_blocks(const int32_t* blocks, int32_t nq, int32_t nb, int32_t block,
                                const int32_t* q_pos, int32_t* tokens, hipStream_t s) {
    const int64_t n = (int64_t)nb * block;
    if (nq == 0 || n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_expand_blocks, dim3((uint32_t)((n + 255) / 256), (uint32_t)nq), dim3(256),
                       0, s, blocks, nb, block, q_pos, tokens);
    return hipGetLastError();
}

}  // namespace csa2

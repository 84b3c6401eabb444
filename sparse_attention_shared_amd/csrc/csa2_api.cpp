// csa2_api.cpp -- the C ABI of libcsa2 (declared in include/csa2.h): argument
// validation, workspace sizing and dispatch to the gfx950 kernels, plus the
// layer-stack driver that applies a Full / Reindex / Reuse schedule ("CED:
// Continuing Context with a Causal Encoder and Decoder", section "What Full,
// Reindex, and Reuse Share", Fig. 5).
//
// Every entry point validates on the host before enqueuing anything, reads no
// device memory, allocates nothing and never synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <new>
#include <vector>

#include "csa2.h"
#include "csa2_kernels.h"

using namespace csa2;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other (a memo, not state)

csa2_status device_ok() {
    int dev = -1;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return CSA2_ERR_NO_DEVICE;
    }
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return CSA2_ERR_NO_DEVICE;
    }
    if (dev < kMaxDevices) {
        const int v = g_arch_ok[dev].load(std::memory_order_relaxed);
        if (v) return v == 1 ? CSA2_OK : CSA2_ERR_UNSUPPORTED;
    }
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
        (void)hipGetLastError();
        return CSA2_ERR_NO_DEVICE;
    }
    const bool ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? CSA2_OK : CSA2_ERR_UNSUPPORTED;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

csa2_status from_hip(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

csa2_status check_cache(const csa2_cache* c, bool need_kv, bool need_idx, CacheView* v) {
    if (!c) return CSA2_ERR_INVALID_ARG;
    if (c->format != CSA2_KV_BF16 && c->format != CSA2_KV_FP4 && c->format != CSA2_KV_FP4_E4M3)
        return CSA2_ERR_INVALID_ARG;
    if (c->n_seq <= 0 || c->t_cap <= 0 || c->t_cap > ((int64_t)1 << 24)) return CSA2_ERR_SHAPE;
    if (c->m < 0 || c->m > 2) return CSA2_ERR_SHAPE;
    if (need_kv) {
        if (!c->data || !aligned16(c->data)) return CSA2_ERR_INVALID_ARG;
        if (c->format != CSA2_KV_BF16 && (!c->scales || !aligned16(c->scales)))
            return CSA2_ERR_INVALID_ARG;
    }
    if (need_idx && (!c->k_idx || !aligned16(c->k_idx))) return CSA2_ERR_INVALID_ARG;
    v->fp4 = c->format == CSA2_KV_FP4 ? 1 : c->format == CSA2_KV_FP4_E4M3 ? 2 : 0;
    v->msh = c->m == 2 ? 1 : 0;
    v->n_seq = c->n_seq;
    v->t_cap = c->t_cap;
    v->data = c->data;
    v->scales = c->scales;
    v->k_idx = c->k_idx;
    return CSA2_OK;
}

csa2_status check_local(const csa2_local* l, LocalView* v) {
    if (!l) return CSA2_ERR_INVALID_ARG;
    if (l->window < 0 || l->lo < 0 || l->cap < 0) return CSA2_ERR_SHAPE;
    if (l->window > l->cap) return CSA2_ERR_SHAPE;
    if (l->window > 0 && (!l->k || !l->v || !aligned16(l->k) || !aligned16(l->v)))
        return CSA2_ERR_INVALID_ARG;
    v->k = l->k;
    v->v = l->v;
    v->cap = l->cap;
    v->window = l->window;
    v->lo = l->lo;
    return CSA2_OK;
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Validate one layer's local append: its ring and both new rows.
csa2_status check_append_local(const csa2_local& l, const uint16_t* kn, const uint16_t* vn) {
    if (l.cap <= 0) return CSA2_ERR_SHAPE;
    if (!l.k || !l.v || !kn || !vn) return CSA2_ERR_INVALID_ARG;
    if (!aligned16(l.k) || !aligned16(l.v) || !aligned16(kn) || !aligned16(vn))
        return CSA2_ERR_INVALID_ARG;
    return CSA2_OK;
}

// Enqueue the append of validated arguments: the global row with the first
// (up to kMaxAppendLayers) local layers, then further launches for the rest.
// Layers whose new rows are both NULL are skipped.
// rows = n_seq with seq = -1 (decode: row b is sequence b's new position), or
// the rows of one sequence's replayed segment (seq >= 0); q_seq_out, when set,
// receives each row's sequence.
// The arguments of one append launch, without local layers.
static AppendArgs append_args(const CacheView& cv, int32_t seq, const int32_t* pos,
                              const uint16_t* kv, const uint16_t* kidx, int32_t* q_seq_out) {
    AppendArgs a{};
    a.pos = pos;
    a.seq = seq;
    a.q_seq_out = q_seq_out;
    a.t_cap = cv.t_cap;
    a.msh = cv.msh;
    a.fp4 = cv.fp4;
    a.kv = kv;
    a.kidx = kidx;
    void* data = const_cast<void*>(cv.data);
    if (cv.fp4) {
        a.codes = static_cast<uint8_t*>(data);
        a.scales = const_cast<uint8_t*>(cv.scales);
    } else {
        a.bf16 = static_cast<uint16_t*>(data);
    }
    a.k_idx = const_cast<uint16_t*>(cv.k_idx);
    return a;
}

// Adds local layers l.. to a (skipping layers without new rows) until it
// holds kMaxAppendLayers; returns the first layer left out.
static int32_t append_locals(AppendArgs& a, int32_t l, int32_t n_local, const csa2_local* local,
                             const uint16_t* const* kn, const uint16_t* const* vn) {
    a.n_local = 0;
    for (; l < n_local && a.n_local < kMaxAppendLayers; ++l) {
        if (!kn[l] && !vn[l]) continue;
        AppendLocal& d = a.local[a.n_local++];
        d.k = const_cast<uint16_t*>(local[l].k);
        d.v = const_cast<uint16_t*>(local[l].v);
        d.k_new = kn[l];
        d.v_new = vn[l];
        d.cap = local[l].cap;
    }
    return l;
}

hipError_t enqueue_append(const CacheView& cv, int32_t rows, int32_t seq, const int32_t* pos,
                          const uint16_t* kv, const uint16_t* kidx, int32_t n_local,
                          const csa2_local* local, const uint16_t* const* kn,
                          const uint16_t* const* vn, int32_t* q_seq_out, hipStream_t s) {
    AppendArgs a = append_args(cv, seq, pos, kv, kidx, q_seq_out);
    bool first = true;
    int32_t l = 0;
    do {
        l = append_locals(a, l, n_local, local, kn, vn);
        if (first || a.n_local > 0) {
            if (hipError_t e = launch_append(a, rows, s)) return e;
        }
        first = false;
        a.kv = nullptr;  // later launches update local rings only
        a.kidx = nullptr;
        a.q_seq_out = nullptr;
    } while (l < n_local);
    return hipSuccess;
}

// Workspace of one stack run.  The regions holding self-resetting counters
// come first, at offsets that depend on the number of queries alone (and not
// at all up to 64 queries): the attention counters, the Reindex select
// counters and the top-k row records; then the scratch regions (scores,
// block scores / block ids, pool scores, pool, the current selection,
// attention partials, replay sequence ids and fused top-k scratch), which no
// call needs cleared.
struct StackWs {
    size_t actr, ctr, topk, scores, bscores, blocks, pscores, pool, sel0, attn, qseq, pf, total;
};

// Whether a Full layer of a one-sequence segment takes the fused prefill top-k
// (scores never written out) instead of dense score rows + top-k.
bool replay_fused_full(int64_t t_cap, int32_t k, int32_t pool, int32_t block) {
    return block == 1 && pool == 0 && k <= kPfMaxK && t_cap <= kPfMaxT;
}

// n_seq = queries (one per sequence for decode, the segment's rows for a
// replay); replay adds the per-query sequence ids and the fused top-k scratch.
StackWs stack_ws_layout(int32_t n_seq, int64_t t_cap, int32_t k, int32_t pool, int32_t block,
                        int32_t max_window, bool replay = false) {
    StackWs w{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align_up(bytes);
        return o;
    };
    const int64_t nb = block > 1 ? (t_cap + block - 1) / block : 0;
    const int32_t nbsel = block > 1 ? pool / block : 0;
    const bool fused = replay && replay_fused_full(t_cap, k, pool, block);
    w.actr = take(kAttnCtrBytes);
    w.ctr = take((size_t)std::max(n_seq, kCtrBlockQueries) * kCtrStride * sizeof(uint32_t));
    size_t tk = topk_ws_bytes(n_seq, t_cap, k, pool);
    if (block > 1) tk = std::max(tk, topk_ws_bytes(n_seq, nb, nbsel, 0));
    if (pool > 0) tk = std::max(tk, topk_ws_bytes(n_seq, pool, k, 0));
    w.topk = take(tk > 0 ? tk : 1);
    w.scores = take(fused ? 1 : (size_t)n_seq * t_cap * sizeof(float));
    w.bscores = take((size_t)n_seq * (nb > 0 ? nb : 1) * sizeof(float));
    w.blocks = take((size_t)n_seq * (nbsel > 0 ? nbsel : 1) * sizeof(int32_t));
    w.pscores = take((size_t)n_seq * score_select_ld(pool > 0 ? pool : 1) * sizeof(float));
    w.pool = take((size_t)n_seq * (pool > 0 ? pool : 1) * sizeof(int32_t));
    w.sel0 = take((size_t)n_seq * k * sizeof(int32_t));
    w.attn = take(std::max<size_t>(attn_part_bytes(n_seq, k, max_window), 1));
    if (replay) {
        w.qseq = take((size_t)n_seq * sizeof(int32_t));
        if (fused) w.pf = take(prefill_topk_ws_bytes(n_seq, t_cap));
    }
    w.total = off;
    return w;
}
}  // namespace

extern "C" {

int csa2_version(void) { return CSA2_VERSION; }

const char* csa2_status_str(csa2_status s) {
    switch (s) {
        case CSA2_OK: return "ok";
        case CSA2_ERR_INVALID_ARG: return "invalid argument";
        case CSA2_ERR_SHAPE: return "inconsistent shape";
        case CSA2_ERR_SCHEDULE: return "invalid layer schedule";
        case CSA2_ERR_WORKSPACE: return "workspace too small";
        case CSA2_ERR_UNSUPPORTED: return "device is not gfx950";
        case CSA2_ERR_NO_DEVICE: return "no HIP device";
        case CSA2_ERR_HIP: return "HIP launch error";
        case CSA2_ERR_TOO_LARGE: return "call larger than the allocation-free scratch";
    }
    return "unknown status";
}

csa2_status csa2_device_check(void) { return device_ok(); }

csa2_status csa2_pack_fp4(const uint16_t* x, int64_t rows, int32_t dim, uint8_t* codes,
                          uint8_t* scales, void* stream) {
    if (rows < 0 || dim <= 0) return CSA2_ERR_SHAPE;
    if (dim % 32) return CSA2_ERR_SHAPE;
    if (rows > 0 && (!x || !codes || !scales || !aligned16(x) || !aligned16(codes)))
        return CSA2_ERR_INVALID_ARG;
    if (csa2_status st = device_ok()) return st;
    return from_hip(launch_pack_fp4(x, rows * (dim / 32), codes, scales, (hipStream_t)stream));
}

csa2_status csa2_pack_fp4_e4m3(const uint16_t* x, int64_t rows, int32_t dim, uint8_t* codes,
                               uint8_t* scales, void* stream) {
    if (rows < 0 || dim <= 0 || dim % 16) return CSA2_ERR_SHAPE;
    if (rows > 0 && (!x || !codes || !scales || !aligned16(x) ||
                     (reinterpret_cast<uintptr_t>(codes) & 7u) != 0))
        return CSA2_ERR_INVALID_ARG;
    if (csa2_status st = device_ok()) return st;
    return from_hip(launch_pack_fp4e(x, rows * (dim / 16), codes, scales, (hipStream_t)stream));
}

csa2_status csa2_unpack_fp4_e4m3(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                 int32_t dim, float* out, void* stream) {
    if (rows < 0 || dim <= 0 || dim % 16) return CSA2_ERR_SHAPE;
    if (rows > 0 && (!codes || !scales || !out || (reinterpret_cast<uintptr_t>(codes) & 7u) != 0 ||
                     !aligned16(out)))
        return CSA2_ERR_INVALID_ARG;
    if (csa2_status st = device_ok()) return st;
    return from_hip(launch_unpack_fp4e(codes, scales, rows * (dim / 16), out, (hipStream_t)stream));
}

csa2_status csa2_unpack_fp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t dim,
                            float* out, void* stream) {
    if (rows < 0 || dim <= 0 || dim % 32) return CSA2_ERR_SHAPE;
    if (rows > 0 && (!codes || !scales || !out || !aligned16(codes) || !aligned16(out)))
        return CSA2_ERR_INVALID_ARG;
    if (csa2_status st = device_ok()) return st;
    return from_hip(launch_unpack_fp4(codes, scales, rows * (dim / 32), out, (hipStream_t)stream));
}

csa2_status csa2_compress(const uint16_t* x, int64_t groups, int32_t m, int32_t dim,
                          uint16_t* out, void* stream) {
    if (groups < 0 || dim <= 0 || dim % 8 || (m != 1 && m != 2)) return CSA2_ERR_SHAPE;
    if (groups > 0 && (!x || !out || !aligned16(x) || !aligned16(out))) return CSA2_ERR_INVALID_ARG;
    if (csa2_status st = device_ok()) return st;
    return from_hip(launch_compress(x, groups, m, dim, out, (hipStream_t)stream));
}

csa2_status csa2_append(const csa2_cache* cache, const int32_t* pos, const uint16_t* kv,
                        const uint16_t* kidx, int32_t n_local, const csa2_local* local,
                        const uint16_t* const* k_new, const uint16_t* const* v_new,
                        void* stream) {
    CacheView cv;
    if (csa2_status st = check_cache(cache, kv != nullptr, kidx != nullptr, &cv)) return st;
    if (n_local < 0) return CSA2_ERR_SHAPE;
    if (!pos) return CSA2_ERR_INVALID_ARG;
    if ((kv && !aligned16(kv)) || (kidx && !aligned16(kidx))) return CSA2_ERR_INVALID_ARG;
    if (n_local > 0 && (!local || !k_new || !v_new)) return CSA2_ERR_INVALID_ARG;
    for (int32_t l = 0; l < n_local; ++l)
        if (csa2_status st = check_append_local(local[l], k_new[l], v_new[l])) return st;
    if (csa2_status st = device_ok()) return st;
    return from_hip(enqueue_append(cv, cv.n_seq, -1, pos, kv, kidx, n_local, local, k_new, v_new,
                                   nullptr, (hipStream_t)stream));
}

csa2_status csa2_index_score(const csa2_cache* cache, const uint16_t* q_idx, const int32_t* q_pos,
                             const int32_t* q_seq, int32_t nq, const int32_t* cand, int64_t n_cand,
                             int32_t block, float* scores, int64_t ld_scores, void* stream) {
    CacheView cv;
    if (csa2_status st = check_cache(cache, false, true, &cv)) return st;
    if (nq < 0) return CSA2_ERR_SHAPE;
    if (nq > 0 && (!q_idx || !q_pos || !scores || !aligned16(q_idx)))
        return CSA2_ERR_INVALID_ARG;
    if (nq > 65535) return CSA2_ERR_SHAPE;
    if (cand) {
        if (block != 1 || n_cand < 0 || ld_scores < n_cand) return CSA2_ERR_SHAPE;
    } else {
        if (block != 1 && block != 64) return CSA2_ERR_SHAPE;
        const int64_t n_out = (cv.t_cap + block - 1) / block;
        if (ld_scores < n_out) return CSA2_ERR_SHAPE;
    }
    if (csa2_status st = device_ok()) return st;
    hipStream_t s = (hipStream_t)stream;
    if (cand)
        return from_hip(launch_score_cand(cv, q_idx, q_pos, q_seq, nq, cand, n_cand, scores,
                                          ld_scores, s));
    return from_hip(launch_score_dense(cv, q_idx, q_pos, q_seq, nq, block, scores, ld_scores, s));
}

csa2_status csa2_prefill_score(const csa2_cache* cache, int32_t seq, const uint16_t* q_idx,
                               const int32_t* q_pos, int32_t nq, float* scores, int64_t ld_scores,
                               void* stream) {
    CacheView cv;
    if (csa2_status st = check_cache(cache, false, true, &cv)) return st;
    if (nq < 0 || seq < 0 || seq >= cv.n_seq || ld_scores < cv.t_cap) return CSA2_ERR_SHAPE;
    if (nq > 65535 * 64) return CSA2_ERR_SHAPE;
    if (nq > 0 && (!q_idx || !q_pos || !scores || !aligned16(q_idx))) return CSA2_ERR_INVALID_ARG;
    if (csa2_status st = device_ok()) return st;
    return from_hip(launch_score_mq(cv, seq, q_idx, q_pos, nq, scores, ld_scores, (hipStream_t)stream));
}

csa2_status csa2_prefill_topk_workspace(int32_t nq, int64_t t_cap, int32_t k, size_t* bytes) {
    if (!bytes) return CSA2_ERR_INVALID_ARG;
    if (nq < 0 || t_cap < 1 || t_cap > kPfMaxT || k < 1 || k > kPfMaxK) return CSA2_ERR_SHAPE;
    *bytes = prefill_topk_ws_bytes(nq, t_cap);
    return CSA2_OK;
}

csa2_status csa2_prefill_topk(const csa2_cache* cache, int32_t seq, const uint16_t* q_idx,
                              const int32_t* q_pos, int32_t nq, int32_t k, int32_t* sel, void* ws,
                              size_t ws_bytes, void* stream) {
    CacheView cv;
    if (csa2_status st = check_cache(cache, false, true, &cv)) return st;
    if (nq < 0 || seq < 0 || seq >= cv.n_seq || k < 1 || k > kPfMaxK || cv.t_cap > kPfMaxT)
        return CSA2_ERR_SHAPE;
    if (nq == 0) return CSA2_OK;
    if (!q_idx || !q_pos || !sel || !ws || !aligned16(q_idx)) return CSA2_ERR_INVALID_ARG;
    if (ws_bytes < prefill_topk_ws_bytes(nq, cv.t_cap)) return CSA2_ERR_WORKSPACE;
    if (csa2_status st = device_ok()) return st;
    return from_hip(launch_prefill_topk(cv, seq, q_idx, q_pos, nq, k, sel, ws, (hipStream_t)stream));
}

csa2_status csa2_topk_workspace(int32_t nq, int64_t n, int32_t k, int32_t k2, size_t* bytes) {
    if (!bytes) return CSA2_ERR_INVALID_ARG;
    if (nq < 0 || n < 0 || k <= 0 || k2 < 0) return CSA2_ERR_SHAPE;
    *bytes = topk_ws_bytes(nq, n, k, k2);
    return CSA2_OK;
}

csa2_status csa2_topk(const float* scores, int32_t nq, int64_t n, int64_t ld, const int32_t* ids,
                      int32_t k, int32_t* out, int32_t k2, int32_t* out2, void* ws,
                      size_t ws_bytes, void* stream) {
    if (nq < 0 || n < 0 || ld < n || k <= 0 || n > ((int64_t)1 << 24)) return CSA2_ERR_SHAPE;
    if (out2 && k2 < k) return CSA2_ERR_SHAPE;
    if (nq > 0 && (!scores || !out)) return CSA2_ERR_INVALID_ARG;
    const size_t need = topk_ws_bytes(nq, n, k, out2 ? k2 : 0);
    if (need > 0 && (!ws || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
    if (csa2_status st = device_ok()) return st;
    return from_hip(launch_topk(scores, nq, n, ld, ids, k, out, out2 ? k2 : 0, out2, ws,
                                (hipStream_t)stream));
}

csa2_status csa2_expand_blocks(const int32_t* blocks, int32_t nq, int32_t nb, int32_t block,
                               const int32_t* q_pos, int32_t* tokens, void* stream) {
    if (nq < 0 || nb < 0 || block <= 0) return CSA2_ERR_SHAPE;
    if ((int64_t)nb * block > (int64_t)INT32_MAX) return CSA2_ERR_SHAPE;
    if (nq > 0 && nb > 0 && (!blocks || !q_pos || !tokens)) return CSA2_ERR_INVALID_ARG;
    if (csa2_status st = device_ok()) return st;
    return from_hip(launch_expand_blocks(blocks, nq, nb, block, q_pos, tokens, (hipStream_t)stream));
}

csa2_status csa2_sparse_attn_workspace(int32_t nq, int32_t k, int32_t window, size_t* bytes) {
    if (!bytes) return CSA2_ERR_INVALID_ARG;
    if (nq < 0 || k < 0 || window < 0) return CSA2_ERR_SHAPE;
    *bytes = attn_ws_bytes(nq, k, window);
    return CSA2_OK;
}

csa2_status csa2_sparse_attn(const csa2_cache* cache, const uint16_t* q, const int32_t* q_pos,
                             const int32_t* q_seq, int32_t nq, const int32_t* sel, int32_t k,
                             const csa2_local* local, float sm_scale, uint16_t* out, void* ws,
                             size_t ws_bytes, void* stream) {
    CacheView cv;
    LocalView lv;
    if (csa2_status st = check_cache(cache, true, false, &cv)) return st;
    if (csa2_status st = check_local(local, &lv)) return st;
    if (nq < 0 || k < 0 || nq > 65535) return CSA2_ERR_SHAPE;
    if (nq > 0 && (!q || !q_pos || !out || !aligned16(q))) return CSA2_ERR_INVALID_ARG;
    if (nq > 0 && k > 0 && !sel) return CSA2_ERR_INVALID_ARG;
    const size_t need = attn_ws_bytes(nq, k, lv.window);
    if (need > 0 && (!ws || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
    if (csa2_status st = device_ok()) return st;
    return from_hip(launch_sparse_attn(cv, q, q_pos, q_seq, nq, sel, k, lv, sm_scale, out, ws,
                                       (hipStream_t)stream));
}

csa2_status csa2_sparse_attn_noalloc(const csa2_cache* cache, const uint16_t* q,
                                     const int32_t* q_pos, const int32_t* q_seq, int32_t nq,
                                     const int32_t* sel, int32_t k, const csa2_local* local,
                                     float sm_scale, uint16_t* out, void* stream) {
    CacheView cv;
    LocalView lv;
    if (csa2_status st = check_cache(cache, true, false, &cv)) return st;
    if (csa2_status st = check_local(local, &lv)) return st;
    if (nq < 0 || k < 0 || nq > 65535) return CSA2_ERR_SHAPE;
    if (nq > 0 && (!q || !q_pos || !out || !aligned16(q))) return CSA2_ERR_INVALID_ARG;
    if (nq > 0 && k > 0 && !sel) return CSA2_ERR_INVALID_ARG;
    if (attn_part_bytes(nq, k, lv.window) > kStaticScratchBytes - kAttnCtrBytes)
        return CSA2_ERR_TOO_LARGE;
    if (csa2_status st = device_ok()) return st;
    return from_hip(launch_sparse_attn_static(cv, q, q_pos, q_seq, nq, sel, k, lv, sm_scale, out,
                                              (hipStream_t)stream));
}

// What one stack run needs, from a decode descriptor (one query per
// sequence) or a replay descriptor (a segment of one sequence).
struct StackJob {
    int32_t n_layers;
    const int32_t* modes;
    int32_t nq;   // queries
    int32_t seq;  // -1: query b is on sequence b; else every query is on `seq`
    const int32_t* q_pos;
    int32_t k, pool, block;
    float sm_scale;
    const uint16_t* const* q;
    const uint16_t* const* q_idx;
    const csa2_local* local;
    uint16_t* const* out;
    int32_t* const* sel_out;
    int32_t* pool_out;
    void* const* scan_events;  // [2] or null (decode only)
    void* const* attn_events;  // [2 n_layers] or null (decode only)
    const uint16_t* app_kv;
    const uint16_t* app_kidx;
    const uint16_t* const* app_k;
    const uint16_t* const* app_v;
};

// Checks shared by both descriptors: schedule, per-layer operands, local
// rings and the rows to write into them.
static csa2_status check_job(const StackJob& j, int32_t* max_window) {
    if (j.n_layers <= 0) return CSA2_ERR_SHAPE;
    if (j.k <= 0 || j.pool < 0 || j.block <= 0) return CSA2_ERR_SHAPE;
    if (j.block != 1 && j.block != 64) return CSA2_ERR_SHAPE;
    if (j.pool > 0 && j.pool < j.k) return CSA2_ERR_SHAPE;
    if (j.block > 1 && (j.pool <= 0 || j.pool % j.block)) return CSA2_ERR_SHAPE;
    if (j.modes[0] != CSA2_MODE_FULL) return CSA2_ERR_SCHEDULE;
    int32_t mw = 0;
    for (int32_t l = 0; l < j.n_layers; ++l) {
        const int32_t m = j.modes[l];
        if (m != CSA2_MODE_FULL && m != CSA2_MODE_REINDEX && m != CSA2_MODE_REUSE)
            return CSA2_ERR_SCHEDULE;
        if (m == CSA2_MODE_REINDEX && j.pool <= 0) return CSA2_ERR_SCHEDULE;
        if (!j.q[l] || !j.out[l] || !aligned16(j.q[l])) return CSA2_ERR_INVALID_ARG;
        if (m != CSA2_MODE_REUSE && (!j.q_idx || !j.q_idx[l] || !aligned16(j.q_idx[l])))
            return CSA2_ERR_INVALID_ARG;
        LocalView lv;
        if (csa2_status st = check_local(&j.local[l], &lv)) return st;
        mw = std::max(mw, lv.window);
    }
    if ((j.app_k != nullptr) != (j.app_v != nullptr)) return CSA2_ERR_INVALID_ARG;
    if (j.app_k)
        for (int32_t l = 0; l < j.n_layers; ++l) {
            if (!j.app_k[l] && !j.app_v[l]) continue;
            if (csa2_status st = check_append_local(j.local[l], j.app_k[l], j.app_v[l])) return st;
            // a segment's rows must land in distinct slots
            if (j.seq >= 0 && j.nq > j.local[l].cap) return CSA2_ERR_SHAPE;
        }
    *max_window = mw;
    return CSA2_OK;
}

static StackJob decode_job(const csa2_stack_desc* d) {
    StackJob j{};
    j.n_layers = d->n_layers;
    j.modes = d->modes;
    j.nq = d->cache->n_seq;
    j.seq = -1;
    j.q_pos = d->q_pos;
    j.k = d->k;
    j.pool = d->pool;
    j.block = d->block;
    j.sm_scale = d->sm_scale;
    j.q = d->q;
    j.q_idx = d->q_idx;
    j.local = d->local;
    j.out = d->out;
    j.sel_out = d->sel_out;
    j.pool_out = d->pool_out;
    j.scan_events = d->scan_events;
    j.attn_events = d->attn_events;
    j.app_kv = d->append_kv;
    j.app_kidx = d->append_kidx;
    j.app_k = d->append_k;
    j.app_v = d->append_v;
    return j;
}

static csa2_status check_stack(const csa2_stack_desc* d, CacheView* cv, int32_t* max_window) {
    if (!d || !d->modes || !d->cache || !d->q_pos || !d->q || !d->local || !d->out)
        return CSA2_ERR_INVALID_ARG;
    if (d->n_layers <= 0) return CSA2_ERR_SHAPE;
    if (csa2_status st = check_cache(d->cache, true, true, cv)) return st;
    if (cv->n_seq > 65535) return CSA2_ERR_SHAPE;
    if (d->append_kidx && !d->append_kv) return CSA2_ERR_INVALID_ARG;
    if (d->append_k && !d->append_kv) return CSA2_ERR_INVALID_ARG;
    if (d->append_kv &&
        (!aligned16(d->append_kv) || (d->append_kidx && !aligned16(d->append_kidx))))
        return CSA2_ERR_INVALID_ARG;
    return check_job(decode_job(d), max_window);
}

static StackJob replay_job(const csa2_replay_desc* d) {
    StackJob j{};
    j.n_layers = d->n_layers;
    j.modes = d->modes;
    j.nq = d->n;
    j.seq = d->seq;
    j.q_pos = d->q_pos;
    j.k = d->k;
    j.pool = d->pool;
    j.block = d->block;
    j.sm_scale = d->sm_scale;
    j.q = d->q;
    j.q_idx = d->q_idx;
    j.local = d->local;
    j.out = d->out;
    j.sel_out = d->sel_out;
    j.pool_out = d->pool_out;
    j.app_k = d->local_k;
    j.app_v = d->local_v;
    return j;
}

static csa2_status check_replay(const csa2_replay_desc* d, CacheView* cv, int32_t* max_window) {
    if (!d || !d->modes || !d->cache || !d->q_pos || !d->q || !d->local || !d->out)
        return CSA2_ERR_INVALID_ARG;
    if (d->n_layers <= 0) return CSA2_ERR_SHAPE;
    if (csa2_status st = check_cache(d->cache, true, true, cv)) return st;
    if (d->seq < 0 || d->seq >= cv->n_seq) return CSA2_ERR_SHAPE;
    if (d->n <= 0 || d->n > 65535) return CSA2_ERR_SHAPE;
    return check_job(replay_job(d), max_window);
}

static StackWs job_ws_layout(const StackJob& j, const CacheView& cv, int32_t mw) {
    return stack_ws_layout(j.nq, cv.t_cap, j.k, j.pool, j.block, mw, j.seq >= 0);
}

csa2_status csa2_stack_workspace(const csa2_stack_desc* d, size_t* bytes) {
    if (!bytes) return CSA2_ERR_INVALID_ARG;
    CacheView cv;
    int32_t mw;
    if (csa2_status st = check_stack(d, &cv, &mw)) return st;
    *bytes = job_ws_layout(decode_job(d), cv, mw).total;
    return CSA2_OK;
}

csa2_status csa2_replay_workspace(const csa2_replay_desc* d, size_t* bytes) {
    if (!bytes) return CSA2_ERR_INVALID_ARG;
    CacheView cv;
    int32_t mw;
    if (csa2_status st = check_replay(d, &cv, &mw)) return st;
    *bytes = job_ws_layout(replay_job(d), cv, mw).total;
    return CSA2_OK;
}

}  // extern "C"

// Enqueue every layer of a validated stack on s.
static csa2_status enqueue_stack(const StackJob& j, const CacheView& cv, const StackWs& W,
                                 void* ws, hipStream_t s) {
    char* base = static_cast<char*>(ws);
    float* scores = reinterpret_cast<float*>(base + W.scores);
    float* bscores = reinterpret_cast<float*>(base + W.bscores);
    int32_t* blocks = reinterpret_cast<int32_t*>(base + W.blocks);
    float* pscores = reinterpret_cast<float*>(base + W.pscores);
    int32_t* pool = j.pool_out ? j.pool_out : reinterpret_cast<int32_t*>(base + W.pool);
    int32_t* selbuf = reinterpret_cast<int32_t*>(base + W.sel0);
    uint32_t* ctr = reinterpret_cast<uint32_t*>(base + W.ctr);
    void* tkws = base + W.topk;
    uint32_t* actr = reinterpret_cast<uint32_t*>(base + W.actr);
    float* apart = reinterpret_cast<float*>(base + W.attn);
    const bool replay = j.seq >= 0;
    // decode: query b reads sequence b; replay: the ids the append step writes
    int32_t* q_seq = replay ? reinterpret_cast<int32_t*>(base + W.qseq) : nullptr;
    const int32_t S = j.nq, k = j.k, P = j.pool, B = j.block;
    const bool fused_full = replay && replay_fused_full(cv.t_cap, k, P, B);
    // A blockwise pool of power-of-two blocks that one scoring launch takes is
    // rescored from its block ids (each candidate's position computed where it
    // is read); the position list is written only for a caller's pool_out.
    int32_t bshift = 0;
    while (B > 1 && (1 << bshift) < B) ++bshift;
    const bool block_pool = B > 1 && (1 << bshift) == B && P <= kFusedSelectMax;
    // score the pool with layer l's indexer query and keep the top k
    auto rescore_pool = [&](int32_t l, int32_t* dst) -> hipError_t {
        if (block_pool)
            return launch_score_select(cv, j.q_idx[l], j.q_pos, q_seq, S, blocks, P, pscores, ctr,
                                       k, dst, s, bshift);
        if (P <= kFusedSelectMax)
            return launch_score_select(cv, j.q_idx[l], j.q_pos, q_seq, S, pool, P, pscores, ctr,
                                       k, dst, s);
        hipError_t e = launch_score_cand(cv, j.q_idx[l], j.q_pos, q_seq, S, pool, P, pscores, P, s);
        if (e == hipSuccess) e = launch_topk(pscores, S, P, P, pool, k, dst, 0, nullptr, tkws, s);
        return e;
    };
    // decode: an append whose rows fit one launch runs inside layer 0's
    // tokenwise scan (the scan takes each query's new key from the rows)
    AppendArgs fused_app{};
    bool fuse_append = false;
    if (!replay && j.app_kv && j.app_kidx && j.n_layers > 0 && j.modes[0] == CSA2_MODE_FULL &&
        B == 1) {
        fused_app = append_args(cv, -1, j.q_pos, j.app_kv, j.app_kidx, nullptr);
        const int32_t nl = j.app_k ? j.n_layers : 0;
        fuse_append = append_locals(fused_app, 0, nl, j.local, j.app_k, j.app_v) >= nl;
    }
    // decode append of the new positions, or the segment's ring rows (the
    // replay always launches it: it also writes the sequence ids)
    if ((j.app_kv || replay) && !fuse_append) {
        const int32_t nl = j.app_k ? j.n_layers : 0;
        if (enqueue_append(cv, S, j.seq, j.q_pos, j.app_kv, j.app_kidx, nl, j.local, j.app_k,
                           j.app_v, q_seq, s) != hipSuccess)
            return CSA2_ERR_HIP;
    }
    const int32_t* cur = nullptr;
    for (int32_t l = 0; l < j.n_layers; ++l) {
        const int32_t m = j.modes[l];
        int32_t* sel_l = (j.sel_out && j.sel_out[l]) ? j.sel_out[l] : nullptr;
        hipError_t e = hipSuccess;
        if (m == CSA2_MODE_FULL || m == CSA2_MODE_REINDEX) {
            int32_t* dst = sel_l ? sel_l : selbuf;
            // layer 0 is Full: on a stream being recorded into a graph the
            // events bracket the scan; otherwise they take the kernel's own
            // start and end times
            const bool timed = l == 0 && j.scan_events && j.scan_events[0] && j.scan_events[1];
            hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
            if (timed) e = hipStreamIsCapturing(s, &cap);
            const bool own = timed && e == hipSuccess && cap == hipStreamCaptureStatusNone;
            hipEvent_t ev0 = own ? (hipEvent_t)j.scan_events[0] : nullptr;
            hipEvent_t ev1 = own ? (hipEvent_t)j.scan_events[1] : nullptr;
            const bool around = timed && !own;
            if (around && e == hipSuccess) e = hipEventRecord((hipEvent_t)j.scan_events[0], s);
            if (e != hipSuccess) return CSA2_ERR_HIP;
            if (m == CSA2_MODE_FULL && fused_full) {
                e = launch_prefill_topk(cv, j.seq, j.q_idx[l], j.q_pos, S, k, dst, base + W.pf, s);
            } else if (m == CSA2_MODE_FULL && B == 1) {
                if (replay)
                    e = launch_score_mq(cv, j.seq, j.q_idx[l], j.q_pos, S, scores, cv.t_cap, s);
                else if (l == 0 && fuse_append)
                    e = launch_score_dense_append(cv, j.q_idx[l], j.q_pos, S, scores, cv.t_cap,
                                                  fused_app, s, ev0, ev1);
                else
                    e = launch_score_dense(cv, j.q_idx[l], j.q_pos, q_seq, S, 1, scores, cv.t_cap,
                                           s, ev0, ev1);
                if (around && e == hipSuccess) e = hipEventRecord((hipEvent_t)j.scan_events[1], s);
                if (e == hipSuccess)
                    e = launch_topk(scores, S, cv.t_cap, cv.t_cap, nullptr, k, dst, P, P ? pool : nullptr,
                                    tkws, s);
            } else if (m == CSA2_MODE_FULL) {
                const int64_t nb = (cv.t_cap + B - 1) / B;
                const int32_t nbsel = P / B;
                e = launch_score_dense(cv, j.q_idx[l], j.q_pos, q_seq, S, B, bscores, nb, s, ev0, ev1);
                if (around && e == hipSuccess) e = hipEventRecord((hipEvent_t)j.scan_events[1], s);
                if (e == hipSuccess)
                    e = launch_topk(bscores, S, nb, nb, nullptr, nbsel, blocks, 0, nullptr, tkws, s);
                if (e == hipSuccess && (!block_pool || j.pool_out))
                    e = launch_expand_blocks(blocks, S, nbsel, B, j.q_pos, pool, s, cv.msh);
                if (e == hipSuccess) e = rescore_pool(l, dst);
            } else {
                e = rescore_pool(l, dst);
            }
            cur = dst;
        } else if (sel_l) {
            e = hipMemcpyAsync(sel_l, cur, sizeof(int32_t) * S * k, hipMemcpyDeviceToDevice, s);
        }
        if (e != hipSuccess) return CSA2_ERR_HIP;
        LocalView lv;
        check_local(&j.local[l], &lv);
        hipEvent_t a0 = nullptr, a1 = nullptr;
        if (j.attn_events && j.attn_events[2 * l] && j.attn_events[2 * l + 1]) {
            hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
            if (hipStreamIsCapturing(s, &cap) != hipSuccess) return CSA2_ERR_HIP;
            if (cap == hipStreamCaptureStatusNone) {  // a plan ignores them
                a0 = (hipEvent_t)j.attn_events[2 * l];
                a1 = (hipEvent_t)j.attn_events[2 * l + 1];
            }
        }
        e = launch_sparse_attn_parts(cv, j.q[l], j.q_pos, q_seq, S, cur, k, lv, j.sm_scale,
                                     j.out[l], actr, apart, s, a0, a1);
        if (e != hipSuccess) return CSA2_ERR_HIP;
    }
    return CSA2_OK;
}

extern "C" {

csa2_status csa2_stack_run(const csa2_stack_desc* d, void* ws, size_t ws_bytes, void* stream) {
    CacheView cv;
    int32_t mw;
    if (csa2_status st = check_stack(d, &cv, &mw)) return st;
    const StackJob j = decode_job(d);
    const StackWs W = job_ws_layout(j, cv, mw);
    if (!ws || ws_bytes < W.total) return CSA2_ERR_WORKSPACE;
    if (csa2_status st = device_ok()) return st;
    return enqueue_stack(j, cv, W, ws, (hipStream_t)stream);
}

csa2_status csa2_replay_run(const csa2_replay_desc* d, void* ws, size_t ws_bytes, void* stream) {
    CacheView cv;
    int32_t mw;
    if (csa2_status st = check_replay(d, &cv, &mw)) return st;
    const StackJob j = replay_job(d);
    const StackWs W = job_ws_layout(j, cv, mw);
    if (!ws || ws_bytes < W.total) return CSA2_ERR_WORKSPACE;
    if (csa2_status st = device_ok()) return st;
    return enqueue_stack(j, cv, W, ws, (hipStream_t)stream);
}

}  // extern "C"

// A recorded stack: the graph captured from one enqueue_stack and its
// executable instance.
struct csa2_stack_plan {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

extern "C" {

csa2_status csa2_stack_plan_create(const csa2_stack_desc* d, void* ws, size_t ws_bytes,
                                   csa2_stack_plan** plan) {
    if (!plan) return CSA2_ERR_INVALID_ARG;
    *plan = nullptr;
    CacheView cv;
    int32_t mw;
    if (csa2_status st = check_stack(d, &cv, &mw)) return st;
    const StackJob j = decode_job(d);
    const StackWs W = job_ws_layout(j, cv, mw);
    if (!ws || ws_bytes < W.total) return CSA2_ERR_WORKSPACE;
    if (csa2_status st = device_ok()) return st;
    hipStream_t cs = nullptr;
    if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return CSA2_ERR_HIP;
    hipGraph_t graph = nullptr;
    csa2_status st = CSA2_OK;
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
        st = CSA2_ERR_HIP;
    } else {
        st = enqueue_stack(j, cv, W, ws, cs);
        // the capture must be ended whatever happened inside it
        if (hipStreamEndCapture(cs, &graph) != hipSuccess && st == CSA2_OK) st = CSA2_ERR_HIP;
    }
    hipStreamDestroy(cs);
    if (st == CSA2_OK && !graph) st = CSA2_ERR_HIP;
    hipGraphExec_t exec = nullptr;
    if (st == CSA2_OK && hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess)
        st = CSA2_ERR_HIP;
    csa2_stack_plan* p = nullptr;
    if (st == CSA2_OK) {
        p = new (std::nothrow) csa2_stack_plan;
        if (!p) st = CSA2_ERR_HIP;
    }
    if (st != CSA2_OK) {
        if (exec) hipGraphExecDestroy(exec);
        if (graph) hipGraphDestroy(graph);
        return st;
    }
    p->graph = graph;
    p->exec = exec;
    *plan = p;
    return CSA2_OK;
}

csa2_status csa2_stack_plan_launch(const csa2_stack_plan* plan, void* stream) {
    if (!plan || !plan->exec) return CSA2_ERR_INVALID_ARG;
    return from_hip(hipGraphLaunch(plan->exec, (hipStream_t)stream));
}

csa2_status csa2_stack_plan_destroy(csa2_stack_plan* plan) {
    if (!plan) return CSA2_OK;
    hipError_t e1 = plan->exec ? hipGraphExecDestroy(plan->exec) : hipSuccess;
    hipError_t e2 = plan->graph ? hipGraphDestroy(plan->graph) : hipSuccess;
    delete plan;
    return (e1 == hipSuccess && e2 == hipSuccess) ? CSA2_OK : CSA2_ERR_HIP;
}

}  // extern "C"

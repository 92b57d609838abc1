// C-ABI layer of libkvq: argument validation, arena layout, split planning.
// Pure host C++ (no HIP headers): every check runs before any launch, so a
// call that fails validation enqueues nothing and leaves the cache unchanged.
#include <cstdlib>
#include <cstring>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr uint64_t kAlign = 256;
constexpr int64_t kMaxQuantSplits = 1000;  // merge keeps per-split weights in LDS

constexpr int64_t kMaxGridY = 65535;  // largest second grid dimension of a launch
uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Words of a unit's eviction bitmap: one bit per token after the sinks.
uint64_t evict_words_of(const kvq_config* c) {
    const int64_t n = c->max_tokens > c->sinks ? c->max_tokens - c->sinks : 0;
    return (uint64_t)(n + 31) / 32;
}

// Key groups the kmeta region holds for C chunks: G = 16 keeps both groups of
// every chunk, so that a half-used last chunk still has a (zeroed) second entry.
uint64_t key_groups_of(uint64_t G, uint64_t C) { return G == 16 ? 2 * C : C * kChunk / G; }

int64_t n_quantized(int64_t T, int64_t R, int64_t G) {
    // Tokens held quantized after T appends: the residual window keeps the
    // last R tokens plus any incomplete group in fp16 ("KV cache quantization
    // and eviction", section "Minimal implementation").
    return T > R ? (T - R) / G * G : 0;
}

kvq_status check_config(const kvq_config* c) {
    if (!c) return KVQ_EINVAL;
    if (c->residual < 0 || c->pool < 0 || c->evict_cap < 0 || c->batch < 1 ||
        c->n_kv_heads < 1 || c->n_q_heads < 1 || c->max_tokens < 1 || c->sinks < 0)
        return KVQ_EINVAL;
    if (c->n_q_heads % c->n_kv_heads != 0) return KVQ_EINVAL;
    const int r = c->n_q_heads / c->n_kv_heads;
    if (c->bits != 2 && c->bits != 4 && c->bits != 8) return KVQ_EUNSUPPORTED;
    // the FP8 codec has no groups or outlier pools; 32 is its chunk size
    if (c->bits == 8 && (c->group != 32 || c->pool != 0)) return KVQ_EUNSUPPORTED;
    if (c->group != 16 && c->group != 32 && c->group != 64 && c->group != 128)
        return KVQ_EUNSUPPORTED;
    if (c->head_dim != kHeadDim) return KVQ_EUNSUPPORTED;
    if (r != 1 && r != 2 && r != 4) return KVQ_EUNSUPPORTED;
    if (c->pool > kMaxPool || c->evict_cap > kMaxEvict || c->sinks > kMaxSinks)
        return KVQ_EUNSUPPORTED;
    if (c->max_tokens > kMaxTokens) return KVQ_EUNSUPPORTED;
    // units index the second grid dimension of the ring and sink stores
    if ((int64_t)c->batch * c->n_kv_heads > kMaxGridY) return KVQ_EUNSUPPORTED;
    if ((int64_t)c->residual + c->group + c->pool + c->evict_cap + c->sinks > kMaxFp16Rows)
        return KVQ_EUNSUPPORTED;
    return KVQ_OK;
}

constexpr int kRegions = 21;

struct Layout {
    uint64_t off[kRegions];
    uint64_t total;
    int64_t q_cap, chunks, ring;
};

Layout layout_of(const kvq_config* c) {
    Layout L{};
    const uint64_t U = (uint64_t)c->batch * c->n_kv_heads;
    const uint64_t d = kHeadDim;
    const uint64_t G = c->group, b = c->bits, N = c->pool, E = c->evict_cap;
    L.q_cap = n_quantized(c->max_tokens > c->sinks ? c->max_tokens - c->sinks : 0, c->residual,
                          c->group);
    L.chunks = (L.q_cap + kChunk - 1) / kChunk;  // G = 16: the last chunk may be half used
    L.ring = (int64_t)c->residual + c->group;
    const uint64_t C = L.chunks, NG = d / G;
    const uint64_t S = c->sinks;
    const uint64_t sizes[kRegions] = {
        U * C * 128 * b * 4,          // kq
        U * C * 128 * b * 4,          // vq
        b == 8 ? 0 : U * key_groups_of(G, C) * d * 4,  // kmeta
        b == 8 ? 0 : U * C * NG * kChunk * 4,          // vmeta
        U * C * 4,                    // mask
        U * L.ring * d * 2,           // kring
        U * L.ring * d * 2,           // vring
        U * N * 4,                    // pool_idx
        U * N * 8,                    // pool_score
        U * N * d * 2,                // pool_k
        U * N * d * 2,                // pool_v
        U * E * 4,                    // ev_idx
        U * E * d * 2,                // ev_k
        U * E * d * 2,                // ev_v
        U * 4 * 4,                    // counters
        N > 0 ? U * L.q_cap * 8 : 0,  // scores
        U * S * d * 2,                // sink_k
        U * S * d * 2,                // sink_v
        U * evict_words_of(c) * 4,    // evict
        (U + 1) / 2 * 8 + U * 16,     // evict_count, then the eviction step's scratch
        (uint64_t)c->n_kv_heads * 8,  // fp8_scales
    };
    uint64_t o = 0;
    for (int i = 0; i < kRegions; ++i) {
        L.off[i] = o;
        o = align_up(o + sizes[i]);
    }
    L.total = o;
    return L;
}

// Quantized tokens after T appends: the residual rule over the tokens after
// the S attention sinks.
int64_t n_quant_of(const kvq_config& c, int64_t T) {
    return n_quantized(T > c.sinks ? T - c.sinks : 0, c.residual, c.group);
}

bool valid_handle(const kvq_cache* h) {
    return h && check_config(&h->cfg) == KVQ_OK && h->arena != 0 && h->tokens >= 0 &&
           h->n_quant == n_quant_of(h->cfg, h->tokens) && h->tokens <= h->cfg.max_tokens;
}

kvq_status launch_status(int e) { return e == 0 ? KVQ_OK : KVQ_ELAUNCH; }

// After a failed launch some of a call's kernels may have run and changed the
// arena, so the handle no longer describes it: it is marked invalid (every
// later call on it returns KVQ_EINVAL) rather than left as it was.
void invalidate(kvq_cache* h) { h->tokens = -1; }

}  // namespace

CacheView view_of(const kvq_cache* h) {
    CacheView v{};
    char* a = reinterpret_cast<char*>(h->arena);
    v.kq = reinterpret_cast<uint32_t*>(a + h->off_kq);
    v.vq = reinterpret_cast<uint32_t*>(a + h->off_vq);
    v.kmeta = reinterpret_cast<uint32_t*>(a + h->off_kmeta);
    v.vmeta = reinterpret_cast<uint32_t*>(a + h->off_vmeta);
    v.mask = reinterpret_cast<uint32_t*>(a + h->off_mask);
    v.kring = reinterpret_cast<uint16_t*>(a + h->off_kring);
    v.vring = reinterpret_cast<uint16_t*>(a + h->off_vring);
    v.pool_idx = reinterpret_cast<int32_t*>(a + h->off_pool_idx);
    v.pool_score = reinterpret_cast<uint64_t*>(a + h->off_pool_score);
    v.pool_k = reinterpret_cast<uint16_t*>(a + h->off_pool_k);
    v.pool_v = reinterpret_cast<uint16_t*>(a + h->off_pool_v);
    v.ev_idx = reinterpret_cast<int32_t*>(a + h->off_ev_idx);
    v.ev_k = reinterpret_cast<uint16_t*>(a + h->off_ev_k);
    v.ev_v = reinterpret_cast<uint16_t*>(a + h->off_ev_v);
    v.counters = reinterpret_cast<int32_t*>(a + h->off_counters);
    v.scores = reinterpret_cast<uint64_t*>(a + h->off_scores);
    v.sink_k = reinterpret_cast<uint16_t*>(a + h->off_sink_k);
    v.sink_v = reinterpret_cast<uint16_t*>(a + h->off_sink_v);
    v.sinks = h->cfg.sinks;
    v.evict = reinterpret_cast<uint32_t*>(a + h->off_evict);
    v.evict_count = reinterpret_cast<int32_t*>(a + h->off_evict_count);
    v.evict_words = (int64_t)evict_words_of(&h->cfg);
    v.fp8_scales = reinterpret_cast<float*>(a + h->off_fp8_scales);
    v.bits = h->cfg.bits;
    v.group = h->cfg.group;
    v.residual = h->cfg.residual;
    v.pool = h->cfg.pool;
    v.evict_cap = h->cfg.evict_cap;
    v.n_q_heads = h->cfg.n_q_heads;
    v.n_kv_heads = h->cfg.n_kv_heads;
    v.batch = h->cfg.batch;
    v.units = h->cfg.batch * h->cfg.n_kv_heads;
    v.ring_slots = (int32_t)h->ring_slots;
    v.q_cap = h->q_cap;
    v.chunks = (h->q_cap + kChunk - 1) / kChunk;
    v.key_groups = (int64_t)key_groups_of(h->cfg.group, v.chunks);
    return v;
}

DecodePlan plan_decode(const kvq_cache* h, bool want_scores) {
    // One resident round of blocks on the current GPU. The fp16 partition
    // (ring + pools) takes about one tile block per compute unit, 16 to 64 rows
    // each; the quantized tokens of each unit are split over the remaining
    // resident blocks, every wavefront of a split taking whole work items
    // (four wavefronts per block, so at most ceil(items / 4) useful splits).
    DecodePlan p{};
    const int64_t U = (int64_t)h->cfg.batch * h->cfg.n_kv_heads;
    const int64_t r = h->cfg.n_q_heads / h->cfg.n_kv_heads;
    int cus = 0, resident = 0;
    decode_launch_shape(h->cfg.bits, (int)r, h->cfg.group, &cus, &resident);
    if (cus < 1) cus = 1;
    if (resident < 1) resident = 1;
    // sinks + ring + full pools (tokens - n_quant counts the sinks and the ring)
    const int64_t fp16_rows = (h->tokens - h->n_quant) +
                              (h->cfg.pool > 0 ? h->cfg.pool + h->cfg.evict_cap : 0);
    const int64_t t_min = fp16_rows > 0 ? (fp16_rows + 63) / 64 : 1;
    int64_t t_max = fp16_rows > 0 ? (fp16_rows + 15) / 16 : 1;
    if (t_max > kMaxFp16Tiles) t_max = kMaxFp16Tiles;
    if (t_max < t_min) t_max = t_min;
    int64_t t = (cus + U - 1) / U;
    if (t > t_max) t = t_max;
    if (t < t_min) t = t_min;
    p.fp16_tiles = (int32_t)t;
    // work items: key groups at G = 32, else chunks (two groups each at
    // G = 16, part of a group at G = 64 and 128)
    const int64_t groups = h->cfg.group == 32 ? h->n_quant / h->cfg.group
                                              : (h->n_quant + kChunk - 1) / kChunk;
    int64_t s = groups > 0 ? (groups + 3) / 4 : 0;
    if (s > kMaxQuantSplits) s = kMaxQuantSplits;
    if (s > 0) {
        int64_t q = (resident - U * t) / U;
        if (q < 1) q = 1;
        if (q < s) s = q;
    }
    p.splits_q = (int32_t)s;
    p.splits = p.splits_q + p.fp16_tiles;
    p.part_floats = U * p.splits * r * kPartRec;
    p.logit_floats = want_scores ? U * r * h->tokens : 0;
    p.ws_bytes = align_up((uint64_t)p.part_floats * 4) + (uint64_t)p.logit_floats * 4;
    return p;
}

}  // namespace kvq

using namespace kvq;

extern "C" {

const char* kvq_status_string(kvq_status s) {
    switch (s) {
        case KVQ_OK: return "ok";
        case KVQ_EINVAL: return "invalid argument";
        case KVQ_EUNSUPPORTED: return "unsupported configuration";
        case KVQ_ECAPACITY: return "cache capacity exceeded";
        case KVQ_EWORKSPACE: return "arena or workspace too small";
        case KVQ_ELAUNCH: return "HIP launch failed";
        case KVQ_ESCRATCH:
            return "decode needs more scratch than the library's static buffer "
                   "(KVQ_NOALLOC_SCRATCH_BYTES) holds; use kvq_decode_attention with a workspace";
        default: return "unknown status";
    }
}

kvq_status kvq_cache_bytes(const kvq_config* cfg, size_t* arena_bytes) {
    kvq_status st = check_config(cfg);
    if (st != KVQ_OK) return st;
    if (!arena_bytes) return KVQ_EINVAL;
    *arena_bytes = (size_t)layout_of(cfg).total;
    return KVQ_OK;
}

kvq_status kvq_cache_init(const kvq_config* cfg, void* d_arena, size_t bytes, kvq_cache* h,
                          void* stream) {
    kvq_status st = check_config(cfg);
    if (st != KVQ_OK) return st;
    if (!d_arena || !h) return KVQ_EINVAL;
    if (reinterpret_cast<uintptr_t>(d_arena) % kAlign != 0) return KVQ_EINVAL;
    const Layout L = layout_of(cfg);
    if (bytes < L.total) return KVQ_EWORKSPACE;
    kvq_cache c{};
    c.cfg = *cfg;
    c.tokens = 0;
    c.n_quant = 0;
    c.arena = reinterpret_cast<uint64_t>(d_arena);
    c.arena_bytes = bytes;
    c.q_cap = L.q_cap;
    c.ring_slots = L.ring;
    uint64_t* offs[kRegions] = {&c.off_kq, &c.off_vq, &c.off_kmeta, &c.off_vmeta, &c.off_mask,
                                &c.off_kring, &c.off_vring, &c.off_pool_idx, &c.off_pool_score,
                                &c.off_pool_k, &c.off_pool_v, &c.off_ev_idx, &c.off_ev_k,
                                &c.off_ev_v, &c.off_counters, &c.off_scores, &c.off_sink_k,
                                &c.off_sink_v, &c.off_evict, &c.off_evict_count,
                                &c.off_fp8_scales};
    for (int i = 0; i < kRegions; ++i) *offs[i] = L.off[i];
    st = launch_status(launch_init(view_of(&c), stream));
    if (st == KVQ_OK) *h = c;
    return st;
}

kvq_status kvq_quantize_append(kvq_cache* h, const void* d_k, const void* d_v, int32_t n_new,
                               void* stream) {
    if (!valid_handle(h) || n_new < 0) return KVQ_EINVAL;
    if (n_new == 0) return KVQ_OK;
    if (!d_k || !d_v) return KVQ_EINVAL;
    const int64_t t_new = h->tokens + n_new;
    if (t_new > h->cfg.max_tokens) return KVQ_ECAPACITY;
    const int64_t nq_new = n_quant_of(h->cfg, t_new);
    kvq_status st = launch_status(launch_append(
        view_of(h), static_cast<const uint16_t*>(d_k), static_cast<const uint16_t*>(d_v),
        h->tokens, n_new, h->n_quant, nq_new, stream));
    if (st == KVQ_OK) {
        h->tokens = t_new;
        h->n_quant = nq_new;
    } else {
        invalidate(h);
    }
    return st;
}

kvq_status kvq_decode_workspace(const kvq_cache* h, int32_t want_scores, size_t* ws_bytes) {
    if (!valid_handle(h) || !ws_bytes) return KVQ_EINVAL;
    *ws_bytes = plan_decode(h, want_scores != 0).ws_bytes;
    return KVQ_OK;
}

kvq_status kvq_decode_attention_timed(const kvq_cache* h, const void* d_q, float* d_out,
                                      float* d_acc, void* d_ws, size_t ws_bytes, void* ev_start,
                                      void* ev_stop, void* stream) {
    if (!valid_handle(h) || !d_q || !d_out || !d_ws) return KVQ_EINVAL;
    if (h->tokens < 1) return KVQ_EINVAL;
    const DecodePlan p = plan_decode(h, d_acc != nullptr);
    if (ws_bytes < p.ws_bytes) return KVQ_EWORKSPACE;
    return launch_status(launch_decode(view_of(h), h->tokens, h->n_quant, p,
                                       static_cast<const uint16_t*>(d_q), d_out, d_acc, d_ws,
                                       ev_start, ev_stop, stream));
}

kvq_status kvq_decode_attention(const kvq_cache* h, const void* d_q, float* d_out, float* d_acc,
                                void* d_ws, size_t ws_bytes, void* stream) {
    return kvq_decode_attention_timed(h, d_q, d_out, d_acc, d_ws, ws_bytes, nullptr, nullptr,
                                      stream);
}

kvq_status kvq_decode_attention_noalloc(const kvq_cache* h, const void* d_q, float* d_out,
                                        float* d_acc, void* stream) {
    if (!valid_handle(h) || !d_q || !d_out) return KVQ_EINVAL;
    if (h->tokens < 1) return KVQ_EINVAL;
    const DecodePlan p = plan_decode(h, d_acc != nullptr);
    if (p.ws_bytes > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ESCRATCH;
    int err = 0;
    void* ws = noalloc_scratch(&err);
    if (!ws) return KVQ_ELAUNCH;
    return launch_status(launch_decode(view_of(h), h->tokens, h->n_quant, p,
                                       static_cast<const uint16_t*>(d_q), d_out, d_acc, ws,
                                       nullptr, nullptr, stream));
}

kvq_status kvq_decode_step_timed(kvq_cache* h, const void* d_k, const void* d_v,
                                 const void* d_q, float* d_out, float* d_acc, void* d_ws,
                                 size_t ws_bytes, void* ev_start, void* ev_stop, void* stream) {
    if (!valid_handle(h) || !d_k || !d_v || !d_q || !d_out || !d_ws) return KVQ_EINVAL;
    const int64_t t_old = h->tokens, t_new = t_old + 1;
    if (t_new > h->cfg.max_tokens) return KVQ_ECAPACITY;
    kvq_cache next = *h;
    next.tokens = t_new;
    next.n_quant = n_quant_of(h->cfg, t_new);
    const DecodePlan p = plan_decode(&next, d_acc != nullptr);
    if (ws_bytes < p.ws_bytes) return KVQ_EWORKSPACE;
    const uint16_t* kn = static_cast<const uint16_t*>(d_k);
    const uint16_t* vn = static_cast<const uint16_t*>(d_v);
    const CacheView v = view_of(h);
    // The new token stays in the fp16 ring unless it is an attention sink or its
    // own group was just quantized; in the ring case the attention kernel stores
    // it, otherwise the append does.
    const int64_t S = h->cfg.sinks;
    const bool in_ring = t_old >= S && t_old - S >= next.n_quant;
    kvq_status st = launch_status(
        launch_append(v, kn, vn, t_old, 1, h->n_quant, next.n_quant, stream, !in_ring));
    if (st != KVQ_OK) {
        invalidate(h);
        return st;
    }
    st = launch_status(launch_decode(v, t_new, next.n_quant, p, static_cast<const uint16_t*>(d_q),
                                     d_out, d_acc, d_ws, ev_start, ev_stop, stream,
                                     in_ring ? kn : nullptr, in_ring ? vn : nullptr));
    if (st == KVQ_OK) *h = next;
    else invalidate(h);
    return st;
}

kvq_status kvq_decode_step(kvq_cache* h, const void* d_k, const void* d_v, const void* d_q,
                           float* d_out, float* d_acc, void* d_ws, size_t ws_bytes,
                           void* stream) {
    return kvq_decode_step_timed(h, d_k, d_v, d_q, d_out, d_acc, d_ws, ws_bytes, nullptr,
                                 nullptr, stream);
}

kvq_status kvq_topk_workspace(int32_t rows, int32_t T, int32_t k, int32_t w, size_t* ws_bytes) {
    if (!ws_bytes || rows < 0 || T < 0 || k < 0 || w < 0 || (int64_t)k + w > T) return KVQ_EINVAL;
    *ws_bytes = rows == 0 || k + w == 0 ? 0 : topk_plan(rows, T, k, w).ws_bytes;
    return KVQ_OK;
}

kvq_status kvq_topk_evict(const float* d_scores, int32_t rows, int32_t T, int32_t k, int32_t w,
                          int32_t* d_idx, void* d_ws, size_t ws_bytes, void* stream) {
    if (rows < 0 || T < 0 || k < 0 || w < 0 || (int64_t)k + w > T) return KVQ_EINVAL;
    if (rows == 0 || k + w == 0) return KVQ_OK;
    if (!d_scores || !d_idx) return KVQ_EINVAL;
    TopkPlan plan{1, T - w, 0};
    if (d_ws) {
        plan = topk_plan(rows, T, k, w);
        if (ws_bytes < plan.ws_bytes) return KVQ_EWORKSPACE;
    }
    return launch_status(launch_topk(d_scores, rows, T, k, w, d_idx, d_ws, plan, stream));
}

kvq_status kvq_unpack_codes(const kvq_cache* h, uint8_t* d_kcodes, uint8_t* d_vcodes,
                            void* stream) {
    if (!valid_handle(h)) return KVQ_EINVAL;
    if (h->n_quant == 0) return KVQ_OK;
    if (!d_kcodes || !d_vcodes) return KVQ_EINVAL;
    return launch_status(launch_unpack(view_of(h), h->n_quant, d_kcodes, d_vcodes, stream));
}

kvq_status kvq_prefill_workspace(int32_t batch, int32_t n_q_heads, int32_t n, size_t* ws_bytes) {
    if (!ws_bytes || batch < 1 || n_q_heads < 1 || n < 0 || n > kMaxTokens) return KVQ_EINVAL;
    // per query row its log-sum-exp, then per (query head, key) a partial
    // column sum (r partials per KV head, added in order)
    *ws_bytes = (size_t)align_up((uint64_t)batch * n_q_heads * n * 4) +
                (size_t)align_up((uint64_t)batch * n_q_heads * n * 4);
    return KVQ_OK;
}

kvq_status kvq_prefill_attention(const void* d_q, const void* d_k, const void* d_v, int32_t batch,
                                 int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                 int32_t n, float* d_out, float* d_acc, void* d_ws,
                                 size_t ws_bytes, void* stream) {
    if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || n < 0 || n > kMaxTokens ||
        n_q_heads % n_kv_heads != 0)
        return KVQ_EINVAL;
    const int r = n_q_heads / n_kv_heads;
    if (head_dim != kHeadDim || (r != 1 && r != 2 && r != 4)) return KVQ_EUNSUPPORTED;
    // query heads and units index the second grid dimension of the kernels
    if ((int64_t)batch * n_q_heads > kMaxGridY) return KVQ_EUNSUPPORTED;
    if (n == 0) return KVQ_OK;
    if (!d_q || !d_k || !d_v || !d_out || !d_ws) return KVQ_EINVAL;
    size_t need = 0;
    kvq_prefill_workspace(batch, n_q_heads, n, &need);
    if (ws_bytes < need) return KVQ_EWORKSPACE;
    return launch_status(launch_prefill(
        static_cast<const uint16_t*>(d_q), static_cast<const uint16_t*>(d_k),
        static_cast<const uint16_t*>(d_v), batch, n_q_heads, n_kv_heads, n, d_out, d_acc,
        static_cast<float*>(d_ws), stream));
}

kvq_status kvq_gather_kv(const void* d_k, const void* d_v, int32_t batch, int32_t n_kv_heads,
                         int32_t head_dim, int32_t n, const int32_t* d_idx, int32_t n_keep,
                         void* d_k_out, void* d_v_out, void* stream) {
    if (batch < 1 || n_kv_heads < 1 || n < 0 || n_keep < 0 || n_keep > n) return KVQ_EINVAL;
    if (head_dim != kHeadDim) return KVQ_EUNSUPPORTED;
    if ((int64_t)batch * n_kv_heads > kMaxGridY) return KVQ_EUNSUPPORTED;  // units: second grid dimension
    if (n_keep == 0) return KVQ_OK;
    if (!d_k || !d_v || !d_idx || !d_k_out || !d_v_out) return KVQ_EINVAL;
    return launch_status(launch_gather(static_cast<const uint16_t*>(d_k),
                                       static_cast<const uint16_t*>(d_v), batch * n_kv_heads, n,
                                       d_idx, n_keep, static_cast<uint16_t*>(d_k_out),
                                       static_cast<uint16_t*>(d_v_out), stream));
}

kvq_status kvq_stream_read(const void* d_buf, size_t bytes, uint32_t* d_sink, void* stream) {
    if (!d_buf || !d_sink || bytes % 16 != 0) return KVQ_EINVAL;
    if (bytes == 0) return KVQ_OK;
    return launch_status(launch_stream_read(d_buf, bytes, d_sink, stream));
}

kvq_status kvq_fp8_set_scales(kvq_cache* h, const float* d_scales, void* stream) {
    if (!valid_handle(h) || !d_scales) return KVQ_EINVAL;
    if (h->cfg.bits != 8) return KVQ_EUNSUPPORTED;
    return launch_status(launch_fp8_scales(view_of(h), d_scales, stream));
}

kvq_status kvq_evict_step(kvq_cache* h, const float* d_acc, int32_t budget, int32_t recent,
                          void* stream) {
    if (!valid_handle(h) || !d_acc || budget < 0 || recent < 0) return KVQ_EINVAL;
    if (h->tokens == 0) return KVQ_OK;
    return launch_status(launch_evict_step(view_of(h), h->tokens, d_acc, budget, recent, stream));
}

kvq_status kvq_pyramid_budgets(int32_t n_layers, int32_t avg_budget, int32_t depth,
                               int32_t* out) {
    if (!out || n_layers < 1 || n_layers > 4096 || avg_budget < 0 || avg_budget > kMaxTokens ||
        depth < 1 || depth > 4096)
        return KVQ_EINVAL;
    // b_l = (2x - x/d) - l (2x - 2x/d) / (L - 1)
    //     = [(2xd - x)(L - 1) - l (2xd - 2x)] / (d (L - 1)), floored; all
    //     terms are non-negative, so integer division floors
    const int64_t x = avg_budget, d = depth, L = n_layers;
    if (L == 1) {
        out[0] = (int32_t)x;
        return KVQ_OK;
    }
    for (int64_t l = 0; l < L; ++l) {
        const int64_t num = (2 * x * d - x) * (L - 1) - l * (2 * x * d - 2 * x);
        out[l] = (int32_t)(num / (d * (L - 1)));
    }
    return KVQ_OK;
}

kvq_status kvq_debug_unpack(const kvq_cache* h, const kvq_debug_view* view, void* stream) {
    if (!valid_handle(h) || !view) return KVQ_EINVAL;
    return launch_status(launch_debug_unpack(view_of(h), h->tokens, h->n_quant, *view, stream));
}

}  // extern "C"

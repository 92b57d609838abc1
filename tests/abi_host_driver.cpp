// Host-only driver for the C-ABI layer (kvq_abi.cpp), built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_abi_sanitize.py.
// The kernel launchers are replaced by stubs that record their arguments and
// return a chosen status, so every validation, layout and planning path runs
// on the host with no GPU. Exit status 0 = every check held.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../kv_cache_compression_kvq_amd/csrc/kvq_internal.h"

static int g_fail_launch = 0;  // status the next stubbed launch returns
static int g_launches = 0;
static int g_checks = 0, g_bad = 0;

#define CHECK(c)                                                         \
    do {                                                                 \
        ++g_checks;                                                      \
        if (!(c)) {                                                      \
            ++g_bad;                                                     \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, \
                         __LINE__, #c);                                  \
        }                                                                \
    } while (0)

namespace kvq {
static int stub() {
    ++g_launches;
    const int e = g_fail_launch;
    g_fail_launch = 0;
    return e;
}
int launch_init(const CacheView&, void*) { return stub(); }
int launch_append(const CacheView& v, const uint16_t*, const uint16_t*, int64_t t_old,
                  int32_t n_new, int64_t nq_old, int64_t nq_new, void*, bool) {
    CHECK(n_new > 0 && nq_new >= nq_old && nq_new <= v.q_cap && t_old >= 0);
    return stub();
}
int launch_decode(const CacheView& v, int64_t T, int64_t n_q, const DecodePlan& p,
                  const uint16_t*, float*, float*, void*, void*, void*, void*,
                  const uint16_t*, const uint16_t*) {
    CHECK(T >= 1 && n_q <= T && n_q <= v.q_cap && p.splits == p.splits_q + p.fp16_tiles);
    return stub();
}
TopkPlan topk_plan(int32_t rows, int32_t T, int32_t k, int32_t w) {
    CHECK(rows > 0 && k + w <= T);
    // the host driver's stand-in: two slices once rows are long
    if (T - w >= 8192 && k > 0 && k < T - w) return TopkPlan{2, (T - w + 7) / 8 * 4, 64};
    return TopkPlan{1, T - w, 0};
}
int launch_topk(const float*, int32_t rows, int32_t T, int32_t k, int32_t w, int32_t*, void* ws,
                const TopkPlan& plan, void*) {
    CHECK(rows > 0 && k + w <= T);
    CHECK(plan.slices == 1 || ws != nullptr);
    return stub();
}
int launch_unpack(const CacheView&, int64_t n_q, uint8_t*, uint8_t*, void*) {
    CHECK(n_q > 0);
    return stub();
}
int launch_prefill(const uint16_t*, const uint16_t*, const uint16_t*, int32_t batch, int32_t hq,
                   int32_t hkv, int32_t n, float*, float*, float*, void*) {
    CHECK(batch >= 1 && hq % hkv == 0 && n >= 1);
    return stub();
}
int launch_gather(const uint16_t*, const uint16_t*, int32_t units, int32_t n, const int32_t*,
                  int32_t n_keep, uint16_t*, uint16_t*, void*) {
    CHECK(units >= 1 && n_keep >= 1 && n_keep <= n);
    return stub();
}
int launch_stream_read(const void*, size_t bytes, uint32_t*, void*) {
    CHECK(bytes % 16 == 0 && bytes > 0);
    return stub();
}
int launch_fp8_scales(const CacheView& v, const float*, void*) {
    CHECK(v.bits == 8);
    return stub();
}
int launch_evict_step(const CacheView& v, int64_t T, const float*, int32_t budget, int32_t recent,
                      void*) {
    CHECK(T >= 1 && budget >= 0 && recent >= 0 && v.evict_words * 32 >= v.q_cap);
    return stub();
}
int launch_debug_unpack(const CacheView&, int64_t T, int64_t n_q, const kvq_debug_view&, void*) {
    CHECK(n_q <= T);
    return stub();
}
void decode_launch_shape(int, int, int, int* cus, int* resident) {
    *cus = 256;
    *resident = 1024;
}
void* noalloc_scratch(int* err) {
    *err = 0;
    return reinterpret_cast<void*>(uintptr_t(1) << 41);
}
}  // namespace kvq

static kvq_config cfg(int bits, int group, int R, int pool, int E, int hq, int hkv, int B,
                      int maxt) {
    kvq_config c{};
    c.bits = bits;
    c.group = group;
    c.residual = R;
    c.pool = pool;
    c.evict_cap = E;
    c.head_dim = 128;
    c.n_q_heads = hq;
    c.n_kv_heads = hkv;
    c.batch = B;
    c.max_tokens = maxt;
    return c;
}

int main() {
    // status strings are static and never null
    for (int s = -7; s <= 1; ++s) CHECK(kvq_status_string(s) != nullptr);

    // configuration checks
    size_t n = 0;
    kvq_config c = cfg(2, 32, 128, 0, 32, 32, 8, 8, 8192);
    CHECK(kvq_cache_bytes(&c, &n) == KVQ_OK && n > 0);
    CHECK(kvq_cache_bytes(nullptr, &n) == KVQ_EINVAL);
    CHECK(kvq_cache_bytes(&c, nullptr) == KVQ_EINVAL);
    const int bad_bits[] = {0, 1, 3, 16, -2};
    for (int b : bad_bits) {
        kvq_config x = c;
        x.bits = b;
        CHECK(kvq_cache_bytes(&x, &n) == KVQ_EUNSUPPORTED);
    }
    kvq_config x = c;
    x.head_dim = 64;
    CHECK(kvq_cache_bytes(&x, &n) == KVQ_EUNSUPPORTED);
    x = c;
    x.n_q_heads = 24;
    x.n_kv_heads = 7;
    CHECK(kvq_cache_bytes(&x, &n) == KVQ_EINVAL);
    x = c;
    x.max_tokens = (1 << 24) + 1;
    CHECK(kvq_cache_bytes(&x, &n) == KVQ_EUNSUPPORTED);
    x = c;
    x.residual = -1;
    CHECK(kvq_cache_bytes(&x, &n) == KVQ_EINVAL);

    // every supported configuration: layout offsets ascending, aligned, inside
    const int groups[] = {16, 32, 64, 128};
    for (int bits : {2, 4, 8})
        for (int g : groups)
            for (int r : {1, 2, 4})
                for (int pool : {0, 3})
                for (int sinks : {0, 5}) {
                    kvq_config k = cfg(bits, g, 40, pool, 8, 2 * r, 2, 3, 1000);
                    k.sinks = sinks;
                    size_t bytes = 0;
                    const kvq_status st = kvq_cache_bytes(&k, &bytes);
                    CHECK(st == KVQ_OK || st == KVQ_EUNSUPPORTED);
                    if (st != KVQ_OK) continue;
                    // a fake, aligned device address: the stubs never touch it
                    void* arena = reinterpret_cast<void*>(uintptr_t(1) << 40);
                    kvq_cache h{};
                    CHECK(kvq_cache_init(&k, arena, bytes - 1, &h, nullptr) == KVQ_EWORKSPACE);
                    CHECK(kvq_cache_init(&k, reinterpret_cast<char*>(arena) + 8, bytes, &h,
                                         nullptr) == KVQ_EINVAL);
                    CHECK(kvq_cache_init(&k, arena, bytes, &h, nullptr) == KVQ_OK);
                    const uint64_t offs[] = {h.off_kq, h.off_vq, h.off_kmeta, h.off_vmeta,
                                             h.off_mask, h.off_kring, h.off_vring,
                                             h.off_pool_idx, h.off_pool_score, h.off_pool_k,
                                             h.off_pool_v, h.off_ev_idx, h.off_ev_k, h.off_ev_v,
                                             h.off_counters, h.off_scores, h.off_sink_k,
                                             h.off_sink_v, h.off_evict, h.off_evict_count,
                                             h.off_fp8_scales};
                    for (size_t i = 0; i < sizeof(offs) / sizeof(offs[0]); ++i) {
                        CHECK(offs[i] % 256 == 0 && offs[i] <= bytes);
                        if (i) CHECK(offs[i] >= offs[i - 1]);
                    }
                    // appends: token counts, capacity, ragged sizes
                    const int16_t dummy = 0;
                    const void* kp = &dummy;
                    int64_t T = 0;
                    const int steps[] = {1, 37, 0, 300, 5, 64};
                    for (int s : steps) {
                        CHECK(kvq_quantize_append(&h, kp, kp, s, nullptr) == KVQ_OK);
                        T += s;
                        CHECK(h.tokens == T);
                        const int64_t nq = T - sinks > 40 ? (T - sinks - 40) / g * g : 0;
                        CHECK(h.n_quant == nq);
                    }
                    CHECK(kvq_quantize_append(&h, kp, kp, -1, nullptr) == KVQ_EINVAL);
                    CHECK(kvq_quantize_append(&h, nullptr, kp, 3, nullptr) == KVQ_EINVAL);
                    CHECK(kvq_quantize_append(&h, kp, kp, 1000, nullptr) == KVQ_ECAPACITY);
                    CHECK(h.tokens == T);
                    // decode: workspace sizing and checks
                    size_t ws = 0, ws2 = 0;
                    CHECK(kvq_decode_workspace(&h, 0, &ws) == KVQ_OK);
                    CHECK(kvq_decode_workspace(&h, 1, &ws2) == KVQ_OK && ws2 >= ws);
                    std::vector<char> hostbuf(16);
                    void* wsp = hostbuf.data();
                    float out = 0.f;
                    CHECK(kvq_decode_attention(&h, kp, &out, nullptr, wsp, ws - 1, nullptr) ==
                          KVQ_EWORKSPACE);
                    CHECK(kvq_decode_attention(&h, kp, &out, nullptr, wsp, ws, nullptr) == KVQ_OK);
                    CHECK(kvq_decode_attention(&h, nullptr, &out, nullptr, wsp, ws, nullptr) ==
                          KVQ_EINVAL);
                    // one decode step, then a failed launch invalidates the handle
                    size_t ws3 = 0;
                    kvq_cache next = h;
                    next.tokens += 1;
                    next.n_quant = next.tokens - sinks > 40 ? (next.tokens - sinks - 40) / g * g : 0;
                    CHECK(kvq_decode_workspace(&next, 1, &ws3) == KVQ_OK);
                    float acc = 0.f;
                    CHECK(kvq_decode_step(&h, kp, kp, kp, &out, &acc, wsp, ws3, nullptr) ==
                          KVQ_OK);
                    CHECK(h.tokens == T + 1);
                    g_fail_launch = 1;
                    CHECK(kvq_decode_step(&h, kp, kp, kp, &out, &acc, wsp, ws3 + (1 << 20),
                                          nullptr) == KVQ_ELAUNCH);
                    CHECK(h.tokens == -1);
                    CHECK(kvq_quantize_append(&h, kp, kp, 1, nullptr) == KVQ_EINVAL);
                    CHECK(kvq_decode_workspace(&h, 0, &ws) == KVQ_EINVAL);
                    CHECK(kvq_unpack_codes(&h, nullptr, nullptr, nullptr) == KVQ_EINVAL);
                    kvq_debug_view dv{};
                    CHECK(kvq_debug_unpack(&h, &dv, nullptr) == KVQ_EINVAL);
                }

    // the no-allocation decode: fits, or KVQ_ESCRATCH with nothing launched
    {
        kvq_config k = cfg(2, 32, 128, 0, 32, 32, 8, 16, 32768);
        size_t bytes = 0;
        CHECK(kvq_cache_bytes(&k, &bytes) == KVQ_OK);
        kvq_cache h{};
        CHECK(kvq_cache_init(&k, reinterpret_cast<void*>(uintptr_t(1) << 40), bytes, &h,
                             nullptr) == KVQ_OK);
        const int16_t dummy = 0;
        CHECK(kvq_quantize_append(&h, &dummy, &dummy, 32768, nullptr) == KVQ_OK);
        size_t ws = 0, ws_h2o = 0;
        CHECK(kvq_decode_workspace(&h, 0, &ws) == KVQ_OK && ws <= KVQ_NOALLOC_SCRATCH_BYTES);
        CHECK(kvq_decode_workspace(&h, 1, &ws_h2o) == KVQ_OK && ws_h2o > KVQ_NOALLOC_SCRATCH_BYTES);
        float out = 0.f, acc = 0.f;
        const int before = g_launches;
        CHECK(kvq_decode_attention_noalloc(&h, &dummy, &out, &acc, nullptr) == KVQ_ESCRATCH);
        CHECK(g_launches == before);
        CHECK(kvq_decode_attention_noalloc(&h, &dummy, &out, nullptr, nullptr) == KVQ_OK);
        CHECK(g_launches == before + 1);
        CHECK(kvq_decode_attention_noalloc(&h, nullptr, &out, nullptr, nullptr) == KVQ_EINVAL);
    }

    // pyramid budgets: argument checks and the closed-form endpoints
    {
        int32_t b[32];
        CHECK(kvq_pyramid_budgets(32, 100, 7, nullptr) == KVQ_EINVAL);
        CHECK(kvq_pyramid_budgets(0, 100, 7, b) == KVQ_EINVAL);
        CHECK(kvq_pyramid_budgets(32, 100, 0, b) == KVQ_EINVAL);
        CHECK(kvq_pyramid_budgets(32, 100, 7, b) == KVQ_OK);
        CHECK(b[0] == 185 && b[31] == 14);  // floor(200 - 100/7), floor(100/7)
        CHECK(kvq_pyramid_budgets(1, 77, 3, b) == KVQ_OK && b[0] == 77);
    }

    // top-k argument checks
    float s = 0.f;
    int32_t idx = 0;
    CHECK(kvq_topk_evict(&s, 2, 100, 90, 20, &idx, nullptr, 0, nullptr) == KVQ_EINVAL);
    CHECK(kvq_topk_evict(&s, -1, 100, 10, 20, &idx, nullptr, 0, nullptr) == KVQ_EINVAL);
    CHECK(kvq_topk_evict(nullptr, 2, 100, 10, 20, &idx, nullptr, 0, nullptr) == KVQ_EINVAL);
    CHECK(kvq_topk_evict(&s, 0, 100, 10, 20, &idx, nullptr, 0, nullptr) == KVQ_OK);
    CHECK(kvq_topk_evict(&s, 2, 100, 10, 20, &idx, nullptr, 0, nullptr) == KVQ_OK);
    // workspace: none needed for short rows; a split plan needs its bytes
    size_t tw = 1;
    CHECK(kvq_topk_workspace(2, 100, 10, 20, &tw) == KVQ_OK && tw == 0);
    CHECK(kvq_topk_workspace(2, 100, 90, 20, &tw) == KVQ_EINVAL);
    CHECK(kvq_topk_workspace(2, 100, 10, 20, nullptr) == KVQ_EINVAL);
    CHECK(kvq_topk_workspace(2, 20000, 4000, 128, &tw) == KVQ_OK && tw == 64);
    char ws[64];
    CHECK(kvq_topk_evict(&s, 2, 20000, 4000, 128, &idx, ws, 63, nullptr) == KVQ_EWORKSPACE);
    CHECK(kvq_topk_evict(&s, 2, 20000, 4000, 128, &idx, ws, 64, nullptr) == KVQ_OK);
    CHECK(kvq_topk_evict(&s, 2, 20000, 4000, 128, &idx, nullptr, 0, nullptr) == KVQ_OK);

    std::printf("%d checks, %d failed, %d stubbed launches\n", g_checks, g_bad, g_launches);
    return g_bad == 0 ? 0 : 1;
}

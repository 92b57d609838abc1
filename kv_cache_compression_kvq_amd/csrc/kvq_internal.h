// Internal declarations shared by the HIP kernels and the C-ABI layer of libkvq.
// Not part of the public interface (include/kvq.h is).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kHeadDim = 128;      // d
constexpr int kChunk = 32;         // tokens per packed chunk
constexpr int kMaxPool = 64;       // N limit
constexpr int kMaxSinks = 64;      // S limit
constexpr int kMaxEvict = 1024;    // E limit
constexpr int kMaxFp16Rows = 2048; // R + G + N + E limit
constexpr int kMaxFp16Tiles = 56;   // fp16-partition tiles per unit (each at most 64 rows)
constexpr int kMaxTokens = 1 << 24; // per-unit capacity: keeps per-unit offsets in 32 bits
constexpr int kPartRec = kHeadDim + 4; // floats per decode partial record: o[d], m, l, 2 pad

// Device pointers of one cache, resolved from the arena and the handle's offsets.
struct CacheView {
    uint32_t* kq;
    uint32_t* vq;
    uint32_t* kmeta;     // (scale | zero << 16) per key group and channel
    uint32_t* vmeta;     // (scale | zero << 16) per chunk, value group, token
    uint32_t* mask;      // one word per chunk
    uint16_t* kring;
    uint16_t* vring;
    int32_t* pool_idx;
    uint64_t* pool_score;
    uint16_t* pool_k;
    uint16_t* pool_v;
    int32_t* ev_idx;
    uint16_t* ev_k;
    uint16_t* ev_v;
    int32_t* counters;
    uint64_t* scores;
    uint16_t* sink_k;    // [U][S][d]
    uint16_t* sink_v;
    uint32_t* evict;     // [U][evict_words]: eviction bits of tokens S, S + 1, ...
    int32_t* evict_count;  // [U]
    int64_t evict_words;
    float* fp8_scales;   // [Hkv][2] (b = 8)
    int32_t sinks;       // S
    int32_t bits, group, residual, pool, evict_cap;
    int32_t n_q_heads, n_kv_heads, batch;
    int32_t units;       // U = batch * n_kv_heads
    int32_t ring_slots;  // RB = R + G
    int64_t q_cap;       // quantized token capacity per unit
    int64_t chunks;      // q_cap / 32
    int64_t key_groups;  // q_cap / G
};

CacheView view_of(const kvq_cache* h);

// Split plan of one decode call.
struct DecodePlan {
    int32_t splits_q;    // quantized-partition splits per unit (0 when n_q == 0): as
                         // many as one resident round of blocks holds
    int32_t fp16_tiles;  // fp16-partition tiles (ring + pools) per unit, 16-64 rows each
    int32_t splits;      // splits_q + fp16_tiles partial records per unit
    int64_t part_floats; // partial records: U * splits * r * kPartRec
    int64_t logit_floats;// U * r * T when scores are wanted
    size_t ws_bytes;
};

DecodePlan plan_decode(const kvq_cache* h, bool want_scores);

// Launchers (return hipError_t as int; 0 = success).
int launch_init(const CacheView& v, void* stream);
// t_old: tokens held before the call (whole sequence, sinks included); the
// first max(0, S - t_old) appended rows go to the sink region. nq_old / nq_new
// count quantized tokens (those after the sinks). ring_store = false leaves
// the appended tokens that stay in the ring out of it (the decode step stores
// its one token itself).
int launch_append(const CacheView& v, const uint16_t* k_new, const uint16_t* v_new,
                  int64_t t_old, int32_t n_new, int64_t nq_old, int64_t nq_new, void* stream,
                  bool ring_store = true);
// k_new / v_new (or null): the newest token (T - 1, fp16, [U][d]) is read
// from there instead of the ring and stored into its ring slot.
int launch_decode(const CacheView& v, int64_t T, int64_t n_q, const DecodePlan& plan,
                  const uint16_t* q, float* out, float* acc, void* ws, void* ev_start,
                  void* ev_stop, void* stream, const uint16_t* k_new = nullptr,
                  const uint16_t* v_new = nullptr);
// Heavy-hitter top-k: rows split over `slices` workgroups of slice_len keys
// each (slices == 1: one workgroup per row, no workspace).
struct TopkPlan {
    int32_t slices;
    int32_t slice_len;
    size_t ws_bytes;
};
TopkPlan topk_plan(int32_t rows, int32_t T, int32_t k, int32_t w);
int launch_topk(const float* scores, int32_t rows, int32_t T, int32_t k, int32_t w, int32_t* idx,
                void* ws, const TopkPlan& plan, void* stream);
int launch_unpack(const CacheView& v, int64_t n_q, uint8_t* kc, uint8_t* vc, void* stream);
int launch_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, int32_t batch,
                   int32_t n_q_heads, int32_t n_kv_heads, int32_t n, float* out, float* acc,
                   float* lse, void* stream);
int launch_gather(const uint16_t* k, const uint16_t* v, int32_t units, int32_t n,
                  const int32_t* idx, int32_t n_keep, uint16_t* ko, uint16_t* vo, void* stream);
int launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
int launch_fp8_scales(const CacheView& v, const float* scales, void* stream);
int launch_evict_step(const CacheView& v, int64_t T, const float* acc, int32_t budget,
                      int32_t recent, void* stream);
int launch_debug_unpack(const CacheView& v, int64_t T, int64_t n_q, const kvq_debug_view& out,
                        void* stream);
// Launch shape of the decode kernel on the current GPU: compute units and the
// blocks of decode_kernel<bits, r, group> resident at once (cached per GPU).
void decode_launch_shape(int bits, int r, int group, int* cus, int* resident);
// Device address of the static decode scratch (KVQ_NOALLOC_SCRATCH_BYTES) on the
// current GPU, looked up once per GPU; null with *err set when the lookup fails.
void* noalloc_scratch(int* err);

}  // namespace kvq

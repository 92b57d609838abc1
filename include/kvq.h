/*
 * kvq.h - C ABI of libkvq: low-bit KV-cache compression and decode attention
 * over the compressed cache, for one AMD Instinct MI355X (gfx950).
 *
 * What the library computes (page citations name the page title and the
 * section on it):
 *
 *  - Asymmetric min-max quantization to b = 2 or 4 bits, step
 *    q = (max - min) / (2^b - 1), zero-point = group minimum
 *    ("Accurate KV Cache Quantization with Outlier Tokens Tracing", section
 *    "Background"; "KV cache quantization and eviction: FP8, INT4, H2O and
 *    attention sinks", section "Minimal implementation").
 *  - KIVI grouping: keys per channel over groups of G tokens, values per
 *    token over groups of min(G, d) channels; codes packed 16 (b = 2) or 8
 *    (b = 4) per 32-bit word; scale and zero kept in fp16 ("MiniKV: Pushing
 *    the Limits of LLM Inference via 2-Bit Layer-Discriminative KV Cache",
 *    section 4.4).
 *  - A full-precision residual window: after T tokens the first
 *    n_q = max(0, floor((T - R) / G) * G) are quantized and the rest stay fp16
 *    ("KV cache quantization and eviction", section "Minimal implementation").
 *  - OTT outlier tracing: the tokens with the smallest key L1 norm are kept in
 *    fp16 in a pool of N, replaced by the group mean before quantization;
 *    displaced members move to an extra pool of E, and tracing stops when that
 *    is full ("Accurate KV Cache Quantization with Outlier Tokens Tracing",
 *    sections "Method details" and "Experimental setup").
 *  - Decode attention over the quantized, fp16-residual and pool partitions
 *    with softmax scale 1/sqrt(d) (MiniKV, section 2 Eq. 1 and Algorithm 1),
 *    and H2O accumulated attention per KV head, summed over the query heads
 *    that share it ("H2O: Heavy-Hitter Oracle for Efficient Generative
 *    Inference of Large Language Models", accumulated attention scores;
 *    "KV cache quantization and eviction", section "Heavy hitters").
 *  - Attention sinks: the first S tokens of every unit stay fp16 and are never
 *    quantized, traced or evicted; the residual rule and the groups apply to
 *    the tokens after them ("KV cache quantization and eviction", section
 *    "Attention sinks and StreamingLLM"; "KV Cache Transform Coding for
 *    Compact Storage in LLM Inference", section 2, s = 4 sinks).
 *  - H2O eviction while decoding: one token per step and KV head, the live
 *    token with the lowest accumulated score outside the sinks and a recent
 *    window, while more than a budget of tokens is live ("H2O: Heavy-Hitter
 *    Oracle", greedy eviction; "KV cache quantization and eviction",
 *    h2o_evict in "Minimal implementation"); per-layer budgets by MiniKV's
 *    pyramid (section 4.2).
 *  - A second codec, FP8 E4M3 (bits = 8): each element stored as the
 *    saturating round-to-nearest-even E4M3 value of x / s, with one fp32
 *    scale s per KV head for keys and one for values ("KV cache quantization
 *    and eviction", sections "FP8, KIVI and KVQuant" and "Failure modes and
 *    how to detect them").
 *  - Heavy-hitter selection: the k highest scores outside a recent window of
 *    w tokens, plus that window (MiniKV, Algorithm 1; "KV cache quantization
 *    and eviction", section "Minimal implementation").
 *  - Prefill selection: causal attention over the prompt that also writes,
 *    per KV head, the column sums of the normalized attention (A_cumul), whose
 *    heavy hitters plus a recent window are gathered and quantized into the
 *    cache (MiniKV, sections 4.3 and 4.1, Algorithm 1).
 *
 * Conventions for every entry point:
 *
 *  - Memory: the caller allocates all device memory (cache arena, inputs,
 *    outputs, workspace). The library never allocates, frees or synchronizes
 *    the device; all work is enqueued on the given stream (a hipStream_t
 *    passed as void*; NULL = the null stream).
 *  - Pointers marked "device" must be device addresses; "host" are host
 *    addresses. Sizes are element counts unless named *_bytes.
 *  - Errors: every call validates its arguments on the host before launching
 *    anything. A call that returns an error has launched nothing and left the
 *    cache unchanged, except KVQ_ELAUNCH, which reports a failed launch: some
 *    of the call's kernels may then have run, so a call that updates a cache
 *    handle marks it invalid (h->tokens = -1; every later call on it returns
 *    KVQ_EINVAL) and the cache must be rebuilt or restored from a snapshot.
 *    Errors left in the HIP runtime by unrelated earlier calls are cleared
 *    before launching and never reported as this call's.
 *  - Threading: calls on distinct caches are independent. Calls on one cache
 *    must be ordered by the caller (same stream, or explicit events).
 *  - Shapes: batch B, query heads Hq, KV heads Hkv with Hq = r * Hkv (query
 *    head h reads KV head h / r), head_dim d = 128. A "unit" is one
 *    (batch, KV head) pair, u = b * Hkv + h_kv; U = B * Hkv. Every unit of a
 *    cache holds the same number of tokens T.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvq_status;

#define KVQ_OK            0
#define KVQ_EINVAL       (-1) /* null pointer, negative or inconsistent size */
#define KVQ_EUNSUPPORTED (-2) /* a configuration the library does not implement */
#define KVQ_ECAPACITY    (-3) /* appending beyond max_tokens */
#define KVQ_EWORKSPACE   (-4) /* arena or workspace smaller than required */
#define KVQ_ELAUNCH      (-5) /* a HIP launch failed (hipGetLastError) */
#define KVQ_ESCRATCH     (-6) /* the no-allocation decode needs more than its static scratch */

/* Bytes of the library's static device scratch used by
 * kvq_decode_attention_noalloc (one copy per GPU, held until the process ends). */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* Static description of a status code. Never returns NULL. */
const char* kvq_status_string(kvq_status status);

/*
 * Cache configuration (host POD).
 *   bits        b in {2, 4}: integer codes; 8: the FP8 E4M3 codec (then group
 *               must be 32 and pool 0: no groups, zero points or OTT)
 *   group       G in {16, 32, 64, 128}: tokens per key group and, capped at d,
 *               channels per value group (one group size for both axes, MiniKV
 *               section 5.1)
 *   residual    R >= 0, fp16 residual window
 *   pool        N in [0, 64], OTT outlier pool size (0 disables tracing; the
 *               page uses 0 for layers 0-1 and 3 elsewhere)
 *   evict_cap   E in [0, 1024], OTT extra pool size (32 on the page)
 *   head_dim    d, must be 128
 *   n_q_heads   Hq, n_kv_heads Hkv: Hq / Hkv = r in {1, 2, 4}
 *   batch       B >= 1, with B * Hkv <= 65535
 *   max_tokens  capacity in tokens per unit, in [1, 2^24]
 *   sinks       S in [0, 64]: attention sinks kept fp16 (4 in StreamingLLM)
 * With S > 0 the token indices of the quantized partition, the ring and the
 * pools are those of the whole sequence (tokens S, S + 1, ...); the residual
 * rule becomes n_q = max(0, floor((T - S - R) / G) * G).
 */
typedef struct kvq_config {
    int32_t bits;
    int32_t group;
    int32_t residual;
    int32_t pool;
    int32_t evict_cap;
    int32_t head_dim;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t batch;
    int32_t max_tokens;
    int32_t sinks;
} kvq_config;

/*
 * Cache handle (caller-owned host POD). Filled by kvq_cache_init; updated by
 * kvq_quantize_append. It holds the device address of the caller's arena,
 * byte offsets of the regions inside it, and the host counters T and n_q.
 * Snapshot / restore of a cache is a copy of the arena bytes plus this struct.
 *
 * Arena regions (each starts 256-byte aligned; u is the unit index, C the
 * number of 32-token chunks of quantized capacity, Qcap = 32 * C,
 * RB = R + G ring slots, NG = d / min(G, d) value groups per token):
 *   kq        packed key codes,   U x C chunks of 16*b*32 bytes (see below)
 *   vq        packed value codes, U x C chunks of 16*b*32 bytes
 *   kmeta     fp16 (scale, zero) per key channel: [U][Qcap/G][d][2]
 *   vmeta     fp16 (scale, zero) per value group:  [U][C][NG][32][2]
 *             (chunk, then value group, then token within the chunk)
 *   mask      uint32 [U][C], bit i of word c set when token 32c+i was admitted
 *             to the outlier pool (its quantized slot holds the group mean)
 *   kring     fp16 [U][RB][d], token t (n_q <= t < T) at slot t % RB
 *   vring     fp16 [U][RB][d]
 *   pool_idx  int32 [U][N] token index of each pool member
 *   pool_score uint64 [U][N] exact key L1 norm in units of 2^-24
 *   pool_k    fp16 [U][N][d] original key row;  pool_v likewise
 *   ev_idx    int32 [U][E]; ev_k, ev_v fp16 [U][E][d] (extra pool, in the
 *             order members were displaced)
 *   counters  int32 [U][4]: pool count, extra-pool count, frozen flag, and a
 *             bound on the unit's value scales (fp16 bits; 0 while nothing
 *             is quantized): the largest scale held, or computed for a token
 *             before it joined the outlier pool; it bounds the decoder's lazy
 *             softmax rescale
 *   scores    uint64 [U][Qcap] scratch for key L1 norms during an append
 *   sink_k    fp16 [U][S][d] the attention-sink rows; sink_v likewise
 *   evict     uint32 [U][ceil((max_tokens - S) / 32)]: bit i of word c set when
 *             token S + 32c + i was evicted (kvq_evict_step)
 *   evict_count int32 [U]: evicted tokens per unit, followed (8-byte aligned)
 *             by uint64 [U][2] of kvq_evict_step scratch, zero between calls
 *   fp8_scales fp32 [Hkv][2] (b = 8): key and value scale per KV head, 1.0
 *             after kvq_cache_init
 * At b = 8, kq / vq hold one E4M3 byte per element (4 KB per chunk each) in
 * the decoder's operand order and kmeta / vmeta are empty.
 * Slots of pool_idx / ev_idx beyond the counters are unspecified.
 *
 * Packed code layout. Codes of 32 consecutive quantized tokens form a chunk
 * laid out for the matrix-core operands of the decode kernel: 64 lanes own
 * 2b 32-bit words each; word w of lane l is stored at word offset
 * (w / 4) * 256 + l * 4 + (w % 4) of the chunk. Inside a word the two 16-bit
 * halves hold the two codes of one operand pair at the same bit position;
 * which pair sits at which position is chosen so that the decoder needs at
 * most one shift or rotate per word position (see kvq_unpack_codes, which
 * returns the canonical view, one byte per code, [token][channel]).
 */
typedef struct kvq_cache {
    kvq_config cfg;
    int64_t tokens;     /* T, tokens held per unit */
    int64_t n_quant;    /* n_q, tokens held quantized per unit */
    uint64_t arena;     /* device address of the arena */
    uint64_t arena_bytes;
    int64_t q_cap;      /* Qcap */
    int64_t ring_slots; /* RB */
    uint64_t off_kq, off_vq, off_kmeta, off_vmeta, off_mask, off_kring, off_vring;
    uint64_t off_pool_idx, off_pool_score, off_pool_k, off_pool_v;
    uint64_t off_ev_idx, off_ev_k, off_ev_v, off_counters, off_scores;
    uint64_t off_sink_k, off_sink_v;
    uint64_t off_evict, off_evict_count;
    uint64_t off_fp8_scales;
} kvq_cache;

/* Bytes of device memory a cache with this configuration needs (host only).
 * Returns KVQ_EINVAL / KVQ_EUNSUPPORTED for a bad configuration. */
kvq_status kvq_cache_bytes(const kvq_config* cfg, size_t* arena_bytes);

/*
 * Bind an empty cache to the caller's arena (device, >= kvq_cache_bytes,
 * 256-byte aligned) and clear its counters, pool masks and eviction state on
 * `stream`.
 * Fills *h (host). The arena stays owned by the caller and must outlive *h.
 */
kvq_status kvq_cache_init(const kvq_config* cfg, void* d_arena, size_t arena_bytes,
                          kvq_cache* h, void* stream);

/*
 * Append n_new >= 0 tokens to every unit: d_k, d_v are device fp16
 * [B][Hkv][n_new][d] (keys as the model caches them, after RoPE). Every group
 * of G tokens that leaves the residual window is quantized: OTT tracing (if
 * N > 0 and not frozen) picks pool members by key L1 norm and replaces them
 * with the group mean, then keys are quantized per channel and values per
 * token. Updates h->tokens and h->n_quant on the host. The inputs may be
 * reused as soon as the enqueued work has run.
 * Errors: KVQ_EINVAL (null pointer with n_new > 0, n_new < 0, invalid
 * handle), KVQ_ECAPACITY (T + n_new > max_tokens), KVQ_ELAUNCH (the handle is
 * then marked invalid).
 */
kvq_status kvq_quantize_append(kvq_cache* h, const void* d_k, const void* d_v,
                               int32_t n_new, void* stream);

/*
 * Workspace bytes kvq_decode_attention needs for the cache's current T, with
 * (want_scores != 0) or without H2O score accumulation.
 */
kvq_status kvq_decode_workspace(const kvq_cache* h, int32_t want_scores, size_t* ws_bytes);

/*
 * One decode step of attention over the cache.
 *   d_q    device fp16 [B][Hq][d] queries
 *   d_out  device fp32 [B][Hq][d] attention outputs (written)
 *   d_acc  device fp32 [B][Hkv][T] H2O accumulated scores, or NULL. When
 *          given, acc[u][j] += sum over the r query heads of KV head u of the
 *          normalized softmax probability of token j (read-modify-write).
 *   d_ws   device workspace of ws_bytes >= kvq_decode_workspace(h, d_acc != NULL)
 * Every cached token counts once: pool members with their fp16 rows (their
 * quantized slots are skipped), tokens at index >= n_q from the fp16 ring,
 * the rest dequantized on the fly from the packed codes; tokens evicted by
 * kvq_evict_step take no part and keep their scores. Softmax scale is
 * 1/sqrt(d).
 * Errors: KVQ_EINVAL (null pointer, T == 0), KVQ_EWORKSPACE.
 */
kvq_status kvq_decode_attention(const kvq_cache* h, const void* d_q, float* d_out,
                                float* d_acc, void* d_ws, size_t ws_bytes, void* stream);

/*
 * kvq_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace taken from a
 * static device array of KVQ_NOALLOC_SCRATCH_BYTES inside the library instead
 * of a caller buffer. The call allocates and frees nothing. The array's device
 * address is looked up once per GPU, on the first call made with that GPU
 * current.
 *   d_q, d_out, d_acc as for kvq_decode_attention (the caller still owns them)
 * Every call on one GPU shares that GPU's array and overwrites what an earlier
 * call left there; calls that overlap in time on one GPU (different streams
 * without ordering) race and give undefined results. Nothing in the array has
 * to start at zero: each call writes every scratch word before reading it.
 * Errors: KVQ_EINVAL (null pointer, T == 0), KVQ_ESCRATCH (the call needs more
 * than KVQ_NOALLOC_SCRATCH_BYTES: kvq_decode_workspace tells how much),
 * KVQ_ELAUNCH (including a failed lookup of the array's address).
 */
kvq_status kvq_decode_attention_noalloc(const kvq_cache* h, const void* d_q, float* d_out,
                                        float* d_acc, void* stream);

/*
 * kvq_decode_attention, additionally recording ev_start and ev_stop (hipEvent_t
 * handles created by the caller, or NULL) at the start and end of the fused
 * attention kernel's own execution, so that it can be timed without the merge
 * kernel and launch gaps. Same arguments, results and errors otherwise.
 */
kvq_status kvq_decode_attention_timed(const kvq_cache* h, const void* d_q, float* d_out,
                                      float* d_acc, void* d_ws, size_t ws_bytes,
                                      void* ev_start, void* ev_stop, void* stream);

/*
 * One decode step: append one token to every unit, then attend with the
 * updated cache. Results and cache state are those of
 *   kvq_quantize_append(h, d_k, d_v, 1, stream);
 *   kvq_decode_attention(h, d_q, d_out, d_acc, d_ws, ws_bytes, stream);
 * (MiniKV, Algorithm 1, one generation step; KIVI-style residual window:
 * "Accurate KV Cache Quantization with Outlier Tokens Tracing", section
 * "Method details", decoding stage). When the new token stays in the fp16
 * window, the attention kernel reads it from d_k / d_v and stores it into the
 * ring itself, so the step costs one kernel less than the two calls.
 *   d_k, d_v  device fp16 [B][Hkv][1][d], the step's key and value
 *   d_ws      ws_bytes >= kvq_decode_workspace of the cache after the append
 *             (T + 1 tokens)
 * Every argument is checked before anything is enqueued; an error leaves
 * *h and the cache unchanged. Updates h->tokens and h->n_quant on success.
 * Errors: KVQ_EINVAL (null pointer), KVQ_ECAPACITY (T + 1 > max_tokens),
 * KVQ_EWORKSPACE, KVQ_ELAUNCH (the handle is then marked invalid).
 */
kvq_status kvq_decode_step(kvq_cache* h, const void* d_k, const void* d_v, const void* d_q,
                           float* d_out, float* d_acc, void* d_ws, size_t ws_bytes,
                           void* stream);

/*
 * kvq_decode_step, additionally recording ev_start and ev_stop (hipEvent_t or
 * NULL) around the attention kernel's own execution, as
 * kvq_decode_attention_timed does.
 */
kvq_status kvq_decode_step_timed(kvq_cache* h, const void* d_k, const void* d_v,
                                 const void* d_q, float* d_out, float* d_acc, void* d_ws,
                                 size_t ws_bytes, void* ev_start, void* ev_stop, void* stream);

/*
 * Workspace bytes kvq_topk_evict can use for these sizes on the current GPU
 * (0 when every row is served by one workgroup). Host only; the same checks
 * as kvq_topk_evict (KVQ_EINVAL).
 */
kvq_status kvq_topk_workspace(int32_t rows, int32_t T, int32_t k, int32_t w, size_t* ws_bytes);

/*
 * Heavy-hitter selection on fp32 scores ("MiniKV: Pushing the Limits of LLM
 * Inference via 2-Bit Layer-Discriminative KV Cache", Algorithm 1, heavy
 * hitters plus recent window; "KV cache quantization and eviction", section
 * "Minimal implementation": evicting the lowest score one token at a time,
 * with ties going to the earlier token, keeps on fixed scores the k largest
 * with ties toward the later index).
 *   d_scores device fp32 [rows][T]
 *   d_idx    device int32 [rows][k + w] (written): for each row the k largest
 *            scores among indices [0, T - w), ties broken toward the larger
 *            index, then the w most recent indices [T - w, T); ascending.
 *   d_ws     device workspace of ws_bytes >= kvq_topk_workspace(rows, T, k, w),
 *            or NULL. With it, rows are split over several workgroups when
 *            one workgroup per row would leave compute units idle; without
 *            it, one workgroup per row. Both give the same indices.
 * +0 and -0 compare equal; a NaN score ranks below every number and all NaNs
 * compare equal. Errors: KVQ_EINVAL (null pointer, rows < 0, k < 0, w < 0,
 * k + w > T), KVQ_EWORKSPACE.
 */
kvq_status kvq_topk_evict(const float* d_scores, int32_t rows, int32_t T, int32_t k,
                          int32_t w, int32_t* d_idx, void* d_ws, size_t ws_bytes,
                          void* stream);

/*
 * Prefill attention of one layer with heavy-hitter scores ("MiniKV: Pushing
 * the Limits of LLM Inference via 2-Bit Layer-Discriminative KV Cache",
 * section 4.3, selective flash-attention; Algorithm 1, prefill):
 *   S = Q K^T / sqrt(d) with the keys after each query masked (causal),
 *   P = softmax(S) per row, d_out = P V, and, when d_acc is given,
 *   d_acc[b][h_kv][j] = sum over the r query heads of KV head h_kv and over
 *   the rows i >= j of P[i][j] (A_cumul, written, not accumulated).
 *   d_q    device fp16 [B][Hq][n][d]; d_k, d_v device fp16 [B][Hkv][n][d]
 *   d_out  device fp32 [B][Hq][n][d]
 *   d_acc  device fp32 [B][Hkv][n] or NULL (then only d_out is computed)
 *   d_ws   device workspace of ws_bytes >= kvq_prefill_workspace (per-row
 *          log-sum-exp of the softmax, per query head partial column sums)
 * d_acc feeds kvq_topk_evict (rows = B * Hkv, T = n), whose kept indices feed
 * kvq_gather_kv and then kvq_quantize_append (MiniKV section 4.1, persistent
 * context selection). Query head h reads KV head h / (Hq / Hkv).
 * Errors: KVQ_EINVAL (null pointer with n > 0, bad sizes), KVQ_EUNSUPPORTED
 * (head_dim != 128, Hq / Hkv not in {1, 2, 4}, B * Hq > 65535), KVQ_EWORKSPACE.
 */
kvq_status kvq_prefill_workspace(int32_t batch, int32_t n_q_heads, int32_t n, size_t* ws_bytes);
kvq_status kvq_prefill_attention(const void* d_q, const void* d_k, const void* d_v, int32_t batch,
                                 int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                 int32_t n, float* d_out, float* d_acc, void* d_ws,
                                 size_t ws_bytes, void* stream);

/*
 * Rows of the kept tokens ("MiniKV", section 4.1, persistent context
 * selection: the heavy hitters chosen at the end of the prefill are the
 * tokens that are quantized): for every unit u = b * Hkv + h,
 *   d_k_out[u][i] = d_k[u][d_idx[u][i]], likewise for values, i < n_keep.
 *   d_k, d_v        device fp16 [B][Hkv][n][d]
 *   d_idx           device int32 [B * Hkv][n_keep] (kvq_topk_evict's output);
 *                   an index outside [0, n) gives a zero row
 *   d_k_out, d_v_out device fp16 [B][Hkv][n_keep][d]
 * Errors: KVQ_EINVAL (null pointer with n_keep > 0, n_keep > n, bad sizes),
 * KVQ_EUNSUPPORTED (head_dim != 128, B * Hkv > 65535).
 */
kvq_status kvq_gather_kv(const void* d_k, const void* d_v, int32_t batch, int32_t n_kv_heads,
                         int32_t head_dim, int32_t n, const int32_t* d_idx, int32_t n_keep,
                         void* d_k_out, void* d_v_out, void* stream);

/*
 * Measurement utility: one read-only pass over d_buf (device, bytes a multiple
 * of 16, 16-byte aligned), every 16-byte word loaded once; writes device
 * uint32 d_sink[4096] (an XOR of the data, so that no load can be dropped).
 * Its bandwidth is the read ceiling the decode kernel is compared with.
 * Errors: KVQ_EINVAL (null pointer, bytes % 16 != 0).
 */
kvq_status kvq_stream_read(const void* d_buf, size_t bytes, uint32_t* d_sink, void* stream);

/*
 * Set the FP8 scales of a b = 8 cache: d_scales is device fp32 [Hkv][2] (key
 * scale, value scale per KV head), finite and positive (not checked on the
 * device). Elements are stored as E4M3(x / s) and read back as E4M3 * s; set
 * the scales before the first append, since stored codes are not re-encoded
 * ("KV cache quantization and eviction", section "FP8, KIVI and KVQuant":
 * scales set to 1.0 or calibrated, optionally per attention head).
 * Errors: KVQ_EINVAL (invalid handle or null d_scales), KVQ_EUNSUPPORTED
 * (b != 8).
 */
kvq_status kvq_fp8_set_scales(kvq_cache* h, const float* d_scales, void* stream);

/*
 * One H2O eviction step ("H2O: Heavy-Hitter Oracle", greedy eviction of the
 * lowest accumulated score, one token per step; "KV cache quantization and
 * eviction", h2o_evict in "Minimal implementation"). For every unit that
 * holds more than `budget` live tokens (sinks included), the live token t in
 * [S, T - recent) with the lowest d_acc[u][t] is evicted: later decode calls
 * skip it and add nothing to its score. Ties go to the older token (a
 * first-occurrence argmin); a NaN score ranks below every number. Evicted
 * tokens keep their storage (a quantized token shares its group's scale).
 *   d_acc   device fp32 [B][Hkv][T], the scores after this step's decode call
 * Errors: KVQ_EINVAL (invalid handle, null d_acc, budget < 0, recent < 0).
 */
kvq_status kvq_evict_step(kvq_cache* h, const float* d_acc, int32_t budget, int32_t recent,
                          void* stream);

/*
 * Heavy-hitter budget per layer by MiniKV's pyramid ("MiniKV", section 4.2,
 * Layer-Specific Selectivity): with average budget x = avg_budget and depth
 * d >= 1 over L = n_layers layers, the budget falls linearly from 2x - x/d at
 * the lowest layer (index 0) to x/d at the highest, each rounded down (exact
 * integer arithmetic). The page names the x/d end "bottom-most" but also
 * gives lower layers more cache; the latter reading is taken. Host only:
 * writes host int32 out[L]. Errors: KVQ_EINVAL (null out, L outside [1, 4096],
 * x outside [0, 2^24], d outside [1, 4096]).
 */
kvq_status kvq_pyramid_budgets(int32_t n_layers, int32_t avg_budget, int32_t depth,
                               int32_t* out);

/*
 * Inspection: canonical codes of the quantized tokens, one byte per code,
 * device uint8 [U][n_q][d] for keys and for values.
 */
kvq_status kvq_unpack_codes(const kvq_cache* h, uint8_t* d_kcodes, uint8_t* d_vcodes,
                            void* stream);

/*
 * Canonical view of everything a cache stores, independent of the arena's
 * internal layout (for parity checks and debugging). Every field is a device
 * buffer owned by the caller, or NULL to skip it. With n_q, T the handle's
 * counts, KG = n_q / G key groups and NG = d / min(G, d) value groups:
 *   kcodes, vcodes  uint8 [U][n_q][d]: one code per element
 *   kscale, kzero   fp16 [U][KG][d]: key scale and zero point per group and
 *                   channel (MiniKV, section 4.4: both kept in FP16)
 *   vscale, vzero   fp16 [U][n_q][NG]: value scale and zero point per token
 *                   and channel group
 *   pooled          uint8 [U][n_q]: 1 when the token was admitted to the
 *                   outlier pool (its quantized slot holds the group mean);
 *                   the quantized tokens are S .. S + n_q - 1
 * Pool and extra-pool indices are indices in the whole sequence.
 *   kres, vres      fp16 [U][T - S - n_q][d]: the fp16 residual rows, token order
 *   ksink, vsink    fp16 [U][min(T, S)][d]: the attention-sink rows
 *   live            uint8 [U][T]: 0 for tokens evicted by kvq_evict_step
 *   counters        int32 [U][4]: pool count, extra-pool count, frozen flag,
 *                   value-scale bound (fp16 bits, as in the arena)
 *   pool_idx        int32 [U][N], pool_score uint64 [U][N] (key L1 norm in
 *                   units of 2^-24), pool_k, pool_v fp16 [U][N][d]
 *   ev_idx          int32 [U][E], ev_k, ev_v fp16 [U][E][d] (extra pool)
 * Pool slots beyond the counters are unspecified.
 */
typedef struct kvq_debug_view {
    uint8_t* kcodes;
    uint8_t* vcodes;
    uint16_t* kscale;
    uint16_t* kzero;
    uint16_t* vscale;
    uint16_t* vzero;
    uint8_t* pooled;
    uint16_t* kres;
    uint16_t* vres;
    int32_t* counters;
    int32_t* pool_idx;
    uint64_t* pool_score;
    uint16_t* pool_k;
    uint16_t* pool_v;
    int32_t* ev_idx;
    uint16_t* ev_k;
    uint16_t* ev_v;
    uint16_t* ksink;
    uint16_t* vsink;
    uint8_t* live;
} kvq_debug_view;

/* Fill the non-NULL fields of *view (host struct of device pointers) on
 * `stream`. Errors: KVQ_EINVAL (invalid handle or null view). */
kvq_status kvq_debug_unpack(const kvq_cache* h, const kvq_debug_view* view, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */

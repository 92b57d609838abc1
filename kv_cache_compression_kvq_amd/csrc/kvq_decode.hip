// Decode attention over the compressed cache on gfx950, plus the H2O score
// accumulation.
//
// One step computes, for every query head h of a unit (MiniKV, section 2
// Eq. 1 and Algorithm 1; "Accurate KV Cache Quantization with Outlier Tokens
// Tracing", section "Method details", decoding stage):
//   s_j = q_h . k_j / sqrt(d),  p = softmax(s),  out_h = sum_j p_j v_j
// over every cached token j exactly once: dequantized quantized tokens (their
// slots skipped when the token sits in the outlier pool), fp16 residual
// tokens and fp16 pool tokens.
//
// Kernel 1 (decode_kernel), one launch:
//  * blocks [0, U * tiles): the fp16 partition (ring + pools), 64 rows each;
//  * blocks [U, U + U*S): split-K over the quantized tokens. Each wavefront
//    takes whole key groups. Per key group the key scale is folded into the
//    query, q~_c = q_c * s_c (split into fp16 hi + lo), and the zero point
//    into one scalar per head; the per-token dot products then run on the
//    matrix cores (v_mfma_f32_16x16x32_f16) against the raw codes, which
//    become the exact fp16 operands 2^b + code with two bit operations.
//    Values go the same way with p_j * s^V_j as the fp16 hi + lo operand.
//    Online softmax in log2 units; partial (o, m, l) per block.
// Kernel 2 (merge_kernel): combines the partials into out and, when asked,
// adds the normalized probabilities of every token, summed over the query
// heads of the KV head, into the H2O accumulator ("H2O: Heavy-Hitter Oracle",
// accumulated attention; "KV cache quantization and eviction", section
// "Heavy hitters").
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;
// Partial record of one (unit, split, head): o[d], m, l, two pad floats, so
// that every record starts 16-byte aligned for the vector stores into it.
constexpr int kRec = kPartRec;
static_assert(kRec % 4 == 0 && kRec >= D + 2, "record holds o, m, l, 16-byte aligned");
constexpr int kMaxSplits = 1056;
constexpr int kH2OChunk = 2048;
// LDS of the fp16 partition: queries, probabilities and value-row addresses
// (4 x 256 B + 4 x 256 B + 4 x 512 B).
constexpr int kFp16Bytes = 4 * D * 2 + 4 * 64 * 4 + 4 * 64 * 8;

// Per-wavefront LDS of the quantized path: a ring of two chunk stages filled
// by direct global->LDS loads (codes, value scales, key scales, pool mask
// word); while chunk k computes, chunk k + 1 is in flight. After the loop the
// same bytes hold the output accumulators. The folded-query table and the
// probability exchange live in LDS objects of their own, so that writing them
// never waits on the ring's copies in flight.
template <int BITS, int G>
struct Ring {
    static constexpr int kStages = 2;
    static constexpr int kCodes = 128 * BITS * 4;          // packed codes of one chunk
    // value scales (32 tokens x d/G groups x 4 B: <= 512 B, 1 KB at G = 16),
    // then key scales (512 B per key group; G = 16: both groups of the chunk)
    static constexpr int kKmOff = G == 16 ? 1024 : 512;
    static constexpr int kMeta = kKmOff + (G == 16 ? 1024 : 512);
    static constexpr int kStage = 2 * kCodes + kMeta + 16;  // + pool mask and eviction words
    static constexpr int kLoads = 2 * (kCodes / 1024) + (G == 16 ? 3 : 2);  // loads per stage
    static constexpr int kWave = kStages * kStage;          // ring bytes per wavefront
    static constexpr int kBlock = 4 * kWave > kFp16Bytes ? 4 * kWave : kFp16Bytes;
    // epilogue: accumulators of tiles 0-5 in the ring, 6-7 in the query table
    static_assert(kWave >= 6 * 64 * 4 * 4, "epilogue fits the wavefront's ring");
};

__device__ __forceinline__ void lds_load16(const void* g, void* lds) {
    // lane i's 16 bytes land at lds + 16 * i
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)g,
        (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_load4(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)g,
        (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}
// Wait until at most N of this wavefront's vector memory operations are in
// flight (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// LDS address of a pointer into a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Load of a wave-uniform word that no kernel writes while this one runs,
// through the scalar data cache (read only).
__device__ __forceinline__ uint32_t scalar_load(const void* p) {
    return *(const __attribute__((address_space(4))) uint32_t*)p;
}
// Reads of a ring stage. They are issued as inline assembly, after the
// stage's explicit vmcnt wait, because the compiler cannot tell which ring
// slot a global->LDS copy in flight targets and would otherwise wait for all
// of them; ring_done() then waits for the reads and ties their results.
template <int OFF = 0>
__device__ __forceinline__ u32x4 ring_read(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
    return v;
}
__device__ __forceinline__ uint32_t ring_read32(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

struct DecodeArgs {
    const uint32_t* kq;
    const uint32_t* vq;
    const uint32_t* kmeta;
    const uint32_t* vmeta;
    const uint32_t* mask;
    const uint16_t* kring;
    const uint16_t* vring;
    const int32_t* pool_idx;
    const uint16_t* pool_k;
    const uint16_t* pool_v;
    const int32_t* ev_idx;
    const uint16_t* ev_k;
    const uint16_t* ev_v;
    const int32_t* counters;
    const uint32_t* evict;   // [U][evict_words] eviction bits of tokens S, S + 1, ...
    const int32_t* evict_count;  // [U]
    int64_t evict_words;
    const uint16_t* sink_k;  // attention sinks [U][sink_cap][d]
    const uint16_t* sink_v;
    const uint16_t* k_new;  // decode step: the newest token's rows [U][d] (else null)
    const uint16_t* v_new;
    const uint16_t* q;
    float* part;
    float* logits;
    float* out;
    float* acc;
    int64_t T, n_q, chunks, key_groups;
    int32_t units, n_kv_heads, ring_slots, splits_q, splits, fp16_tiles, pool, evict_cap;
    int32_t tile_rows;  // rows per fp16-partition tile (<= 64)
    int32_t sink_cap;   // S: sinks per unit; the quantized tokens are S .. S + n_q - 1
    int32_t sink_rows;  // min(T, S): sink rows present
    float qscale;  // log2(e) / sqrt(d)
    const float* fp8_scales;  // b = 8: [Hkv][2] key and value scale per KV head
};

__device__ __forceinline__ float h2f(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t hbits(_Float16 x) { return __builtin_bit_cast(uint16_t, x); }

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(half8, v);
}

template <int N>
__device__ __forceinline__ float row_ror(float x) {
    // DPP row_ror:N within each row of 16 lanes
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x120 + N, 0xF, 0xF, false));
}
template <int H>
__device__ __forceinline__ float quad_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, x), H | (H << 2) | (H << 4) | (H << 6),
                                         0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, false));
}
// x at lanes l and l ^ 32 (swap32) or l and l ^ 16 (swap16), returned as the
// pair (a, b) in either order: the gfx950 permlane swaps exchange rows of two
// registers on the VALU, with no LDS round trip. Written as inline asm because
// the compiler's builtin for these drops the second result.
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
    a = x;
    b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
    a = x;
    b = x;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_x32(float x) { float a, b; swap32(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float max_x16(float x) { float a, b; swap16(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float sum_x32(float x) { float a, b; swap32(x, a, b); return a + b; }
__device__ __forceinline__ float sum_x16(float x) { float a, b; swap16(x, a, b); return a + b; }
__device__ __forceinline__ float readlane(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
// Wavefront reductions: DPP within each row of 16 lanes, then the four row
// results through scalar registers (no LDS round trips).
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<0x128>(x));  // row_ror:8
    x = fmaxf(x, dpp<0x124>(x));  // row_ror:4
    x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
    return fmaxf(fmaxf(readlane(x, 0), readlane(x, 16)), fmaxf(readlane(x, 32), readlane(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<0x128>(x);
    x += dpp<0x124>(x);
    x += dpp<0x4E>(x);
    x += dpp<0xB1>(x);
    return (readlane(x, 0) + readlane(x, 16)) + (readlane(x, 32) + readlane(x, 48));
}

// fp16 pair (f16(a0 * s0), f16(a1 * s1)), s0 and s1 the low fp16 halves of
// their words, each a fused multiply rounded once (v_fma_mixlo / mixhi).
__device__ __forceinline__ uint32_t mul_pk(float a0, uint32_t s0, float a1, uint32_t s1) {
    uint32_t d;
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a0), "v"(s0));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(d) : "v"(a1), "v"(s1));
    return d;
}
// Residual pair (f16(a0 * s0 - h.lo), f16(a1 * s1 - h.hi)), fused and rounded once.
__device__ __forceinline__ uint32_t mul_pk_res(float a0, uint32_t s0, float a1, uint32_t s1,
                                               uint32_t h) {
    uint32_t d;
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a0), "v"(s0), "v"(h));
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,1,1]"
        : "+v"(d)
        : "v"(a1), "v"(s1), "v"(h));
    return d;
}

// Words 0-3 shifted left by 4, right by 4 and rotated left by 8 bits: the
// three moves that bring every 2-bit code position to bits 6-9 (positions 3, 4).
__device__ __forceinline__ void moved4(const uint32_t* w, uint32_t* l4, uint32_t* r4,
                                       uint32_t* o8) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        l4[m] = w[m] << 4;
        r4[m] = w[m] >> 4;
        o8[m] = __builtin_amdgcn_alignbit(w[m], w[m], 24);
    }
}

__device__ __forceinline__ void wave_lds_fence() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

// One 64-row tile of the fp16 partition of unit u: rows are the residual
// ring tokens [n_q, T), then the pool members, then the extra-pool members.
// Wavefront h < r takes query head h. Logits: one row per lane, the row read
// straight from memory and dotted with the query (fp16 x fp16 products are
// exact in the fp32 dot2 accumulation). Each lane also resolves its row's
// value address once and leaves it in LDS. Outputs: lane (row phase l / 16,
// channel block l % 16) accumulates 8 channels over every fourth row, then the
// four row phases are summed across lanes.
template <int R>
__device__ void fp16_tile(const DecodeArgs& a, int u, int tile, float* smem) {
    const int tid = threadIdx.x, lane = tid & 63, h = tid >> 6;
    uint32_t* qh = reinterpret_cast<uint32_t*>(smem);      // [R][D/2] fp16 pairs
    float* ps = reinterpret_cast<float*>(qh + R * D / 2);  // [R][64]
    const uint4** vp = reinterpret_cast<const uint4**>(ps + 4 * 64);  // [R][64] value rows
    const int b = u / a.n_kv_heads, hk = u % a.n_kv_heads;
    const uint32_t* qsrc =
        reinterpret_cast<const uint32_t*>(a.q + ((int64_t)b * a.n_kv_heads * R + hk * R) * D);
    for (int e = tid; e < R * D / 2; e += 256) qh[e] = qsrc[e];
    // Rows of the partition: the attention sinks, the residual ring tokens
    // (sequence index S + n_q onwards), the pool, the extra pool.
    const int64_t ns = a.sink_rows;
    const int64_t nres = a.T - ns - a.n_q;
    const int pc = a.pool > 0 ? a.counters[(int64_t)u * 4] : 0;
    const int ec = a.pool > 0 ? a.counters[(int64_t)u * 4 + 1] : 0;
    const int64_t ntot = ns + nres + pc + ec;
    const int N = a.pool, E = a.evict_cap, RB = a.ring_slots;
    const int64_t base = (int64_t)tile * a.tile_rows;
    const int cnt = (int)(ntot - base < 0 ? 0 : ntot - base < a.tile_rows ? ntot - base : a.tile_rows);
    // Row i of the tile: kind 0 sink, 1 ring (slot (n_q + ring row) % RB),
    // 2 pool, 3 extra pool; returns the row's element offset in its array.
    // The ring rows of a tile are fewer than RB, so one slot computed per tile
    // and at most one wrap give every row's slot.
    const int64_t ring_first = base > ns ? base : ns;
    const int32_t slot_first = (int32_t)((a.n_q + (ring_first - ns)) % RB);
    auto row_off = [&](int i, int& kind) -> int64_t {
        const int64_t li = base + i;
        if (li < ns) {
            kind = 0;
            return ((int64_t)u * a.sink_cap + li) * D;
        }
        if (li < ns + nres) {
            kind = 1;
            int32_t sl = slot_first + (int32_t)(li - ring_first);
            if (sl >= RB) sl -= RB;
            return ((int64_t)u * RB + sl) * D;
        }
        if (li < ns + nres + pc) {
            kind = 2;
            return ((int64_t)u * N + (li - ns - nres)) * D;
        }
        kind = 3;
        return ((int64_t)u * E + (li - ns - nres - pc)) * D;
    };
    // With a decode step's input, the newest token (the last ring row) is read
    // from it; its ring slot is written below.
    const bool new_row = a.k_new != nullptr;
    const int64_t last_ring = ns + nres - 1;
    auto row_ptr = [&](int i, const uint16_t* sink, const uint16_t* ring, const uint16_t* pool,
                       const uint16_t* ev, const uint16_t* nw) -> const uint16_t* {
        int kind;
        const int64_t o = row_off(i, kind);
        if (kind == 1) return new_row && base + i == last_ring ? nw + (int64_t)u * D : ring + o;
        return (kind == 0 ? sink : kind == 2 ? pool : ev) + o;
    };
    if (new_row && h == 0 && lane < 32 && base <= last_ring && last_ring < base + cnt) {
        // store the step's token (sequence index T - 1, ring token T - 1 - S)
        // into its ring slot: lanes 0-15 the key, 16-31 the value, 16 bytes each
        const int64_t dst = ((int64_t)u * RB + (a.T - 1 - a.sink_cap) % RB) * D;
        const int part = lane & 15;
        const uint16_t* src = (lane < 16 ? a.k_new : a.v_new) + (int64_t)u * D;
        uint16_t* ring = const_cast<uint16_t*>(lane < 16 ? a.kring : a.vring);
        reinterpret_cast<uint4*>(ring + dst)[part] = reinterpret_cast<const uint4*>(src)[part];
    }
    __syncthreads();
    if (h >= R) return;
    const bool any_evicted = scalar_load(a.evict_count + u) != 0u;
    float s = -INFINITY;
    if (lane < cnt) {
        // the row's token index after the sinks (-1 for a sink) and whether it
        // was evicted, requested together with the row itself
        const int64_t li = base + lane;
        const int64_t tau = li < ns ? -1
                            : li < ns + nres ? a.n_q + (li - ns)
                            : li < ns + nres + pc
                                ? a.pool_idx[(int64_t)u * N + (li - ns - nres)]
                                : a.ev_idx[(int64_t)u * E + (li - ns - nres - pc)];
        const uint32_t evw = tau >= 0 && any_evicted
                                 ? a.evict[(int64_t)u * a.evict_words + (tau >> 5)] : 0u;
        const uint4* kr = reinterpret_cast<const uint4*>(
            row_ptr(lane, a.sink_k, a.kring, a.pool_k, a.ev_k, a.k_new));
        vp[h * 64 + lane] = reinterpret_cast<const uint4*>(
            row_ptr(lane, a.sink_v, a.vring, a.pool_v, a.ev_v, a.v_new));
        uint4 x[16];
#pragma unroll
        for (int c8 = 0; c8 < 16; ++c8) x[c8] = kr[c8];
        const uint4* qr = reinterpret_cast<const uint4*>(qh + h * (D / 2));
        float acc = 0.f;
#pragma unroll
        for (int c8 = 0; c8 < 16; ++c8) {
            const uint4 y = qr[c8];
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, x[c8].x),
                                         __builtin_bit_cast(half2_t, y.x), acc, false);
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, x[c8].y),
                                         __builtin_bit_cast(half2_t, y.y), acc, false);
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, x[c8].z),
                                         __builtin_bit_cast(half2_t, y.z), acc, false);
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, x[c8].w),
                                         __builtin_bit_cast(half2_t, y.w), acc, false);
        }
        s = acc * a.qscale;
        if (tau >= 0 && ((evw >> (tau & 31)) & 1u)) s = -INFINITY;  // evicted
        if (a.logits) {
            // sequence index of the row's token
            const int64_t t = tau < 0 ? li : a.sink_cap + tau;
            a.logits[((int64_t)u * R + h) * a.T + t] = s;
        }
    }
    const float m = cnt > 0 ? wave_max(s) : -INFINITY;
    const float p = s == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s - m);
    const float l = wave_sum(p);
    ps[h * 64 + lane] = p;
    wave_lds_fence();
    // Outputs: lane (phase rp, block cb) takes channels 8 cb .. 8 cb + 7 of rows
    // rp, rp + 4, ...; p is 0 past cnt.
    const int rp = lane >> 4, cb = lane & 15;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float* ph = ps + h * 64;
    const uint4* const* vh = vp + h * 64;
    for (int i0 = 0; i0 < cnt; i0 += 16) {
        uint4 w[4];
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 4 * r + rp;
            pv[r] = ph[i < 64 ? i : 63];
            w[r] = i < cnt ? vh[i][cb] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t ww[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                o[2 * c] += pv[r] * h2f(ww[c] & 0xFFFF);
                o[2 * c + 1] += pv[r] * h2f(ww[c] >> 16);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = sum_x32(sum_x16(o[c]));
    float* rec = a.part + (((int64_t)u * a.splits + a.splits_q + tile) * R + h) * kRec;
    if (rp == 0) {
        *reinterpret_cast<floatx4*>(rec + 8 * cb) = floatx4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<floatx4*>(rec + 8 * cb + 4) = floatx4{o[4], o[5], o[6], o[7]};
    }
    if (lane == 0) {
        rec[D] = m;
        rec[D + 1] = l;
    }
}

template <int BITS, int R, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void decode_kernel(DecodeArgs a) {
    constexpr bool kG16 = G == 16;   // two key groups per 32-token chunk
    constexpr int NG = D / G;        // value groups per token
    // A wavefront's work item is a key group of CPG chunks, or with G = 16 one
    // chunk holding KPC = 2 key groups (16-token tiles 0 and 1).
    constexpr int CPG = kG16 ? 1 : G / 32;
    constexpr int KPC = kG16 ? 2 : 1;
    // Value-operand rows are (head, value group) pairs: 16 per matrix-core
    // operand, so r = 4 with 8 value groups (G = 16) needs two row sets, set s
    // holding groups 4s .. 4s + 3 for the channel tiles 4s .. 4s + 3.
    constexpr int GPS = 16 / R < NG ? 16 / R : NG;  // value groups per row set
    constexpr int VSETS = NG / GPS;
    static_assert(VSETS == 1 || VSETS == 2, "at most two value row sets");
    constexpr int WPC = 128 * BITS;  // words per chunk
    // With r = 4 the 16 MFMA columns hold 4 copies of each head's logits;
    // each copy then exponentiates a quarter of the tokens.
    constexpr bool kSplitExp = R == 4;
    constexpr bool kMirror = kSplitExp;
    // Code operands. A code masked in place at bits [p, p + b) of both 16-bit
    // halves is the pair of fp16 subnormals code * 2^(p - 24): exact, one AND.
    // The matrix cores align products by the encoded exponent, so codes are
    // kept at bits 6-9 (at most two leading zero bits; lower positions cost
    // precision): at b = 2 every pair is moved to bits 6-7 or 8-9, at b = 4
    // value nibbles are shifted to bits 4-7. Each matrix-core operand takes all
    // its pairs from one position, so the weight 2^(p - 24) is common to the
    // operand and is taken out elsewhere (keys: in the folded query; values:
    // in the epilogue). At b = 4 keys are shifted to bits 6-9 and become
    // 16 + code (v_and_or_b32 with the exponent of 16).
    constexpr float kAccW = BITS == 2 ? 65536.f : 1.f;  // keys: 2^16 removes the operand weight
    constexpr uint32_t kMaskA = 0x03C003C0u;
    constexpr uint32_t kMagicA = 0x4C004C00u;
    using RG = Ring<BITS, G>;
    __shared__ __align__(16) float smem[RG::kBlock / 4];
    __shared__ __align__(16) unsigned char s_btab[4][2048 * KPC];
    __shared__ __align__(16) float s_pbuf[4][128];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if ((int)blockIdx.x < a.units * a.fp16_tiles) {
        fp16_tile<R>(a, blockIdx.x / a.fp16_tiles, blockIdx.x % a.fp16_tiles, smem);
        return;
    }
    uint32_t vmaskA, vmagicA;
    asm volatile("v_mov_b32 %0, %1" : "=v"(vmaskA) : "i"(kMaskA));
    asm volatile("v_mov_b32 %0, %1" : "=v"(vmagicA) : "i"(kMagicA));
    auto cvt4 = [&](uint32_t w, int sh) -> uint32_t {  // b = 4 keys; sh > 0: left shift
        const uint32_t x = sh >= 0 ? (w << sh) : (w >> -sh);
        return (x & vmaskA) | vmagicA;
    };

    const int idx = blockIdx.x - a.units * a.fp16_tiles;
    const int u = idx / a.splits_q, split = idx % a.splits_q;
    const int b = u / a.n_kv_heads, hk = u % a.n_kv_heads;
    // Work items: key groups (wavefronts of a block interleaved), or with
    // G = 16 chunks (two groups each); with groups of several chunks (G = 64,
    // 128) single chunks, each wavefront taking a contiguous quarter of its
    // block's range, so that no wavefront holds a whole extra group; a
    // wavefront that starts inside a group folds that group's scales first.
    constexpr bool kChunkItems = CPG > 1;
    const uint32_t items = (uint32_t)(kG16 || kChunkItems ? (a.n_q + 31) / 32 : a.n_q / G);
    const uint32_t gs0 = (uint32_t)((int64_t)split * items / a.splits_q);
    const uint32_t gs1 = (uint32_t)((int64_t)(split + 1) * items / a.splits_q);
    const uint32_t wc0 = gs0 + (uint32_t)wave * (gs1 - gs0) / 4;  // chunk items: first chunk
    const uint32_t wc1 = gs0 + (uint32_t)(wave + 1) * (gs1 - gs0) / 4;
    const uint32_t my_groups = gs1 - gs0 > (uint32_t)wave ? (gs1 - gs0 - wave + 3) / 4 : 0;
    const uint32_t n_items = kChunkItems ? wc1 - wc0 : my_groups * CPG;
    // chunk k of this wavefront: its index, key group and place in the group
    auto chunk_of = [&](uint32_t k, uint32_t& gi, uint32_t& cc) {
        if (kChunkItems) {
            const uint32_t ch = wc0 + k;
            gi = ch / CPG;
            cc = ch % CPG;
        } else {
            gi = gs0 + wave + 4 * (k / CPG);
            cc = k % CPG;
        }
    };

    // Per-unit base pointers (wave-uniform); per-lane offsets stay 32-bit.
    const uint32_t* kq_u = a.kq + (int64_t)u * a.chunks * WPC;
    const uint32_t* vq_u = a.vq + (int64_t)u * a.chunks * WPC;
    const uint32_t* km_u = a.kmeta + (int64_t)u * a.key_groups * D;
    const uint32_t* vm_u = a.vmeta + (int64_t)u * a.chunks * NG * 32;
    const uint32_t* mk_u = a.mask + (int64_t)u * a.chunks;
    const uint32_t* ev_u = a.evict + (int64_t)u * a.evict_words;

    // MFMA lane roles: j = column / row within a 16-lane row, kb = k-block.
    const int j = lane & 15, kb = lane >> 4, jj = j & 7;
    // Logit columns. With r = 4 (kMirror) column j holds head hq, the hi
    // (pq = 0) or lo (pq = 1) half of the folded query, copy cq: within each
    // half-row of 8 lanes, the lo column of a head mirrors its hi column, so
    // one row_half_mirror add gives both lanes the full logit. Otherwise the
    // columns repeat head j % r and hi/lo are two k-steps.
    const int hq = kMirror ? (jj < 4 ? jj : 7 - jj) : j % R;
    const int pq = jj < 4 ? 0 : 1;
    const int cq = kMirror ? pq + 2 * (j >> 3) : j >> 2;
    // Query-fold role: head hb, channels cb0 .. cb0+7 (k-step ksb, k-block kbb);
    // with kMirror the lanes of one head in a row are its four logit columns.
    const int hb = kMirror ? hq : lane % R, kap = (lane >> 2) & 15, ksb = kap >> 2, kbb = kap & 3;
    const int cb0 = 32 * ksb + 8 * kbb;
    // Value-operand role: row j = (head ha = j % r, value group gs); with
    // kSplitExp, copy cq of head hq owns token slots 2cq, 2cq+1.
    const int ha = j % R;
    const int gs = (j / R) % NG;
    const int own_tok = 16 * (cq >> 1) + 4 * kb + 2 * (cq & 1);  // first owned token

    // The query row is requested first (inline assembly, so that the
    // compiler's counter bookkeeping does not wait for every ring stage before
    // it is used) and converted once the first ring stages are in flight.
    u32x4 qraw;
    asm volatile("global_load_dwordx4 %0, %1, off"
                 : "=v"(qraw)
                 : "v"(a.q + ((int64_t)b * a.n_kv_heads * R + hk * R + hb) * D + cb0)
                 : "memory");
    float qv[8];

    // Stage k (chunk k of this wavefront) lands in ring slot k % kStages.
    char* wlds = reinterpret_cast<char*>(smem) + wave * RG::kWave;
    auto issue = [&](uint32_t k) {
        uint32_t gi, cc;
        chunk_of(k, gi, cc);
        const uint32_t ch = gi * CPG + cc;
        const bool fold = cc == 0 || (kChunkItems && k == 0);  // the group's key scales
        char* st = wlds + (k % RG::kStages) * RG::kStage;
        lds_load16(kq_u + ch * WPC + lane * 4, st);
        if (BITS == 4) lds_load16(kq_u + ch * WPC + 256 + lane * 4, st + 1024);
        lds_load16(vq_u + ch * WPC + lane * 4, st + RG::kCodes);
        if (BITS == 4) lds_load16(vq_u + ch * WPC + 256 + lane * 4, st + RG::kCodes + 1024);
        if (kG16) {
            // value scales (1 KB), then the key scales of both groups (1 KB)
            lds_load16(vm_u + ch * NG * 32 + lane * 4, st + 2 * RG::kCodes);
            lds_load16(km_u + 2 * ch * D + lane * 4, st + 2 * RG::kCodes + RG::kKmOff);
        } else {
            // value scales (lanes < 8 NG) and, at a key group's first chunk, key
            // scales (lanes >= 32)
            const uint32_t* src =
                lane < 32 ? vm_u + ch * NG * 32 + lane * 4 : km_u + gi * D + (lane - 32) * 4;
            if (lane < 8 * NG || (lane >= 32 && fold)) lds_load16(src, st + 2 * RG::kCodes);
        }
        // lane 0: the chunk's pool mask word; lane 1: its eviction word
        if (lane < 2) lds_load4(lane == 0 ? mk_u + ch : ev_u + ch, st + 2 * RG::kCodes + RG::kMeta);
    };
    float* wsm = reinterpret_cast<float*>(wlds);
    unsigned char* btab = s_btab[wave];  // folded query, 2 KB per key group of a chunk
    float* pbuf = s_pbuf[wave];          // [4][32] probabilities
    // beta0 / beta1: zero-point terms of the chunk's key groups (tiles 0 / 1);
    // zc / zc2: sum_t p_t z^V_t of the lane's value rows in row set 0 / 1
    float m_run = -INFINITY, lsum = 0.f, zc = 0.f, zc2 = 0.f, beta0 = 0.f, beta1 = 0.f;
    floatx4 O[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    // Lazy rescale: the running max m_run only moves when a logit exceeds it
    // by more than tau (log2 units), so probabilities stay below 2^tau; tau is
    // bounded so that p * s^V, s^V below the unit's value-scale bound, stays
    // far inside fp16 (< 2^15).
    float m_thr = -INFINITY;
    float tau = 8.f;
    {
        // wave-uniform and constant during the kernel: a scalar load, so that it
        // never waits on the ring's vector-memory counter
        const uint32_t smax = scalar_load(a.counters + (int64_t)u * 4 + 3) & 0x7FFFu;
        if (smax >= 0x0400u) {  // normal: s < 2^(e+1)
            const int e = (int)(smax >> 10) - 15;
            tau = (float)min(8, max(0, 14 - e));
        }
    }

    // per-lane parts of the ring-stage addresses: codes, value scales of this
    // lane's value-operand row, key scales of its query-fold channels
    const uint32_t lane_codes = lane * 16;
    const uint32_t lane_vm = 2 * RG::kCodes + (gs * 32 + 4 * kb) * 4;
    const uint32_t lane_km = 2 * RG::kCodes + RG::kKmOff + cb0 * 4;
    auto step = [&](uint32_t k, uint32_t later) {
        uint32_t gi, cc;
        chunk_of(k, gi, cc);
        const bool fold = cc == 0 || (kChunkItems && k == 0);
        const int64_t tb = (int64_t)(gi * CPG + cc) * 32;
        const uint32_t st = lds_addr(wlds + (k % RG::kStages) * RG::kStage);
        const uint32_t meta = st + 2 * RG::kCodes;
        // the stage issued after this one (if any) may stay in flight
        if (later >= 1) wait_vm<RG::kLoads>();
        else wait_vm<0>();
        // three per-lane bases, every other offset an immediate
        const uint32_t a_codes = st + lane_codes, a_vm = st + lane_vm, a_km = st + lane_km;
        u32x4 wk0 = ring_read<0>(a_codes), wk1;
        u32x4 wv0 = ring_read<RG::kCodes>(a_codes), wv1;
        if (BITS == 4) {
            wk1 = ring_read<1024>(a_codes);
            wv1 = ring_read<RG::kCodes + 1024>(a_codes);
        }
        u32x4 vm0 = ring_read<0>(a_vm);
        u32x4 vm1 = ring_read<64>(a_vm);
        u32x4 km0 = vm0, km1 = vm1, km2 = vm0, km3 = vm1, vm2 = vm0, vm3 = vm1;
        if (fold) {
            km0 = ring_read<0>(a_km);
            km1 = ring_read<16>(a_km);
        }
        if (kG16) {
            // the second key group's scales, and the value rows of set 1
            km2 = ring_read<512>(a_km);
            km3 = ring_read<528>(a_km);
            vm2 = ring_read<GPS * 128>(a_vm);
            vm3 = ring_read<GPS * 128 + 64>(a_vm);
        }
        uint32_t mwv = ring_read32(meta + RG::kMeta);
        uint32_t ewv = ring_read32(meta + RG::kMeta + 4);
        if (kG16 && BITS == 4) {
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(wk0), "+v"(wk1), "+v"(wv0), "+v"(wv1), "+v"(vm0), "+v"(vm1),
                           "+v"(km0), "+v"(km1), "+v"(mwv), "+v"(ewv), "+v"(km2), "+v"(km3), "+v"(vm2),
                           "+v"(vm3)
                         :
                         : "memory");
        } else if (kG16) {
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(wk0), "+v"(wv0), "+v"(vm0), "+v"(vm1), "+v"(km0), "+v"(km1),
                           "+v"(mwv), "+v"(ewv), "+v"(km2), "+v"(km3), "+v"(vm2), "+v"(vm3)
                         :
                         : "memory");
            wk1 = wk0;
            wv1 = wv0;
        } else if (BITS == 4) {
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(wk0), "+v"(wk1), "+v"(wv0), "+v"(wv1), "+v"(vm0), "+v"(vm1),
                           "+v"(km0), "+v"(km1), "+v"(mwv), "+v"(ewv)
                         :
                         : "memory");
        } else {
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(wk0), "+v"(wv0), "+v"(vm0), "+v"(vm1), "+v"(km0), "+v"(km1),
                           "+v"(mwv), "+v"(ewv)
                         :
                         : "memory");
            wk1 = wk0;  // one 16-byte word group per lane at b = 2
            wv1 = wv0;
        }
        if (fold) {
            // Fold the key scale into the query: B = hi/lo of q~_c * s_c, and
            // the zero point into beta_h = sum_c q~_c (z_c - 2^b s_c); with
            // G = 16 once per key group of the chunk.
            wave_lds_fence();  // previous group's B reads are done
#pragma unroll
            for (int kg = 0; kg < KPC; ++kg) {
                const u32x4 ka = kg == 0 ? km0 : km2, kc = kg == 0 ? km1 : km3;
                const uint32_t kmw[8] = {ka.x, ka.y, ka.z, ka.w, kc.x, kc.y, kc.z, kc.w};
                uint32_t hiw[4], low[4];
                float bp = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    hiw[i] = mul_pk(qv[2 * i], kmw[2 * i], qv[2 * i + 1], kmw[2 * i + 1]);
                    low[i] = mul_pk_res(qv[2 * i], kmw[2 * i], qv[2 * i + 1], kmw[2 * i + 1], hiw[i]);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float zk = h2f(kmw[i] >> 16);
                    if (BITS == 2) {
                        bp += qv[i] * zk;
                    } else {
                        const float sk = h2f(kmw[i] & 0xFFFF);
                        bp += qv[i] * (zk - 16.f * sk);
                    }
                }
                if (BITS == 2 && ksb % 2 == 0) bp *= 0.25f;  // undo the query weight
                unsigned char* e0 = btab + kg * 2048 + ((((ksb * 4 + kbb) * 2) * 4) + hb) * 16;
                *reinterpret_cast<u32x4*>(e0) = u32x4{hiw[0], hiw[1], hiw[2], hiw[3]};
                *reinterpret_cast<u32x4*>(e0 + 4 * 16) = u32x4{low[0], low[1], low[2], low[3]};
                bp += row_ror<8>(bp);
                bp += kMirror ? dpp<0x141>(bp) : row_ror<4>(bp);  // row_half_mirror
                (kg == 0 ? beta0 : beta1) = sum_x32(sum_x16(bp));
            }
            if (!kG16) beta1 = beta0;
            wave_lds_fence();
        }

        // Logits S^T[token][(head, g)] on the matrix cores: two 16-token tiles,
        // K = 128 channels x {hi, lo}.
        const uint32_t wk[8] = {wk0.x, wk0.y, wk0.z, wk0.w, wk1.x, wk1.y, wk1.z, wk1.w};
        uint32_t wkL4[4], wkR4[4], wkO8[4];
        moved4(wk, wkL4, wkR4, wkO8);
        floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            half8 A0, A1;
            if (BITS == 2) {
                // pair m from word m: tile 0 at positions 3, 4, 1, 2 (k-steps
                // 0..3), tile 1 at 5, 6, 7, 0; even k-steps end at bits 6-7
                const uint32_t mk = ks % 2 == 0 ? 0x00C000C0u : 0x03000300u;
                const uint32_t* x0 = ks < 2 ? wk : wkL4;
                const uint32_t* x1 = ks < 2 ? wkR4 : wkO8;
                A0 = as_half8(x0[0] & mk, x0[1] & mk, x0[2] & mk, x0[3] & mk);
                A1 = as_half8(x1[0] & mk, x1[1] & mk, x1[2] & mk, x1[3] & mk);
            } else {
                const uint32_t w0 = wk[ks], w1 = wk[4 + ks];
                A0 = as_half8(cvt4(w0, 6), cvt4(w0, 2), cvt4(w0, -2), cvt4(w0, -6));
                A1 = as_half8(cvt4(w1, 6), cvt4(w1, 2), cvt4(w1, -2), cvt4(w1, -6));
            }
            // tile 1 takes the folded query of the chunk's second key group (G = 16)
            constexpr int kT1 = (KPC - 1) * 2048;
            if (kMirror) {
                const int ob = ((((ks * 4 + kb) * 2 + pq) * 4) + hq) * 16;
                const half8 B0 = *reinterpret_cast<const half8*>(btab + ob);
                const half8 B1 = *reinterpret_cast<const half8*>(btab + kT1 + ob);
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, B0, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, B1, acc1, 0, 0, 0);
            } else {
                const int oh = ((((ks * 4 + kb) * 2 + 0) * 4) + hq) * 16;
                const int ol = ((((ks * 4 + kb) * 2 + 1) * 4) + hq) * 16;
                const half8 Bh0 = *reinterpret_cast<const half8*>(btab + oh);
                const half8 Bl0 = *reinterpret_cast<const half8*>(btab + ol);
                const half8 Bh1 = *reinterpret_cast<const half8*>(btab + kT1 + oh);
                const half8 Bl1 = *reinterpret_cast<const half8*>(btab + kT1 + ol);
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, Bh0, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, Bh1, acc1, 0, 0, 0);
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, Bl0, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, Bl1, acc1, 0, 0, 0);
            }
        }
        if (kMirror) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc0[i] += dpp<0x141>(acc0[i]);  // hi + lo of the head
                acc1[i] += dpp<0x141>(acc1[i]);
            }
        }
        // pool members (attended through their fp16 rows) and evicted tokens
        // are skipped; the same words in every lane
        uint32_t mw = __builtin_amdgcn_readfirstlane(mwv | ewv);
        // G = 16: a last chunk whose second group is not quantized yet (its
        // tokens are in the fp16 ring) has that half masked out
        if (kG16 && tb + 32 > a.n_q) mw |= 0xFFFF0000u;
        float p[8];
        if constexpr (kSplitExp) {
            // This lane's two tokens (slots 2cq, 2cq+1 of its k-block).
            const float a0 = cq & 1 ? acc0[2] : acc0[0], b0 = cq & 1 ? acc1[2] : acc1[0];
            const float a1 = cq & 1 ? acc0[3] : acc0[1], b1 = cq & 1 ? acc1[3] : acc1[1];
            const float bt = cq < 2 ? beta0 : beta1;  // tile 0 or 1
            float s0 = fmaf(cq < 2 ? a0 : b0, kAccW, bt), s1 = fmaf(cq < 2 ? a1 : b1, kAccW, bt);
            if (mw) {
                if ((mw >> own_tok) & 1u) s0 = -INFINITY;
                if ((mw >> (own_tok + 1)) & 1u) s1 = -INFINITY;
            }
            if (a.logits) {
                float* lg = a.logits + ((int64_t)u * R + hq) * a.T + a.sink_cap + tb + own_tok;
                if (s0 != -INFINITY) lg[0] = s0;
                if (s1 != -INFINITY) lg[1] = s1;
            }
            // The wavefront max is only needed when some logit passes the
            // threshold (always on the first chunk, rarely afterwards).
            const float lm = fmaxf(s0, s1);
            if (__any(lm > m_thr)) {
                float cm = fmaxf(lm, row_ror<8>(lm));
                cm = fmaxf(cm, dpp<0x141>(cm));  // row_half_mirror: the head's four columns
                cm = max_x32(max_x16(cm));
                const float mnew = fmaxf(m_run, cm);
                if (__builtin_amdgcn_readfirstlane(m_run != -INFINITY)) {
                    const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
                    // per head h, from lane h (whose logit head is h)
                    const float ah[4] = {readlane(alpha, 0), readlane(alpha, 1), readlane(alpha, 2),
                                         readlane(alpha, 3)};
                    lsum *= alpha;
                    const float az = (lane & 3) == 0   ? ah[0]
                                     : (lane & 3) == 1 ? ah[1]
                                     : (lane & 3) == 2 ? ah[2]
                                                       : ah[3];
                    zc *= az;  // rows j of both value row sets belong to head j % 4
                    zc2 *= az;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int nt = 0; nt < 8; ++nt) O[nt][i] *= ah[i];
                }
                m_run = mnew;
                m_thr = mnew + tau;
            }
            const float mu = m_run == -INFINITY ? 0.f : m_run;
            const float p0 = __builtin_amdgcn_exp2f(s0 - mu), p1 = __builtin_amdgcn_exp2f(s1 - mu);
            lsum += p0 + p1;
            *reinterpret_cast<float2*>(pbuf + hq * 32 + own_tok) = float2{p0, p1};
            wave_lds_fence();
            const float* ph = pbuf + ha * 32;
            const floatx4 pa = *reinterpret_cast<const floatx4*>(ph + 4 * kb);
            const floatx4 pb = *reinterpret_cast<const floatx4*>(ph + 16 + 4 * kb);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = pa[i];
                p[4 + i] = pb[i];
            }
        } else {
            float s[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s[i] = fmaf(acc0[i], kAccW, beta0);
                s[4 + i] = fmaf(acc1[i], kAccW, beta1);
            }
            if (mw) {
#pragma unroll
                for (int sl = 0; sl < 8; ++sl) {
                    const int tok = 16 * (sl / 4) + 4 * kb + sl % 4;
                    if ((mw >> tok) & 1u) s[sl] = -INFINITY;
                }
            }
            if (a.logits && j < R) {
                float* lg = a.logits + ((int64_t)u * R + j) * a.T + a.sink_cap + tb + 4 * kb;
#pragma unroll
                for (int sl = 0; sl < 8; ++sl)
                    if (s[sl] != -INFINITY) lg[16 * (sl / 4) + sl % 4] = s[sl];
            }
            float lm = s[0];
#pragma unroll
            for (int sl = 1; sl < 8; ++sl) lm = fmaxf(lm, s[sl]);
            if (__any(lm > m_thr)) {
                const float cm = max_x32(max_x16(lm));
                const float mnew = fmaxf(m_run, cm);
                if (__builtin_amdgcn_readfirstlane(m_run != -INFINITY)) {
                    const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
                    lsum *= alpha;
                    zc *= alpha;
                    zc2 *= alpha;
                    float ah[4];
                    ah[0] = quad_bcast<0>(alpha);
                    if (R > 1) ah[1] = quad_bcast<1>(alpha);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int nt = 0; nt < 8; ++nt) O[nt][i] *= ah[i % R];
                }
                m_run = mnew;
                m_thr = mnew + tau;
            }
            const float mu = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                p[sl] = __builtin_amdgcn_exp2f(s[sl] - mu);
                lsum += p[sl];
            }
        }

        // Value operand rows (head, value group): hi/lo of p_t * s^V_t. The
        // zero points go to zc = sum_t p_t z^V_t. Value codes enter as fp16
        // subnormals code * 2^(pos - 24), masked in place: every operand of
        // tile nt has the same position, so the tile's sum carries one exact
        // power-of-two weight that the epilogue removes.
        half8 Ahi, Alo, Ahi2, Alo2;
#pragma unroll
        for (int vs = 0; vs < VSETS; ++vs) {
            const u32x4 va = vs == 0 ? vm0 : vm2, vc = vs == 0 ? vm1 : vm3;
            const uint32_t vmw[8] = {va.x, va.y, va.z, va.w, vc.x, vc.y, vc.z, vc.w};
            float z = 0.f;
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) z += p[sl] * h2f(vmw[sl] >> 16);
            (vs == 0 ? zc : zc2) += z;
            uint32_t ahw[4], alw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ahw[i] = mul_pk(p[2 * i], vmw[2 * i], p[2 * i + 1], vmw[2 * i + 1]);
                alw[i] = mul_pk_res(p[2 * i], vmw[2 * i], p[2 * i + 1], vmw[2 * i + 1], ahw[i]);
            }
            (vs == 0 ? Ahi : Ahi2) = as_half8(ahw[0], ahw[1], ahw[2], ahw[3]);
            (vs == 0 ? Alo : Alo2) = as_half8(alw[0], alw[1], alw[2], alw[3]);
        }
        const uint32_t wv[8] = {wv0.x, wv0.y, wv0.z, wv0.w, wv1.x, wv1.y, wv1.z, wv1.w};
        uint32_t wvL4[4], wvR4[4], wvO8[4];
        if (BITS == 2) moved4(wv, wvL4, wvR4, wvO8);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            uint32_t x[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (BITS == 2) {
                    // tile nt at position 3, 4, 1, 2, 5, 6, 7, 0 of word m
                    const uint32_t r = nt < 2 ? wv[m] : nt < 4 ? wvL4[m] : nt < 6 ? wvR4[m] : wvO8[m];
                    x[m] = r & (nt % 2 == 0 ? 0x00C000C0u : 0x03000300u);
                } else {
                    // nibble j of word 4*(nt/4) + m, moved to bits 4-7
                    const uint32_t w = wv[4 * (nt / 4) + m];
                    const int j = nt % 4;
                    const uint32_t r = j == 0 ? w << 4 : j == 1 ? w : j == 2 ? w >> 4 : w >> 8;
                    x[m] = r & 0x00F000F0u;
                }
            }
            const half8 Bv = as_half8(x[0], x[1], x[2], x[3]);
            // tile nt's channels belong to value group nt * 16 / G, in row set
            // (nt * 16 / G) / GPS
            const bool set1 = VSETS == 2 && (nt * 16 / G) / GPS == 1;
            O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(set1 ? Ahi2 : Ahi, Bv, O[nt], 0, 0, 0);
            O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(set1 ? Alo2 : Alo, Bv, O[nt], 0, 0, 0);
        }
    };

    // Pipeline start: the first chunk is requested right after the query row;
    // the wait below is for the query row only, the chunk stays in flight.
    if (n_items > 0) {
        issue(0);
        wait_vm<RG::kLoads>();
    } else {
        wait_vm<0>();
    }
    asm volatile("" : "+v"(qraw));
    {
        // b = 2: this lane's channels (k-step ksb) sit at bits 6-7 (even ksb,
        // weight 2^-18) or 8-9 (odd ksb, 2^-16); the folded query takes 2^2 or
        // 2^0 so that every key product carries 2^-16
        const uint32_t w[4] = {qraw.x, qraw.y, qraw.z, qraw.w};
        const float wq = BITS == 2 && ksb % 2 == 0 ? 4.f * a.qscale : a.qscale;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qv[2 * i] = h2f(w[i] & 0xFFFF) * wq;
            qv[2 * i + 1] = h2f(w[i] >> 16) * wq;
        }
    }
    for (uint32_t k = 0; k < n_items; ++k) {
        // Issue priority from the work left: the arbiter otherwise favours the
        // oldest wavefronts, and the youngest ones finish last, alone.
        const uint32_t left = n_items - k;
        if (left >= 3) __builtin_amdgcn_s_setprio(3);
        else if (left >= 2) __builtin_amdgcn_s_setprio(2);
        else __builtin_amdgcn_s_setprio(1);
        // chunk k + 1 in flight while chunk k computes
        if (k + 1 < n_items) issue(k + 1);
        step(k, n_items - 1 - k);  // stages issued after k: min(1, n_items - 1 - k)
    }
    __builtin_amdgcn_s_setprio(0);
    wave_lds_fence();

    // Wavefront epilogue: per-head l, per-row zero-point totals, outputs to LDS
    // as they sit in the accumulators; the block combine picks the valid rows.
    float lt = lsum;
    if (kSplitExp) {
        lt += row_ror<8>(lt);
        lt += dpp<0x141>(lt);  // row_half_mirror
    }
    lt = sum_x32(sum_x16(lt));
    const float zt = sum_x32(sum_x16(zc));
    const float zt2 = VSETS == 2 ? sum_x32(sum_x16(zc2)) : 0.f;
    // Accumulators as they sit in the registers: tiles 0-5 in the ring, 6-7 in
    // the query table; row totals in the probability buffer.
    float* obuf = wsm;                               // [6][64][4]
    float* obuf2 = reinterpret_cast<float*>(btab);   // [2][64][4]
    float* Zs = pbuf;                                // [2][16] sum_t p z^V per row and set
    float* ms = Zs + 32;                             // [4]
    float* ls = ms + 4;                              // [4]
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
        *reinterpret_cast<floatx4*>((nt < 6 ? obuf + nt * 256 : obuf2 + (nt - 6) * 256) + lane * 4) = O[nt];
    if (kb == 0) {
        Zs[j] = zt;
        Zs[16 + j] = zt2;
        if (j < R) {
            ms[j] = m_run;
            ls[j] = lt;
        }
    }
    __syncthreads();
    // Block combine of the four wavefronts.
    for (int e = threadIdx.x; e < R * D; e += 256) {
        const int h = e / D, c = e % D;
        const int gv = c / G;                       // value group of channel c
        const int ir = h + R * (gv % GPS);          // accumulator row (head, value group)
        const int zi = 16 * (gv / GPS) + ir;        // its zero-point total (row set)
        const int nt = c / 16;
        const int src = ((nt % 6) * 64 + (c % 16) + 16 * (ir / 4)) * 4 + ir % 4;
        // weight of tile nt's code operands: 2^(pos - 24)
        const int pos = BITS == 2 ? (nt % 2 == 0 ? 6 : 8) : 4;
        float mw[4], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            mw[w] = s_pbuf[w][32 + h];
            M = fmaxf(M, mw[w]);
        }
        float o = 0.f, l = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float* ob = nt < 6 ? smem + w * (RG::kWave / 4)
                                         : reinterpret_cast<const float*>(s_btab[w]);
                const float f = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
                o += (ldexpf(ob[src], 24 - pos) + s_pbuf[w][zi]) * f;
                l += s_pbuf[w][36 + h] * f;
            }
        }
        float* rec = a.part + (((int64_t)u * a.splits + split) * R + h) * kRec;
        rec[c] = o;
        if (c == 0) {
            rec[D] = M;
            rec[D + 1] = l;
        }
    }
}

// FP8 E4M3 cache (b = 8): decode over 32-token chunks of E4M3 bytes, 4 KB of
// keys and 4 KB of values each, in the operand order pack8_kernel writes.
// Same block roles, split plan, softmax and partial records as decode_kernel;
// differences: the key scale is one number per KV head, so the query is folded
// (and split into fp16 hi + lo) once per wavefront; codes become exact fp16
// operands with one v_cvt_scalef32_pk_f16_fp8 per pair (every E4M3 value is an
// fp16 value); there are no zero points; the value scale multiplies the
// block's output. A wavefront's chunks are loaded straight into registers one
// chunk ahead ("KV cache quantization and eviction", section "FP8, KIVI and
// KVQuant"; MiniKV, section 4.4: dequantization fused into the attention).
__device__ __forceinline__ half8 fp8x8_to_half8(uint32_t w0, uint32_t w1) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    return half8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

template <int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(R == 4 ? 3 : 2))) void decode8_kernel(DecodeArgs a) {
    constexpr bool kSplitExp = R == 4;
    constexpr bool kMirror = kSplitExp;
    constexpr int kWaveAcc = 8 * 64 * 4;  // floats: a wavefront's output accumulators
    __shared__ __align__(16) float smem[4 * kWaveAcc > kFp16Bytes / 4 ? 4 * kWaveAcc : kFp16Bytes / 4];
    __shared__ __align__(16) float s_pbuf[4][128];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if ((int)blockIdx.x < a.units * a.fp16_tiles) {
        fp16_tile<R>(a, blockIdx.x / a.fp16_tiles, blockIdx.x % a.fp16_tiles, smem);
        return;
    }
    const int idx = blockIdx.x - a.units * a.fp16_tiles;
    const int u = idx / a.splits_q, split = idx % a.splits_q;
    const int b = u / a.n_kv_heads, hk = u % a.n_kv_heads;
    const uint32_t items = (uint32_t)(a.n_q / 32);
    const uint32_t gs0 = (uint32_t)((int64_t)split * items / a.splits_q);
    const uint32_t gs1 = (uint32_t)((int64_t)(split + 1) * items / a.splits_q);
    const uint32_t n_items = gs1 - gs0 > (uint32_t)wave ? (gs1 - gs0 - wave + 3) / 4 : 0;
    const uint4* kq_u = reinterpret_cast<const uint4*>(a.kq) + (int64_t)u * a.chunks * 256;
    const uint4* vq_u = reinterpret_cast<const uint4*>(a.vq) + (int64_t)u * a.chunks * 256;
    const uint32_t* mk_u = a.mask + (int64_t)u * a.chunks;
    const uint32_t* ev_u = a.evict + (int64_t)u * a.evict_words;

    // lane roles as in decode_kernel
    const int j = lane & 15, kb = lane >> 4, jj = j & 7;
    const int hq = kMirror ? (jj < 4 ? jj : 7 - jj) : j % R;
    const int pq = jj < 4 ? 0 : 1;
    const int cq = kMirror ? pq + 2 * (j >> 3) : j >> 2;
    const int ha = j % R;
    const int own_tok = 16 * (cq >> 1) + 4 * kb + 2 * (cq & 1);
    const float sk = __builtin_bit_cast(float, scalar_load(a.fp8_scales + 2 * hk));
    const float sv = __builtin_bit_cast(float, scalar_load(a.fp8_scales + 2 * hk + 1));

    // Folded query, B operand of the key products: column j holds head hq,
    // channels 32 ks + 8 kb .. + 7 of q * log2(e) / sqrt(d) * s_K, fp16 hi
    // (pq = 0) or lo (pq = 1) with kMirror (kept in Bh); both hi (Bh) and lo
    // (Bl) otherwise.
    half8 Bh[4], Bl[4];
    {
        const uint32_t one = 0x3C00u;  // fp16 1.0 in the low half
        const float f = a.qscale * sk;
        const uint4* qr = reinterpret_cast<const uint4*>(
            a.q + ((int64_t)b * a.n_kv_heads * R + hk * R + hq) * D);
        uint4 qw[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qw[ks] = qr[(32 * ks + 8 * kb) / 8];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint32_t w[4] = {qw[ks].x, qw[ks].y, qw[ks].z, qw[ks].w};
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x0 = h2f(w[i] & 0xFFFF) * f, x1 = h2f(w[i] >> 16) * f;
                hi[i] = mul_pk(x0, one, x1, one);
                lo[i] = mul_pk_res(x0, one, x1, one, hi[i]);
            }
            Bh[ks] = kMirror && pq ? as_half8(lo[0], lo[1], lo[2], lo[3])
                                   : as_half8(hi[0], hi[1], hi[2], hi[3]);
            Bl[ks] = as_half8(lo[0], lo[1], lo[2], lo[3]);
        }
    }
    float* pbuf = s_pbuf[wave];
    float m_run = -INFINITY, lsum = 0.f, m_thr = -INFINITY;
    constexpr float tau = 8.f;  // lazy rescale threshold: p < 2^8 in fp16
    floatx4 O[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto load = [&](uint32_t k, uint4 (&kr)[4], uint4 (&vr)[4]) {
        const uint32_t ch = gs0 + wave + 4 * k;
#pragma unroll
        for (int w = 0; w < 4; ++w) kr[w] = kq_u[ch * 256 + w * 64 + lane];
#pragma unroll
        for (int w = 0; w < 4; ++w) vr[w] = vq_u[ch * 256 + w * 64 + lane];
    };
    auto compute = [&](uint32_t k, const uint4 (&kr)[4], const uint4 (&vr)[4]) {
        const uint32_t ch = gs0 + wave + 4 * k;
        const int64_t tb = (int64_t)ch * 32;
        floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint4 r0 = kr[ks / 2], r1 = kr[2 + ks / 2];  // tiles 0 and 1
            const half8 A0 = ks % 2 ? fp8x8_to_half8(r0.z, r0.w) : fp8x8_to_half8(r0.x, r0.y);
            const half8 A1 = ks % 2 ? fp8x8_to_half8(r1.z, r1.w) : fp8x8_to_half8(r1.x, r1.y);
            if (kMirror) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, Bh[ks], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, Bh[ks], acc1, 0, 0, 0);
            } else {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, Bh[ks], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, Bh[ks], acc1, 0, 0, 0);
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, Bl[ks], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, Bl[ks], acc1, 0, 0, 0);
            }
        }
        if (kMirror) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc0[i] += dpp<0x141>(acc0[i]);  // hi + lo of the head
                acc1[i] += dpp<0x141>(acc1[i]);
            }
        }
        // pool members are never set at b = 8; evicted tokens are skipped
        const uint32_t mw = scalar_load(mk_u + ch) | scalar_load(ev_u + ch);
        float p[8];
        if constexpr (kSplitExp) {
            const float a0 = cq & 1 ? acc0[2] : acc0[0], b0 = cq & 1 ? acc1[2] : acc1[0];
            const float a1 = cq & 1 ? acc0[3] : acc0[1], b1 = cq & 1 ? acc1[3] : acc1[1];
            float s0 = cq < 2 ? a0 : b0, s1 = cq < 2 ? a1 : b1;
            if (mw) {
                if ((mw >> own_tok) & 1u) s0 = -INFINITY;
                if ((mw >> (own_tok + 1)) & 1u) s1 = -INFINITY;
            }
            if (a.logits) {
                float* lg = a.logits + ((int64_t)u * R + hq) * a.T + a.sink_cap + tb + own_tok;
                if (s0 != -INFINITY) lg[0] = s0;
                if (s1 != -INFINITY) lg[1] = s1;
            }
            const float lm = fmaxf(s0, s1);
            if (__any(lm > m_thr)) {
                float cm = fmaxf(lm, row_ror<8>(lm));
                cm = fmaxf(cm, dpp<0x141>(cm));
                cm = max_x32(max_x16(cm));
                const float mnew = fmaxf(m_run, cm);
                if (__builtin_amdgcn_readfirstlane(m_run != -INFINITY)) {
                    const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
                    const float ah[4] = {readlane(alpha, 0), readlane(alpha, 1), readlane(alpha, 2),
                                         readlane(alpha, 3)};
                    lsum *= alpha;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int nt = 0; nt < 8; ++nt) O[nt][i] *= ah[i];
                }
                m_run = mnew;
                m_thr = mnew + tau;
            }
            const float mu = m_run == -INFINITY ? 0.f : m_run;
            const float p0 = __builtin_amdgcn_exp2f(s0 - mu), p1 = __builtin_amdgcn_exp2f(s1 - mu);
            lsum += p0 + p1;
            *reinterpret_cast<float2*>(pbuf + hq * 32 + own_tok) = float2{p0, p1};
            wave_lds_fence();
            const float* ph = pbuf + ha * 32;
            const floatx4 pa = *reinterpret_cast<const floatx4*>(ph + 4 * kb);
            const floatx4 pb = *reinterpret_cast<const floatx4*>(ph + 16 + 4 * kb);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = pa[i];
                p[4 + i] = pb[i];
            }
        } else {
            float s[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s[i] = acc0[i];
                s[4 + i] = acc1[i];
            }
            if (mw) {
#pragma unroll
                for (int sl = 0; sl < 8; ++sl) {
                    const int tok = 16 * (sl / 4) + 4 * kb + sl % 4;
                    if ((mw >> tok) & 1u) s[sl] = -INFINITY;
                }
            }
            if (a.logits && j < R) {
                float* lg = a.logits + ((int64_t)u * R + j) * a.T + a.sink_cap + tb + 4 * kb;
#pragma unroll
                for (int sl = 0; sl < 8; ++sl)
                    if (s[sl] != -INFINITY) lg[16 * (sl / 4) + sl % 4] = s[sl];
            }
            float lm = s[0];
#pragma unroll
            for (int sl = 1; sl < 8; ++sl) lm = fmaxf(lm, s[sl]);
            if (__any(lm > m_thr)) {
                const float cm = max_x32(max_x16(lm));
                const float mnew = fmaxf(m_run, cm);
                if (__builtin_amdgcn_readfirstlane(m_run != -INFINITY)) {
                    const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
                    lsum *= alpha;
                    float ah[4];
                    ah[0] = quad_bcast<0>(alpha);
                    if (R > 1) ah[1] = quad_bcast<1>(alpha);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int nt = 0; nt < 8; ++nt) O[nt][i] *= ah[i % R];
                }
                m_run = mnew;
                m_thr = mnew + tau;
            }
            const float mu = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                p[sl] = __builtin_amdgcn_exp2f(s[sl] - mu);
                lsum += p[sl];
            }
        }
        // values: A = fp16 hi / lo of p (rows: head j % r), B = the value codes
        const uint32_t one = 0x3C00u;
        uint32_t ahw[4], alw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ahw[i] = mul_pk(p[2 * i], one, p[2 * i + 1], one);
            alw[i] = mul_pk_res(p[2 * i], one, p[2 * i + 1], one, ahw[i]);
        }
        const half8 Ahi = as_half8(ahw[0], ahw[1], ahw[2], ahw[3]);
        const half8 Alo = as_half8(alw[0], alw[1], alw[2], alw[3]);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const uint4 r = vr[nt / 2];
            const half8 Bv = nt % 2 ? fp8x8_to_half8(r.z, r.w) : fp8x8_to_half8(r.x, r.y);
            O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Bv, O[nt], 0, 0, 0);
            O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Bv, O[nt], 0, 0, 0);
        }
    };
    // two register sets, one chunk ahead
    uint4 kA[4], vA[4], kB[4], vB[4];
    if (n_items > 0) load(0, kA, vA);
    for (uint32_t k = 0; k < n_items; k += 2) {
        if (k + 1 < n_items) load(k + 1, kB, vB);
        compute(k, kA, vA);
        if (k + 1 < n_items) {
            if (k + 2 < n_items) load(k + 2, kA, vA);
            compute(k + 1, kB, vB);
        }
    }

    // Wavefront epilogue, then the block combine of the four wavefronts.
    float lt = lsum;
    if (kSplitExp) {
        lt += row_ror<8>(lt);
        lt += dpp<0x141>(lt);
    }
    lt = sum_x32(sum_x16(lt));
    float* obuf = smem + wave * kWaveAcc;  // [8][64][4] as in the accumulators
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
        *reinterpret_cast<floatx4*>(obuf + nt * 256 + lane * 4) = O[nt];
    if (kb == 0 && j < R) {
        pbuf[32 + j] = m_run;
        pbuf[36 + j] = lt;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < R * D; e += 256) {
        const int h = e / D, c = e % D, nt = c / 16;
        const int src = (nt * 64 + (c % 16) + 16 * (h / 4)) * 4 + h % 4;  // accumulator row h
        float mw[4], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            mw[w] = s_pbuf[w][32 + h];
            M = fmaxf(M, mw[w]);
        }
        float o = 0.f, l = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
                o += smem[w * kWaveAcc + src] * f;
                l += s_pbuf[w][36 + h] * f;
            }
        }
        float* rec = a.part + (((int64_t)u * a.splits + split) * R + h) * kRec;
        rec[c] = o * sv;
        if (c == 0) {
            rec[D] = M;
            rec[D + 1] = l;
        }
    }
}

// Merge of the split partials. Block x serves unit x / r. Blocks y = 0 write
// the outputs of head x % r: wavefront w sums a contiguous quarter of the
// splits, and the four partial sums are added in order, so results do not
// depend on timing. Blocks y >= 1 add the H2O increments of the
// (x % r)-th part of a 2048-token slice.
template <int R>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
    constexpr int kML = 4;  // (m, l) pairs per lane kept in registers
    __shared__ float wsp[kMaxSplits + 1];
    __shared__ float opart[4][D];
    __shared__ float Ms[R], Linv[R];
    const int u = blockIdx.x / R, hb = blockIdx.x % R;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int S = a.splits;
    const float* base = a.part + (int64_t)u * S * R * kRec;
    // Global max and normaliser of head h over all splits; split weights of
    // [s_lo, s_hi) go to wsp.
    auto softmax_terms = [&](int h, int s_lo, int s_hi, float& m, float& l) {
        float mr[kML], lr[kML];
        m = -INFINITY;
#pragma unroll
        for (int j = 0; j < kML; ++j) {
            const int s = lane + 64 * j;
            mr[j] = s < S ? base[(s * R + h) * kRec + D] : -INFINITY;
            lr[j] = s < S ? base[(s * R + h) * kRec + D + 1] : 0.f;
            m = fmaxf(m, mr[j]);
        }
        for (int s = lane + 64 * kML; s < S; s += 64) m = fmaxf(m, base[(s * R + h) * kRec + D]);
        m = wave_max(m);
        l = 0.f;
#pragma unroll
        for (int j = 0; j < kML; ++j) {
            const int s = lane + 64 * j;
            const float f = mr[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mr[j] - m);
            if (s >= s_lo && s < s_hi) wsp[s] = f;
            l += lr[j] * f;
        }
        for (int s = lane + 64 * kML; s < S; s += 64) {
            const float ms = base[(s * R + h) * kRec + D];
            const float f = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - m);
            if (s >= s_lo && s < s_hi) wsp[s] = f;
            l += base[(s * R + h) * kRec + D + 1] * f;
        }
        l = wave_sum(l);
    };
    if (blockIdx.y == 0) {
        const int h = hb;
        const int s_lo = S * wave / 4, s_hi = S * (wave + 1) / 4;
        auto row = [&](int s) {
            return *reinterpret_cast<const float2*>(base + (s * R + h) * kRec + 2 * lane);
        };
        // the range's first rows are requested together with the (m, l) pairs
        constexpr int kPre = 16;
        float2 xp[kPre];
#pragma unroll
        for (int j = 0; j < kPre; ++j) xp[j] = s_lo + j < s_hi ? row(s_lo + j) : make_float2(0.f, 0.f);
        float m, l;
        softmax_terms(h, s_lo, s_hi, m, l);
        wave_lds_fence();  // this wavefront's split weights are in LDS
        // lane owns channels 2 lane, 2 lane + 1
        float o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int j = 0; j < kPre; ++j) {
            const float f = s_lo + j < s_hi ? wsp[s_lo + j] : 0.f;
            o0 += xp[j].x * f;
            o1 += xp[j].y * f;
        }
        for (int s0 = s_lo + kPre; s0 < s_hi; s0 += 16) {
            float2 x[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) x[j] = s0 + j < s_hi ? row(s0 + j) : make_float2(0.f, 0.f);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float f = s0 + j < s_hi ? wsp[s0 + j] : 0.f;
                o0 += x[j].x * f;
                o1 += x[j].y * f;
            }
        }
        *reinterpret_cast<float2*>(&opart[wave][2 * lane]) = make_float2(o0, o1);
        __syncthreads();
        if (wave == 0) {
            float t0 = 0.f, t1 = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                t0 += opart[w][2 * lane];
                t1 += opart[w][2 * lane + 1];
            }
            const float linv = 1.0f / l;
            const int b = u / a.n_kv_heads, hk = u % a.n_kv_heads;
            *reinterpret_cast<float2*>(a.out + ((int64_t)b * a.n_kv_heads * R + hk * R + h) * D + 2 * lane) =
                make_float2(t0 * linv, t1 * linv);
        }
        return;
    }
    if (wave < R) {
        float m, l;
        softmax_terms(wave, 0, 0, m, l);
        if (lane == 0) {
            Ms[wave] = m;
            Linv[wave] = 1.0f / l;
        }
    }
    __syncthreads();
    // H2O increments of this block's part of a 2048-token slice: sum over the
    // r query heads of the normalized probabilities.
    constexpr int kPart = kH2OChunk / R;
    const int64_t t0 = (int64_t)(blockIdx.y - 1) * kH2OChunk + (int64_t)hb * kPart;
    const uint32_t* ev_u = a.evict + (int64_t)u * a.evict_words;
    const bool any_evicted = a.evict_count[u] != 0;
    for (int64_t t = t0 + threadIdx.x; t < t0 + kPart && t < a.T; t += 256) {
        const int64_t tau = t - a.sink_cap;
        if (any_evicted && tau >= 0 && ((ev_u[tau >> 5] >> (tau & 31)) & 1u))
            continue;  // evicted: no score
        float d = 0.f;
#pragma unroll
        for (int h = 0; h < R; ++h)
            d += __builtin_amdgcn_exp2f(a.logits[((int64_t)u * R + h) * a.T + t] - Ms[h]) * Linv[h];
        a.acc[(int64_t)u * a.T + t] += d;
    }
}

// Blocks of decode_kernel<BITS, R, G> resident on the current device at once
// (occupancy x compute units), cached per device.
template <int BITS, int R, int G>
int resident_blocks() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cached[dev] == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per, reinterpret_cast<const void*>(decode_kernel<BITS, R, G>), 256, 0) !=
                hipSuccess)
            cus = per = 0;
        cached[dev] = cus * per > 0 ? cus * per : 512;
    }
    return cached[dev];
}

int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

template <int BITS, int R, int G>
void launch_decode_t(DecodeArgs a, hipEvent_t e0, hipEvent_t e1, hipStream_t s) {
    // fp16 tile rows: the partition's rows (ring tokens plus full pools) over
    // the plan's tile count
    const int64_t fp16_rows = (a.T - a.n_q) + (a.pool > 0 ? (int64_t)a.pool + a.evict_cap : 0);
    a.tile_rows = fp16_rows > 0 ? (int32_t)((fp16_rows + a.fp16_tiles - 1) / a.fp16_tiles) : 1;
    const unsigned blocks = (unsigned)(a.units * a.fp16_tiles + a.units * a.splits_q);
    // the device queries of the plan may have left an error that is not a launch's
    (void)hipGetLastError();
    if (e0 || e1)
        hipExtLaunchKernelGGL((decode_kernel<BITS, R, G>), dim3(blocks), dim3(256), 0, s, e0, e1, 0,
                              a);
    else
        hipLaunchKernelGGL((decode_kernel<BITS, R, G>), dim3(blocks), dim3(256), 0, s, a);
    const unsigned ny = 1 + (a.acc ? (unsigned)((a.T + kH2OChunk - 1) / kH2OChunk) : 0u);
    hipLaunchKernelGGL((merge_kernel<R>), dim3(a.units * R, ny), dim3(256), 0, s, a);
}

template <int R>
int resident8_blocks() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cached[dev] == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per, reinterpret_cast<const void*>(decode8_kernel<R>), 256, 0) != hipSuccess)
            cus = per = 0;
        cached[dev] = cus * per > 0 ? cus * per : 512;
    }
    return cached[dev];
}

template <int R>
void launch_decode8_t(DecodeArgs a, hipEvent_t e0, hipEvent_t e1, hipStream_t s) {
    const int64_t fp16_rows = (a.T - a.n_q) + (a.pool > 0 ? (int64_t)a.pool + a.evict_cap : 0);
    a.tile_rows = fp16_rows > 0 ? (int32_t)((fp16_rows + a.fp16_tiles - 1) / a.fp16_tiles) : 1;
    const unsigned blocks = (unsigned)(a.units * a.fp16_tiles + a.units * a.splits_q);
    (void)hipGetLastError();  // the device queries of the plan may have left an error
    if (e0 || e1)
        hipExtLaunchKernelGGL((decode8_kernel<R>), dim3(blocks), dim3(256), 0, s, e0, e1, 0, a);
    else
        hipLaunchKernelGGL((decode8_kernel<R>), dim3(blocks), dim3(256), 0, s, a);
    const unsigned ny = 1 + (a.acc ? (unsigned)((a.T + kH2OChunk - 1) / kH2OChunk) : 0u);
    hipLaunchKernelGGL((merge_kernel<R>), dim3(a.units * R, ny), dim3(256), 0, s, a);
}

template <int BITS, int R>
void dispatch_g(const DecodeArgs& a, int G, hipEvent_t e0, hipEvent_t e1, hipStream_t s) {
    if (G == 16) launch_decode_t<BITS, R, 16>(a, e0, e1, s);
    else if (G == 32) launch_decode_t<BITS, R, 32>(a, e0, e1, s);
    else if (G == 64) launch_decode_t<BITS, R, 64>(a, e0, e1, s);
    else launch_decode_t<BITS, R, 128>(a, e0, e1, s);
}

template <int BITS>
void dispatch_r(const DecodeArgs& a, int R, int G, hipEvent_t e0, hipEvent_t e1, hipStream_t s) {
    if (R == 1) dispatch_g<BITS, 1>(a, G, e0, e1, s);
    else if (R == 2) dispatch_g<BITS, 2>(a, G, e0, e1, s);
    else dispatch_g<BITS, 4>(a, G, e0, e1, s);
}

template <int BITS, int R>
int resident_g(int G) {
    return G == 16   ? resident_blocks<BITS, R, 16>()
           : G == 32 ? resident_blocks<BITS, R, 32>()
           : G == 64 ? resident_blocks<BITS, R, 64>()
                     : resident_blocks<BITS, R, 128>();
}

}  // namespace

void decode_launch_shape(int bits, int r, int group, int* cus, int* resident) {
    *cus = cu_count();
    if (bits == 8)
        *resident = r == 1 ? resident8_blocks<1>() : r == 2 ? resident8_blocks<2>()
                                                            : resident8_blocks<4>();
    else if (bits == 2)
        *resident = r == 1 ? resident_g<2, 1>(group) : r == 2 ? resident_g<2, 2>(group)
                                                              : resident_g<2, 4>(group);
    else
        *resident = r == 1 ? resident_g<4, 1>(group) : r == 2 ? resident_g<4, 2>(group)
                                                              : resident_g<4, 4>(group);
}

// Workspace of kvq_decode_attention_noalloc: a file-scope device array, one
// copy per GPU. Host code never uses this name as an address (on the host it
// is only a stand-in); it uses the device address hipGetSymbolAddress returns
// for the current GPU.
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

void* noalloc_scratch(int* err) {
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        *err = e != hipSuccess ? (int)e : (int)hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            *err = e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
            return nullptr;
        }
        addr[dev] = p;
    }
    *err = 0;
    return addr[dev];
}

int launch_decode(const CacheView& v, int64_t T, int64_t n_q, const DecodePlan& plan,
                  const uint16_t* q, float* out, float* acc, void* ws, void* ev_start,
                  void* ev_stop, void* stream, const uint16_t* k_new, const uint16_t* v_new) {
    if (plan.splits > kMaxSplits) return (int)hipErrorInvalidValue;
    DecodeArgs a{};
    a.kq = v.kq;
    a.vq = v.vq;
    a.kmeta = v.kmeta;
    a.vmeta = v.vmeta;
    a.mask = v.mask;
    a.kring = v.kring;
    a.vring = v.vring;
    a.pool_idx = v.pool_idx;
    a.pool_k = v.pool_k;
    a.pool_v = v.pool_v;
    a.ev_idx = v.ev_idx;
    a.ev_k = v.ev_k;
    a.ev_v = v.ev_v;
    a.counters = v.counters;
    a.evict = v.evict;
    a.evict_count = v.evict_count;
    a.evict_words = v.evict_words;
    a.sink_k = v.sink_k;
    a.sink_v = v.sink_v;
    a.sink_cap = v.sinks;
    a.sink_rows = (int32_t)(T < v.sinks ? T : v.sinks);
    a.k_new = k_new;
    a.v_new = v_new;
    a.q = q;
    a.part = static_cast<float*>(ws);
    a.logits = acc ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                              (plan.ws_bytes - (size_t)plan.logit_floats * 4))
                   : nullptr;
    a.out = out;
    a.acc = acc;
    a.T = T;
    a.n_q = n_q;
    a.chunks = v.chunks;
    a.key_groups = v.key_groups;
    a.units = v.units;
    a.n_kv_heads = v.n_kv_heads;
    a.ring_slots = v.ring_slots;
    a.splits_q = plan.splits_q;
    a.splits = plan.splits;
    a.fp16_tiles = plan.fp16_tiles;
    a.pool = v.pool;
    a.evict_cap = v.evict_cap;
    a.qscale = 1.4426950408889634f / sqrtf((float)kHeadDim);
    const int R = v.n_q_heads / v.n_kv_heads;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t e0 = static_cast<hipEvent_t>(ev_start), e1 = static_cast<hipEvent_t>(ev_stop);
    a.fp8_scales = v.fp8_scales;
    if (v.bits == 8) {
        if (R == 1) launch_decode8_t<1>(a, e0, e1, s);
        else if (R == 2) launch_decode8_t<2>(a, e0, e1, s);
        else launch_decode8_t<4>(a, e0, e1, s);
    } else if (v.bits == 2) {
        dispatch_r<2>(a, R, v.group, e0, e1, s);
    } else {
        dispatch_r<4>(a, R, v.group, e0, e1, s);
    }
    return (int)hipGetLastError();
}

}  // namespace kvq

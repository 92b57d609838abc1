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

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;
constexpr int kRec = D + 2;  // partial record: o[d], m, l
constexpr int kMaxSplits = 1056;
constexpr int kH2OChunk = 2048;
constexpr int kWaveFloats = 1024;  // per-wavefront LDS of the quantized path (4 KB)
// LDS of one block: the fp16 partition's K/V tiles, queries and probabilities
// (64 rows x 2 x 256 B + 4 x 256 B + 4 x 256 B), or 4 wavefronts x 4 KB.
constexpr int kSmemFloats = (64 * D * 2 * 2 + 4 * D * 2 + 4 * 64 * 4) / 4;
static_assert(kSmemFloats >= 4 * kWaveFloats, "LDS layout");

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
    const uint16_t* q;
    float* part;
    float* logits;
    float* out;
    float* acc;
    int64_t T, n_q, chunks, key_groups;
    int32_t units, n_kv_heads, ring_slots, splits_q, splits, fp16_tiles, pool, evict_cap;
    float qscale;  // log2(e) / sqrt(d)
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

__device__ __forceinline__ void wave_lds_fence() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

// One 64-row tile of the fp16 partition of unit u: rows are the residual
// ring tokens [n_q, T), then the pool members, then the extra-pool members.
// The block stages the tile's K and V rows in LDS; wavefront h < r then takes
// query head h (one token per lane for the logits, two channels per lane for
// the outputs) and writes one partial record.
template <int R>
__device__ void fp16_tile(const DecodeArgs& a, int u, int tile, float* smem) {
    const int tid = threadIdx.x, lane = tid & 63, h = tid >> 6;
    uint16_t* kt = reinterpret_cast<uint16_t*>(smem);  // [64][D] fp16
    uint16_t* vt = kt + 64 * D;                         // [64][D] fp16
    uint32_t* qh = reinterpret_cast<uint32_t*>(vt + 64 * D);  // [R][D/2] fp16 pairs
    float* ps = reinterpret_cast<float*>(qh + R * D / 2);     // [R][64]
    const int b = u / a.n_kv_heads, hk = u % a.n_kv_heads;
    const uint32_t* qsrc =
        reinterpret_cast<const uint32_t*>(a.q + ((int64_t)b * a.n_kv_heads * R + hk * R) * D);
    for (int e = tid; e < R * D / 2; e += 256) qh[e] = qsrc[e];
    const int64_t nres = a.T - a.n_q;
    const int pc = a.pool > 0 ? a.counters[(int64_t)u * 4] : 0;
    const int ec = a.pool > 0 ? a.counters[(int64_t)u * 4 + 1] : 0;
    const int64_t ntot = nres + pc + ec;
    const int N = a.pool, E = a.evict_cap, RB = a.ring_slots;
    const int64_t base = (int64_t)tile * 64;
    const int cnt = (int)(ntot - base < 0 ? 0 : ntot - base < 64 ? ntot - base : 64);
    auto row_of = [&](int64_t li, const uint16_t* ring, const uint16_t* pool,
                      const uint16_t* ev) -> const uint16_t* {
        if (li < nres) return ring + ((int64_t)u * RB + (a.n_q + li) % RB) * D;
        if (li < nres + pc) return pool + ((int64_t)u * N + (li - nres)) * D;
        return ev + ((int64_t)u * E + (li - nres - pc)) * D;
    };
    for (int e = tid; e < cnt * 16; e += 256) {
        const int i = e / 16, part = e % 16;
        reinterpret_cast<uint4*>(kt)[e] =
            reinterpret_cast<const uint4*>(row_of(base + i, a.kring, a.pool_k, a.ev_k))[part];
        reinterpret_cast<uint4*>(vt)[e] =
            reinterpret_cast<const uint4*>(row_of(base + i, a.vring, a.pool_v, a.ev_v))[part];
    }
    __syncthreads();
    if (h >= R) return;
    float s = -INFINITY;
    if (lane < cnt) {
        // fp16 x fp16 products are exact in the fp32 dot2 accumulation
        float acc = 0.f;
        const uint32_t* qr = qh + h * (D / 2);
#pragma unroll
        for (int c8 = 0; c8 < D / 8; ++c8) {
            const int cx = (c8 + lane) & 15;  // rotate to spread LDS banks
            const uint4 x = reinterpret_cast<const uint4*>(kt + lane * D)[cx];
            const uint4 y = reinterpret_cast<const uint4*>(qr)[cx];
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, x.x),
                                         __builtin_bit_cast(half2_t, y.x), acc, false);
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, x.y),
                                         __builtin_bit_cast(half2_t, y.y), acc, false);
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, x.z),
                                         __builtin_bit_cast(half2_t, y.z), acc, false);
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, x.w),
                                         __builtin_bit_cast(half2_t, y.w), acc, false);
        }
        s = acc * a.qscale;
        if (a.logits) {
            const int64_t li = base + lane;
            const int64_t t = li < nres ? a.n_q + li
                              : li < nres + pc ? a.pool_idx[(int64_t)u * N + (li - nres)]
                                               : a.ev_idx[(int64_t)u * E + (li - nres - pc)];
            a.logits[((int64_t)u * R + h) * a.T + t] = s;
        }
    }
    const float m = cnt > 0 ? wave_max(s) : -INFINITY;
    const float p = s == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s - m);
    const float l = wave_sum(p);
    ps[h * 64 + lane] = p;
    wave_lds_fence();
    float o0 = 0.f, o1 = 0.f;
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(vt) + lane;
    for (int i = 0; i < cnt; ++i) {
        const uint32_t w = vw[i * (D / 2)];
        const float pi = ps[h * 64 + i];
        o0 += pi * h2f(w & 0xFFFF);
        o1 += pi * h2f(w >> 16);
    }
    float* rec = a.part + (((int64_t)u * a.splits + a.splits_q + tile) * R + h) * kRec;
    rec[2 * lane] = o0;
    rec[2 * lane + 1] = o1;
    if (lane == 0) {
        rec[D] = m;
        rec[D + 1] = l;
    }
}

// Per-lane data of one 32-token chunk (and, at the first chunk of a key
// group, the lane's eight key scale/zero pairs), loaded one chunk ahead.
struct Chunk {
    u32x4 km0, km1;  // key (scale, zero) of channels cb0 .. cb0+7
    u32x4 wk0, wk1;  // packed key codes (second half only for 4-bit)
    u32x4 wv0, wv1;  // packed value codes
    u32x4 vm0, vm1;  // value (scale, zero) of the lane's 8 token slots
    uint32_t mw;     // pool mask of the chunk (wave-uniform)
};

template <int BITS, int R, int G>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    constexpr int NG = D / G;        // value groups per token
    constexpr int CPG = G / 32;      // chunks per key group
    constexpr int WPC = 128 * BITS;  // words per chunk
    constexpr float F = (float)(1 << BITS);
    // Codes become fp16 operands F + code with two bit operations; the masks
    // live in VGPRs so that the pair becomes one v_and_or_b32.
    constexpr uint32_t kMagicC = BITS == 2 ? 0x44004400u : 0x4C004C00u;
    constexpr uint32_t kMaskC = BITS == 2 ? 0x03000300u : 0x03C003C0u;
    __shared__ __align__(16) float smem[kSmemFloats];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if ((int)blockIdx.x < a.units * a.fp16_tiles) {
        fp16_tile<R>(a, blockIdx.x / a.fp16_tiles, blockIdx.x % a.fp16_tiles, smem);
        return;
    }
    uint32_t vmask, vmagic;
    asm volatile("v_mov_b32 %0, %1" : "=v"(vmask) : "i"(kMaskC));
    asm volatile("v_mov_b32 %0, %1" : "=v"(vmagic) : "i"(kMagicC));
    auto cvt = [&](uint32_t w, int sh) -> uint32_t {  // sh > 0: left shift
        const uint32_t x = sh >= 0 ? (w << sh) : (w >> -sh);
        return (x & vmask) | vmagic;
    };

    const int idx = blockIdx.x - a.units * a.fp16_tiles;
    const int u = idx / a.splits_q, split = idx % a.splits_q;
    const int b = u / a.n_kv_heads, hk = u % a.n_kv_heads;
    const int64_t groups = a.n_q / G;
    const int64_t gs0 = split * groups / a.splits_q, gs1 = (split + 1) * groups / a.splits_q;
    const int64_t my_groups = gs1 - gs0 > wave ? (gs1 - gs0 - wave + 3) / 4 : 0;
    const int64_t n_items = my_groups * CPG;

    // MFMA lane roles: j = column / row within a 16-lane row, kb = k-block.
    const int j = lane & 15, kb = lane >> 4;
    // Query-fold role: head hb, channels cb0 .. cb0+7 (k-step ksb, k-block kbb).
    const int hb = lane % R, kap = (lane >> 2) & 15, ksb = kap >> 2, kbb = kap & 3;
    const int cb0 = 32 * ksb + 8 * kbb;
    // Softmax / value-operand role: row j = (head j % R, value group gs).
    const int gs = (j / R) % NG;

    float qv[8];
    {
        const uint16_t* qrow = a.q + ((int64_t)b * a.n_kv_heads * R + hk * R + hb) * D + cb0;
        const uint4 x = *reinterpret_cast<const uint4*>(qrow);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qv[2 * i] = h2f(w[i] & 0xFFFF) * a.qscale;
            qv[2 * i + 1] = h2f(w[i] >> 16) * a.qscale;
        }
    }

    auto load = [&](int64_t k, Chunk& c) {
        const int64_t gi = gs0 + wave + 4 * (k / CPG);
        const int cc = (int)(k % CPG);
        const int64_t ch = gi * CPG + cc;
        if (cc == 0) {
            const uint32_t* km = a.kmeta + ((int64_t)u * a.key_groups + gi) * D + cb0;
            c.km0 = *reinterpret_cast<const u32x4*>(km);
            c.km1 = *reinterpret_cast<const u32x4*>(km + 4);
        }
        const uint32_t* kc = a.kq + ((int64_t)u * a.chunks + ch) * WPC;
        const uint32_t* vc = a.vq + ((int64_t)u * a.chunks + ch) * WPC;
        c.wk0 = *reinterpret_cast<const u32x4*>(kc + lane * 4);
        c.wv0 = *reinterpret_cast<const u32x4*>(vc + lane * 4);
        if (BITS == 4) {
            c.wk1 = *reinterpret_cast<const u32x4*>(kc + 256 + lane * 4);
            c.wv1 = *reinterpret_cast<const u32x4*>(vc + 256 + lane * 4);
        }
        const uint32_t* vm = a.vmeta + (((int64_t)u * a.chunks + ch) * NG + gs) * 32 + 4 * kb;
        c.vm0 = *reinterpret_cast<const u32x4*>(vm);
        c.vm1 = *reinterpret_cast<const u32x4*>(vm + 16);
        c.mw = a.pool > 0 ? a.mask[(int64_t)u * a.chunks + ch] : 0u;
    };

    unsigned char* btab = reinterpret_cast<unsigned char*>(smem + wave * kWaveFloats);
    float m_run = -INFINITY, lsum = 0.f, zc = 0.f, beta = 0.f;
    floatx4 O[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};

    Chunk cur, nxt;
    if (n_items > 0) load(0, nxt);
    for (int64_t k = 0; k < n_items; ++k) {
        cur = nxt;
        if (k + 1 < n_items) load(k + 1, nxt);
        const int64_t gi = gs0 + wave + 4 * (k / CPG);
        const int cc = (int)(k % CPG);
        const int64_t tb = (gi * CPG + cc) * 32;
        if (cc == 0) {
            // Fold the key scale into the query: B = hi/lo of q~_c * s_c, and
            // the zero point into beta_h = sum_c q~_c (z_c - 2^b s_c).
            wave_lds_fence();  // previous group's B reads are done
            const uint32_t kmw[8] = {cur.km0.x, cur.km0.y, cur.km0.z, cur.km0.w,
                                     cur.km1.x, cur.km1.y, cur.km1.z, cur.km1.w};
            uint32_t hiw[4], low[4];
            float bp = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hiw[i] = mul_pk(qv[2 * i], kmw[2 * i], qv[2 * i + 1], kmw[2 * i + 1]);
                low[i] = mul_pk_res(qv[2 * i], kmw[2 * i], qv[2 * i + 1], kmw[2 * i + 1], hiw[i]);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float sk = h2f(kmw[i] & 0xFFFF), zk = h2f(kmw[i] >> 16);
                bp += qv[i] * (zk - F * sk);
            }
            unsigned char* e0 = btab + ((((ksb * 4 + kbb) * 2) * 4) + hb) * 16;
            *reinterpret_cast<u32x4*>(e0) = u32x4{hiw[0], hiw[1], hiw[2], hiw[3]};
            *reinterpret_cast<u32x4*>(e0 + 4 * 16) = u32x4{low[0], low[1], low[2], low[3]};
            bp += row_ror<8>(bp);
            bp += row_ror<4>(bp);
            bp += __shfl_xor(bp, 16);
            bp += __shfl_xor(bp, 32);
            beta = bp;
            wave_lds_fence();
        }

        // Logits S^T[token][(head, g)] on the matrix cores: two 16-token tiles,
        // K = 128 channels x {hi, lo}.
        const uint32_t wk[8] = {cur.wk0.x, cur.wk0.y, cur.wk0.z, cur.wk0.w,
                                cur.wk1.x, cur.wk1.y, cur.wk1.z, cur.wk1.w};
        floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            half8 A0, A1;
            if (BITS == 2) {
                const uint32_t w0 = wk[ks / 2], w1 = wk[2 + ks / 2];
                const int q0 = (ks % 2) * 4;
                A0 = as_half8(cvt(w0, 8 - 2 * q0), cvt(w0, 6 - 2 * q0), cvt(w0, 4 - 2 * q0),
                              cvt(w0, 2 - 2 * q0));
                A1 = as_half8(cvt(w1, 8 - 2 * q0), cvt(w1, 6 - 2 * q0), cvt(w1, 4 - 2 * q0),
                              cvt(w1, 2 - 2 * q0));
            } else {
                const uint32_t w0 = wk[ks], w1 = wk[4 + ks];
                A0 = as_half8(cvt(w0, 6), cvt(w0, 2), cvt(w0, -2), cvt(w0, -6));
                A1 = as_half8(cvt(w1, 6), cvt(w1, 2), cvt(w1, -2), cvt(w1, -6));
            }
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const half8 B = *reinterpret_cast<const half8*>(
                    btab + ((((ks * 4 + kb) * 2 + x) * 4) + (j % R)) * 16);
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, B, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, B, acc1, 0, 0, 0);
            }
        }
        float s[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = acc0[i] + beta;
            s[4 + i] = acc1[i] + beta;
        }
        const uint32_t mw = __builtin_amdgcn_readfirstlane(cur.mw);  // same word in every lane
        if (mw) {
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                const int tok = 16 * (sl / 4) + 4 * kb + sl % 4;
                if ((mw >> tok) & 1u) s[sl] = -INFINITY;
            }
        }
        if (a.logits && j < R) {
            float* lg = a.logits + ((int64_t)u * R + j) * a.T + tb + 4 * kb;
            if (!mw) {
                *reinterpret_cast<floatx4*>(lg) = floatx4{s[0], s[1], s[2], s[3]};
                *reinterpret_cast<floatx4*>(lg + 16) = floatx4{s[4], s[5], s[6], s[7]};
            } else {
#pragma unroll
                for (int sl = 0; sl < 8; ++sl) {
                    const int tok = 16 * (sl / 4) + 4 * kb + sl % 4;
                    if (!((mw >> tok) & 1u)) lg[16 * (sl / 4) + sl % 4] = s[sl];
                }
            }
        }

        // Online softmax (log2 units); rescale only when the running max grows.
        float cm = s[0];
#pragma unroll
        for (int sl = 1; sl < 8; ++sl) cm = fmaxf(cm, s[sl]);
        cm = fmaxf(cm, __shfl_xor(cm, 16));
        cm = fmaxf(cm, __shfl_xor(cm, 32));
        const float mnew = fmaxf(m_run, cm);
        if (__any(mnew > m_run)) {
            const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mnew);
            lsum *= alpha;
            zc *= alpha;
            float ah[4];
            ah[0] = quad_bcast<0>(alpha);
            if (R > 1) ah[1] = quad_bcast<1>(alpha);
            if (R > 2) {
                ah[2] = quad_bcast<2>(alpha);
                ah[3] = quad_bcast<3>(alpha);
            }
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) O[nt][i] *= ah[i % R];
            m_run = mnew;
        }
        const float mu = m_run == -INFINITY ? 0.f : m_run;

        // Value operand rows (head, value group): hi/lo of p_t * s^V_t; the
        // offsets go to zc = sum_t p_t (z^V_t - 2^b s^V_t).
        const uint32_t vmw[8] = {cur.vm0.x, cur.vm0.y, cur.vm0.z, cur.vm0.w,
                                 cur.vm1.x, cur.vm1.y, cur.vm1.z, cur.vm1.w};
        float p[8];
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            p[sl] = __builtin_amdgcn_exp2f(s[sl] - mu);
            lsum += p[sl];
            const float sv = h2f(vmw[sl] & 0xFFFF), zv = h2f(vmw[sl] >> 16);
            zc += p[sl] * (zv - F * sv);
        }
        uint32_t ahw[4], alw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ahw[i] = mul_pk(p[2 * i], vmw[2 * i], p[2 * i + 1], vmw[2 * i + 1]);
            alw[i] = mul_pk_res(p[2 * i], vmw[2 * i], p[2 * i + 1], vmw[2 * i + 1], ahw[i]);
        }
        const half8 Ahi = as_half8(ahw[0], ahw[1], ahw[2], ahw[3]);
        const half8 Alo = as_half8(alw[0], alw[1], alw[2], alw[3]);
        const uint32_t wv[8] = {cur.wv0.x, cur.wv0.y, cur.wv0.z, cur.wv0.w,
                                cur.wv1.x, cur.wv1.y, cur.wv1.z, cur.wv1.w};
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            half8 Bv;
            if (BITS == 2) {
                const uint32_t w = wv[nt / 2];
                const int q0 = (nt % 2) * 4;
                Bv = as_half8(cvt(w, 8 - 2 * q0), cvt(w, 6 - 2 * q0), cvt(w, 4 - 2 * q0),
                              cvt(w, 2 - 2 * q0));
            } else {
                const uint32_t w = wv[nt];
                Bv = as_half8(cvt(w, 6), cvt(w, 2), cvt(w, -2), cvt(w, -6));
            }
            O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Bv, O[nt], 0, 0, 0);
            O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Bv, O[nt], 0, 0, 0);
        }
    }
    wave_lds_fence();

    // Wavefront epilogue: l per head, value corrections per row, outputs to LDS.
    float lt = lsum;
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    float zt = zc;
    zt += __shfl_xor(zt, 16);
    zt += __shfl_xor(zt, 32);
    float* ws = smem + wave * kWaveFloats;  // [R][D] outputs, then Z[16], m[4], l[4]
    float* Zs = ws + R * D;
    float* ms = Zs + 16;
    float* ls = ms + 4;
    if (kb == 0) {
        Zs[j] = zt;
        if (j < R) {
            ms[j] = m_run;
            ls[j] = lt;
        }
    }
    wave_lds_fence();
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ir = 4 * kb + i;
            const int c = 16 * nt + j;
            if (ir / R == c / G) ws[(ir % R) * D + c] = O[nt][i] + Zs[ir];
        }
    __syncthreads();
    // Block combine of the four wavefronts.
    for (int e = threadIdx.x; e < R * D; e += 256) {
        const int h = e / D, c = e % D;
        float mw[4], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            mw[w] = smem[w * kWaveFloats + R * D + 16 + h];
            M = fmaxf(M, mw[w]);
        }
        float o = 0.f, l = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
                o += smem[w * kWaveFloats + h * D + c] * f;
                l += smem[w * kWaveFloats + R * D + 20 + h] * f;
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

// Merge the split partials of unit blockIdx.x: block y = 0 writes the
// outputs, blocks y >= 1 add the H2O increments of a 2048-token slice.
template <int R>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
    __shared__ float wsp[R][kMaxSplits + 1];
    __shared__ float Ms[R], Linv[R];
    const int u = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int S = a.splits;
    const float* base = a.part + (int64_t)u * S * R * kRec;
    if (wave < R) {
        const int h = wave;
        float m = -INFINITY;
        for (int s = lane; s < S; s += 64) m = fmaxf(m, base[(s * R + h) * kRec + D]);
        m = wave_max(m);
        float l = 0.f;
        for (int s = lane; s < S; s += 64) {
            const float ms = base[(s * R + h) * kRec + D];
            const float f = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - m);
            wsp[h][s] = f;
            l += base[(s * R + h) * kRec + D + 1] * f;
        }
        l = wave_sum(l);
        if (lane == 0) {
            Ms[h] = m;
            Linv[h] = 1.0f / l;
        }
    }
    __syncthreads();
    if (blockIdx.y == 0) {
        const int b = u / a.n_kv_heads, hk = u % a.n_kv_heads;
        for (int e = threadIdx.x; e < R * D; e += 256) {
            const int h = e / D, c = e % D;
            float o = 0.f;
            for (int s = 0; s < S; ++s) o += base[(s * R + h) * kRec + c] * wsp[h][s];
            a.out[((int64_t)b * a.n_kv_heads * R + hk * R + h) * D + c] = o * Linv[h];
        }
    } else {
        const int64_t t0 = (int64_t)(blockIdx.y - 1) * kH2OChunk;
        for (int64_t t = t0 + threadIdx.x; t < t0 + kH2OChunk && t < a.T; t += 256) {
            float d = 0.f;
#pragma unroll
            for (int h = 0; h < R; ++h)
                d += __builtin_amdgcn_exp2f(a.logits[((int64_t)u * R + h) * a.T + t] - Ms[h]) * Linv[h];
            a.acc[(int64_t)u * a.T + t] += d;
        }
    }
}

template <int BITS, int R, int G>
void launch_decode_t(const DecodeArgs& a, hipEvent_t e0, hipEvent_t e1, hipStream_t s) {
    const unsigned blocks = (unsigned)(a.units * a.fp16_tiles + a.units * a.splits_q);
    if (e0 || e1)
        hipExtLaunchKernelGGL((decode_kernel<BITS, R, G>), dim3(blocks), dim3(256), 0, s, e0, e1, 0,
                              a);
    else
        hipLaunchKernelGGL((decode_kernel<BITS, R, G>), dim3(blocks), dim3(256), 0, s, a);
    const unsigned ny = 1 + (a.acc ? (unsigned)((a.T + kH2OChunk - 1) / kH2OChunk) : 0u);
    hipLaunchKernelGGL((merge_kernel<R>), dim3(a.units, ny), dim3(256), 0, s, a);
}

template <int BITS, int R>
void dispatch_g(const DecodeArgs& a, int G, hipEvent_t e0, hipEvent_t e1, hipStream_t s) {
    if (G == 32) launch_decode_t<BITS, R, 32>(a, e0, e1, s);
    else if (G == 64) launch_decode_t<BITS, R, 64>(a, e0, e1, s);
    else launch_decode_t<BITS, R, 128>(a, e0, e1, s);
}

template <int BITS>
void dispatch_r(const DecodeArgs& a, int R, int G, hipEvent_t e0, hipEvent_t e1, hipStream_t s) {
    if (R == 1) dispatch_g<BITS, 1>(a, G, e0, e1, s);
    else if (R == 2) dispatch_g<BITS, 2>(a, G, e0, e1, s);
    else dispatch_g<BITS, 4>(a, G, e0, e1, s);
}

}  // namespace

int launch_decode(const CacheView& v, int64_t T, int64_t n_q, const DecodePlan& plan,
                  const uint16_t* q, float* out, float* acc, void* ws, void* ev_start,
                  void* ev_stop, void* stream) {
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
    if (v.bits == 2) dispatch_r<2>(a, R, v.group, e0, e1, s);
    else dispatch_r<4>(a, R, v.group, e0, e1, s);
    return (int)hipGetLastError();
}

}  // namespace kvq

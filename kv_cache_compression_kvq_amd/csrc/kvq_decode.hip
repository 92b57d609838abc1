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
//  * blocks [0, U): the fp16 partition of each unit (ring + pools);
//  * blocks [U, U + U*S): split-K over the quantized tokens. Each wavefront
//    takes whole key groups. Per key group the key scale is folded into the
//    query, q~_c = q_c * s_c * 2^b (split into fp16 hi + lo), and the zero
//    point into one scalar per head; the per-token dot products then run on
//    the matrix cores (v_mfma_f32_16x16x32_f16) against the raw codes, which
//    become fp16 operands 1 + code/2^b with two bit operations. Values go the
//    same way with p_j * s^V_j * 2^b as the fp16 hi + lo operand. Online
//    softmax in log2 units; partial (o, m, l) per block.
// Kernel 2 (merge_kernel): combines the partials into out and, when asked,
// adds the normalized probabilities of every token, summed over the query
// heads of the KV head, into the H2O accumulator ("H2O: Heavy-Hitter Oracle",
// accumulated attention; "KV cache quantization and eviction", section
// "Heavy hitters").
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = kHeadDim;
constexpr int kRec = D + 2;  // partial record: o[d], m, l
constexpr int kMaxSplits = 1024;
constexpr int kH2OChunk = 2048;

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
    int32_t units, n_kv_heads, ring_slots, splits_q, splits, pool, evict_cap;
    float qscale;  // log2(e) / sqrt(d)
};

__device__ __forceinline__ float h2f(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t hbits(_Float16 x) { return __builtin_bit_cast(uint16_t, x); }

// Codes of a pair slot -> two fp16 operands 1 + code / 2^b (exact).
// b = 2: the pair sits at bits (2q, 16 + 2q) of the word.
__device__ __forceinline__ uint32_t cvt2(uint32_t w, int q) {
    const uint32_t x = q <= 4 ? (w << (8 - 2 * q)) : (w >> (2 * q - 8));
    return (x & 0x03000300u) | 0x3C003C00u;
}
// b = 4: the pair sits at bits (4m, 16 + 4m).
__device__ __forceinline__ uint32_t cvt4(uint32_t w, int m) {
    const uint32_t x = m <= 1 ? (w << (6 - 4 * m)) : (w >> (4 * m - 6));
    return (x & 0x03C003C0u) | 0x3C003C00u;
}

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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ void wave_lds_fence() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

// fp16 partition of unit u: residual ring tokens [n_q, T), then pool members,
// then extra-pool members. One wavefront per query head, 64 tokens at a time.
template <int R>
__device__ void fp16_partition(const DecodeArgs& a, int u, float* smem) {
    const int lane = threadIdx.x & 63, h = threadIdx.x >> 6;
    if (h >= R) return;
    const int b = u / a.n_kv_heads, hk = u % a.n_kv_heads;
    const int hq = hk * R + h;
    float* qs = smem + h * (D + 64);
    float* ps = qs + D;
    const uint16_t* qrow = a.q + ((int64_t)b * a.n_kv_heads * R + hq) * D;
    qs[2 * lane] = h2f(qrow[2 * lane]) * a.qscale;
    qs[2 * lane + 1] = h2f(qrow[2 * lane + 1]) * a.qscale;
    const int64_t nres = a.T - a.n_q;
    const int pc = a.pool > 0 ? a.counters[(int64_t)u * 4] : 0;
    const int ec = a.pool > 0 ? a.counters[(int64_t)u * 4 + 1] : 0;
    const int64_t ntot = nres + pc + ec;
    const int N = a.pool, E = a.evict_cap, RB = a.ring_slots;
    wave_lds_fence();
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int64_t base = 0; base < ntot; base += 64) {
        const int64_t li = base + lane;
        float s = -INFINITY;
        if (li < ntot) {
            const uint16_t* kr;
            int64_t t;
            if (li < nres) {
                t = a.n_q + li;
                kr = a.kring + ((int64_t)u * RB + t % RB) * D;
            } else if (li < nres + pc) {
                const int64_t p = (int64_t)u * N + (li - nres);
                t = a.pool_idx[p];
                kr = a.pool_k + p * D;
            } else {
                const int64_t e = (int64_t)u * E + (li - nres - pc);
                t = a.ev_idx[e];
                kr = a.ev_k + e * D;
            }
            float acc = 0.f;
#pragma unroll 4
            for (int c8 = 0; c8 < D / 8; ++c8) {
                const uint4 x = reinterpret_cast<const uint4*>(kr)[c8];
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc += qs[8 * c8 + 2 * i] * h2f(w[i] & 0xFFFF);
                    acc += qs[8 * c8 + 2 * i + 1] * h2f(w[i] >> 16);
                }
            }
            s = acc;
            if (a.logits) a.logits[((int64_t)u * R + h) * a.T + t] = s;
        }
        const float mn = fmaxf(m, wave_max(s));
        const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        const float p = s == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s - mn);
        l = l * alpha + wave_sum(p);
        o0 *= alpha;
        o1 *= alpha;
        m = mn;
        ps[lane] = p;
        wave_lds_fence();
        const int64_t cnt = ntot - base < 64 ? ntot - base : 64;
        for (int i = 0; i < cnt; ++i) {
            const int64_t li2 = base + i;
            const uint16_t* vr;
            if (li2 < nres) vr = a.vring + ((int64_t)u * RB + (a.n_q + li2) % RB) * D;
            else if (li2 < nres + pc) vr = a.pool_v + ((int64_t)u * N + (li2 - nres)) * D;
            else vr = a.ev_v + ((int64_t)u * E + (li2 - nres - pc)) * D;
            const uint32_t w = reinterpret_cast<const uint32_t*>(vr)[lane];
            const float pi = ps[i];
            o0 += pi * h2f(w & 0xFFFF);
            o1 += pi * h2f(w >> 16);
        }
        wave_lds_fence();
    }
    float* rec = a.part + (((int64_t)u * a.splits + a.splits_q) * R + h) * kRec;
    rec[2 * lane] = o0;
    rec[2 * lane + 1] = o1;
    if (lane == 0) {
        rec[D] = m;
        rec[D + 1] = l;
    }
}

template <int BITS, int R, int G>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    constexpr int NG = D / G;        // value groups per token
    constexpr int CPG = G / 32;      // chunks per key group
    constexpr int WPC = 128 * BITS;  // words per chunk
    constexpr float F = (float)(1 << BITS);
    __shared__ __align__(16) float smem[4 * 1024];  // 4 KB per wavefront
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if ((int)blockIdx.x < a.units) {
        fp16_partition<R>(a, blockIdx.x, smem);
        return;
    }
    const int idx = blockIdx.x - a.units;
    const int u = idx / a.splits_q, split = idx % a.splits_q;
    const int b = u / a.n_kv_heads, hk = u % a.n_kv_heads;
    const int64_t groups = a.n_q / G;
    const int64_t gs0 = split * groups / a.splits_q, gs1 = (split + 1) * groups / a.splits_q;

    // MFMA lane roles: j = column / row within a 16-lane row, kb = k-block.
    const int j = lane & 15, kb = lane >> 4;
    // Query-fold role: head hb, channels cb0 .. cb0+7 (k-step ksb, k-block kbb).
    const int hb = lane % R, kap = (lane >> 2) & 15, ksb = kap >> 2, kbb = kap & 3;
    const int cb0 = 32 * ksb + 8 * kbb;
    // Value-operand role: row j = (head j % R, value group gs).
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

    unsigned char* btab = reinterpret_cast<unsigned char*>(smem + wave * 1024);
    float m_run = -INFINITY, lsum = 0.f, zc = 0.f;
    floatx4 O[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int64_t gi = gs0 + wave; gi < gs1; gi += 4) {
        // Fold the key scale into the query: B[c][(h, x)] = hi/lo of q~_c * s_c * 2^b,
        // and the zero-point into beta_h = sum_c q~_c z_c - sum_c (hi + lo).
        const uint32_t* km = a.kmeta + ((int64_t)u * a.key_groups + gi) * D + cb0;
        const u32x4 m0 = *reinterpret_cast<const u32x4*>(km);
        const u32x4 m1 = *reinterpret_cast<const u32x4*>(km + 4);
        const uint32_t kmw[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        uint32_t hiw[4], low[4];
        float bp = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float sk = h2f(kmw[i] & 0xFFFF), zk = h2f(kmw[i] >> 16);
            const float x = qv[i] * F * sk;
            const _Float16 hi = (_Float16)x;
            const float hf = (float)hi;
            const _Float16 lo = (_Float16)(x - hf);
            bp += qv[i] * zk - (hf + (float)lo);
            if (i % 2 == 0) {
                hiw[i / 2] = hbits(hi);
                low[i / 2] = hbits(lo);
            } else {
                hiw[i / 2] |= hbits(hi) << 16;
                low[i / 2] |= hbits(lo) << 16;
            }
        }
#pragma unroll
        for (int x = 0; x < 16 / R; ++x) {
            const int jj = hb + R * x;
            u32x4 val = (x & 1) ? u32x4{low[0], low[1], low[2], low[3]}
                                : u32x4{hiw[0], hiw[1], hiw[2], hiw[3]};
            *reinterpret_cast<u32x4*>(btab + ((ksb * 4 + kbb) * 16 + jj) * 16) = val;
        }
        bp += __shfl_xor(bp, 4);
        bp += __shfl_xor(bp, 8);
        bp += __shfl_xor(bp, 16);
        bp += __shfl_xor(bp, 32);
        const float beta = bp;
        wave_lds_fence();
        half8 Bk[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            Bk[ks] = *reinterpret_cast<const half8*>(btab + ((ks * 4 + kb) * 16 + j) * 16);

        for (int cc = 0; cc < CPG; ++cc) {
            const int64_t ch = gi * CPG + cc;
            const int64_t tb = ch * 32;
            const uint32_t* kc = a.kq + ((int64_t)u * a.chunks + ch) * WPC;
            const uint32_t* vc = a.vq + ((int64_t)u * a.chunks + ch) * WPC;
            u32x4 wk0 = *reinterpret_cast<const u32x4*>(kc + lane * 4);
            u32x4 wv0 = *reinterpret_cast<const u32x4*>(vc + lane * 4);
            u32x4 wk1 = wk0, wv1 = wv0;
            if (BITS == 4) {
                wk1 = *reinterpret_cast<const u32x4*>(kc + 256 + lane * 4);
                wv1 = *reinterpret_cast<const u32x4*>(vc + 256 + lane * 4);
            }
            const uint32_t* vm = a.vmeta + (((int64_t)u * a.chunks + ch) * NG + gs) * 32 + 4 * kb;
            const u32x4 vm0 = *reinterpret_cast<const u32x4*>(vm);
            const u32x4 vm1 = *reinterpret_cast<const u32x4*>(vm + 16);
            const uint32_t mw = a.pool > 0 ? a.mask[(int64_t)u * a.chunks + ch] : 0u;
            const uint32_t wk[8] = {wk0.x, wk0.y, wk0.z, wk0.w, wk1.x, wk1.y, wk1.z, wk1.w};
            const uint32_t wv[8] = {wv0.x, wv0.y, wv0.z, wv0.w, wv1.x, wv1.y, wv1.z, wv1.w};

            // Logits: S^T[token][(h, x)] on the matrix cores, two 16-token tiles.
            float s[8];
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    half8 A;
                    if (BITS == 2) {
                        const uint32_t w = wk[2 * tau + ks / 2];
                        const int q0 = (ks % 2) * 4;
                        A = as_half8(cvt2(w, q0), cvt2(w, q0 + 1), cvt2(w, q0 + 2), cvt2(w, q0 + 3));
                    } else {
                        const uint32_t w = wk[4 * tau + ks];
                        A = as_half8(cvt4(w, 0), cvt4(w, 1), cvt4(w, 2), cvt4(w, 3));
                    }
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bk[ks], acc, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) s[4 * tau + i] = acc[i] + row_ror<R>(acc[i]) + beta;
            }
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
            float p[8];
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                p[sl] = __builtin_amdgcn_exp2f(s[sl] - mu);
                lsum += p[sl];
            }

            // Value operand: hi/lo of p_t * s^V_t * 2^b per (head, value group) row.
            const uint32_t vmw[8] = {vm0.x, vm0.y, vm0.z, vm0.w, vm1.x, vm1.y, vm1.z, vm1.w};
            uint32_t ahw[4], alw[4];
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                const float sv = h2f(vmw[sl] & 0xFFFF), zv = h2f(vmw[sl] >> 16);
                const float x = p[sl] * F * sv;
                const _Float16 hi = (_Float16)x;
                const float hf = (float)hi;
                const _Float16 lo = (_Float16)(x - hf);
                zc += p[sl] * zv - (hf + (float)lo);
                if (sl % 2 == 0) {
                    ahw[sl / 2] = hbits(hi);
                    alw[sl / 2] = hbits(lo);
                } else {
                    ahw[sl / 2] |= hbits(hi) << 16;
                    alw[sl / 2] |= hbits(lo) << 16;
                }
            }
            const half8 Ahi = as_half8(ahw[0], ahw[1], ahw[2], ahw[3]);
            const half8 Alo = as_half8(alw[0], alw[1], alw[2], alw[3]);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                half8 Bv;
                if (BITS == 2) {
                    const uint32_t w = wv[nt / 2];
                    const int q0 = (nt % 2) * 4;
                    Bv = as_half8(cvt2(w, q0), cvt2(w, q0 + 1), cvt2(w, q0 + 2), cvt2(w, q0 + 3));
                } else {
                    const uint32_t w = wv[nt];
                    Bv = as_half8(cvt4(w, 0), cvt4(w, 1), cvt4(w, 2), cvt4(w, 3));
                }
                O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Bv, O[nt], 0, 0, 0);
                O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Bv, O[nt], 0, 0, 0);
            }
        }
        wave_lds_fence();
    }

    // Wavefront epilogue: l per head, value corrections per row, outputs to LDS.
    float lt = lsum;
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    float zt = zc;
    zt += __shfl_xor(zt, 16);
    zt += __shfl_xor(zt, 32);
    float* ws = smem + wave * 1024;  // [R][D] outputs, then Z[16], m[R], l[R]
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
            mw[w] = smem[w * 1024 + R * D + 16 + h];
            M = fmaxf(M, mw[w]);
        }
        float o = 0.f, l = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
                o += smem[w * 1024 + h * D + c] * f;
                l += smem[w * 1024 + R * D + 20 + h] * f;
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
void launch_decode_t(const DecodeArgs& a, hipStream_t s) {
    const unsigned blocks = (unsigned)(a.units + a.units * a.splits_q);
    hipLaunchKernelGGL((decode_kernel<BITS, R, G>), dim3(blocks), dim3(256), 0, s, a);
    const unsigned ny = 1 + (a.acc ? (unsigned)((a.T + kH2OChunk - 1) / kH2OChunk) : 0u);
    hipLaunchKernelGGL((merge_kernel<R>), dim3(a.units, ny), dim3(256), 0, s, a);
}

template <int BITS, int R>
void dispatch_g(const DecodeArgs& a, int G, hipStream_t s) {
    if (G == 32) launch_decode_t<BITS, R, 32>(a, s);
    else if (G == 64) launch_decode_t<BITS, R, 64>(a, s);
    else launch_decode_t<BITS, R, 128>(a, s);
}

template <int BITS>
void dispatch_r(const DecodeArgs& a, int R, int G, hipStream_t s) {
    if (R == 1) dispatch_g<BITS, 1>(a, G, s);
    else if (R == 2) dispatch_g<BITS, 2>(a, G, s);
    else dispatch_g<BITS, 4>(a, G, s);
}

}  // namespace

int launch_decode(const CacheView& v, int64_t T, int64_t n_q, const DecodePlan& plan,
                  const uint16_t* q, float* out, float* acc, void* ws, void* stream) {
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
    a.pool = v.pool;
    a.evict_cap = v.evict_cap;
    a.qscale = 1.4426950408889634f / sqrtf((float)kHeadDim);
    const int R = v.n_q_heads / v.n_kv_heads;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (v.bits == 2) dispatch_r<2>(a, R, v.group, s);
    else dispatch_r<4>(a, R, v.group, s);
    return (int)hipGetLastError();
}

}  // namespace kvq

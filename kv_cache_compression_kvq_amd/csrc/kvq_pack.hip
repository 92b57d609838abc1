// Append path of libkvq on gfx950: OTT outlier tracing, KIVI quantize + pack,
// fp16 residual ring, plus cache initialisation and the canonical code view.
//
// Quantizer ("Accurate KV Cache Quantization with Outlier Tokens Tracing",
// section "Background"; "KV cache quantization and eviction", section
// "Minimal implementation"): for a group with minimum mn and maximum mx the
// step is q = max(mx - mn, 1e-8) / (2^b - 1) in IEEE fp32, each code is
// clamp(rint((x - mn) / q), 0, 2^b - 1) with ties to even, and the group keeps
// fp16(q) and mn (MiniKV, section 4.4: scale and zero-point in FP16). Every
// fp32 operation here is a single correctly rounded IEEE operation: nothing
// is contracted into an FMA, and division is built correctly rounded.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int D = kHeadDim;
constexpr int kPackRow = D + 8;  // LDS row stride of the pack kernel, in fp16 elements

__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
}

// An fp16 value as an exact integer multiple of 2^-24 (every finite binary16
// number is one).
__device__ __forceinline__ int64_t half_fixed(uint16_t h) {
    const uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
    const int64_t mag = e ? (int64_t)(1024 + m) << (e - 1) : (int64_t)m;
    return (h & 0x8000) ? -mag : mag;
}

// Round S * 2^-(24 + sh) to the nearest binary16 value, ties to even, from
// the exact integer S. Used for the group mean, which is exact before this one
// rounding (sum of fixed-point values divided by a power of two).
__device__ uint16_t fixed_to_half(int64_t S, int sh) {
    const uint16_t sign = S < 0 ? 0x8000 : 0;
    const uint64_t A = S < 0 ? (uint64_t)(-S) : (uint64_t)S;
    if (A == 0) return 0;
    const int lg = 63 - __builtin_clzll(A) - sh;  // floor(log2) of the value in 2^-24 units
    const int qe = lg > 10 ? lg - 10 : 0;         // log2 of the binary16 quantum there
    const int shift = sh + qe;
    uint64_t n = A;
    if (shift > 0) {
        n = A >> shift;
        const uint64_t rem = A & ((1ull << shift) - 1), half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (n & 1))) ++n;
    }
    const uint64_t vu = n << qe;  // rounded value, 2^-24 units
    if (vu < 1024) return sign | (uint16_t)vu;  // subnormal
    const int p = 63 - __builtin_clzll(vu);
    const int e = p - 9;  // biased exponent
    if (e >= 31) return sign | 0x7C00;
    const uint32_t f = (uint32_t)(vu >> (e - 1)) - 1024;
    return sign | (uint16_t)(e << 10) | (uint16_t)f;
}

// Codes of N elements of one group: clamp(rint(fl32(fl32(x - mn) / q)), 0,
// levels), exactly. The quotient is first taken as fl32(d * rq) with
// rq = fl32(1 / q): for quotients below 16 that lies within 2^-18.6 of the
// correctly rounded quotient (two roundings of 2^-24 relative each, plus half
// an ulp of the quotient), so whenever it is at least 2^-17 away from every
// half-integer both round to the same integer. Closer than that (rare), the
// correctly rounded division decides; that branch is taken by the whole
// wavefront or not at all.
__device__ __forceinline__ bool near_tie(float t) {
    return fabsf(fabsf(t - rintf(t)) - 0.5f) < 0x1p-17f;
}
template <int N>
__device__ __forceinline__ void quant_codes(const float (&x)[N], float mn, float q, float rq,
                                            float levels, uint32_t (&c)[N]) {
    float d[N], t[N], r[N];
    float dist = 1.0f;  // smallest distance of a quotient to a half-integer
#pragma unroll
    for (int m = 0; m < N; ++m) {
        d[m] = x[m] - mn;
        t[m] = d[m] * rq;
        r[m] = rintf(t[m]);
        dist = fminf(dist, fabsf(fabsf(t[m] - r[m]) - 0.5f));
    }
    if (__any(dist < 0x1p-17f)) {
#pragma unroll
        for (int m = 0; m < N; ++m)
            if (near_tie(t[m])) r[m] = rintf(d[m] / q);
    }
#pragma unroll
    for (int m = 0; m < N; ++m) c[m] = (uint32_t)fminf(fmaxf(r[m], 0.0f), levels);
}

// Lower bound on the range before dividing (the reference quantizer clamps
// max - min at 1e-8); bit pattern of the fp32 nearest to 1e-8.
__device__ __forceinline__ float range_floor() { return __builtin_bit_cast(float, 0x322BCC77u); }

// Source row of token t of unit u during an append: the residual ring holds
// tokens appended by earlier calls, the caller's buffer holds this call's.
__device__ __forceinline__ const uint16_t* src_row(const uint16_t* ring, const uint16_t* fresh,
                                                   const CacheView& v, int u, int64_t t,
                                                   int64_t t_old, int32_t n_new) {
    return t < t_old ? ring + ((int64_t)u * v.ring_slots + t % v.ring_slots) * D
                     : fresh + ((int64_t)u * n_new + (t - t_old)) * D;
}

// The eviction step's per-unit scratch, after the eviction counts (8-byte
// aligned): word 0 the complement of the best (key, index) found so far (an
// atomic maximum), word 1 the count of the unit's workgroups that are done.
// Both are zero between calls: the unit's last workgroup resets them.
__device__ __forceinline__ uint64_t* evict_scratch(const CacheView& v) {
    return reinterpret_cast<uint64_t*>(v.evict_count + ((v.units + 1) & ~1));
}

// Counters and pool masks start at zero. With G = 16 the key and value
// scale/zero words are zeroed too: a chunk whose second group is not yet
// quantized is read by the decoder with that half masked out, and its
// parameters must then be finite.
__global__ void init_kernel(CacheView v) {
    const int64_t nc = (int64_t)v.units * 4, nm = (int64_t)v.units * v.chunks;
    const int64_t nk = v.group == 16 ? (int64_t)v.units * v.key_groups * D : 0;
    const int64_t nv = v.group == 16 ? (int64_t)v.units * v.chunks * (D / 16) * kChunk : 0;
    const int64_t ne = (int64_t)v.units * v.evict_words, nu = v.units;
    const int64_t n1 = nc + nm, n2 = n1 + nk, n3 = n2 + nv, n4 = n3 + ne, n5 = n4 + nu;
    const int64_t n6 = n5 + 4 * nu;  // the eviction step's scratch, as 32-bit words
    if (v.bits == 8 && blockIdx.x == 0 && (int)threadIdx.x < 2 * v.n_kv_heads)
        v.fp8_scales[threadIdx.x] = 1.0f;  // FP8 scales: 1.0 until set
    uint32_t* esc = reinterpret_cast<uint32_t*>(evict_scratch(v));
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n6;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (i < nc) v.counters[i] = 0;
        else if (i < n1) v.mask[i - nc] = 0;
        else if (i < n2) v.kmeta[i - n1] = 0;
        else if (i < n3) v.vmeta[i - n2] = 0;
        else if (i < n4) v.evict[i - n3] = 0;
        else if (i < n5) v.evict_count[i - n4] = 0;
        else esc[i - n5] = 0;
    }
}

// OTT pool competition, one wavefront per unit, groups in token order.
// For each group the tokens ranked by (score, index) together with the pool
// members and falling among the N best are admitted in that order; an
// admission into a full pool moves the pool's worst member to the extra pool;
// when that needs a move and the extra pool already holds E tokens, tracing
// stops for good ("Accurate KV Cache Quantization with Outlier Tokens
// Tracing", section "Method details" and appendix E). Admitted tokens get
// their bit in the chunk mask and their original fp16 rows copied to the pool.
__global__ __launch_bounds__(64) void ott_scan_kernel(CacheView v, const uint16_t* knew,
                                                      const uint16_t* vnew, int64_t t_old,
                                                      int32_t n_new, int64_t g0, int64_t g1) {
    const int u = blockIdx.x, lane = threadIdx.x;
    const int G = v.group, N = v.pool, E = v.evict_cap;
    // scores of up to kScanBatch tokens are staged at once, so that the serial
    // walk over the groups reads them from LDS
    constexpr int kScanBatch = 2048;
    __shared__ uint64_t sc_all[kScanBatch];
    __shared__ uint32_t mbatch[kScanBatch / 32];  // chunk mask words of the staged groups
    // members displaced in this call: token and the pool slot it left
    __shared__ int32_t ev_tok[kMaxEvict], ev_from[kMaxEvict];
    // The block is one wavefront: LDS ordering needs the LDS counter and a wave
    // barrier only (no wait for global stores in flight).
    auto wave_sync = [] {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
    };
    int32_t* cnt = v.counters + (int64_t)u * 4;
    int pc = cnt[0], ec = cnt[1], frozen = cnt[2];
    const int ec0 = ec;
    // group and token indices fit in 32 bits (per-unit capacity below 2^24)
    const int32_t t_first = (int32_t)g0 * G;  // tokens from here on are admitted in this call
    // Pool member p lives in lane p (N <= 64): its exact score and token index.
    uint64_t psl = lane < N ? v.pool_score[(int64_t)u * N + lane] : 0ull;
    int32_t pil = lane < N ? v.pool_idx[(int64_t)u * N + lane] : -1;
    auto rl64 = [](uint64_t x, int l) -> uint64_t {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
        return (uint64_t)lo | ((uint64_t)hi << 32);
    };
    // The pool's worst member (largest (score, index)) and its slot once the
    // pool is full: only tokens ordered before it can rank among the N best.
    uint64_t wsc = ~0ull;
    int32_t widx = INT32_MAX;
    int wslot = 0;
    auto find_worst = [&] {
        wsc = ~0ull;
        widx = INT32_MAX;
        if (pc < N) return;
        uint64_t bs = 0;
        int32_t bi = -1;
        for (int p = 0; p < N; ++p) {
            const uint64_t sp = rl64(psl, p);
            const int32_t ip = __builtin_amdgcn_readlane(pil, p);
            if (sp > bs || (sp == bs && ip > bi)) {
                bs = sp;
                bi = ip;
                wslot = p;
            }
        }
        wsc = bs;
        widx = bi;
    };
    find_worst();
    const int32_t gend = (int32_t)g1;
    int32_t gb = (int32_t)g0, gb_end = gb, g = gb;
    // Chunk-mask words: group g's bits start at bit g*G of the unit's mask.
    // With G = 16 two groups share a word (the odd group in the high half).
    auto wfirst = [&](int32_t gg) { return (int32_t)(((int64_t)gg * G) >> 5); };
    auto wend = [&](int32_t gg) { return (int32_t)(((int64_t)gg * G + 31) >> 5); };
    // mask words of groups [gb, ge) to memory (none for an empty range: with
    // G = 16 and an odd gb, wend(gb) - wfirst(gb) would otherwise be 1)
    auto flush = [&](int32_t ge) {
        if (ge <= gb) return;
        for (int i = lane; i < wend(ge) - wfirst(gb); i += 64)
            v.mask[(int64_t)u * v.chunks + wfirst(gb) + i] = mbatch[i];
    };
    // the group's mask bits (mword holds group word w in lane w; G = 16: lane 0)
    auto put_mask = [&](int32_t gg, uint32_t mword) {
        if (G >= 32) {
            if (lane < G / 32) mbatch[wfirst(gg) - wfirst(gb) + lane] = mword;
        } else if (lane == 0 && mword) {
            mbatch[wfirst(gg) - wfirst(gb)] |= mword << (16 * (gg & 1));
        }
    };
    // Lane l holds the smallest score of the staged batch's group gb + l. A
    // group can admit a token only if the pool is not full or that minimum is
    // at most the pool's worst score, so the walk goes from one such group to
    // the next with a ballot (a tie on the score is checked in full there);
    // the groups in between keep mask words of zero.
    uint64_t gms = ~0ull;
    for (; g < gend && !frozen; ++g) {
        if (g == gb_end) {
            flush(g);
            gb = g;
            // At most 64 groups (lane l holds the minimum score of group
            // gb + l). G = 16: batches after the first start at an even group,
            // so that no mask word is shared by two batches of this launch.
            const int32_t bmax = kScanBatch / G < 64 ? kScanBatch / G : 64;
            gb_end = g + bmax < gend ? g + bmax : gend;
            if (G < 32 && gb_end < gend && (gb_end & 1)) --gb_end;
            wave_sync();  // the previous batch is no longer read
            // eight loads in flight per lane before any is stored
            const int32_t nb = (gb_end - g) * G, tb = g * G;
            for (int i0 = 0; i0 < nb; i0 += 8 * 64) {
                uint64_t x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = i0 + 64 * j + lane;
                    x[j] = i < nb ? v.scores[(int64_t)u * v.q_cap + tb + i] : 0ull;
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = i0 + 64 * j + lane;
                    if (i < nb) sc_all[i] = x[j];
                }
            }
            for (int i = lane; i < wend(gb_end) - wfirst(gb); i += 64) mbatch[i] = 0u;
            // G = 16, odd first group: the low half of its word belongs to the
            // group before, quantized by an earlier call
            if (G < 32 && (gb & 1) && lane == 0)
                mbatch[0] = v.mask[(int64_t)u * v.chunks + wfirst(gb)];
            wave_sync();
            gms = ~0ull;
            if (lane < gb_end - gb) {
                // tokens visited from a lane-dependent start, so that the
                // lanes' LDS reads fall into different banks
                const uint64_t* sg = sc_all + (int64_t)lane * G;
                for (int i0 = 0; i0 < G; i0 += 8) {  // G is a multiple of 8
                    uint64_t x[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) x[j] = sg[(i0 + j + lane) & (G - 1)];
#pragma unroll
                    for (int j = 0; j < 8; ++j) gms = x[j] < gms ? x[j] : gms;
                }
            }
        }
        {
            const uint64_t m = __ballot(lane < gb_end - gb && lane >= g - gb && (pc < N || gms <= wsc));
            if (m == 0) {  // no group left in the batch can admit a token
                g = gb_end - 1;
                continue;
            }
            g = gb + __builtin_ctzll(m);
        }
        const int32_t t0 = g * G;
        const uint64_t* sc = sc_all + (g - gb) * G;
        // this lane's tokens of the group: lane and lane + 64 (G = 128)
        uint64_t sl[2];
        bool cand[2], any = false;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int i = lane + 64 * j;
            sl[j] = i < G ? sc[i] : ~0ull;
            cand[j] = i < G && (pc < N || sl[j] < wsc || (sl[j] == wsc && t0 + i < widx));
            any |= cand[j];
        }
        if (!__any(any)) continue;  // nothing enters the pool: the common case
        // Chunk mask word w of the group lives in lane w (G / 32 words), so
        // marking a token is one masked OR in a register.
        uint32_t mword = 0;
        auto mark = [&](int i) {
            if (lane == (i >> 5)) mword |= 1u << (i & 31);
        };
        if (pc == N) {
            // Full pool: the candidates order before the worst member, hence
            // before every other token of the group. Taking them in ascending
            // (score, index) order, the k-th enters iff it still orders before
            // the current worst member, i.e. iff (pool members before it) +
            // k - 1 < N: the same admissions, in the same order, as by rank.
            uint64_t m0 = __ballot(cand[0]), m1 = __ballot(cand[1]);
            while (m0 | m1) {
                uint64_t bs = ~0ull;
                int32_t bt = INT32_MAX;
                int bl = 0;
                for (uint64_t m = m0; m; m &= m - 1) {
                    const int l = __builtin_ctzll(m);
                    const uint64_t sq = rl64(sl[0], l);
                    if (sq < bs || (sq == bs && t0 + l < bt)) {
                        bs = sq;
                        bt = t0 + l;
                        bl = l;
                    }
                }
                for (uint64_t m = m1; m; m &= m - 1) {
                    const int l = __builtin_ctzll(m);
                    const uint64_t sq = rl64(sl[1], l);
                    if (sq < bs || (sq == bs && t0 + 64 + l < bt)) {
                        bs = sq;
                        bt = t0 + 64 + l;
                        bl = 64 + l;
                    }
                }
                if (!(bs < wsc || (bs == wsc && bt < widx))) break;
                if (ec == E) {
                    frozen = 1;
                    break;
                }
                if (lane == 0) {
                    v.ev_idx[(int64_t)u * E + ec] = widx;
                    ev_tok[ec - ec0] = widx;
                    ev_from[ec - ec0] = wslot;
                }
                ++ec;
                if (lane == wslot) {
                    psl = bs;
                    pil = (int32_t)bt;
                }
                mark(bl);
                if (bl < 64) m0 &= ~(1ull << bl);
                else m1 &= ~(1ull << (bl - 64));
                find_worst();
            }
            put_mask(g, mword);
            continue;
        }
        // Pool still filling: rank of each token among the pool members and
        // the group, by (score, index).
        int rank[2] = {0, 0};
        for (int p = 0; p < pc; ++p) {
            const uint64_t sp = rl64(psl, p);
            const int32_t ip = __builtin_amdgcn_readlane(pil, p);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                rank[j] += (sp < sl[j]) || (sp == sl[j] && ip < t0 + lane + 64 * j);
        }
        for (int q = 0; q < G; ++q) {
            const uint64_t sq = rl64(q < 64 ? sl[0] : sl[1], q & 63);
#pragma unroll
            for (int j = 0; j < 2; ++j) rank[j] += (sq < sl[j]) || (sq == sl[j] && q < lane + 64 * j);
        }
        // Admissions in rank order; a full pool gives up its worst member.
        for (int rk = 0; rk < N; ++rk) {
            const uint64_t m0 = __ballot(cand[0] && rank[0] == rk);
            const uint64_t m1 = __ballot(cand[1] && rank[1] == rk);
            if (m0 == 0 && m1 == 0) continue;
            const int i = m0 ? __builtin_ctzll(m0) : 64 + __builtin_ctzll(m1);
            const int32_t t = t0 + i;
            const uint64_t si = rl64(i < 64 ? sl[0] : sl[1], i & 63);
            int dst;
            if (pc == N) {
                if (ec == E) {
                    frozen = 1;
                    break;
                }
                if (lane == 0) {
                    v.ev_idx[(int64_t)u * E + ec] = widx;
                    ev_tok[ec - ec0] = widx;
                    ev_from[ec - ec0] = wslot;
                }
                ++ec;
                dst = wslot;
            } else {
                dst = pc++;
            }
            if (lane == dst) {
                psl = si;
                pil = (int32_t)t;
            }
            mark(i);
            find_worst();
        }
        put_mask(g, mword);
    }
    flush(g);
    wave_sync();
    // Row copies, after the walk. Displaced members first: a member admitted
    // in this call still has its rows in the input or the ring; an older one
    // has them in the pool slot it left, which no copy below has overwritten yet.
    // Four rows at a time: all loads, then all stores.
    for (int e0 = ec0; e0 < ec; e0 += 4) {
        uint32_t kx[4], vx[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (e0 + j >= ec) break;
            const int64_t t = ev_tok[e0 + j - ec0];
            const int64_t ps = (int64_t)u * N + ev_from[e0 + j - ec0];
            const uint16_t* kr = t >= t_first ? src_row(v.kring, knew, v, u, t, t_old, n_new) : v.pool_k + ps * D;
            const uint16_t* vr = t >= t_first ? src_row(v.vring, vnew, v, u, t, t_old, n_new) : v.pool_v + ps * D;
            kx[j] = reinterpret_cast<const uint32_t*>(kr)[lane];
            vx[j] = reinterpret_cast<const uint32_t*>(vr)[lane];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (e0 + j >= ec) break;
            const int64_t es = (int64_t)u * E + e0 + j;
            reinterpret_cast<uint32_t*>(v.ev_k + es * D)[lane] = kx[j];
            reinterpret_cast<uint32_t*>(v.ev_v + es * D)[lane] = vx[j];
        }
    }
    __syncthreads();  // every old pool row is read before the slots are rewritten
    for (int p0 = 0; p0 < pc; p0 += 4) {
        uint32_t kx[4], vx[4];
        bool cp[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // members from an earlier call keep their rows in place
            const int p = p0 + j;
            const int64_t t = p < pc ? __builtin_amdgcn_readlane(pil, p) : -1;
            cp[j] = p < pc && t >= t_first;
            if (cp[j]) {
                kx[j] = reinterpret_cast<const uint32_t*>(src_row(v.kring, knew, v, u, t, t_old, n_new))[lane];
                vx[j] = reinterpret_cast<const uint32_t*>(src_row(v.vring, vnew, v, u, t, t_old, n_new))[lane];
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (!cp[j]) continue;
            const int64_t pd = (int64_t)u * N + p0 + j;
            reinterpret_cast<uint32_t*>(v.pool_k + pd * D)[lane] = kx[j];
            reinterpret_cast<uint32_t*>(v.pool_v + pd * D)[lane] = vx[j];
        }
    }
    if (lane < N) {
        v.pool_idx[(int64_t)u * N + lane] = pil;
        v.pool_score[(int64_t)u * N + lane] = psl;
    }
    if (lane == 0) {
        cnt[0] = pc;
        cnt[1] = ec;
        cnt[2] = frozen;
    }
}

// 2-bit position of operand pair j (0..7) inside a packed word: the decoder
// uses positions 3 and 4 (bits 6-9 of each half) in place, brings 1-2 there
// by a 4-bit left shift, 5-6 by a 4-bit right shift, and 0 and 7 by one 8-bit
// left rotate, which also swaps the two halves of position 7 (stored swapped
// for that reason). Even j ends at bits 6-7, odd j at bits 8-9.
__device__ constexpr int kPos2[8] = {3, 4, 1, 2, 5, 6, 7, 0};

// Quantize and pack one key group (G tokens) of one unit; 256 threads.
// Pool members' rows are first replaced, for keys and values alike, by the
// per-channel mean of all G rows of the group, computed exactly and rounded
// once to fp16 ("Accurate KV Cache Quantization with Outlier Tokens Tracing",
// section "Method details"). Keys are then quantized per channel over the G
// tokens, values per token over runs of G channels (KIVI grouping; MiniKV,
// section 4.4), and the codes written in the chunk layout of kvq.h.
// Block x takes group g0 + gstride * (x / U). With G = 16 a 32-token chunk
// holds two groups: the even and the odd groups of an append run as two
// launches (gstride 2), and a 2-bit key word, which holds codes of both
// halves of its chunk, is rewritten keeping the other half's bits.
// With an outlier pool the groups of an append are packed twice around the
// pool scan (modes): mode 1 writes every token's exact key L1 score (OTT,
// appendix E) from the rows it already holds and quantizes with no pool
// member; the scan then admits tokens; mode 2 repacks the groups that
// admitted one (mean replacement). Mode 0: one pass (no pool). The unit's
// value-scale bound (counters[3]) is raised in every pass, so it also covers
// the first-pass scales of tokens later replaced by the group mean.
// Threads of a pack block: groups of 64 and 128 tokens take 512 and 1024, so
// that each thread holds two 16-byte row pieces per tensor and the per-channel
// and per-token passes split over several threads.
template <int G>
constexpr int pack_threads() { return G <= 32 ? 256 : G == 64 ? 512 : 1024; }

template <int BITS, int G>
__device__ void pack_group(const CacheView& v, const uint16_t* knew, const uint16_t* vnew,
                           int64_t t_old, int32_t n_new, int u, int64_t g, int32_t mode,
                           uint32_t vmax_seen) {
    constexpr int NT = pack_threads<G>();
    constexpr int KSL = NT / (2 * D);  // token slices per key channel
    constexpr int VPP = NT / (2 * D);  // threads per (token, value group): D pairs per group
    constexpr int NG = D / G;          // value groups per token
    constexpr bool kHalf = G == 16;    // the group is half a chunk
    constexpr int CPG = kHalf ? 1 : G / kChunk;  // chunks the group touches
    constexpr int WPC = 128 * BITS;    // 32-bit words per chunk
    constexpr int LG = G == 16 ? 4 : G == 32 ? 5 : G == 64 ? 6 : 7;
    const float levels = (float)((1 << BITS) - 1);
    extern __shared__ __align__(16) uint16_t smem[];
    // [G][RS] fp16 rows, overwritten by their codes. The row stride of 272
    // bytes puts the 16-byte value reads of a quarter wavefront (4 tokens x
    // 4 value groups at G = 32) on disjoint LDS banks.
    constexpr int RS = kPackRow;
    uint16_t* kx = smem;
    uint16_t* vx = smem + G * RS;
    __shared__ uint16_t meank[D], meanv[D];
    __shared__ uint32_t vmax_w[NT / 128];
    __shared__ float kmin_s[KSL][D], kmax_s[KSL][D];  // key slices' extremes (KSL > 1)
    const int tid = threadIdx.x;
    const int64_t t0 = g * G;
    const int hf = kHalf ? (int)(g & 1) : 0;  // G = 16: which half of its chunk

    {
        // all of this thread's row pieces are requested before any is stored
        constexpr int kPer = G * 16 / NT;  // 16-byte pieces per thread and tensor
        uint4 kr[kPer], vr[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int e = tid + NT * j, i = e / 16, part = e % 16;
            kr[j] = reinterpret_cast<const uint4*>(src_row(v.kring, knew, v, u, t0 + i, t_old, n_new))[part];
            vr[j] = reinterpret_cast<const uint4*>(src_row(v.vring, vnew, v, u, t0 + i, t_old, n_new))[part];
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int e = tid + NT * j, i = e / 16, part = e % 16;
            reinterpret_cast<uint4*>(kx + i * RS)[part] = kr[j];
            reinterpret_cast<uint4*>(vx + i * RS)[part] = vr[j];
        }
    }
    uint32_t mw[CPG];
    bool any = false;
#pragma unroll
    for (int c = 0; c < CPG; ++c) {
        mw[c] = v.pool > 0 && mode != 1 ? v.mask[(int64_t)u * v.chunks + t0 / kChunk + c] : 0u;
        if (kHalf) mw[c] = (mw[c] >> (16 * hf)) & 0xFFFFu;
        any |= mw[c] != 0;
    }
    __syncthreads();
    if (mode == 1) {
        // OTT token score: sum of |k_c| over the row, exact, as an integer in
        // units of 2^-24; 256 / G threads per token
        // (any partial sum is a multiple of 2^-24 below 2^23 with at most 47
        // significant bits, so the fp64 sum is exact in any order)
        constexpr int TPT = NT / G, CPT = D / TPT;
        const int i = tid / TPT, part = tid % TPT;
        double sc = 0.0;
#pragma unroll
        for (int c8 = 0; c8 < CPT / 8; ++c8) {
            const uint4 x = reinterpret_cast<const uint4*>(kx + i * RS + part * CPT)[c8];
            const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                sc += fabs((double)h2f((uint16_t)(w[m] & 0xFFFF)));
                sc += fabs((double)h2f((uint16_t)(w[m] >> 16)));
            }
        }
#pragma unroll
        for (int off = TPT / 2; off > 0; off >>= 1) sc += __shfl_xor(sc, off, TPT);
        if (part == 0) v.scores[(int64_t)u * v.q_cap + t0 + i] = (uint64_t)(sc * 16777216.0);
    }
    if (any) {
        if (tid < 2 * D) {
            const uint16_t* x = tid < D ? kx + tid : vx + (tid - D);
            int64_t s = 0;
            for (int i = 0; i < G; ++i) s += half_fixed(x[i * RS]);
            (tid < D ? meank[tid] : meanv[tid - D]) = fixed_to_half(s, LG);
        }
        __syncthreads();
        for (int e = tid; e < G * D; e += NT) {
            const int i = e / D, c = e % D;
            if ((mw[i / kChunk] >> (i % kChunk)) & 1u) {
                kx[i * RS + c] = meank[c];
                vx[i * RS + c] = meanv[c];
            }
        }
        __syncthreads();
    }
    if constexpr (KSL == 1) {
        // 256 threads: thread tid < D takes key channel tid over the G tokens,
        // thread D + j the value pair (token j / NG, group j % NG)
        if (tid < D) {
            // keys: channel c over the G tokens
            const int c = tid;
            float mn = INFINITY, mx = -INFINITY;
            for (int i = 0; i < G; ++i) {
                const float x = h2f(kx[i * RS + c]);
                mn = fminf(mn, x);
                mx = fmaxf(mx, x);
            }
            const float q = fmaxf(mx - mn, range_floor()) / levels;
            const float rq = 1.0f / q;
            v.kmeta[((int64_t)u * v.key_groups + g) * D + c] = (uint32_t)f2h(q) | ((uint32_t)f2h(mn) << 16);
            for (int i0 = 0; i0 < G; i0 += 8) {
                float x[8];
                uint32_t cd[8];
    #pragma unroll
                for (int m = 0; m < 8; ++m) x[m] = h2f(kx[(i0 + m) * RS + c]);
                quant_codes(x, mn, q, rq, levels, cd);
    #pragma unroll
                for (int m = 0; m < 8; ++m) kx[(i0 + m) * RS + c] = (uint16_t)cd[m];
            }
        } else {
            // values: token i, channels [gq*G, gq*G + G), eight at a time
            const int j = tid - D, i = j / NG, gq = j % NG;
            uint4* row = reinterpret_cast<uint4*>(vx + i * RS + gq * G);
            float mn = INFINITY, mx = -INFINITY;
            for (int c8 = 0; c8 < G / 8; ++c8) {
                const uint4 x = row[c8];
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    #pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float a = h2f((uint16_t)(w[m] & 0xFFFF)), b = h2f((uint16_t)(w[m] >> 16));
                    mn = fminf(mn, fminf(a, b));
                    mx = fmaxf(mx, fmaxf(a, b));
                }
            }
            const float q = fmaxf(mx - mn, range_floor()) / levels;
            const float rq = 1.0f / q;
            const int64_t t = t0 + i;
            const uint16_t qh = f2h(q);
            v.vmeta[(((int64_t)u * v.chunks + t / kChunk) * NG + gq) * kChunk + t % kChunk] =
                (uint32_t)qh | ((uint32_t)f2h(mn) << 16);
            // Largest value scale of the unit (fp16 bits of a positive number order
            // like the numbers): bounds the lazy softmax rescale of the decoder.
            uint32_t mq = qh;
            for (int off = 32; off > 0; off >>= 1) mq = max(mq, (uint32_t)__shfl_xor((int)mq, off));
            if ((tid & 63) == 0) vmax_w[(tid - D) >> 6] = mq;
            for (int c8 = 0; c8 < G / 8; ++c8) {
                const uint4 x = row[c8];
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
                float xf[8];
                uint32_t cd[8];
    #pragma unroll
                for (int m = 0; m < 4; ++m) {
                    xf[2 * m] = h2f((uint16_t)(w[m] & 0xFFFF));
                    xf[2 * m + 1] = h2f((uint16_t)(w[m] >> 16));
                }
                quant_codes(xf, mn, q, rq, levels, cd);
                row[c8] = make_uint4(cd[0] | cd[1] << 16, cd[2] | cd[3] << 16, cd[4] | cd[5] << 16,
                                     cd[6] | cd[7] << 16);
            }
        }
    } else {
        // Keys: thread tid < NT / 2 takes channel tid % D over token slice
        // tid / D (G / KSL tokens). Values: thread NT / 2 + j takes (token, value
        // group) pair j / VPP, channel part j % VPP (G / VPP channels); the parts of
        // a pair are adjacent lanes.
        constexpr int KT = G / KSL, VC = G / VPP;
        const bool is_key = tid < NT / 2;
        const int c = tid % D, ksl = (tid / D) % KSL;
        const int j = tid - NT / 2, vpair = j / VPP, vpart = j % VPP;
        const int vi = vpair / NG, vgq = vpair % NG;
        float mn = INFINITY, mx = -INFINITY;
        if (is_key) {
            for (int i = ksl * KT; i < ksl * KT + KT; ++i) {
                const float x = h2f(kx[i * RS + c]);
                mn = fminf(mn, x);
                mx = fmaxf(mx, x);
            }
            if (KSL > 1) {
                kmin_s[ksl][c] = mn;
                kmax_s[ksl][c] = mx;
            }
        } else {
            const uint4* row = reinterpret_cast<const uint4*>(vx + vi * RS + vgq * G + vpart * VC);
            for (int c8 = 0; c8 < VC / 8; ++c8) {
                const uint4 x = row[c8];
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    #pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float a = h2f((uint16_t)(w[m] & 0xFFFF)), b = h2f((uint16_t)(w[m] >> 16));
                    mn = fminf(mn, fminf(a, b));
                    mx = fmaxf(mx, fmaxf(a, b));
                }
            }
    #pragma unroll
            for (int off = 1; off < VPP; off <<= 1) {
                mn = fminf(mn, __shfl_xor(mn, off, VPP));
                mx = fmaxf(mx, __shfl_xor(mx, off, VPP));
            }
        }
        if (KSL > 1) {
            __syncthreads();
            if (is_key) {
                mn = kmin_s[0][c];
                mx = kmax_s[0][c];
    #pragma unroll
                for (int sl = 1; sl < KSL; ++sl) {
                    mn = fminf(mn, kmin_s[sl][c]);
                    mx = fmaxf(mx, kmax_s[sl][c]);
                }
            }
        }
        const float q = fmaxf(mx - mn, range_floor()) / levels;
        const float rq = 1.0f / q;
        if (is_key) {
            // keys: channel c over its token slice
            if (ksl == 0)
                v.kmeta[((int64_t)u * v.key_groups + g) * D + c] = (uint32_t)f2h(q) | ((uint32_t)f2h(mn) << 16);
            for (int i0 = ksl * KT; i0 < ksl * KT + KT; i0 += 8) {
                float x[8];
                uint32_t cd[8];
    #pragma unroll
                for (int m = 0; m < 8; ++m) x[m] = h2f(kx[(i0 + m) * RS + c]);
                quant_codes(x, mn, q, rq, levels, cd);
    #pragma unroll
                for (int m = 0; m < 8; ++m) kx[(i0 + m) * RS + c] = (uint16_t)cd[m];
            }
        } else {
            // values: token vi, channels vgq * G + vpart * VC .. + VC - 1, eight at a time
            uint4* row = reinterpret_cast<uint4*>(vx + vi * RS + vgq * G + vpart * VC);
            const int64_t t = t0 + vi;
            const uint16_t qh = f2h(q);
            if (vpart == 0)
                v.vmeta[(((int64_t)u * v.chunks + t / kChunk) * NG + vgq) * kChunk + t % kChunk] =
                    (uint32_t)qh | ((uint32_t)f2h(mn) << 16);
            // Largest value scale of the unit (fp16 bits of a positive number order
            // like the numbers): bounds the lazy softmax rescale of the decoder.
            uint32_t mq = qh;
            for (int off = 32; off > 0; off >>= 1) mq = max(mq, (uint32_t)__shfl_xor((int)mq, off));
            if ((j & 63) == 0) vmax_w[j >> 6] = mq;
            for (int c8 = 0; c8 < VC / 8; ++c8) {
                const uint4 x = row[c8];
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
                float xf[8];
                uint32_t cd[8];
    #pragma unroll
                for (int m = 0; m < 4; ++m) {
                    xf[2 * m] = h2f((uint16_t)(w[m] & 0xFFFF));
                    xf[2 * m + 1] = h2f((uint16_t)(w[m] >> 16));
                }
                quant_codes(xf, mn, q, rq, levels, cd);
                row[c8] = make_uint4(cd[0] | cd[1] << 16, cd[2] | cd[3] << 16, cd[4] | cd[5] << 16,
                                     cd[6] | cd[7] << 16);
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t mq = vmax_w[0];
#pragma unroll
        for (int w = 1; w < NT / 128; ++w) mq = max(mq, vmax_w[w]);
        if (mq > vmax_seen) atomicMax(reinterpret_cast<uint32_t*>(v.counters) + (int64_t)u * 4 + 3, mq);
    }

    // Pack. Word w of lane l sits at (w/4)*256 + l*4 + w%4 within its chunk.
    // LDS row of the token at position tc of chunk cc (with G = 16 only the
    // block's own half of the chunk is in LDS).
    auto row_of = [&](int cc, int tc) { return kHalf ? tc - 16 * hf : cc * kChunk + tc; };
    for (int e = tid; e < 2 * CPG * WPC; e += NT) {
        const bool isv = e >= CPG * WPC;
        const int r = isv ? e - CPG * WPC : e;
        const int cc = r / WPC, o = r % WPC;
        const int w = (o / 256) * 4 + (o % 4), l = (o % 256) / 4;
        const int kb = l / 16, n = l % 16;
        // With G = 16, the half (16-token tile) a word's codes belong to: 2-bit
        // key words hold both halves (merged below), the others one half.
        if (kHalf && !(BITS == 2 && !isv)) {
            const int tau = isv ? (w % 4) / 2 : w / 4;
            if (tau != hf) continue;
        }
        uint32_t word = 0;
        if (!isv) {
            // lane (token row n of tile tau, channel block kb): codes of channels
            // 32*ks + 8*kb + {2m, 2m+1} in the low/high halves of the word
            if (BITS == 2) {
                // Word m holds pair m of every (tile tau, k-step ks) at 2-bit
                // position kPos2[4 tau + ks]: one matrix-core operand takes its
                // four pairs from one position of the four words.
                const int m = w;
#pragma unroll
                for (int tau = 0; tau < 2; ++tau) {
                    if (kHalf && tau != hf) continue;
                    const int tok = row_of(cc, 16 * tau + n);
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const int ch = 32 * ks + 8 * kb + 2 * m, q = kPos2[4 * tau + ks];
                        const int sw = q == 7 ? 1 : 0;
                        word |= (uint32_t)kx[tok * RS + ch + sw] << (2 * q);
                        word |= (uint32_t)kx[tok * RS + ch + 1 - sw] << (16 + 2 * q);
                    }
                }
            } else {
                const int tau = w / 4, ks = w % 4;
                const int tok = row_of(cc, 16 * tau + n);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int ch = 32 * ks + 8 * kb + 2 * m;
                    word |= (uint32_t)kx[tok * RS + ch] << (4 * m);
                    word |= (uint32_t)kx[tok * RS + ch + 1] << (16 + 4 * m);
                }
            }
        } else {
            // lane (channel n of each 16-channel tile nt, token block kb): slot s
            // holds token 16*(s/4) + 4*kb + s%4; slots {2m, 2m+1} share a word.
            // The position inside the word depends on the tile only (b = 2: word
            // m, position kPos2[nt]; b = 4: word 4*(nt/4) + m, nibble nt%4), so
            // that every operand of one tile carries the same power-of-two weight.
            const int m = w % 4;
            const int sa = 2 * m, sb = 2 * m + 1;
            const int ta = row_of(cc, 16 * (sa / 4) + 4 * kb + sa % 4);
            const int tb = row_of(cc, 16 * (sb / 4) + 4 * kb + sb % 4);
            if (BITS == 2) {
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) {
                    const int c = 16 * nt + n, q = kPos2[nt];
                    const int xa = q == 7 ? tb : ta, xb = q == 7 ? ta : tb;
                    word |= (uint32_t)vx[xa * RS + c] << (2 * q);
                    word |= (uint32_t)vx[xb * RS + c] << (16 + 2 * q);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = 16 * (4 * (w / 4) + j) + n;
                    word |= (uint32_t)vx[ta * RS + c] << (4 * j);
                    word |= (uint32_t)vx[tb * RS + c] << (16 + 4 * j);
                }
            }
        }
        const int64_t chunk = kHalf ? g / 2 : g * CPG + cc;
        const int64_t base = ((int64_t)u * v.chunks + chunk) * WPC;
        if (kHalf && BITS == 2 && !isv) {
            // keep the other half's codes: tile 1 - hf sits at the 2-bit
            // positions kPos2[4 (1 - hf) + ks] of both 16-bit halves
            uint32_t keep = 0;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int q = kPos2[4 * (1 - hf) + ks];
                keep |= (3u << (2 * q)) | (3u << (16 + 2 * q));
            }
            word |= v.kq[base + o] & keep;
        }
        (isv ? v.vq : v.kq)[base + o] = word;
    }
}

// One block per (unit, group), units fastest so that the blocks resident at
// once spread over all units (and their counter words); in mode 2 one block
// per (unit, batch of kRepairBatch groups), repacking only the groups whose
// tokens the scan admitted to the pool (a small share).
constexpr int kRepairBatch = 4;
template <int BITS, int G>
__global__ __launch_bounds__(pack_threads<G>()) __attribute__((amdgpu_waves_per_eu(G == 128 ? 8 : 1)))
void pack_kernel(CacheView v, const uint16_t* knew,
                                                   const uint16_t* vnew, int64_t t_old,
                                                   int32_t n_new, int64_t g0, int32_t gstride,
                                                   int64_t ng, int32_t mode) {
    constexpr bool kHalf = G == 16;
    constexpr int CPG = kHalf ? 1 : G / kChunk;
    const int u = (int)(blockIdx.x % (uint32_t)v.units);
    const int64_t b = blockIdx.x / (uint32_t)v.units;
    // The unit's largest value scale so far, read at device scope (past this
    // XCD's L2, where the atomics of the pack do not land); a block only
    // raises it with an atomic when its own maximum is larger. A stale value
    // costs one atomic, no more.
    const uint32_t vmax_seen =
        threadIdx.x == 0
            ? __hip_atomic_load(reinterpret_cast<const uint32_t*>(v.counters) + (int64_t)u * 4 + 3,
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
            : 0u;
    if (mode != 2) {
        pack_group<BITS, G>(v, knew, vnew, t_old, n_new, u, g0 + gstride * b, mode, vmax_seen);
        return;
    }
    // lane j of every wavefront reads the pool mask words of the batch's
    // group j at once; one ballot lists the groups to repack
    static_assert(kRepairBatch <= 64, "one lane per group of the batch");
    const int lane = threadIdx.x & 63;
    bool admitted = false;
    if (lane < kRepairBatch && b * kRepairBatch + lane < ng) {
        const int64_t g = g0 + gstride * (b * kRepairBatch + lane), t0 = g * G;
#pragma unroll
        for (int c = 0; c < CPG; ++c) {
            uint32_t w = v.mask[(int64_t)u * v.chunks + t0 / kChunk + c];
            if (kHalf) w = (w >> (16 * (int)(g & 1))) & 0xFFFFu;
            admitted |= w != 0;
        }
    }
    uint64_t todo = __ballot(admitted);
    while (todo) {
        const int j = __builtin_ctzll(todo);
        todo &= todo - 1;
        __syncthreads();  // the previous group's LDS reads are done
        pack_group<BITS, G>(v, knew, vnew, t_old, n_new, u, g0 + gstride * (b * kRepairBatch + j),
                            2, vmax_seen);
    }
}

// FP8 E4M3 code of an fp32 value, exactly: round to nearest, ties to even,
// saturating at +-448 (OCP E4M3: bias 7, no infinity, S.1111.111 is NaN;
// "KV cache quantization and eviction", sections "FP8, KIVI and KVQuant" and
// "Failure modes and how to detect them": casts must saturate). Every step
// below is exact in fp32 except the final rounding to the 3-bit mantissa.
__device__ __forceinline__ uint32_t e4m3_sat(float x) {
    const uint32_t sign = (__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u;
    const float a = fabsf(x);
    if (a != a) return sign | 0x7Fu;
    if (a >= 448.0f) return sign | 0x7Eu;
    if (a < 0x1p-6f) return sign | (uint32_t)rintf(a * 512.0f);  // subnormal steps of 2^-9
    int e = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xFF) - 127;  // a is a normal fp32
    const float mant = ldexpf(a, -e);                                    // in [1, 2)
    uint32_t m = (uint32_t)rintf((mant - 1.0f) * 8.0f);
    if (m == 8) {
        m = 0;
        ++e;
    }
    return sign | (uint32_t)((e + 7) << 3) | m;
}

// Correctly rounded fp32 quotient x / s from y = RN(1 / s): q0 = RN(x y) is
// within 1.5 ulp of x / s; one correction q1 = RN(q0 + r0 y), with the exact
// residual r0 = x - q0 s (one FMA), is within one ulp, and a second
// correction then rounds correctly (Markstein's theorem for a correctly
// rounded reciprocal and a quotient within one ulp). With |x| <= 65504 and
// 2^-100 <= s <= 2^100 nothing overflows and the residuals stay normal or 0.
__device__ __forceinline__ float div_rn(float x, float s, float y) {
    const float q0 = x * y;
    const float q1 = fmaf(fmaf(-q0, s, x), y, q0);
    return fmaf(fmaf(-q1, s, x), y, q1);
}

// E4M3 code of a finite x / s, saturating: the magnitude's quotient, clamped
// to 448, converted by the hardware's round-to-nearest-even conversion, with
// the sign of x (so -0 keeps its sign). Two codes per call, into bytes 2 hi,
// 2 hi + 1 of w.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t w, float x0, float x1, float s, float y) {
    const float a0 = copysignf(fminf(div_rn(fabsf(x0), s, y), 448.0f), x0);
    const float a1 = copysignf(fminf(div_rn(fabsf(x1), s, y), 448.0f), x1);
    return __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, w, HI);
}

// FP8 codec: one block per (unit, 32-token chunk). Keys and values are
// encoded element by element as E4M3(x / s) with the KV head's scales and
// written in the decoder's operand order: 4 KB per chunk and tensor, lane l
// of 16-byte group w at byte w * 1024 + l * 16. A wavefront whose elements
// are all finite, with scales in [2^-100, 2^100], takes the reciprocal
// quotient and the hardware conversion; any other takes the IEEE division
// and the encoder above (the same codes).
//   keys:   group w = 2 tau + ks / 2; bytes 8 (ks % 2) + e hold channel
//           32 ks + 8 (l / 16) + e of token 16 tau + l % 16;
//   values: group w; bytes 8 i + sl hold channel 16 (2 w + i) + l % 16 of
//           token 16 (sl / 4) + 4 (l / 16) + sl % 4.
__global__ __launch_bounds__(256) void pack8_kernel(CacheView v, const uint16_t* knew,
                                                    const uint16_t* vnew, int64_t t_old,
                                                    int32_t n_new, int64_t c0) {
    __shared__ __align__(16) uint16_t kx[kChunk][kPackRow], vx[kChunk][kPackRow];
    const int u = (int)(blockIdx.x % (uint32_t)v.units), tid = threadIdx.x;
    const int64_t ch = c0 + blockIdx.x / (uint32_t)v.units, t0 = ch * kChunk;
    {
        uint4 kr[2], vr[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid + 256 * j, i = e / 16, part = e % 16;
            kr[j] = reinterpret_cast<const uint4*>(src_row(v.kring, knew, v, u, t0 + i, t_old, n_new))[part];
            vr[j] = reinterpret_cast<const uint4*>(src_row(v.vring, vnew, v, u, t0 + i, t_old, n_new))[part];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid + 256 * j, i = e / 16, part = e % 16;
            reinterpret_cast<uint4*>(&kx[i][0])[part] = kr[j];
            reinterpret_cast<uint4*>(&vx[i][0])[part] = vr[j];
        }
    }
    __syncthreads();
    const int hk = u % v.n_kv_heads;
    const float sk = v.fp8_scales[2 * hk], sv = v.fp8_scales[2 * hk + 1];
    const int w = tid / 64, l = tid % 64, n = l % 16, kb = l / 16;
    float xk[16], xv[16];
    bool special = false;
#pragma unroll
    for (int byte = 0; byte < 16; ++byte) {
        // key byte: k-step ks = 2 (w % 2) + byte / 8, element e = byte % 8
        const int tau = w / 2, ks = 2 * (w % 2) + byte / 8, e = byte % 8;
        xk[byte] = h2f(kx[16 * tau + n][32 * ks + 8 * kb + e]);
        // value byte: tile 2 w + byte / 8, token slot sl = byte % 8
        const int nt = 2 * w + byte / 8, sl = byte % 8;
        xv[byte] = h2f(vx[16 * (sl / 4) + 4 * kb + sl % 4][16 * nt + n]);
        special |= !__builtin_isfinite(xk[byte]) || !__builtin_isfinite(xv[byte]);
    }
    uint32_t kw[4] = {0, 0, 0, 0}, vw[4] = {0, 0, 0, 0};
    const bool in_range = sk >= 0x1p-100f && sk <= 0x1p100f && sv >= 0x1p-100f && sv <= 0x1p100f;
    if (in_range && !__any(special)) {
        const float yk = 1.0f / sk, yv = 1.0f / sv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kw[i] = e4m3_pair<false>(0u, xk[4 * i], xk[4 * i + 1], sk, yk);
            kw[i] = e4m3_pair<true>(kw[i], xk[4 * i + 2], xk[4 * i + 3], sk, yk);
            vw[i] = e4m3_pair<false>(0u, xv[4 * i], xv[4 * i + 1], sv, yv);
            vw[i] = e4m3_pair<true>(vw[i], xv[4 * i + 2], xv[4 * i + 3], sv, yv);
        }
    } else {
#pragma unroll
        for (int byte = 0; byte < 16; ++byte) {
            kw[byte / 4] |= e4m3_sat(xk[byte] / sk) << (8 * (byte % 4));
            vw[byte / 4] |= e4m3_sat(xv[byte] / sv) << (8 * (byte % 4));
        }
    }
    const int64_t base = ((int64_t)u * v.chunks + ch) * 1024 + w * 256 + l * 4;  // words
    *reinterpret_cast<uint4*>(v.kq + base) = make_uint4(kw[0], kw[1], kw[2], kw[3]);
    *reinterpret_cast<uint4*>(v.vq + base) = make_uint4(vw[0], vw[1], vw[2], vw[3]);
}

// Copy the appended rows that are attention sinks (tokens t_old .. t_old +
// n_sink - 1 of the sequence, the first rows of each unit's input) to the
// sink region.
__global__ __launch_bounds__(256) void sink_store_kernel(CacheView v, const uint16_t* knew,
                                                         const uint16_t* vnew, int64_t t_old,
                                                         int32_t n_new, int32_t n_sink) {
    const int u = blockIdx.y;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (int64_t)n_sink * 16) return;
    const int64_t i = e / 16;
    const int part = (int)(e % 16);
    const int64_t src = ((int64_t)u * n_new + i) * D;
    const int64_t dst = ((int64_t)u * v.sinks + t_old + i) * D;
    reinterpret_cast<uint4*>(v.sink_k + dst)[part] = reinterpret_cast<const uint4*>(knew + src)[part];
    reinterpret_cast<uint4*>(v.sink_v + dst)[part] = reinterpret_cast<const uint4*>(vnew + src)[part];
}

// Copy this call's tokens that stay fp16 into the residual ring (slot t % RB).
__global__ __launch_bounds__(256) void ring_store_kernel(CacheView v, const uint16_t* knew,
                                                         const uint16_t* vnew, int64_t t_old,
                                                         int32_t n_new, int64_t ts, int64_t ntok) {
    const int u = blockIdx.y;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= ntok * 16) return;
    const int64_t t = ts + e / 16;
    const int part = (int)(e % 16);
    const int64_t src = ((int64_t)u * n_new + (t - t_old)) * D;
    const int64_t dst = ((int64_t)u * v.ring_slots + t % v.ring_slots) * D;
    reinterpret_cast<uint4*>(v.kring + dst)[part] = reinterpret_cast<const uint4*>(knew + src)[part];
    reinterpret_cast<uint4*>(v.vring + dst)[part] = reinterpret_cast<const uint4*>(vnew + src)[part];
}

// Canonical view: one byte per code, [unit][token][channel] (a null output is skipped).
__global__ __launch_bounds__(256) void unpack_kernel(CacheView v, int64_t n_q, uint8_t* kc,
                                                     uint8_t* vc) {
    const int64_t total = (int64_t)v.units * n_q * D;
    const int b = v.bits;
    const int wpc = 128 * b;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(e % D);
        const int64_t t = (e / D) % n_q;
        const int u = (int)(e / (D * n_q));
        const int64_t chunk = t / kChunk;
        const int tt = (int)(t % kChunk);
        const uint32_t* kbase = v.kq + ((int64_t)u * v.chunks + chunk) * wpc;
        const uint32_t* vbase = v.vq + ((int64_t)u * v.chunks + chunk) * wpc;
        const uint32_t mask = (1u << b) - 1;
        if (b == 8) {
            // FP8: byte offsets inside the chunk's 4 KB (see pack8_kernel)
            const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(kbase);
            const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(vbase);
            const int tau = tt / 16, n = tt % 16, ks = c / 32, kbl = (c % 32) / 8, e8 = c % 8;
            const int kw = 2 * tau + ks / 2, kl = n + 16 * kbl;
            if (kc) kc[e] = kb8[kw * 1024 + kl * 16 + 8 * (ks % 2) + e8];
            const int nt = c / 16, cn = c % 16, r16 = tt % 16, vkb = r16 / 4;
            const int sl = 4 * tau + r16 % 4, vl = cn + 16 * vkb;
            if (vc) vc[e] = vb8[(nt / 2) * 1024 + vl * 16 + 8 * (nt % 2) + sl];
            continue;
        }
        {   // key code
            const int tau = tt / 16, row = tt % 16;
            const int ks = c / 32, kb = (c % 32) / 8, s = c % 8, m = s / 2, hi = s % 2;
            const int l = row + 16 * kb;
            int w, bit;
            if (b == 2) {
                const int q = kPos2[4 * tau + ks];
                w = m;
                bit = 2 * q + 16 * (q == 7 ? 1 - hi : hi);
            } else {
                w = 4 * tau + ks;
                bit = 4 * m + 16 * hi;
            }
            if (kc) kc[e] = (uint8_t)((kbase[(w / 4) * 256 + l * 4 + w % 4] >> bit) & mask);
        }
        {   // value code
            const int tau = tt / 16, r16 = tt % 16, kb = r16 / 4, s = 4 * tau + r16 % 4;
            const int m = s / 2, hi = s % 2, nt = c / 16, n = c % 16;
            const int l = n + 16 * kb;
            int w, bit;
            if (b == 2) {
                const int q = kPos2[nt];
                w = m;
                bit = 2 * q + 16 * (q == 7 ? 1 - hi : hi);
            }
            else { w = 4 * (nt / 4) + m; bit = 4 * (nt % 4) + 16 * hi; }
            if (vc) vc[e] = (uint8_t)((vbase[(w / 4) * 256 + l * 4 + w % 4] >> bit) & mask);
        }
    }
}

// The rest of the canonical view: scale/zero words split into fp16 arrays,
// pool marks as bytes, residual rows in token order. One thread per output
// element of the largest array it serves.
__global__ __launch_bounds__(256) void debug_view_kernel(CacheView v, int64_t T, int64_t n_q,
                                                         kvq_debug_view o) {
    const int G = v.group, NG = D / (G < D ? G : D);
    const int64_t KG = n_q / G, nres = T - (T < v.sinks ? T : v.sinks) - n_q;
    const int64_t nk = (int64_t)v.units * KG * D, nv = (int64_t)v.units * n_q * NG;
    const int64_t np = (int64_t)v.units * n_q, nr = (int64_t)v.units * nres * D;
    const int64_t n = nk > nv ? nk : nv;
    const int64_t m = (np > nr ? np : nr) > n ? (np > nr ? np : nr) : n;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < m;
         e += (int64_t)gridDim.x * blockDim.x) {
        if (e < nk && (o.kscale || o.kzero)) {
            const int64_t u = e / (KG * D), r = e % (KG * D);
            const uint32_t w = v.kmeta[u * v.key_groups * D + r];
            if (o.kscale) o.kscale[e] = (uint16_t)(w & 0xFFFF);
            if (o.kzero) o.kzero[e] = (uint16_t)(w >> 16);
        }
        if (e < nv && (o.vscale || o.vzero)) {
            const int64_t u = e / (n_q * NG), t = (e / NG) % n_q, gq = e % NG;
            const uint32_t w =
                v.vmeta[((u * v.chunks + t / kChunk) * NG + gq) * kChunk + t % kChunk];
            if (o.vscale) o.vscale[e] = (uint16_t)(w & 0xFFFF);
            if (o.vzero) o.vzero[e] = (uint16_t)(w >> 16);
        }
        if (e < np && o.pooled) {
            const int64_t u = e / n_q, t = e % n_q;
            o.pooled[e] = (uint8_t)((v.mask[u * v.chunks + t / kChunk] >> (t % kChunk)) & 1u);
        }
        if (e < nr && (o.kres || o.vres)) {
            const int64_t u = e / (nres * D), i = (e / D) % nres, c = e % D;
            const int64_t src = (u * v.ring_slots + (n_q + i) % v.ring_slots) * D + c;  // ring token n_q + i
            if (o.kres) o.kres[e] = v.kring[src];
            if (o.vres) o.vres[e] = v.vring[src];
        }
    }
}

// One H2O eviction step. If more than `budget` tokens of a unit are live,
// the live token in [S, T - recent) with the lowest score is evicted ("H2O:
// Heavy-Hitter Oracle", greedy eviction; "KV cache quantization and
// eviction", h2o_evict). Scores compare through an order-preserving key with
// every NaN lowest and -0 equal to +0; the smallest (key, index) wins, so ties
// go to the older token. A unit's range is cut into slices of
// kEvictThreads x kEvictGroups 4-token groups, one 256-thread workgroup each
// (every compute unit pulls part of the scores: one workgroup per unit would
// leave most idle). Each thread reads four consecutive scores at a time
// (16-byte loads when the row allows it), all of its loads in flight before
// any is compared. A workgroup folds its minimum into the unit's scratch word
// with an atomic maximum of the complement, then takes a ticket; the unit's
// last workgroup reads the result, resets the scratch and marks the token.
__device__ __forceinline__ uint64_t evict_key(float f, int64_t t) {
    uint32_t b = __builtin_bit_cast(uint32_t, f);
    uint32_t key;
    if (f != f) {
        key = 0u;  // NaN: lowest
    } else {
        if (f == 0.0f) b = 0u;  // -0 == +0
        key = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    }
    return ((uint64_t)key << 32) | (uint64_t)t;
}

constexpr int kEvictThreads = 256;
constexpr int kEvictGroups = 8;  // 4-token groups per thread
constexpr int64_t kEvictSlice = (int64_t)kEvictThreads * kEvictGroups;
__global__ __launch_bounds__(kEvictThreads) void evict_step_kernel(CacheView v, int64_t T,
                                                                   const float* acc, int32_t budget,
                                                                   int32_t recent) {
    const int u = blockIdx.x, tid = threadIdx.x;  // slice blockIdx.y of unit u
    const int64_t live = T - v.evict_count[u];
    if (live <= budget) return;  // uniform over the unit's workgroups
    const int64_t S = v.sinks, end = T - recent;
    const uint32_t* ev = v.evict + (int64_t)u * v.evict_words;
    const float* sc = acc + (int64_t)u * T;
    uint64_t best = ~0ull;
    // groups of 4 tokens t = 4 g .. 4 g + 3 (sequence indices); this
    // workgroup's slice starts at group gs
    const int64_t g_first = S / 4, g_end = (end + 3) / 4;
    const int64_t gs = g_first + (int64_t)blockIdx.y * kEvictSlice;
    const bool aligned = (T % 4) == 0;  // row start 16-byte aligned
    const bool any_evicted = v.evict_count[u] != 0;
    {
        float4 x[kEvictGroups];
        uint32_t ew0[kEvictGroups], ew1[kEvictGroups];  // eviction words of a group's first and last token
#pragma unroll
        for (int k = 0; k < kEvictGroups; ++k) {
            const int64_t g = gs + tid + (int64_t)k * kEvictThreads;
            if (g < g_end && aligned && 4 * g + 3 < T) {
                x[k] = reinterpret_cast<const float4*>(sc)[g];
            } else {
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = g < g_end && 4 * g + e < T ? sc[4 * g + e] : 0.f;
                x[k] = make_float4(y[0], y[1], y[2], y[3]);
            }
            // the group's first and last token inside the row (indices after the sinks)
            const int64_t ta = 4 * g - S, tb = (4 * g + 3 < T ? 4 * g + 3 : T - 1) - S;
            ew0[k] = any_evicted && g < g_end && ta >= 0 ? ev[ta >> 5] : 0u;
            ew1[k] = any_evicted && g < g_end && tb >= 0 ? ev[tb >> 5] : 0u;
        }
#pragma unroll
        for (int k = 0; k < kEvictGroups; ++k) {
            const int64_t g = gs + tid + (int64_t)k * kEvictThreads;
            if (g >= g_end) break;
            const float y[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t t = 4 * g + e;
                if (t < S || t >= end) continue;
                const int64_t tau = t - S;
                const uint32_t w = (tau >> 5) == ((4 * g - S) >> 5) ? ew0[k] : ew1[k];
                if ((w >> (tau & 31)) & 1u) continue;
                const uint64_t kk = evict_key(y[e], t);
                best = kk < best ? kk : best;
            }
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor(best, off);
        best = o < best ? o : best;
    }
    __shared__ uint64_t wbest[kEvictThreads / 64];
    if ((tid & 63) == 0) wbest[tid >> 6] = best;
    __syncthreads();
    if (tid == 0) {
        uint64_t b = wbest[0];
        for (int w = 1; w < kEvictThreads / 64; ++w) b = wbest[w] < b ? wbest[w] : b;
        uint64_t* scr = evict_scratch(v) + 2 * u;
        // device-scope atomics: performed where every die sees them; the
        // maximum has returned (so it is performed) before the ticket is taken
        const uint64_t prev =
            __hip_atomic_fetch_max(&scr[0], ~b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" ::"v"(prev) : "memory");
        const uint64_t ticket =
            __hip_atomic_fetch_add(&scr[1], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (ticket == gridDim.y - 1) {
            // the unit's last workgroup: every other one has folded its minimum
            const uint64_t nb = __hip_atomic_exchange(&scr[0], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&scr[1], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (nb != 0ull) {
                const int64_t tau = (int64_t)((~nb) & 0xFFFFFFFFu) - S;
                uint32_t* word = v.evict + (int64_t)u * v.evict_words + (tau >> 5);
                *word |= 1u << (tau & 31);
                v.evict_count[u] += 1;
            }
        }
    }
}

// Read-only streaming pass over a buffer, the memory ceiling the decode kernel
// is compared with: every 16-byte word is loaded once (eight loads in flight
// per thread), folded with XOR so no load can be dropped, one word written per
// block.
constexpr int kStreamBlocks = 4096;
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* buf, int64_t n16,
                                                          uint32_t* sink) {
    uint32_t f = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < n16; i0 += 8 * stride) {
        uint4 x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t i = i0 + k * stride;
            x[k] = i < n16 ? buf[i] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) f ^= x[k].x ^ x[k].y ^ x[k].z ^ x[k].w;
    }
    for (int off = 32; off > 0; off >>= 1) f ^= __shfl_xor(f, off);
    __shared__ uint32_t wf[4];
    if ((threadIdx.x & 63) == 0) wf[threadIdx.x >> 6] = f;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = wf[0] ^ wf[1] ^ wf[2] ^ wf[3];
}

// Pool and extra-pool indices of the canonical view: sequence indices, i.e.
// the stored index (counted from the first token after the sinks) plus S.
__global__ __launch_bounds__(256) void index_view_kernel(int32_t* dst, const int32_t* src,
                                                         int64_t n, int32_t add) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x)
        dst[e] = src[e] + add;
}

// Liveness of the canonical view: [U][T] bytes, 0 for evicted tokens.
__global__ __launch_bounds__(256) void live_view_kernel(CacheView v, int64_t T, uint8_t* live) {
    const int64_t n = (int64_t)v.units * T;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t u = e / T, t = e % T, tau = t - v.sinks;
        live[e] = tau < 0 ? 1
                          : (uint8_t)(((v.evict[u * v.evict_words + (tau >> 5)] >> (tau & 31)) & 1u) ^ 1u);
    }
}

// Sink rows of the canonical view: [U][rows][d] from the sink region [U][S][d].
__global__ __launch_bounds__(256) void sink_view_kernel(CacheView v, int32_t rows, uint16_t* kd,
                                                        uint16_t* vd) {
    const int64_t n = (int64_t)v.units * rows * D;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t u = e / ((int64_t)rows * D), r = e % ((int64_t)rows * D);
        const int64_t src = u * v.sinks * D + r;
        if (kd) kd[e] = v.sink_k[src];
        if (vd) vd[e] = v.sink_v[src];
    }
}

template <int BITS, int G>
hipError_t launch_pack_t(const CacheView& v, const uint16_t* kn, const uint16_t* vn, int64_t t_old,
                         int32_t n_new, int64_t g0, int64_t ng, hipStream_t s, int32_t gstride,
                         int32_t mode) {
    const size_t lds = 2 * (size_t)G * kPackRow * sizeof(uint16_t);
    // the dynamic LDS limit is raised once per process; a failure is reported
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(pack_kernel<BITS, G>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    // one block per (unit, group) or, in mode 2, per (unit, batch of groups),
    // units fastest; at most 2^22 blocks a launch. ng groups g0, g0 + gstride, ...
    const int64_t per = mode == 2 ? kRepairBatch : 1;
    const int64_t step = ((int64_t)1 << 22 >= v.units ? ((int64_t)1 << 22) / v.units : 1) * per;
    for (int64_t gs = 0; gs < ng; gs += step) {
        const int64_t n = ng - gs < step ? ng - gs : step;
        hipLaunchKernelGGL((pack_kernel<BITS, G>), dim3((unsigned)((n + per - 1) / per * v.units)),
                           dim3(pack_threads<G>()), lds, s, v, kn, vn, t_old, n_new, g0 + gs * gstride,
                           gstride, n, mode);
    }
    return hipSuccess;
}

// Every group g0 .. g1 - 1 of an append through pack_kernel in `mode`. With
// G = 16 the even groups, then the odd ones: the two halves of a chunk are
// never written by one launch.
hipError_t launch_pack_groups(const CacheView& v, const uint16_t* kn, const uint16_t* vn,
                              int64_t t_old, int32_t n_new, int64_t g0, int64_t g1, hipStream_t s,
                              int32_t mode) {
    const int G = v.group;
    const int64_t ng = g1 - g0;
    if (G == 16) {
        const int64_t ge = g0 + (g0 & 1), go = g0 + 1 - (g0 & 1);
        const int64_t ne = ge < g1 ? (g1 - ge + 1) / 2 : 0, no = go < g1 ? (g1 - go + 1) / 2 : 0;
        hipError_t e = hipSuccess;
        for (int pass = 0; pass < 2 && e == hipSuccess; ++pass) {
            const int64_t gp = pass == 0 ? ge : go, np = pass == 0 ? ne : no;
            if (np == 0) continue;
            e = v.bits == 2 ? launch_pack_t<2, 16>(v, kn, vn, t_old, n_new, gp, np, s, 2, mode)
                            : launch_pack_t<4, 16>(v, kn, vn, t_old, n_new, gp, np, s, 2, mode);
        }
        return e;
    }
#define KVQ_PACK(B_, G_)                                                                  \
    if (v.bits == B_ && G == G_) return launch_pack_t<B_, G_>(v, kn, vn, t_old, n_new, g0, ng, s, 1, mode);
    KVQ_PACK(2, 32) KVQ_PACK(2, 64) KVQ_PACK(2, 128)
    KVQ_PACK(4, 32) KVQ_PACK(4, 64) KVQ_PACK(4, 128)
#undef KVQ_PACK
    return hipErrorInvalidValue;
}

}  // namespace

int launch_init(const CacheView& v, void* stream) {
    (void)hipGetLastError();  // an error left by an earlier call is not this call's
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n = (int64_t)v.units * (4 + v.chunks + v.evict_words + 1);
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(init_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0,
                       s, v);
    return (int)hipGetLastError();
}

int launch_append(const CacheView& v, const uint16_t* kn, const uint16_t* vn, int64_t t_seq,
                  int32_t n_new, int64_t nq_old, int64_t nq_new, void* stream, bool ring_store) {
    (void)hipGetLastError();  // an error left by an earlier call is not this call's
    hipStream_t s = static_cast<hipStream_t>(stream);
    // Attention sinks first: rows of tokens below S go to the sink region.
    const int64_t S = v.sinks;
    const int32_t n_sink = t_seq < S ? (int32_t)(S - t_seq < n_new ? S - t_seq : n_new) : 0;
    if (n_sink > 0) {
        hipLaunchKernelGGL(sink_store_kernel, dim3((unsigned)((n_sink * 16 + 255) / 256), v.units),
                           dim3(256), 0, s, v, kn, vn, t_seq, n_new, n_sink);
        if (n_sink == n_new) return (int)hipGetLastError();
    }
    // The rest is a cache of the tokens after the sinks, in its own token
    // numbering tau = t - S. Its rows sit n_sink rows into each unit's input
    // (unit stride n_new): with n_sink > 0 that cache was empty, and the
    // kernels address fresh row tau of the input at tau - t_old = tau + n_sink.
    const int64_t t_old = (t_seq > S ? t_seq - S : 0) - n_sink;
    const int G = v.group;
    const int64_t g0 = nq_old / G, g1 = nq_new / G, ng = g1 - g0;
    if (ng > 0) {
        hipError_t e = hipSuccess;
        if (v.bits == 8) {
            // FP8 codec: one block per (unit, chunk); ng groups of 32 tokens
            hipLaunchKernelGGL(pack8_kernel, dim3((unsigned)(ng * v.units)), dim3(256), 0, s, v, kn,
                               vn, t_old, n_new, g0);
        } else {
            // With a pool: first pass with scores, the scan, then the repair
            // pass; otherwise one pass.
            const int npass = v.pool > 0 ? 2 : 1;
            for (int pass = 0; pass < npass && e == hipSuccess; ++pass) {
                const int32_t mode = v.pool > 0 ? 1 + pass : 0;
                if (pass == 1)
                    hipLaunchKernelGGL(ott_scan_kernel, dim3(v.units), dim3(64), 0, s, v, kn, vn,
                                       t_old, n_new, g0, g1);
                e = launch_pack_groups(v, kn, vn, t_old, n_new, g0, g1, s, mode);
            }
        }
        if (e != hipSuccess) return (int)e;
    }
    const int64_t ts = t_old > nq_new ? t_old : nq_new, te = t_old + n_new;
    if (ring_store && te > ts) {
        const int64_t ntok = te - ts;
        hipLaunchKernelGGL(ring_store_kernel, dim3((unsigned)((ntok * 16 + 255) / 256), v.units),
                           dim3(256), 0, s, v, kn, vn, t_old, n_new, ts, ntok);
    }
    return (int)hipGetLastError();
}

int launch_unpack(const CacheView& v, int64_t n_q, uint8_t* kc, uint8_t* vc, void* stream) {
    (void)hipGetLastError();  // an error left by an earlier call is not this call's
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t total = (int64_t)v.units * n_q * D;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, v, n_q, kc, vc);
    return (int)hipGetLastError();
}

int launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    (void)hipGetLastError();  // an error left by an earlier call is not this call's
    hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamBlocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf),
                       (int64_t)(bytes / 16), sink);
    return (int)hipGetLastError();
}

int launch_fp8_scales(const CacheView& v, const float* scales, void* stream) {
    (void)hipGetLastError();  // an error left by an earlier call is not this call's
    return (int)hipMemcpyAsync(v.fp8_scales, scales, (size_t)v.n_kv_heads * 2 * sizeof(float),
                               hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream));
}

int launch_evict_step(const CacheView& v, int64_t T, const float* acc, int32_t budget,
                      int32_t recent, void* stream) {
    (void)hipGetLastError();  // an error left by an earlier call is not this call's
    hipStream_t s = static_cast<hipStream_t>(stream);
    // slices of the groups [S / 4, (T - recent + 3) / 4), at least one per unit
    const int64_t groups = (T - recent + 3) / 4 - v.sinks / 4;
    const int64_t slices = groups > kEvictSlice ? (groups + kEvictSlice - 1) / kEvictSlice : 1;
    hipLaunchKernelGGL(evict_step_kernel, dim3(v.units, (unsigned)slices), dim3(kEvictThreads), 0, s, v,
                       T, acc, budget, recent);
    return (int)hipGetLastError();
}

int launch_debug_unpack(const CacheView& v, int64_t T, int64_t n_q, const kvq_debug_view& o,
                        void* stream) {
    (void)hipGetLastError();  // an error left by an earlier call is not this call's
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n_q > 0 && (o.kcodes || o.vcodes)) {
        const int64_t total = (int64_t)v.units * n_q * D;
        int64_t blocks = (total + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, v, n_q,
                           o.kcodes, o.vcodes);
    }
    {
        const int64_t KG = n_q / v.group, NG = D / (v.group < D ? v.group : D);
        const int64_t ns = T < v.sinks ? T : v.sinks;
        int64_t m = (int64_t)v.units * KG * D;
        const int64_t m2 = (int64_t)v.units * n_q * NG, m3 = (int64_t)v.units * (T - ns - n_q) * D;
        if (m2 > m) m = m2;
        if (m3 > m) m = m3;
        if (v.bits == 8) m = m3 > (int64_t)v.units * n_q ? m3 : (int64_t)v.units * n_q;  // no meta
        kvq_debug_view oo = o;
        if (v.bits == 8) oo.kscale = oo.kzero = oo.vscale = oo.vzero = nullptr;
        if (m > 0 && (oo.kscale || oo.kzero || oo.vscale || oo.vzero || oo.pooled || oo.kres || oo.vres)) {
            int64_t blocks = (m + 255) / 256;
            if (blocks > 65536) blocks = 65536;
            hipLaunchKernelGGL(debug_view_kernel, dim3((unsigned)blocks), dim3(256), 0, s, v, T, n_q,
                               oo);
        }
    }
    const size_t U = (size_t)v.units, N = (size_t)v.pool, E = (size_t)v.evict_cap;
    const int32_t ns = (int32_t)(T < v.sinks ? T : v.sinks);
    if (o.live && U * T)
        hipLaunchKernelGGL(live_view_kernel, dim3((unsigned)((U * T + 255) / 256)), dim3(256), 0, s,
                           v, T, o.live);
    if (ns > 0 && (o.ksink || o.vsink))
        hipLaunchKernelGGL(sink_view_kernel, dim3((unsigned)((U * ns * D + 255) / 256)), dim3(256),
                           0, s, v, ns, o.ksink, o.vsink);
    if (o.pool_idx && U * N)
        hipLaunchKernelGGL(index_view_kernel, dim3((unsigned)((U * N + 255) / 256)), dim3(256), 0,
                           s, o.pool_idx, v.pool_idx, (int64_t)(U * N), v.sinks);
    if (o.ev_idx && U * E)
        hipLaunchKernelGGL(index_view_kernel, dim3((unsigned)((U * E + 255) / 256)), dim3(256), 0,
                           s, o.ev_idx, v.ev_idx, (int64_t)(U * E), v.sinks);
    struct {
        void* dst;
        const void* src;
        size_t bytes;
    } cp[] = {
        {o.counters, v.counters, U * 4 * 4},     {o.pool_score, v.pool_score, U * N * 8},
        {o.pool_k, v.pool_k, U * N * D * 2},     {o.pool_v, v.pool_v, U * N * D * 2},
        {o.ev_k, v.ev_k, U * E * D * 2},         {o.ev_v, v.ev_v, U * E * D * 2},
    };
    for (const auto& c : cp) {
        if (!c.dst || c.bytes == 0) continue;
        const hipError_t e = hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return (int)e;
    }
    return (int)hipGetLastError();
}

}  // namespace kvq

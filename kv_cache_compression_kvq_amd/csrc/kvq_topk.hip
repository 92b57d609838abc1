// Heavy-hitter selection on gfx950: per row of fp32 scores keep the k largest
// among indices [0, T - w) plus the w most recent indices (MiniKV,
// Algorithm 1, heavy-hitter selection; "KV cache quantization and eviction",
// section "Minimal implementation": evicting the lowest-scoring non-recent
// token one at a time with a first-occurrence argmin leaves, on fixed scores,
// the k largest with ties going to the larger index).
//
// Without a workspace: one 1024-thread workgroup per row. Scores become
// order-preserving 32-bit keys. Rows of up to 32768 keys are held in registers
// (16 or 32 keys per thread, all loads in flight at once); a radix select over
// key - min(key) with 11-bit digits from the top of the row's key range
// finds the k-th largest key tau and how many keys equal to tau are kept.
// Taking digits from the row's own range spreads the first histogram over
// more bins than the fixed top bits would and needs fewer passes when the
// range is short. The first pass's bins spread well enough for plain LDS
// atomics; the keys left for the later passes lie close together, and lanes
// of a wavefront that share a bin there add once, by their count. Each
// wavefront owns a contiguous index range and writes its kept indices in
// ascending order from ballot prefix counts.
// Longer rows are read from memory in every pass, with a candidate list after
// the first digit.
// With a workspace, rows are split over several workgroups (below) where one
// workgroup per row would leave compute units idle, and always when they are
// longer than the register kernels hold.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;  // histogram bins (11-bit digits)
constexpr int kCand = 4096;  // candidate list after the first digit (long rows)
constexpr int kFast = 512;   // first-digit bin resolved by one wavefront (register rows)
constexpr int kMaxRegKeys = 32 * kThreads;  // rows held in registers

// Order-preserving key of a score, in [0, 0xFF800000]: -0 and +0 compare
// equal, and every NaN ranks below -inf.
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7FFFFFFFu) == 0) u = 0;
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63; }
// The wavefront's LDS accesses issued so far are complete and visible to it.
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}
// Lanes below this one whose bit is set in m.
__device__ __forceinline__ uint32_t rank_in(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// hist[bin] += 1 for every active lane. The bins of the first kLeaders
// distinct values among the active lanes get one add each (with fixed top
// bits as the digit, scores of similar size share a bin, which would
// serialize on one LDS address); the remaining lanes add individually.
template <int kLeaders>
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
    uint64_t todo = __ballot(active);
#pragma unroll
    for (int it = 0; it < kLeaders; ++it) {
        if (todo == 0) return;
        const int leader = __builtin_ctzll(todo);
        const uint32_t lb = __builtin_amdgcn_readlane(bin, leader);
        const uint64_t same = __ballot(active && bin == lb) & todo;
        if ((int)lane_id() == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
        todo &= ~same;
    }
    if ((todo >> lane_id()) & 1ull) atomicAdd(&hist[bin], 1u);
}

// Digit of the k-th largest among the counted keys: the bin where the count
// from the top reaches `need`; also the keys still needed inside that bin.
// Wavefront 0 only: lane l holds bins NB/64 l .. NB/64 (l + 1) - 1.
// `top_excess` is taken off the top bin first.
template <int NB = kBins>
__device__ __forceinline__ void pick_digit(const uint32_t* hist, uint32_t need, uint32_t* sel,
                                           uint32_t top_excess = 0) {
    constexpr int kPer = NB / 64;
    const int lane = threadIdx.x & 63;
    uint32_t b[kPer], c = 0;
#pragma unroll
    for (int j = 0; j < kPer; j += 4) {
        const uint4 x = *reinterpret_cast<const uint4*>(hist + kPer * lane + j);
        b[j] = x.x;
        b[j + 1] = x.y;
        b[j + 2] = x.z;
        b[j + 3] = x.w;
    }
    if (lane == 63) b[kPer - 1] -= top_excess;
#pragma unroll
    for (int j = 0; j < kPer; ++j) c += b[j];
    uint32_t s = c;  // sum over lanes >= l
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_down(s, o);
        if (lane + o < 64) s += y;
    }
    if (s >= need && s - c < need) {
        // walk this lane's bins from the top, in registers
        uint32_t cum = s - c, d = kPer * lane, left = 0;
        bool found = false;
#pragma unroll
        for (int j = kPer - 1; j >= 0; --j) {
            const bool hit = !found && cum + b[j] >= need;
            if (hit) {
                d = kPer * lane + j;
                left = need - cum;
            }
            found |= hit;
            if (!found) cum += b[j];
        }
        sel[0] = d;
        sel[1] = left;
    }
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = min(x, (uint32_t)__shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = max(x, (uint32_t)__shfl_xor(x, o));
    return x;
}

// Rows of n <= 1024 R keys. Thread (wavefront v, lane l) holds the keys of
// indices v 64R + 256 j + 4 l + c for j < R/4, c < 4, so each wavefront owns
// one contiguous index range and reads it with 16-byte loads.
template <int R>
__global__ __launch_bounds__(kThreads) void topk_reg_kernel(const float* scores, int32_t T,
                                                            int32_t k, int32_t w, int32_t* idx) {
    constexpr int kJ = R / 4;
    __shared__ __align__(16) uint32_t hist[3][kBins];  // one per digit pass
    __shared__ uint32_t sel[2];                       // chosen digit, keys still needed
    __shared__ uint32_t wmin[kWaves], wmax[kWaves], cnt_gt[kWaves], cnt_eq[kWaves], tau_sh;
    __shared__ uint32_t cand[kFast], ncand;           // keys of the first digit's bin
    const int row = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = T - w;
    const float* sc = scores + (int64_t)row * T;
    int32_t* out = idx + (int64_t)row * (k + w);
    for (int i = tid; i < w; i += kThreads) out[k + i] = n + i;
    if (k == 0) return;
    if (k == n) {
        for (int i = tid; i < n; i += kThreads) out[i] = i;
        return;
    }
    const int base = wave * 64 * R + 4 * lane;  // index of key[0][0]
    uint32_t key[kJ][4];
    if ((reinterpret_cast<uintptr_t>(sc) & 15) == 0) {
        float4 x[kJ];
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            const int i = base + 256 * j;
            if (i + 3 < n) {
                x[j] = *reinterpret_cast<const float4*>(sc + i);
            } else {
                x[j].x = i < n ? sc[i] : 0.f;
                x[j].y = i + 1 < n ? sc[i + 1] : 0.f;
                x[j].z = i + 2 < n ? sc[i + 2] : 0.f;
                x[j].w = 0.f;
            }
        }
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            key[j][0] = order_key(x[j].x);
            key[j][1] = order_key(x[j].y);
            key[j][2] = order_key(x[j].z);
            key[j][3] = order_key(x[j].w);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kJ; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int i = base + 256 * j + c;
                key[j][c] = order_key(i < n ? sc[i] : 0.f);
            }
    }
    for (int i = tid; i < 3 * kBins / 4; i += kThreads)
        reinterpret_cast<uint4*>(&hist[0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
    if (tid == 0) ncand = 0;
    // range of the row's keys (slots past n take no part)
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (base + 256 * j + c < n) {
                mn = min(mn, key[j][c]);
                mx = max(mx, key[j][c]);
            }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
        wmin[wave] = mn;
        wmax[wave] = mx;
    }
    __syncthreads();
    mn = 0xFFFFFFFFu;
    mx = 0u;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        mn = min(mn, wmin[v]);
        mx = max(mx, wmax[v]);
    }
    // Offsets from the minimum: at most range < 2^L. Slots past n get the
    // offset kPast, above every key's (keys are at most 0xFF800000), so no
    // per-slot index test is needed after this point.
    constexpr uint32_t kPast = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) key[j][c] = base + 256 * j + c < n ? key[j][c] - mn : kPast;
    const uint32_t range = mx - mn;
    const int L = range == 0 ? 0 : 32 - __builtin_clz(range);
    // Digits from bit L down, 11 bits at a time: after the pass over bits
    // [lo, hi) the top L - lo bits of tau's offset are `pref`. A slot past n
    // has (kPast >> hi) != pref for hi < 32; for hi = 32 it lands in the top
    // bin (2047), which no key reaches, and is taken off there.
    uint32_t pref = 0, need = (uint32_t)k;
    int hi = L, pass = 0;
    while (hi > 0) {
        const int lo = hi > 11 ? hi - 11 : 0;
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        uint32_t* h = hist[pass];
        if (pass == 0) {
            // every key counts; the bins spread over the row's range
#pragma unroll
            for (int j = 0; j < kJ; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t v = key[j][c];
                    hist_add<0>(h, (v >> lo) & dmask, hi >= 32 || (v >> hi) == pref);
                }
        } else {
            // only the keys of the chosen bin count (hi < 32 here); they lie
            // close together, so equal bins are aggregated first
#pragma unroll
            for (int j = 0; j < kJ; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t v = key[j][c];
                    hist_add<2>(h, (v >> lo) & dmask, (v >> hi) == pref);
                }
        }
        __syncthreads();
        if (wave == 0) pick_digit(h, need, sel, hi >= 32 ? (uint32_t)(kThreads * R - n) : 0u);
        __syncthreads();
        pref = (pref << (hi - lo)) | sel[0];
        need = sel[1];
        hi = lo;
        ++pass;
        if (pass == 1 && hi > 0) {
            // The keys of the chosen bin (a few hundred on H2O scores) are
            // copied to an LDS list, and when they fit, one wavefront resolves
            // the remaining hi bits on them bit by bit from the top, with one
            // compare and ballot per held candidate and bit: no histogram
            // passes over the registers, whose atomics collide on keys that
            // lie close together.
            const uint32_t lmask = (1u << hi) - 1u;
#pragma unroll
            for (int j = 0; j < kJ; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const bool m = (key[j][c] >> hi) == pref;
                    const uint64_t bm = __ballot(m);
                    if (bm) {
                        const int leader = __builtin_ctzll(bm);
                        uint32_t base = 0;
                        if (lane == leader) base = atomicAdd(&ncand, (uint32_t)__popcll(bm));
                        base = __builtin_amdgcn_readlane(base, leader);
                        const uint32_t at = base + rank_in(bm);
                        if (m && at < kFast) cand[at] = key[j][c] & lmask;
                    }
                }
            __syncthreads();
            const uint32_t nc = ncand;
            if (nc <= kFast) {
                if (wave == 0) {
                    constexpr int kPer = kFast / 64;
                    const int held = (int)(nc + 63) / 64;  // slots that hold candidates
                    uint32_t cv[kPer];
#pragma unroll
                    for (int i = 0; i < kPer; ++i) {
                        const uint32_t at = (uint32_t)(lane + 64 * i);
                        // past the list: all ones above bit hi, never a match
                        cv[i] = at < nc ? cand[at] : 0xFFFFFFFFu;
                    }
                    uint32_t sofar = 0, nd = need;  // the chosen bits above b
                    for (int b = hi - 1; b >= 0; --b) {
                        // candidates whose bits above b are sofar and whose bit b is set
                        const uint32_t want = (sofar << 1) | 1u;
                        uint32_t ones = 0;
#pragma unroll
                        for (int i = 0; i < kPer; ++i)
                            if (i < held) ones += (uint32_t)__popcll(__ballot((cv[i] >> b) == want));
                        if (nd <= ones) {
                            sofar = want;
                        } else {
                            nd -= ones;
                            sofar = want - 1u;
                        }
                    }
                    if (lane == 0) {
                        sel[0] = sofar;
                        sel[1] = nd;
                    }
                }
                __syncthreads();
                pref = (pref << hi) | sel[0];
                need = sel[1];
                hi = 0;
            }
        }
    }
    const uint32_t tau = pref;  // offset of the k-th largest key

    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // tau < v <= range (slots past n excluded), v == tau
            gt += __popcll(__ballot(key[j][c] - tau - 1u < range - tau));
            eq += __popcll(__ballot(key[j][c] == tau));
        }
    if (lane == 0) {
        cnt_gt[wave] = gt;
        cnt_eq[wave] = eq;
    }
    if (tid == 0) tau_sh = tau;
    __syncthreads();
    // tau read back: the comparisons below are then not merged with the
    // counting ones above, whose lane masks would stay live across the
    // barrier (128 slots x 2 masks exceed the scalar registers)
    const uint32_t tk = tau_sh;
    uint32_t gt_before = 0, eq_before = 0, eq_total = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        if (v < wave) {
            gt_before += cnt_gt[v];
            eq_before += cnt_eq[v];
        }
        eq_total += cnt_eq[v];
    }
    // keys equal to tau: the last `need` of them (largest indices) are kept
    const uint32_t eq_first_kept = eq_total - need;
    uint32_t pos = gt_before + (eq_before > eq_first_kept ? eq_before - eq_first_kept : 0u);
    uint32_t er = eq_before;
    // Writes this lane's kept slots of register row j: position = kept keys
    // of the lanes below (all four slots), then this lane's earlier slots.
    auto emit = [&](int j, const bool (&keep)[4]) {
        uint64_t mk[4];
        uint32_t p = pos;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            mk[c] = __ballot(keep[c]);
            p += rank_in(mk[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (keep[c]) out[p] = base + 256 * j + c;
            p += keep[c];
            pos += __popcll(mk[c]);
        }
    };
    if (eq_first_kept == 0) {
        // every key equal to tau is kept: keep tau <= v <= range
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            bool keep[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) keep[c] = key[j][c] - tk <= range - tk;
            emit(j, keep);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            // rank of each equal key among the row's equal keys, in index order
            bool is_eq[4], keep[4];
            uint64_t me[4];
            uint32_t r = er;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                is_eq[c] = key[j][c] == tk;
                me[c] = __ballot(is_eq[c]);
                r += rank_in(me[c]);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                keep[c] = (key[j][c] - tk - 1u < range - tk) | (is_eq[c] & (r >= eq_first_kept));
                r += is_eq[c];
                er += __popcll(me[c]);
            }
            emit(j, keep);
        }
    }
}

// Rows longer than kMaxRegKeys: keys are re-read from memory in every pass.
// The first digit is bits 21-31 of the key; the keys sharing the chosen first
// digit are copied to a candidate list, and the two remaining digits are
// resolved on that list (on the whole row if it overflows).
__global__ __launch_bounds__(kThreads) void topk_global_kernel(const float* scores, int32_t T,
                                                               int32_t k, int32_t w, int32_t* idx) {
    __shared__ __align__(16) uint32_t hist[kBins];
    __shared__ uint32_t cand[kCand];
    __shared__ uint32_t sel[2];  // chosen digit, keys still needed
    __shared__ uint32_t cnt_gt[kWaves], cnt_eq[kWaves];
    const int row = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = T - w;
    const float* sc = scores + (int64_t)row * T;
    int32_t* out = idx + (int64_t)row * (k + w);
    for (int i = tid; i < w; i += kThreads) out[k + i] = n + i;
    if (k == 0) return;
    if (k == n) {
        for (int i = tid; i < n; i += kThreads) out[i] = i;
        return;
    }
    auto key_at = [&](int i) -> uint32_t { return order_key(sc[i]); };
    for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
    __syncthreads();
    // Keys i0 + j * stride (+ this thread's offset) for j < 4, read together
    // before they are used; 0 past lim.
    auto load4 = [&](int i0, int stride, int lim, uint32_t (&kk)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) kk[j] = i0 + j * stride < lim ? key_at(i0 + j * stride) : 0u;
    };
    // First digit (bits 21-31). Every wavefront runs the same trip count, so
    // ballots see whole waves.
    for (int i0 = 0; i0 < n; i0 += 4 * kThreads) {
        uint32_t kk[4];
        load4(i0 + tid, kThreads, n, kk);
#pragma unroll
        for (int j = 0; j < 4; ++j) hist_add<2>(hist, kk[j] >> 21, i0 + j * kThreads + tid < n);
    }
    __syncthreads();
    if (wave == 0) pick_digit(hist, (uint32_t)k, sel);
    __syncthreads();
    uint32_t prefix = sel[0] << 21, need = sel[1];
    // Candidates: the keys with that first digit, counted per wavefront, then
    // written at the wavefront's offset.
    uint32_t mine = 0;
    for (int i0 = 0; i0 < n; i0 += 4 * kThreads) {
        uint32_t kk[4];
        load4(i0 + tid, kThreads, n, kk);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            mine += __popcll(__ballot(i0 + j * kThreads + tid < n && (kk[j] >> 21) == (prefix >> 21)));
    }
    if (lane == 0) cnt_gt[wave] = mine;
    __syncthreads();
    uint32_t at0 = 0, nc = 0;
    for (int v = 0; v < kWaves; ++v) {
        at0 += v < wave ? cnt_gt[v] : 0u;
        nc += cnt_gt[v];
    }
    if (nc <= (uint32_t)kCand) {
        for (int i0 = 0; i0 < n; i0 += 4 * kThreads) {
            uint32_t kk[4];
            load4(i0 + tid, kThreads, n, kk);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool c = i0 + j * kThreads + tid < n && (kk[j] >> 21) == (prefix >> 21);
                const uint64_t m = __ballot(c);
                if (c) cand[at0 + rank_in(m)] = kk[j];
                at0 += __popcll(m);
            }
        }
    }
    __syncthreads();
    const bool use_cand = nc <= (uint32_t)kCand;
    // Remaining digits: bits 10-20, then 0-9.
    uint32_t pmask = 0xFFE00000u;
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = pass == 0 ? 10 : 0;
        const uint32_t dmask = pass == 0 ? 0x7FFu : 0x3FFu;
        for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
        __syncthreads();
        const int m = use_cand ? (int)nc : n;
        for (int i0 = 0; i0 < m; i0 += kThreads) {
            const int i = i0 + tid;
            const uint32_t key = i < m ? (use_cand ? cand[i] : key_at(i)) : 0u;
            hist_add<2>(hist, (key >> shift) & dmask, i < m && (key & pmask) == prefix);
        }
        __syncthreads();
        if (wave == 0) pick_digit(hist, need, sel);
        __syncthreads();
        prefix |= sel[0] << shift;
        pmask |= dmask << shift;
        need = sel[1];
        __syncthreads();
    }
    const uint32_t tau = prefix;

    // Wavefront ranges: contiguous, multiples of 64 indices.
    const int per = ((n + kWaves - 1) / kWaves + 63) & ~63;
    const int lo = wave * per < n ? wave * per : n;
    const int hi = lo + per < n ? lo + per : n;
    uint32_t gt = 0, eq = 0;
    for (int i0 = lo; i0 < hi; i0 += 256) {
        uint32_t kk[4];
        load4(i0 + lane, 64, hi, kk);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool in = i0 + 64 * j + lane < hi;
            gt += __popcll(__ballot(in && kk[j] > tau));
            eq += __popcll(__ballot(in && kk[j] == tau));
        }
    }
    if (lane == 0) {
        cnt_gt[wave] = gt;
        cnt_eq[wave] = eq;
    }
    __syncthreads();
    uint32_t gt_before = 0, eq_before = 0, eq_total = 0;
    for (int v = 0; v < kWaves; ++v) {
        if (v < wave) {
            gt_before += cnt_gt[v];
            eq_before += cnt_eq[v];
        }
        eq_total += cnt_eq[v];
    }
    // keys equal to tau: the last `need` of them (largest indices) are kept
    const uint32_t eq_first_kept = eq_total - need;
    uint32_t pos = gt_before + (eq_before > eq_first_kept ? eq_before - eq_first_kept : 0u);
    uint32_t er = eq_before;
    for (int i0 = lo; i0 < hi; i0 += 256) {
        uint32_t kk[4];
        load4(i0 + lane, 64, hi, kk);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = i0 + 64 * j + lane;
            const bool is_eq = i < hi && kk[j] == tau;
            const uint64_t me = __ballot(is_eq);
            const bool keep = (i < hi && kk[j] > tau) || (is_eq && er + rank_in(me) >= eq_first_kept);
            const uint64_t mk = __ballot(keep);
            if (keep) out[pos + rank_in(mk)] = i;
            pos += __popcll(mk);
            er += __popcll(me);
        }
    }
}

// ---------------------------------------------------------------------------
// Rows split over several workgroups, for row counts that would leave most
// compute units idle with one workgroup per row (one compute unit pulls a
// row through its own load path at a small share of the chip's bandwidth),
// and for rows longer than the register kernels hold. A row's indices
// [0, n) are cut into P slices of L <= 16384 keys.
//
// topk_slice_hist_kernel, workgroup (slice, row), the only pass over the
// scores: counts the slice's keys per value of their top 12 bits (order flag,
// exponent, three mantissa bits) and writes to the workspace
//   * the cumulative counts from the top, C_s(b) = keys with digit >= b, over
//     the occupied range [lo, hi] (below lo C_s is the slice total, above hi
//     zero), and
//   * the slice's local indices ordered by digit (a counting sort through
//     LDS; the order inside a digit is arbitrary), as uint16.
//
// topk_slice_select_kernel, workgroup (slice, row): sums C_s over the slices,
// so the digit b* of the k-th largest key is where the row's C crosses k;
// gathers the keys of digit b* (on H2O scores a few hundred of 32768) through
// the ordered index lists; resolves their remaining 20 bits with two 10-bit
// digits; counts per slice the keys above and equal to the k-th key; marks
// its slice's kept indices (all of digits above b*, read from the tail of its
// list, and those of b*) in an LDS bitmap; and writes them in ascending order
// after those of the earlier slices. Every workgroup of a row takes the same
// decisions from the same data, so none waits on another, and none reads more
// than its slice's list tail and the keys of b* again. When digit b* holds
// more keys than the LDS list (long runs of equal scores), the workgroup
// instead takes the two digits and the counts from the whole row and its
// slice's keys from the scores.

constexpr int kSlicePer = 16;                     // keys per thread in a slice
constexpr int kSliceKeys = kSlicePer * kThreads;  // longest slice
constexpr int kTopBins = 4096;                    // first digit: key bits 20-31
constexpr int kListOff = 3 + kTopBins;            // words: lo, hi, total, C_s(0 .. 4095)
constexpr int kSliceWords = kListOff + kSliceKeys / 2;  // + uint16 index list
constexpr int kMaxSlices = 64;
constexpr int kCandCap = 8192;                    // LDS list of the keys of digit b*

// Keys of slice [beg, end) in registers: thread (wavefront v, lane l) holds
// indices beg + 1024 v + 256 j + 4 l + c (j < 4, c < 4); 0 past end.
__device__ __forceinline__ void load_slice(const float* sc, int beg, int end,
                                           uint32_t (&key)[kSlicePer / 4][4]) {
    constexpr int kJ = kSlicePer / 4;
    const int first = beg + (threadIdx.x >> 6) * 64 * kSlicePer + 4 * (threadIdx.x & 63);
    if ((reinterpret_cast<uintptr_t>(sc + beg) & 15) == 0) {
        float4 x[kJ];
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            const int i = first + 256 * j;
            if (i + 3 < end) {
                x[j] = *reinterpret_cast<const float4*>(sc + i);
            } else {
                x[j].x = i < end ? sc[i] : 0.f;
                x[j].y = i + 1 < end ? sc[i + 1] : 0.f;
                x[j].z = i + 2 < end ? sc[i + 2] : 0.f;
                x[j].w = 0.f;
            }
        }
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            key[j][0] = order_key(x[j].x);
            key[j][1] = order_key(x[j].y);
            key[j][2] = order_key(x[j].z);
            key[j][3] = order_key(x[j].w);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kJ; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int i = first + 256 * j + c;
                key[j][c] = order_key(i < end ? sc[i] : 0.f);
            }
    }
}

// Sum of x over the threads above (dir > 0) or below (dir < 0) this one in
// the workgroup. wtot: kWaves words of LDS; ends with a barrier passed.
template <int Dir>
__device__ __forceinline__ uint32_t sum_beyond(uint32_t x, uint32_t* wtot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t s = x;  // inclusive over this side of the wavefront
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        if (Dir > 0) {
            const uint32_t y = __shfl_down(s, o);
            if (lane + o < 64) s += y;
        } else {
            const uint32_t y = __shfl_up(s, o);
            if (lane >= o) s += y;
        }
    }
    if (lane == (Dir > 0 ? 0 : 63)) wtot[wave] = s;
    __syncthreads();
    uint32_t r = s - x;
    if (Dir > 0)
        for (int v = wave + 1; v < kWaves; ++v) r += wtot[v];
    else
        for (int v = 0; v < wave; ++v) r += wtot[v];
    return r;
}

__global__ __launch_bounds__(kThreads) void topk_slice_hist_kernel(const float* scores, int32_t T,
                                                                   int32_t w, int32_t L,
                                                                   uint32_t* ws) {
    constexpr int kJ = kSlicePer / 4;
    __shared__ __align__(16) uint32_t hist[kTopBins];  // counts, then C(b)
    __shared__ __align__(16) uint16_t order[kSliceKeys];
    __shared__ uint32_t wlo[kWaves], whi[kWaves], wtot[kWaves], s_total;
    const int sl = blockIdx.x, row = blockIdx.y, P = gridDim.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = T - w, beg = sl * L, end = min(beg + L, n);
    const float* sc = scores + (int64_t)row * T;
    uint32_t* out = ws + ((int64_t)row * P + sl) * kSliceWords;
    uint32_t key[kJ][4];
    load_slice(sc, beg, end, key);
    reinterpret_cast<uint4*>(hist)[tid] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    const int first = beg + wave * 64 * kSlicePer + 4 * lane;
    uint32_t dlo = 0xFFFFFFFFu, dhi = 0u;
    uint32_t rank[kJ][4];  // place among the slice's keys of the same digit
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            rank[j][c] = 0;
            if (first + 256 * j + c < end) {
                const uint32_t d = key[j][c] >> 20;
                rank[j][c] = atomicAdd(&hist[d], 1u);
                dlo = min(dlo, d);
                dhi = max(dhi, d);
            }
        }
    dlo = wave_min(dlo);
    dhi = wave_max(dhi);
    if (lane == 0) {
        wlo[wave] = dlo;
        whi[wave] = dhi;
    }
    __syncthreads();
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        lo = min(lo, wlo[v]);
        hi = max(hi, whi[v]);
    }
    // cumulative counts from the top; thread t owns bins 4t .. 4t + 3
    const uint4 hv = reinterpret_cast<const uint4*>(hist)[tid];
    const uint32_t above = sum_beyond<1>(hv.x + hv.y + hv.z + hv.w, wtot);
    const uint32_t c3 = above + hv.w, c2 = c3 + hv.z, c1 = c2 + hv.y, c0 = c1 + hv.x;
    reinterpret_cast<uint4*>(hist)[tid] = make_uint4(c0, c1, c2, c3);
    if (tid == 0) s_total = c0;
    const uint32_t cv[4] = {c0, c1, c2, c3};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t b = 4 * tid + i;
        if (b >= lo && b <= hi) out[3 + b] = cv[i];
    }
    if (tid == 0) {
        out[0] = lo;  // lo > hi: empty slice
        out[1] = hi;
        out[2] = c0;  // slice total
    }
    __syncthreads();
    // counting sort: digit d starts at total - C(d)
    const uint32_t total = s_total;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int i = first + 256 * j + c;
            if (i < end) order[total - hist[key[j][c] >> 20] + rank[j][c]] = (uint16_t)(i - beg);
        }
    __syncthreads();
    uint32_t* list = out + kListOff;
    const uint32_t* ow = reinterpret_cast<const uint32_t*>(order);
    for (uint32_t e = tid; 2 * e < total; e += kThreads) list[e] = ow[e];
}

__global__ __launch_bounds__(kThreads) void topk_slice_select_kernel(const float* scores,
                                                                     int32_t T, int32_t k,
                                                                     int32_t w, int32_t L,
                                                                     const uint32_t* ws,
                                                                     int32_t* idx) {
    constexpr int kJ = kSlicePer / 4;
    __shared__ __align__(16) uint32_t hist[1024];
    __shared__ uint32_t cand_low[kCandCap];  // bits 0-19 of the keys of digit b*
    __shared__ int32_t cand_idx[kCandCap];
    __shared__ uint32_t keepb[kSliceKeys / 32], eqb[kSliceKeys / 32];
    __shared__ uint32_t sgt[kMaxSlices], seq[kMaxSlices], sseg[kMaxSlices], soff[kMaxSlices + 1];
    __shared__ uint32_t slo[kMaxSlices], shi[kMaxSlices], stot[kMaxSlices];
    __shared__ uint32_t sel[3], wtot[kWaves], cnt_gt[kWaves], cnt_eq[kWaves];
    const int sl = blockIdx.x, row = blockIdx.y, P = gridDim.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = T - w, beg = sl * L, end = min(beg + L, n);
    const float* sc = scores + (int64_t)row * T;
    int32_t* out = idx + (int64_t)row * (k + w);
    if (sl == 0)
        for (int i = tid; i < w; i += kThreads) out[k + i] = n + i;
    if (k == 0) return;
    if (k == n) {
        for (int i = beg + tid; i < end; i += kThreads) out[i] = i;
        return;
    }
    const uint32_t* base = ws + (int64_t)row * P * kSliceWords;
    // C_q(b) from the slice headers in LDS; only counts inside a slice's
    // occupied range are read
    if (tid == 0) {
        sel[0] = 0;
        sel[1] = 0;
        sel[2] = 0;
    }
    if (tid < P) {
        slo[tid] = base[tid * kSliceWords];
        shi[tid] = base[tid * kSliceWords + 1];
        stot[tid] = base[tid * kSliceWords + 2];
    }
    __syncthreads();
    auto cum = [&](int q, uint32_t b) -> uint32_t {
        return b < slo[q] ? stot[q] : b > shi[q] ? 0u : base[q * kSliceWords + 3 + b];
    };
    auto list_at = [&](int q, uint32_t e) -> uint32_t {  // entry e of slice q's list
        const uint16_t* l = reinterpret_cast<const uint16_t*>(base + q * kSliceWords + kListOff);
        return l[e];
    };
    // The row's C(b) = sum over slices of C_q(b). Counts inside each slice's
    // occupied range are added into LDS, the (slice, bin) pairs spread over
    // the threads so that their loads are requested together; below its range
    // a slice adds its total, through a difference array summed from the top.
    uint32_t* rowc = cand_low;                               // free until the
    uint32_t* lowd = reinterpret_cast<uint32_t*>(cand_idx);  // gather below
    reinterpret_cast<uint4*>(rowc)[tid] = make_uint4(0u, 0u, 0u, 0u);
    reinterpret_cast<uint4*>(lowd)[tid] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    if (tid == 0) {
        uint32_t o = 0;
        for (int q = 0; q < P; ++q) {
            soff[q] = o;
            o += slo[q] <= shi[q] ? shi[q] - slo[q] + 1 : 0u;
        }
        soff[P] = o;
    }
    if (tid < P && slo[tid] <= shi[tid] && slo[tid] > 0) atomicAdd(&lowd[slo[tid] - 1], stot[tid]);
    __syncthreads();
    // the slice q with soff[q] <= e < soff[q + 1]
    auto slice_of = [&](uint32_t e) -> int {
        int lo = 0, hi = P - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (soff[mid] <= e) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    };
    {
        const uint32_t npairs = soff[P];
        for (uint32_t e0 = 0; e0 < npairs; e0 += 8 * kThreads) {
            uint32_t v[8];
            int bb[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t e = e0 + tid + u * kThreads;
                bb[u] = -1;
                v[u] = 0;
                if (e < npairs) {
                    const int q = slice_of(e);
                    bb[u] = (int)(slo[q] + (e - soff[q]));
                    v[u] = base[q * kSliceWords + 3 + bb[u]];
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (bb[u] >= 0) atomicAdd(&rowc[bb[u]], v[u]);
        }
    }
    __syncthreads();
    // b* is where C crosses k; thread t checks bins 4t .. 4t + 3
    {
        const uint4 ld = reinterpret_cast<const uint4*>(lowd)[tid];
        const uint4 rc = reinterpret_cast<const uint4*>(rowc)[tid];
        // a slice whose range starts above bin b counts whole there: its total
        // sits at lowd[lo - 1], so the slices below b sum lowd from b upwards
        const uint32_t s_up = sum_beyond<1>(ld.x + ld.y + ld.z + ld.w, wtot);
        const uint32_t nxt_rc = tid + 1 < kThreads ? rowc[4 * tid + 4] : 0u;
        uint32_t c[5];
        c[3] = rc.w + s_up + ld.w;
        c[2] = rc.z + s_up + ld.w + ld.z;
        c[1] = rc.y + s_up + ld.w + ld.z + ld.y;
        c[0] = rc.x + s_up + ld.w + ld.z + ld.y + ld.x;
        c[4] = tid + 1 < kThreads ? nxt_rc + s_up : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (c[i] >= (uint32_t)k && c[i + 1] < (uint32_t)k) {
                sel[0] = 4 * tid + i;
                sel[1] = (uint32_t)k - c[i + 1];  // keys still needed inside digit b*
                sel[2] = c[i] - c[i + 1];         // keys of the row with digit b*
            }
    }
    __syncthreads();
    const uint32_t bstar = sel[0], nb = sel[2];
    uint32_t need = sel[1];
    // per slice: keys above digit b*, and where its digit-b* entries sit
    if (tid < P) {
        const uint32_t total = stot[tid];
        const uint32_t cb = cum(tid, bstar);
        const uint32_t ch = bstar + 1 < (uint32_t)kTopBins ? cum(tid, bstar + 1) : 0u;
        sgt[tid] = ch;
        seq[tid] = 0;
        sseg[tid] = total - cb;
        soff[tid + 1] = cb - ch;
    }
    __syncthreads();
    if (tid == 0) {
        soff[0] = 0;
        for (int q = 0; q < P; ++q) soff[q + 1] += soff[q];
    }
    __syncthreads();
    const bool fits = nb <= (uint32_t)kCandCap;
    // The tail of this slice's list (its keys of every digit above b*, all
    // kept) is requested together with the keys of digit b*.
    constexpr int kTailPer = 8;
    const uint32_t my_total = stot[sl], my_ch = sgt[sl];
    uint32_t tail[kTailPer];
    if (fits) {
#pragma unroll
        for (int u = 0; u < kTailPer; ++u) {
            const uint32_t e = tid + u * kThreads;
            tail[u] = e < my_ch ? list_at(sl, my_total - my_ch + e) : 0xFFFFFFFFu;
        }
        // the keys of digit b*, through the slices' ordered lists: every
        // list entry of this thread, then every score
        constexpr int kPer = kCandCap / kThreads;
        int gi[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const uint32_t e = tid + u * kThreads;
            gi[u] = -1;
            if (e < nb) {
                const int q = slice_of(e);
                const uint32_t at = sseg[q] + e - soff[q];
                if (at < stot[q]) gi[u] = q * L + (int)list_at(q, at);
            }
        }
        float xs[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) xs[u] = gi[u] >= 0 && gi[u] < n ? sc[gi[u]] : 0.f;
#pragma unroll
        for (int u = 0; u < kPer; ++u)
            if (gi[u] >= 0) {
                const uint32_t e = tid + u * kThreads;
                cand_low[e] = order_key(xs[u]) & 0xFFFFFu;
                cand_idx[e] = gi[u];
            }
    }
    // Keys of digit b* of the whole row from memory (when the list is too
    // short): fn(key, index) for each.
    auto scan_bin = [&](auto&& fn) {
        for (int i0 = 0; i0 < n; i0 += 4 * kThreads) {
            float x[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int i = i0 + c * kThreads + tid;
                x[c] = i < n ? sc[i] : 0.f;
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int i = i0 + c * kThreads + tid;
                const uint32_t kk = order_key(x[c]);
                if (i < n && (kk >> 20) == bstar) fn(kk, i);
            }
        }
    };
    // bits 10-19, then 0-9, of the k-th key
    uint32_t d0 = 0, d1 = 0;
    if (fits) {
        // a few hundred keys: wavefront 0 alone, without workgroup barriers
        __syncthreads();  // the candidate list is complete
        if (wave == 0) {
            for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    reinterpret_cast<uint4*>(hist)[lane + 64 * i] = make_uint4(0u, 0u, 0u, 0u);
                wave_lds_sync();
                for (uint32_t e = lane; e < nb; e += 64) {
                    const uint32_t low = cand_low[e];
                    if (pass == 0) atomicAdd(&hist[low >> 10], 1u);
                    else if ((low >> 10) == d0) atomicAdd(&hist[low & 0x3FFu], 1u);
                }
                wave_lds_sync();
                pick_digit<1024>(hist, need, sel);
                wave_lds_sync();
                (pass == 0 ? d0 : d1) = sel[0];
                need = sel[1];
                wave_lds_sync();
            }
            if (lane == 0) {
                sel[0] = d0;
                sel[1] = d1;
                sel[2] = need;
            }
        }
        __syncthreads();
        d0 = sel[0];
        d1 = sel[1];
        need = sel[2];
    } else {
        for (int pass = 0; pass < 2; ++pass) {
            hist[tid] = 0;
            __syncthreads();
            scan_bin([&](uint32_t kk, int) {
                const uint32_t low = kk & 0xFFFFFu;
                if (pass == 0) atomicAdd(&hist[low >> 10], 1u);
                else if ((low >> 10) == d0) atomicAdd(&hist[low & 0x3FFu], 1u);
            });
            __syncthreads();
            if (wave == 0) pick_digit<1024>(hist, need, sel);
            __syncthreads();
            (pass == 0 ? d0 : d1) = sel[0];
            need = sel[1];
            __syncthreads();
        }
    }
    const uint32_t tlow = (d0 << 10) | d1, tau = (bstar << 20) | tlow;
    // per slice: keys of digit b* above and equal to tau
    auto tally = [&](uint32_t low, int i) {
        const int q = i / L;
        if (low > tlow) atomicAdd(&sgt[q], 1u);
        else if (low == tlow) atomicAdd(&seq[q], 1u);
    };
    if (fits) {
        for (uint32_t e = tid; e < nb; e += kThreads) tally(cand_low[e], cand_idx[e]);
    } else {
        scan_bin([&](uint32_t kk, int i) { tally(kk & 0xFFFFFu, i); });
    }
    __syncthreads();
    // keys equal to tau: the last `need` of them in index order are kept
    uint32_t gt_before = 0, eq_before = 0, eq_total = 0;
    for (int q = 0; q < P; ++q) {
        if (q < sl) {
            gt_before += sgt[q];
            eq_before += seq[q];
        }
        eq_total += seq[q];
    }
    const uint32_t eq_first_kept = eq_total - need;
    if (fits) {
        // this slice's kept indices as bitmaps: above tau (every digit above
        // b*: the tail of its list; digit b*: from the candidates) and equal
        const int ns = end - beg;
        for (int e = tid; e < kSliceKeys / 32; e += kThreads) {
            keepb[e] = 0;
            eqb[e] = 0;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kTailPer; ++u)
            if (tail[u] < (uint32_t)ns) atomicOr(&keepb[tail[u] >> 5], 1u << (tail[u] & 31));
        for (uint32_t e = tid + kTailPer * kThreads; e < my_ch; e += kThreads) {
            const uint32_t li = list_at(sl, my_total - my_ch + e);
            if (li < (uint32_t)ns) atomicOr(&keepb[li >> 5], 1u << (li & 31));
        }
        for (uint32_t e = tid; e < nb; e += kThreads) {
            const int gi = cand_idx[e];
            if (gi >= beg && gi < end) {
                const uint32_t li = (uint32_t)(gi - beg), low = cand_low[e];
                if (low > tlow) atomicOr(&keepb[li >> 5], 1u << (li & 31));
                else if (low == tlow) atomicOr(&eqb[li >> 5], 1u << (li & 31));
            }
        }
        __syncthreads();
        // thread t: local indices 16 t .. 16 t + 15
        const uint32_t sh = 16 * (tid & 1);
        const uint32_t kb = (keepb[tid >> 1] >> sh) & 0xFFFFu, ebits = (eqb[tid >> 1] >> sh) & 0xFFFFu;
        const uint32_t below = sum_beyond<-1>(((uint32_t)__popc(kb) << 16) | (uint32_t)__popc(ebits), wtot);
        uint32_t er = eq_before + (below & 0xFFFFu);
        uint32_t pos = gt_before + (below >> 16) + (er > eq_first_kept ? er - eq_first_kept : 0u);
        for (int bit = 0; bit < 16; ++bit) {
            const int li = 16 * tid + bit;
            if (li >= ns) break;
            bool take = (kb >> bit) & 1u;
            if (!take && ((ebits >> bit) & 1u)) {
                take = er >= eq_first_kept;
                ++er;
            }
            if (take) {
                if (pos < (uint32_t)k) out[pos] = beg + li;
                ++pos;
            }
        }
        return;
    }
    // long runs of equal keys: this slice's keys from the scores
    uint32_t key[kJ][4];
    load_slice(sc, beg, end, key);
    const int first = beg + wave * 64 * kSlicePer + 4 * lane;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool valid = first + 256 * j + c < end;
            gt += __popcll(__ballot(valid && key[j][c] > tau));
            eq += __popcll(__ballot(valid && key[j][c] == tau));
        }
    if (lane == 0) {
        cnt_gt[wave] = gt;
        cnt_eq[wave] = eq;
    }
    __syncthreads();
    for (int v = 0; v < wave; ++v) {
        gt_before += cnt_gt[v];
        eq_before += cnt_eq[v];
    }
    uint32_t pos = gt_before + (eq_before > eq_first_kept ? eq_before - eq_first_kept : 0u);
    uint32_t er = eq_before;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
        bool is_eq[4], keep[4];
        uint64_t me[4], mk[4];
        uint32_t r = er;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool valid = first + 256 * j + c < end;
            is_eq[c] = valid && key[j][c] == tau;
            keep[c] = valid && key[j][c] > tau;
            me[c] = __ballot(is_eq[c]);
            r += rank_in(me[c]);
        }
        uint32_t p = pos;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            keep[c] = keep[c] || (is_eq[c] && r >= eq_first_kept);
            r += is_eq[c];
            er += __popcll(me[c]);
            mk[c] = __ballot(keep[c]);
            p += rank_in(mk[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (keep[c] && p < (uint32_t)k) out[p] = first + 256 * j + c;
            p += keep[c];
            pos += __popcll(mk[c]);
        }
    }
}
}  // namespace

int topk_cu_count() {
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

TopkPlan topk_plan(int32_t rows, int32_t T, int32_t k, int32_t w) {
    // Split a row when one workgroup per row would leave compute units idle:
    // about one workgroup per compute unit in all, each slice at most 16384
    // keys (held in registers) and at least 4096.
    // Rows longer than the register kernels hold are always split; shorter
    // rows only when there are at most a quarter as many rows as compute
    // units. (At 128 rows of 32768 on 256 compute units the split measured
    // 27 us against 26 us for one workgroup per row: the one pass over the
    // scores costs about the same either way, and the second launch's chain
    // of dependent reads takes what the halved slices save.)
    TopkPlan p{1, T - w, 0};
    const int64_t n = (int64_t)T - w;
    if (rows <= 0 || k <= 0 || k >= n || n < 2 * 4096) return p;
    const int64_t cus = topk_cu_count();
    if (n <= kMaxRegKeys && 4 * (int64_t)rows > cus) return p;
    int64_t P = rows >= cus ? 1 : (cus + rows - 1) / rows;
    const int64_t pmin = (n + kSliceKeys - 1) / kSliceKeys, pmax = n / 4096;
    if (P < pmin) P = pmin;
    if (P > pmax) P = pmax;
    if (P > kMaxSlices || P < 2) return p;
    int64_t L = ((n + P - 1) / P + 3) / 4 * 4;
    P = (n + L - 1) / L;
    if (P < 2) return p;
    p.slices = (int32_t)P;
    p.slice_len = (int32_t)L;
    p.ws_bytes = (size_t)rows * P * kSliceWords * 4;
    return p;
}

int launch_topk(const float* scores, int32_t rows, int32_t T, int32_t k, int32_t w, int32_t* idx,
                void* ws, const TopkPlan& plan, void* stream) {
    (void)hipGetLastError();  // an error left by an earlier call is not this call's
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int n = T - w;
    if (ws && plan.slices > 1) {
        const dim3 grid(plan.slices, rows), block(kThreads);
        uint32_t* h = static_cast<uint32_t*>(ws);
        hipLaunchKernelGGL(topk_slice_hist_kernel, grid, block, 0, s, scores, T, w,
                           plan.slice_len, h);
        hipLaunchKernelGGL(topk_slice_select_kernel, grid, block, 0, s, scores, T, k, w,
                           plan.slice_len, static_cast<const uint32_t*>(h), idx);
        return (int)hipGetLastError();
    }
    const dim3 grid(rows), block(kThreads);
    if (n <= 16 * kThreads)
        hipLaunchKernelGGL(topk_reg_kernel<16>, grid, block, 0, s, scores, T, k, w, idx);
    else if (n <= kMaxRegKeys)
        hipLaunchKernelGGL(topk_reg_kernel<32>, grid, block, 0, s, scores, T, k, w, idx);
    else
        hipLaunchKernelGGL(topk_global_kernel, grid, block, 0, s, scores, T, k, w, idx);
    return (int)hipGetLastError();
}

}  // namespace kvq

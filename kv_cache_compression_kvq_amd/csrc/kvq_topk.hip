// Heavy-hitter selection on gfx950: per row of fp32 scores keep the k largest
// among indices [0, T - w) plus the w most recent indices (MiniKV,
// Algorithm 1, heavy-hitter selection; "KV cache quantization and eviction",
// section "Minimal implementation": evicting the lowest-scoring non-recent
// token one at a time with a first-occurrence argmin leaves, on fixed scores,
// the k largest with ties going to the larger index).
//
// One 1024-thread workgroup per row. Scores become order-preserving 32-bit
// keys. Rows of up to 65536 keys are held in registers (16, 32 or 64 keys
// per thread, all loads in flight at once); a radix select over
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
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;  // histogram bins (11-bit digits)
constexpr int kCand = 4096;  // candidate list after the first digit (long rows)
constexpr int kMaxRegKeys = 64 * kThreads;  // rows held in registers

// Order-preserving key of a score, in [0, 0xFF800000]: -0 and +0 compare
// equal, and every NaN ranks below -inf.
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7FFFFFFFu) == 0) u = 0;
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63; }
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
// Wavefront 0 only: lane l holds bins 32 l .. 32 l + 31. `top_excess` is
// taken off the top bin first.
__device__ __forceinline__ void pick_digit(const uint32_t* hist, uint32_t need, uint32_t* sel,
                                           uint32_t top_excess = 0) {
    constexpr int kPer = kBins / 64;
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

}  // namespace

int launch_topk(const float* scores, int32_t rows, int32_t T, int32_t k, int32_t w, int32_t* idx,
                void* stream) {
    (void)hipGetLastError();  // an error left by an earlier call is not this call's
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int n = T - w;
    const dim3 grid(rows), block(kThreads);
    if (n <= 16 * kThreads)
        hipLaunchKernelGGL(topk_reg_kernel<16>, grid, block, 0, s, scores, T, k, w, idx);
    else if (n <= 32 * kThreads)
        hipLaunchKernelGGL(topk_reg_kernel<32>, grid, block, 0, s, scores, T, k, w, idx);
    else if (n <= kMaxRegKeys)
        hipLaunchKernelGGL(topk_reg_kernel<64>, grid, block, 0, s, scores, T, k, w, idx);
    else
        hipLaunchKernelGGL(topk_global_kernel, grid, block, 0, s, scores, T, k, w, idx);
    return (int)hipGetLastError();
}

}  // namespace kvq

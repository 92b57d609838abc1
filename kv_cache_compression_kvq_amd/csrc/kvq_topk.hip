// Heavy-hitter selection on gfx950: per row of fp32 scores keep the k largest
// among indices [0, T - w) plus the w most recent indices (MiniKV,
// Algorithm 1, heavy-hitter selection; "KV cache quantization and eviction",
// section "Minimal implementation": evicting the lowest-scoring non-recent
// token one at a time with a first-occurrence argmin leaves, on fixed scores,
// the k largest with ties going to the larger index).
//
// One 1024-thread workgroup per row. The row's order-preserving 32-bit keys
// are staged once in LDS (rows longer than the LDS share are read from
// memory in every pass instead). A radix select with 11-, 11- and 10-bit
// digits finds the k-th largest key tau and how many of the keys equal to
// tau are kept: after the first digit's histogram, the keys sharing the
// chosen first digit (usually a few percent of the row) are copied to a
// candidate list, and the two remaining digits are resolved on that list (on
// the whole row if it overflows). Lanes of a
// wavefront that fall into the same histogram bin add once, by their count.
// Each wavefront then owns a contiguous index range and writes its kept
// indices in ascending order from ballot prefix counts.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsKeys = 33280;  // keys staged in LDS (130 KB)
constexpr int kBins = 2048;      // histogram bins (11-bit digits)
constexpr int kCand = 4096;      // candidate list after the first digit

__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7FFFFFFFu) == 0) u = 0;  // -0 and +0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63; }
// Lanes below this one whose bit is set in m.
__device__ __forceinline__ uint32_t rank_in(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// hist[bin] += 1 for every active lane. The bins of the first two distinct
// values among the active lanes get one add each (scores of similar size
// share their leading digits, which would serialize on one LDS address);
// the remaining lanes add individually.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
    uint64_t todo = __ballot(active);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
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
// Wavefront 0 only: lane l holds bins 32 l .. 32 l + 31.
__device__ __forceinline__ void pick_digit(const uint32_t* hist, uint32_t need, uint32_t* sel) {
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
        c += (x.x + x.y) + (x.z + x.w);
    }
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

template <bool kLds>
__global__ __launch_bounds__(kThreads) void topk_kernel(const float* scores, int32_t T, int32_t k,
                                                        int32_t w, int32_t* idx) {
    extern __shared__ __align__(16) uint32_t keys[];  // [n] when kLds
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
    auto key_at = [&](int i) -> uint32_t { return kLds ? keys[i] : order_key(sc[i]); };
    for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
    __syncthreads();
    // Staging first, in a loop of independent loads (the histogram's LDS
    // atomics would otherwise sit between consecutive loads).
    if (kLds) {
        // 16-byte loads when the row is 16-byte aligned
        int done = 0;
        if ((reinterpret_cast<uintptr_t>(sc) & 15) == 0) {
            // four 16-byte loads in flight per thread before any is stored
            const float4* s4 = reinterpret_cast<const float4*>(sc);
            const int n4 = n / 4;
            for (int i0 = 0; i0 < n4; i0 += 4 * kThreads) {
                float4 x[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = i0 + j * kThreads + tid;
                    x[j] = i < n4 ? s4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = i0 + j * kThreads + tid;
                    if (i < n4)
                        *reinterpret_cast<uint4*>(keys + 4 * i) = make_uint4(
                            order_key(x[j].x), order_key(x[j].y), order_key(x[j].z), order_key(x[j].w));
                }
            }
            done = n4 * 4;
        }
        for (int i = done + tid; i < n; i += kThreads) keys[i] = order_key(sc[i]);
        __syncthreads();
    }
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
        for (int j = 0; j < 4; ++j) hist_add(hist, kk[j] >> 21, i0 + j * kThreads + tid < n);
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
            hist_add(hist, (key >> shift) & dmask, i < m && (key & pmask) == prefix);
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
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int n = T - w;
    if (n <= kLdsKeys) {
        static bool attr = [] {
            (void)hipFuncSetAttribute(reinterpret_cast<const void*>(topk_kernel<true>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, kLdsKeys * 4);
            return true;
        }();
        (void)attr;
        hipLaunchKernelGGL(topk_kernel<true>, dim3(rows), dim3(kThreads), (size_t)n * 4, s, scores,
                           T, k, w, idx);
    } else {
        hipLaunchKernelGGL(topk_kernel<false>, dim3(rows), dim3(kThreads), 0, s, scores, T, k, w,
                           idx);
    }
    return (int)hipGetLastError();
}

}  // namespace kvq

// Heavy-hitter selection on gfx950: per row of fp32 scores keep the k largest
// among indices [0, T - w) plus the w most recent indices (MiniKV,
// Algorithm 1, heavy-hitter selection; "KV cache quantization and eviction",
// section "Minimal implementation": evicting the lowest-scoring non-recent
// token one at a time with a first-occurrence argmin leaves, on fixed scores,
// the k largest with ties going to the larger index).
//
// One 1024-thread workgroup per row. The row's order-preserving 32-bit keys
// are staged once in LDS (rows longer than the LDS share are read from
// memory in every pass instead). An 8-bit-digit radix select finds the k-th
// largest key tau and how many of the keys equal to tau are kept; lanes of a
// wavefront that fall into the same histogram bin add once, by their count.
// Each wavefront then owns a contiguous index range and writes its kept
// indices in ascending order from ballot prefix counts.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsKeys = 36864;  // keys staged in LDS (144 KB)

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

template <bool kLds>
__global__ __launch_bounds__(kThreads) void topk_kernel(const float* scores, int32_t T, int32_t k,
                                                        int32_t w, int32_t* idx) {
    extern __shared__ uint32_t keys[];  // [n] when kLds
    __shared__ uint32_t hist[256];
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
    if (kLds)
        for (int i = tid; i < n; i += kThreads) keys[i] = order_key(sc[i]);
    auto key_at = [&](int i) -> uint32_t { return kLds ? keys[i] : order_key(sc[i]); };

    // Radix select: tau = the k-th largest key, need = keys equal to tau kept.
    uint32_t prefix = 0, pmask = 0, need = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        // every wavefront runs the same trip count, so ballots see whole waves
        for (int i0 = 0; i0 < n; i0 += kThreads) {
            const int i = i0 + tid;
            const uint32_t key = i < n ? key_at(i) : 0u;
            hist_add(hist, (key >> shift) & 255u, i < n && (key & pmask) == prefix);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l holds bins 4l .. 4l+3; suffix sums from the top bin down
            uint32_t b[4], c = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b[j] = hist[4 * lane + j];
                c += b[j];
            }
            uint32_t s = c;  // sum over lanes >= l
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_down(s, o);
                if (lane + o < 64) s += y;
            }
            if (s >= need && s - c < need) {
                uint32_t cum = s - c, d = 4 * lane;
#pragma unroll
                for (int j = 3; j >= 0; --j) {
                    if (cum + b[j] >= need) {
                        d = 4 * lane + j;
                        break;
                    }
                    cum += b[j];
                }
                sel[0] = d;
                sel[1] = need - cum;
            }
        }
        __syncthreads();
        prefix |= sel[0] << shift;
        pmask |= 255u << shift;
        need = sel[1];
        __syncthreads();
    }
    const uint32_t tau = prefix;

    // Wavefront ranges: contiguous, multiples of 64 indices.
    const int per = ((n + kWaves - 1) / kWaves + 63) & ~63;
    const int lo = wave * per < n ? wave * per : n;
    const int hi = lo + per < n ? lo + per : n;
    uint32_t gt = 0, eq = 0;
    for (int i0 = lo; i0 < hi; i0 += 64) {
        const int i = i0 + lane;
        const uint32_t key = i < hi ? key_at(i) : 0u;
        gt += __popcll(__ballot(i < hi && key > tau));
        eq += __popcll(__ballot(i < hi && key == tau));
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
    for (int i0 = lo; i0 < hi; i0 += 64) {
        const int i = i0 + lane;
        const uint32_t key = i < hi ? key_at(i) : 0u;
        const bool is_eq = i < hi && key == tau;
        const uint64_t me = __ballot(is_eq);
        const bool keep = (i < hi && key > tau) || (is_eq && er + rank_in(me) >= eq_first_kept);
        const uint64_t mk = __ballot(keep);
        if (keep) out[pos + rank_in(mk)] = i;
        pos += __popcll(mk);
        er += __popcll(me);
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

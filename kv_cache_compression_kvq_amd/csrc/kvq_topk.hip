// Heavy-hitter selection on gfx950: per row of fp32 scores keep the k largest
// among indices [0, T - w) plus the w most recent indices (MiniKV,
// Algorithm 1, heavy-hitter selection; "KV cache quantization and eviction",
// section "Minimal implementation": evicting the lowest-scoring non-recent
// token one at a time with a first-occurrence argmin leaves, on fixed scores,
// the k largest with ties going to the larger index).
//
// One 1024-thread workgroup per row: an 8-bit-digit radix select on
// order-preserving 32-bit keys finds the k-th largest key tau and how many of
// the keys equal to tau are kept, then two block-wide scans place the kept
// indices in ascending order.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 1024;

__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7FFFFFFFu) == 0) u = 0;  // -0 and +0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive block-wide prefix sum of one value per thread; returns the total.
__device__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* prefix, uint32_t* wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t run = 0;
        for (int w = 0; w < kThreads / 64; ++w) {
            const uint32_t t = wsum[w];
            wsum[w] = run;
            run += t;
        }
        wsum[kThreads / 64] = run;
    }
    __syncthreads();
    *prefix = wsum[wave] + incl - x;
    const uint32_t total = wsum[kThreads / 64];
    __syncthreads();
    return total;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* scores, int32_t T, int32_t k,
                                                        int32_t w, int32_t* idx) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sel[2];  // chosen digit, keys still needed
    __shared__ uint32_t wsum[kThreads / 64 + 1];
    const int row = blockIdx.x, tid = threadIdx.x;
    const int n = T - w;
    const float* sc = scores + (int64_t)row * T;
    int32_t* out = idx + (int64_t)row * (k + w);
    for (int i = tid; i < w; i += kThreads) out[k + i] = n + i;
    if (k == 0) return;
    if (k == n) {
        for (int i = tid; i < n; i += kThreads) out[i] = i;
        return;
    }
    // Radix select: tau = the k-th largest key, need = keys equal to tau kept.
    uint32_t prefix = 0, pmask = 0, need = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kThreads) hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            const uint32_t key = order_key(sc[i]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t cum = 0, d = 0;
            for (int bin = 255; bin >= 0; --bin) {
                if (cum + hist[bin] >= need) {
                    d = (uint32_t)bin;
                    break;
                }
                cum += hist[bin];
            }
            sel[0] = d;
            sel[1] = need - cum;
        }
        __syncthreads();
        prefix |= sel[0] << shift;
        pmask |= 255u << shift;
        need = sel[1];
        __syncthreads();
    }
    const uint32_t tau = prefix;
    // Contiguous index range per thread, so scans give index order.
    const int per = (n + kThreads - 1) / kThreads;
    const int lo = tid * per < n ? tid * per : n;
    const int hi = lo + per < n ? lo + per : n;
    uint32_t eq = 0;
    for (int i = lo; i < hi; ++i) eq += order_key(sc[i]) == tau;
    uint32_t eq_before;
    const uint32_t eq_total = block_exclusive_scan(eq, &eq_before, wsum);
    const uint32_t eq_first_kept = eq_total - need;  // keep the last `need` equal keys
    uint32_t kept = 0, e = eq_before;
    for (int i = lo; i < hi; ++i) {
        const uint32_t key = order_key(sc[i]);
        if (key > tau) ++kept;
        else if (key == tau) kept += (e++ >= eq_first_kept);
    }
    uint32_t pos;
    block_exclusive_scan(kept, &pos, wsum);
    e = eq_before;
    for (int i = lo; i < hi; ++i) {
        const uint32_t key = order_key(sc[i]);
        bool keep = key > tau;
        if (key == tau) keep = (e++ >= eq_first_kept);
        if (keep && pos < (uint32_t)k) out[pos++] = i;
    }
}

}  // namespace

int launch_topk(const float* scores, int32_t rows, int32_t T, int32_t k, int32_t w, int32_t* idx,
                void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(topk_kernel, dim3(rows), dim3(kThreads), 0, s, scores, T, k, w, idx);
    return (int)hipGetLastError();
}

}  // namespace kvq

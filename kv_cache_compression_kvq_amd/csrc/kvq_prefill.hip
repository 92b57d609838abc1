// Prefill of one attention layer on gfx950: causal attention over the n prompt
// tokens and the per-KV-head column sums of the normalized attention that
// select the heavy hitters ("MiniKV: Pushing the Limits of LLM Inference via
// 2-Bit Layer-Discriminative KV Cache", section 4.3, selective flash-attention,
// and Algorithm 1, prefill; section 4.1, persistent context selection).
//
//   S = Q K^T / sqrt(d) (keys after the query masked), P = softmax(S) per row,
//   X_O = P V,  A_cumul[j] = sum over the KV head's query heads and over the
//   query rows i >= j of P[i][j].
//
// Kernel 1 (prefill_fwd_kernel) computes X_O flash-style, one pass over the
// keys with an online softmax, and keeps each row's log-sum-exp. Kernel 2
// (prefill_colsum_kernel) recomputes S for one 16-key tile per wavefront and
// sums exp(S - lse) over the rows below it, so every column sum is produced by
// one wavefront in a fixed order (no atomics).
//
// Matrix-core layouts. The forward kernel computes S^T = K Q^T on
// v_mfma_f32_32x32x16_f16, so a lane of an S^T tile holds sixteen keys of one
// query row, and O^T = V^T P^T on the same shape, so a lane's P values are
// already its B operand and a lane's output accumulators all belong to its
// own query row (rescaling needs no cross-lane exchange). The column-sum
// kernel computes S^T on v_mfma_f32_16x16x32_f16, four keys of one row per
// lane.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int D = kHeadDim;
constexpr int KB = 64;           // keys per block step
// Value tile as copied, row-major (64 keys x 256 B), 16-byte chunk c of key
// row r at position c ^ v_swz(r). The value operand is read with the gfx950
// transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// 4 r + s reads 8 bytes, and lane i receives element i of the 16 values read
// by lanes 4 r' .. 4 r' + 3, for r' = 0..3. Lane (16 g + 4 r + s) reads key
// row 16 k + 4 (g / 2) + r (and the row 8 below), channels 32 nt + 16 (g % 2)
// + 4 s .. + 3, so lane l gets channel 32 nt + l % 32 of four consecutive
// keys: the A operand layout of the 32x32x16 product. A 32-lane half reads
// four rows r = 0..3 (mod 4) and chunks 4 nt .. 4 nt + 3; the swizzle puts
// those 16 pieces on 16 distinct chunk positions (and each 16-lane group's 8
// on 8 distinct positions mod 8), so the reads are free of bank conflicts.
__device__ __forceinline__ int v_swz(int r) { return 2 * (r & 3) + 8 * (r & 1); }
// Lazy rescaling ("online softmax" with a threshold): a row's reference
// maximum moves only when a logit exceeds it by more than this (log2 units),
// so its probabilities stay below 2^8 in the fp16 operand.
constexpr float kLazyTau = 8.0f;

// x at lanes l and l ^ 32 as the pair (a, b) in either order, through the
// gfx950 permlane swap (VALU, no LDS round trip); inline asm because the
// compiler's builtin drops one result.
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
    a = x;
    b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_x32(float x) { float a, b; swap32(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float sum_x32(float x) { float a, b; swap32(x, a, b); return a + b; }

// Block coordinates with all blocks of one unit on one compute die when the
// unit count is a multiple of 8: workgroups are dealt to the 8 dies round
// robin by linear index, so the unit's K/V (forward) or Q (column sums) stays
// in that die's L2 instead of passing through all eight. A bijection of the
// grid; only placement (speed) depends on the dealing order.
__device__ __forceinline__ void die_local_block(int& x, int& y) {
    x = blockIdx.x;
    y = blockIdx.y;
    if (gridDim.y % 8 == 0) {
        const int lin = blockIdx.x + gridDim.x * blockIdx.y, die = lin % 8, idx = lin / 8;
        y = die + 8 * (idx / (int)gridDim.x);
        x = idx % (int)gridDim.x;
    }
}

__device__ __forceinline__ void lds_load16(const void* g, void* lds) {
    // lane i's 16 bytes land at lds + 16 * i
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
// Buffer-resource form of the same copy: a wave-uniform descriptor (base and
// size in bytes, raw access), a per-lane byte offset and a wave-uniform byte
// offset, so a loop adds nothing per lane; every access here stays inside the
// described range.
constexpr uint32_t kRawBufferWord3 = 0x00020000u;  // raw (untyped) 32-bit access
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             (int)kRawBufferWord3);
}
__device__ __forceinline__ void lds_load16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                               void* lds) {
    // lane i's 16 bytes land at lds + 16 * i
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff,
                                             soff, 0, 0);
}
__device__ __forceinline__ void lds_load4(const void* g, void* lds) {
    // lane i's 4 bytes land at lds + 4 * i
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}
// Wait until at most N of this wavefront's vector memory operations are in
// flight (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier without the memory fence of __syncthreads, whose release
// would wait for every LDS copy in flight (the ring's later stages too); the
// ring's own waits order the copies.
__device__ __forceinline__ void bare_barrier() { asm volatile("s_barrier" ::: "memory"); }
// Reads of a ring stage, issued as inline assembly so that the compiler does
// not wait for the copies in flight into other stages; lds_wait() then waits
// for them and ties their results.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
__device__ __forceinline__ uint32_t lds_read4(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

struct PrefillArgs {
    const uint16_t* q;  // [B][Hq][n][d]
    const uint16_t* k;  // [B][Hkv][n][d]
    const uint16_t* v;
    float* out;         // [B][Hq][n][d]
    float* acc;         // [B][Hkv][n] or null
    float* lse;         // [B][Hq][n]: log2 of each row's softmax normaliser (log2 units)
    float* part;        // [B][Hq][n]: column sums of each query head (added per KV head)
    int32_t n, n_kv_heads;
    float qscale;       // log2(e) / sqrt(d)
};

// Block (query block x, unit y = b * Hkv + h_kv): 128 / r query rows of each of
// the r query heads of the KV head. Wavefront w takes head w % r and the 32
// rows (w / r) * 32 .. + 31 of the block: lane l holds row (l % 32) of the
// S^T tiles and of the output, the two 32-lane halves different keys
// (S^T) or channels (O^T) of it.
template <int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_fwd_kernel(PrefillArgs a) {
    constexpr int QR = 128 / R;  // query rows per block
    // key tiles, double-buffered and filled by direct global->LDS copies:
    // 64 rows of 256 B, 16-byte chunk c of key row r at position c ^ (r % 16)
    __shared__ __align__(16) unsigned char ks[2][KB * D * 2];
    // value tiles as copied (row-major, chunks swizzled by v_swz), double-buffered
    __shared__ __align__(16) unsigned char vs[2][KB * D * 2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = a.n;
    int bx, by;
    die_local_block(bx, by);
    const int unit = by, b = unit / a.n_kv_heads, hkv = unit % a.n_kv_heads;
    // the last query blocks see the most keys: they are dispatched first
    const int q0 = ((int)gridDim.x - 1 - bx) * QR;
    const int hl = wave % R, row0 = q0 + (wave / R) * 32;
    const int hq = hkv * R + hl;
    const int64_t qbase = ((int64_t)b * a.n_kv_heads * R + hq) * n;
    const int64_t kvbase = (int64_t)unit * n;
    const uint16_t* kunit = a.k + kvbase * D;  // this unit's rows; offsets below are 32-bit
    const uint16_t* vunit = a.v + kvbase * D;
    const float qs = a.qscale;
    const int j = lane & 31, h = lane >> 5;
    const int row = row0 + j;  // this lane's query row

    // query operands (B of S^T), k-step kst: row `row`, channels 16 kst + 8 h
    // .. + 7 (zero rows past n)
    half8 Qo[8];
#pragma unroll
    for (int kst = 0; kst < 8; ++kst) {
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (row < n) w = *reinterpret_cast<const uint4*>(a.q + (qbase + row) * D + 16 * kst + 8 * h);
        Qo[kst] = __builtin_bit_cast(half8, w);
    }
    // O^T tile nt: lane holds channels 32 nt + 8 (i / 4) + 4 h + i % 4 of `row`
    floatx16 O[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[nt][i] = 0.f;
    // the row's reference maximum and this lane's part of its sum (the two
    // halves hold different keys; they are added at the end)
    float m = -INFINITY, l = 0.f;

    const int kend = n < q0 + QR ? n : q0 + QR;  // keys any row of the block sees
    const int nkb = (kend + KB - 1) / KB;
    // this thread's copies (i = 0..3): key row p / 16 of the tile, p = tid + 256 i;
    // lane position p % 16 receives chunk (p % 16) ^ (row % 16) (K) or
    // (p % 16) ^ v_swz(row) (V).
    // Byte offsets from the tile's first row, fixed for the whole loop; the
    // tile's own offset is wave-uniform.
    uint32_t koff[4], voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = tid + 256 * i, key = p / 16, pc = p % 16;
        koff[i] = (uint32_t)(2 * (key * D + 8 * (pc ^ (key & 15))));
        voff[i] = (uint32_t)(2 * (key * D + 8 * (pc ^ v_swz(key))));
    }
    // a unit's K (V) rows in bytes; 2^32 at n = 2^24 saturates (every offset
    // the loop forms stays below 2^32)
    const uint64_t ub = (uint64_t)n * D * 2;
    const uint32_t unit_bytes = ub > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)ub;
    const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(kunit, unit_bytes), vrs = buffer_rsrc(vunit, unit_bytes);
    const int wbase = __builtin_amdgcn_readfirstlane(tid - lane);  // first thread of the wave
    auto fetch = [&](int t) {
        const int k0 = t * KB;
        unsigned char* kdst = &ks[t & 1][0];
        unsigned char* vdst = &vs[t & 1][0];
        const uint32_t tb = (uint32_t)k0 * D * 2;  // the tile's first row
        if (k0 + KB <= n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_load16_buf(krs, koff[i], tb, kdst + (wbase + 256 * i) * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_load16_buf(vrs, voff[i], tb, vdst + (wbase + 256 * i) * 16);
        } else {
            // last tile: rows past n repeat row n - 1 (their logits are masked,
            // their probabilities 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = (tid + 256 * i) / 16;
                const uint32_t back = k0 + key < n ? 0u : (uint32_t)((k0 + key - (n - 1)) * D * 2);
                lds_load16_buf(krs, koff[i] - back, tb, kdst + (wbase + 256 * i) * 16);
                lds_load16_buf(vrs, voff[i] - back, tb, vdst + (wbase + 256 * i) * 16);
            }
        }
    };
    if (nkb > 0) fetch(0);
    // key-operand reads (A of S^T): key row 32 kt + j, chunk 2 kst + h at
    // position (2 kst + h) ^ (j % 16)
    // value-operand reads: lane (16 g + 4 r + s) reads key row 4 (g / 2) + r
    // (+ 16 k, + 8), chunk 4 nt + 2 (g % 2) + s / 2, 8-byte half s % 2; the
    // chunk's position is swizzled by v_swz(r) (rows differ from r by
    // multiples of 4); the four tiles' lane offsets are fixed for the loop
    const int vg = lane >> 4, vr = (lane >> 2) & 3, vsl = lane & 3;
    const int vsw = v_swz(vr);
    uint32_t vlane[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
        vlane[nt] = (uint32_t)((4 * (vg >> 1) + vr) * 256 + 16 * ((4 * nt + 2 * (vg & 1) + (vsl >> 1)) ^ vsw) +
                               8 * (vsl & 1));
    for (int t = 0; t < nkb; ++t) {
        // every wavefront is done with tile t - 1 (whose buffers the next
        // copies refill), and tile t's copies have landed (the barrier's fence
        // waits for them)
        __syncthreads();
        if (t + 1 < nkb) fetch(t + 1);
        const int k0 = t * KB;
        if (k0 > row0 + 31 || row0 >= n) continue;  // every key of the tile is after this wave's rows
        const unsigned char* kt_lds = &ks[t & 1][0];
        // S^T tiles kt = 0, 1: lane holds keys k0 + 32 kt + 8 (i / 4) + 4 h + i % 4
        // of `row`; the two tiles as interleaved independent chains
        floatx16 St[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) St[kt][i] = 0.f;
        // key operands requested two k-steps ahead of their products
        half8 Ak[8][2];
#pragma unroll
        for (int kst = 0; kst < 8; ++kst)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                Ak[kst][kt] = *reinterpret_cast<const half8*>(
                    kt_lds + (32 * kt + j) * 256 + 16 * ((2 * kst + h) ^ (j & 15)));
#pragma unroll
        for (int kst = 0; kst < 8; ++kst)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                St[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ak[kst][kt], Qo[kst], St[kt], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
        // the row's maximum logit over the tile, from the unscaled products
        // (the scale is positive) with masked keys at -inf
        float mx = -INFINITY;
        if (k0 + KB - 1 <= row0 && row0 + 31 < n) {
            // every key of the tile at or before every row of the wavefront
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, St[kt][i]);
        } else {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = k0 + 32 * kt + 8 * (i >> 2) + 4 * h + (i & 3);
                    if (key > row || key >= n || row >= n) St[kt][i] = -INFINITY;
                    mx = fmaxf(mx, St[kt][i]);
                }
        }
        mx = max_x32(mx) * qs;
        // the reference maximum moves (and the row's sums are rescaled) only
        // when some row of the wavefront passes its own by more than tau
        if (__any(mx > m + kLazyTau)) {
            const float mnew = mx > m + kLazyTau ? mx : m;
            // rows with nothing unmasked yet keep alpha = 1 and p = 0
            const float alpha = m == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
            l *= alpha;
            m = mnew;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int i = 0; i < 16; ++i) O[nt][i] *= alpha;
        }
        const float nmu = m == -INFINITY ? 0.f : -m;
        // P^T operands of the four 16-key k-steps: k-step s takes S^T tile
        // s / 2, values 8 (s % 2) .. + 7, i.e. keys 16 s + 4 h + 0..3 and
        // 16 s + 8 + 4 h + 0..3
        half8 Bp[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = __builtin_amdgcn_exp2f(fmaf(St[s >> 1][8 * (s & 1) + e], qs, nmu));
                l += p[e];
            }
            Bp[s] = half8{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3],
                          (_Float16)p[4], (_Float16)p[5], (_Float16)p[6], (_Float16)p[7]};
        }
        // O^T += V^T P^T: value operand of tile nt, k-step s: channel 32 nt + j,
        // keys 16 s + 4 h + 0..3 and 16 s + 8 + 4 h + 0..3
        const unsigned char* vtile = &vs[t & 1][0];
        half4 Vr[4][4][2];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const unsigned char* vb = vtile + vlane[nt] + (16 * s) * 256;
                Vr[s][nt][0] = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) short4_t*)vb));
                Vr[s][nt][1] = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) short4_t*)(vb + 8 * 256)));
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const half4 v0 = Vr[s][nt][0], v1 = Vr[s][nt][1];
                const half8 Av = half8{v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                O[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Av, Bp[s], O[nt], 0, 0, 0);
            }
        }
        // value reads: the first k-step's 8 first, then each k-step's products
        // with the next k-step's reads behind them
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
    }
    // outputs: channels 32 nt + 8 (i / 4) + 4 h .. + 3 of `row`; log-sum-exp per row
    const float lt = sum_x32(l);
    if (row < n) {
        const float linv = lt > 0.f ? 1.0f / lt : 0.f;
        float* o = a.out + (qbase + row) * D + 4 * h;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int ig = 0; ig < 4; ++ig)
                *reinterpret_cast<float4*>(o + 32 * nt + 8 * ig) =
                    make_float4(O[nt][4 * ig] * linv, O[nt][4 * ig + 1] * linv, O[nt][4 * ig + 2] * linv,
                                O[nt][4 * ig + 3] * linv);
        if (h == 0) a.lse[qbase + row] = m + log2f(lt);
    }
}

// Column sums: block (key block x of 64 keys, query head y = unit * r + h).
// The query rows of the head from the block's first key on pass through a
// ring of LDS stages, 64 rows with their log-sum-exp each, copied straight
// from memory two stages ahead of use. Wavefront w owns keys k0 + 32 (w % 2)
// .. + 31 and rows 32 (w / 2) .. + 31 of every stage: it recomputes S^T for
// them on v_mfma_f32_32x32x16_f16 (a lane holds sixteen keys of one row) and
// adds exp2(s - lse_row) over the rows at or after each key. The two
// wavefronts of a key half are added in a fixed order at the end, so every
// column sum is produced in a fixed order (no atomics).
template <int R>
__global__ __launch_bounds__(256) void prefill_colsum_kernel(PrefillArgs a) {
    constexpr int QT = 64;                       // query rows per stage
    constexpr int kStages = 3;                   // stages in flight
    constexpr int kTileBytes = QT * D * 2;       // 16 KB of query rows
    __shared__ __align__(16) unsigned char ring[kStages][kTileBytes + QT * 4];
    __shared__ float half_sums[2][32];           // the second row half's sums per key half
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = a.n;
    int bx, by;
    die_local_block(bx, by);
    const int unit = by / R, hh = by % R, b = unit / a.n_kv_heads, hkv = unit % a.n_kv_heads;
    const int kg = wave & 1, rh = wave >> 1;     // key half, row half
    const int k0 = bx * KB, kt0 = k0 + 32 * kg;  // first key of the block, of this wavefront
    const int64_t qhead = (int64_t)b * a.n_kv_heads * R + hkv * R + hh;
    const int64_t kvbase = (int64_t)unit * n;
    const float qs = a.qscale;
    const int j = lane & 31, h = lane >> 5;
    // key operands (A of S^T): key kt0 + j, channels 16 kst + 8 h .. + 7
    half8 Ak[8];
#pragma unroll
    for (int kst = 0; kst < 8; ++kst) {
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (kt0 + j < n)
            w = *reinterpret_cast<const uint4*>(a.k + (kvbase + kt0 + j) * D + 16 * kst + 8 * h);
        Ak[kst] = __builtin_bit_cast(half8, w);
    }
    // keys kt0 + 8 (i / 4) + 4 h + i % 4, partial over this lane's rows
    float cs[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) cs[i] = 0.f;
    const int t_first = k0 / QT, ntiles = (n + QT - 1) / QT, iters = ntiles - t_first;
    // Stage it (rows r0 .. r0 + 63 of query head hh): 64 rows of 256 B
    // with the 16-byte chunk c of row r stored at position c ^ (r % 16), so the
    // rows of an operand read sit on distinct banks, then the rows'
    // log-sum-exp. Each wavefront copies a quarter of both (five copies), and
    // waits for its own copies of a stage before the barrier that publishes it.
    const int64_t qbase = qhead * n;
    // this thread's copies: row (16 wave + 4 i + lane / 16) of the stage, its
    // chunk, as an element offset from the stage's first row
    int coff[4], crow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int slot = (4 * wave + i) * 64 + lane, row = slot / 16;
        crow[i] = row;
        coff[i] = row * D + 8 * ((slot % 16) ^ (row & 15));
    }
    auto issue = [&](int it) {
        const int r0 = (t_first + it) * QT;
        unsigned char* st = &ring[it % kStages][0];
        const uint16_t* q0p = a.q + (qbase + r0) * D;
        if (r0 + QT <= n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_load16(q0p + coff[i], st + (4 * wave + i) * 1024);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // rows past n are read from row n - 1 (masked below)
                const int back = r0 + crow[i] < n ? 0 : (r0 + crow[i] - (n - 1)) * D;
                lds_load16(q0p + coff[i] - back, st + (4 * wave + i) * 1024);
            }
        }
        if ((lane >> 4) == wave) {
            const int rr = r0 + lane < n ? r0 + lane : n - 1;
            lds_load4(a.lse + qbase + rr, st + kTileBytes);
        }
    };
    // query-operand reads (B of S^T): row 32 rh + j of a stage, chunk 2 kst + h
    // at position (2 kst + h) ^ (j % 16); byte offsets from the stage's start
    uint32_t qoff[8];
#pragma unroll
    for (int kst = 0; kst < 8; ++kst)
        qoff[kst] = (uint32_t)((32 * rh + j) * 256 + 16 * ((2 * kst + h) ^ (j & 15)));
    const uint32_t loff = (uint32_t)(kTileBytes + 4 * (32 * rh + j));
    for (int p = 0; p < kStages - 1 && p < iters; ++p) issue(p);
    for (int it = 0; it < iters; ++it) {
        bare_barrier();  // stage (it - 1) % kStages is no longer read
        if (it + kStages - 1 < iters) issue(it + kStages - 1);
        const int later = min(kStages - 1, iters - 1 - it);  // stages requested after this one
        if (later >= 3) wait_vm<15>();
        else if (later == 2) wait_vm<10>();
        else if (later == 1) wait_vm<5>();
        else wait_vm<0>();
        bare_barrier();  // every wavefront's copies of stage it have landed
        const int rb = (t_first + it) * QT + 32 * rh;  // this wavefront's first row of the stage
        if (kt0 >= n || rb + 31 < kt0 || rb >= n) continue;  // no row at or after a key, or past n
        const uint32_t st = lds_addr(&ring[it % kStages][0]);
        u32x4 bw[8];
#pragma unroll
        for (int kst = 0; kst < 8; ++kst) bw[kst] = lds_read16(st + qoff[kst]);
        uint32_t lsw = lds_read4(st + loff);
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(bw[0]), "+v"(bw[1]), "+v"(bw[2]), "+v"(bw[3]), "+v"(bw[4]), "+v"(bw[5]),
                       "+v"(bw[6]), "+v"(bw[7]), "+v"(lsw)
                     :
                     : "memory");
        floatx16 acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
        for (int kst = 0; kst < 8; ++kst)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ak[kst], __builtin_bit_cast(half8, bw[kst]), acc, 0, 0,
                                                         0);
        const float nl = -__builtin_bit_cast(float, lsw);
        const int row = rb + j;
        if (rb >= kt0 + 31 && rb + 31 < n && kt0 + 31 < n) {
            // every row of the wavefront at or after every key of it
#pragma unroll
            for (int i = 0; i < 16; ++i) cs[i] += __builtin_amdgcn_exp2f(fmaf(acc[i], qs, nl));
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kt0 + 8 * (i >> 2) + 4 * h + (i & 3);
                if (key <= row && row < n && key < n) cs[i] += __builtin_amdgcn_exp2f(fmaf(acc[i], qs, nl));
            }
        }
    }
    // sum over the 32 rows of the lane half (lanes j = 0..31 of each h)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float x = cs[i];
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 8);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 1);
        cs[i] = x;
    }
    // the second row half's sums, then the first half adds them (fixed order)
    if (rh == 1 && j == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) half_sums[kg][8 * (i >> 2) + 4 * h + (i & 3)] = cs[i];
    }
    __syncthreads();
    if (rh == 0 && j == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kl = 8 * (i >> 2) + 4 * h + (i & 3), key = kt0 + kl;
            if (key < n) a.part[qhead * n + key] = cs[i] + half_sums[kg][kl];
        }
    }
}

// A_cumul of each KV head: its r query heads' column sums, added in head order.
template <int R>
__global__ __launch_bounds__(256) void prefill_colsum_add_kernel(PrefillArgs a, int64_t total) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // unit * n + key
    if (e >= total) return;
    const int64_t unit = e / a.n, key = e % a.n;
    const float* p = a.part + unit * R * a.n + key;
    float s = p[0];
#pragma unroll
    for (int h = 1; h < R; ++h) s += p[(int64_t)h * a.n];
    a.acc[e] = s;
}

template <int R>
void launch_prefill_t(const PrefillArgs& a, int batch, hipStream_t s) {
    const unsigned units = (unsigned)(batch * a.n_kv_heads);
    const unsigned qblocks = (unsigned)((a.n + 128 / R - 1) / (128 / R));
    hipLaunchKernelGGL((prefill_fwd_kernel<R>), dim3(qblocks, units), dim3(256), 0, s, a);
    if (a.acc) {
        const unsigned kblocks = (unsigned)((a.n + KB - 1) / KB);
        hipLaunchKernelGGL((prefill_colsum_kernel<R>), dim3(kblocks, units * R), dim3(256), 0, s, a);
        const int64_t total = (int64_t)units * a.n;
        hipLaunchKernelGGL((prefill_colsum_add_kernel<R>), dim3((unsigned)((total + 255) / 256)),
                           dim3(256), 0, s, a, total);
    }
}

// Rows idx[u][i] of each unit's K and V ([U][n][d]) to [U][n_keep][d].
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t* k, const uint16_t* v,
                                                     int32_t n, const int32_t* idx, int32_t n_keep,
                                                     uint16_t* ko, uint16_t* vo) {
    const int u = blockIdx.y;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 16-byte piece
    if (e >= (int64_t)n_keep * 16) return;
    const int64_t i = e / 16;
    const int part = (int)(e % 16);
    const int32_t t = idx[(int64_t)u * n_keep + i];
    const int64_t dst = ((int64_t)u * n_keep + i) * D;
    if (t < 0 || t >= n) {  // an index outside the prompt gives a zero row
        reinterpret_cast<uint4*>(ko + dst)[part] = make_uint4(0u, 0u, 0u, 0u);
        reinterpret_cast<uint4*>(vo + dst)[part] = make_uint4(0u, 0u, 0u, 0u);
        return;
    }
    const int64_t src = ((int64_t)u * n + t) * D;
    reinterpret_cast<uint4*>(ko + dst)[part] = reinterpret_cast<const uint4*>(k + src)[part];
    reinterpret_cast<uint4*>(vo + dst)[part] = reinterpret_cast<const uint4*>(v + src)[part];
}

}  // namespace

int launch_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, int32_t batch,
                   int32_t n_q_heads, int32_t n_kv_heads, int32_t n, float* out, float* acc,
                   float* lse, void* stream) {
    (void)hipGetLastError();  // an error left by an earlier call is not this call's
    PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.acc = acc;
    a.lse = lse;
    // the partial column sums follow the log-sum-exp, 256-byte aligned
    a.part = lse + ((int64_t)batch * n_q_heads * n * 4 + 255) / 256 * 64;
    a.n = n;
    a.n_kv_heads = n_kv_heads;
    a.qscale = 1.4426950408889634f / sqrtf((float)D);
    const int r = n_q_heads / n_kv_heads;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (r == 1) launch_prefill_t<1>(a, batch, s);
    else if (r == 2) launch_prefill_t<2>(a, batch, s);
    else launch_prefill_t<4>(a, batch, s);
    return (int)hipGetLastError();
}

int launch_gather(const uint16_t* k, const uint16_t* v, int32_t units, int32_t n,
                  const int32_t* idx, int32_t n_keep, uint16_t* ko, uint16_t* vo, void* stream) {
    (void)hipGetLastError();  // an error left by an earlier call is not this call's
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)(((int64_t)n_keep * 16 + 255) / 256), units),
                       dim3(256), 0, s, k, v, n, idx, n_keep, ko, vo);
    return (int)hipGetLastError();
}

}  // namespace kvq

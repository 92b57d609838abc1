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
// Matrix-core layout (v_mfma_f32_16x16x32_f16): S^T = K Q^T is computed, so a
// lane of an S^T tile holds four keys of one query row; two key tiles give
// exactly the eight keys one lane contributes to a 32-key k-step of P V. The
// value operand is read from V^T in LDS with the same key order.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int D = kHeadDim;
constexpr int KB = 64;           // keys per block step
constexpr int KROW = D + 8;      // LDS row stride of the key tile (fp16)
constexpr int VROW = KB + 4;     // LDS row stride of the transposed value tile (fp16)

__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float max_x16(float x) {
    return fmaxf(x, __shfl_xor(x, 16));
}
__device__ __forceinline__ float max_x32(float x) {
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum_x16(float x) { return x + __shfl_xor(x, 16); }
__device__ __forceinline__ float sum_x32(float x) { return x + __shfl_xor(x, 32); }

struct PrefillArgs {
    const uint16_t* q;  // [B][Hq][n][d]
    const uint16_t* k;  // [B][Hkv][n][d]
    const uint16_t* v;
    float* out;         // [B][Hq][n][d]
    float* acc;         // [B][Hkv][n] or null
    float* lse;         // [B][Hq][n]: log2 of each row's softmax normaliser (log2 units)
    int32_t n, n_kv_heads;
    float qscale;       // log2(e) / sqrt(d)
};

// Block (query block x, unit y = b * Hkv + h_kv): 128 / r query rows of each of
// the r query heads of the KV head. Wavefront w takes head w % r and the 32
// rows (w / r) * 32 .. + 31 of the block (two 16-row tiles).
template <int R>
__global__ __launch_bounds__(256) void prefill_fwd_kernel(PrefillArgs a) {
    constexpr int QR = 128 / R;  // query rows per block
    __shared__ __align__(16) uint16_t ks[KB][KROW];
    __shared__ __align__(16) uint16_t vt[D][VROW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = a.n;
    const int unit = blockIdx.y, b = unit / a.n_kv_heads, hkv = unit % a.n_kv_heads;
    const int q0 = blockIdx.x * QR;
    const int hl = wave % R, row0 = q0 + (wave / R) * 32;
    const int hq = hkv * R + hl;
    const int64_t qbase = ((int64_t)b * a.n_kv_heads * R + hq) * n;
    const int64_t kvbase = (int64_t)unit * n;
    const int j = lane & 15, kb = lane >> 4;

    // query operands: tile rt, k-step kst: row row0 + 16 rt + j, channels
    // 32 kst + 8 kb .. + 7 (zero rows past n)
    half8 Qo[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int row = row0 + 16 * rt + j;
#pragma unroll
        for (int kst = 0; kst < 4; ++kst) {
            uint4 w = make_uint4(0u, 0u, 0u, 0u);
            if (row < n)
                w = *reinterpret_cast<const uint4*>(a.q + (qbase + row) * D + 32 * kst + 8 * kb);
            Qo[rt][kst] = __builtin_bit_cast(half8, w);
        }
    }
    floatx4 O[2][8];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) O[rt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};  // of row row0 + 16 rt + j

    const int kend = n < q0 + QR ? n : q0 + QR;  // keys any row of the block sees
    const int nkb = (kend + KB - 1) / KB;
    // tile staging: 64 keys x 128 channels of K (row-major) and V (transposed)
    uint4 kr[4], vr[4];
    auto fetch = [&](int t) {
        const int k0 = t * KB;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = tid + 256 * i, key = p / 16, c8 = p % 16;
            const bool ok = k0 + key < n;
            kr[i] = ok ? *reinterpret_cast<const uint4*>(a.k + (kvbase + k0 + key) * D + 8 * c8)
                       : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            // two consecutive keys of the same 8 channels, stored as key pairs
            const int p = tid + 256 * i, kp = p / 16, c8 = p % 16;
            const int key = 2 * kp;
            vr[2 * i] = k0 + key < n
                            ? *reinterpret_cast<const uint4*>(a.v + (kvbase + k0 + key) * D + 8 * c8)
                            : make_uint4(0u, 0u, 0u, 0u);
            vr[2 * i + 1] = k0 + key + 1 < n ? *reinterpret_cast<const uint4*>(
                                                   a.v + (kvbase + k0 + key + 1) * D + 8 * c8)
                                             : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = tid + 256 * i, key = p / 16, c8 = p % 16;
            *reinterpret_cast<uint4*>(&ks[key][8 * c8]) = kr[i];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = tid + 256 * i, kp = p / 16, c8 = p % 16;
            const uint32_t a0[4] = {vr[2 * i].x, vr[2 * i].y, vr[2 * i].z, vr[2 * i].w};
            const uint32_t a1[4] = {vr[2 * i + 1].x, vr[2 * i + 1].y, vr[2 * i + 1].z,
                                    vr[2 * i + 1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t lo = (a0[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
                const uint32_t hi = (a1[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
                *reinterpret_cast<uint32_t*>(&vt[8 * c8 + e][2 * kp]) = lo | (hi << 16);
            }
        }
    };
    if (nkb > 0) fetch(0);
    for (int t = 0; t < nkb; ++t) {
        __syncthreads();  // the previous tile is no longer read
        stage();
        __syncthreads();
        if (t + 1 < nkb) fetch(t + 1);
        const int k0 = t * KB;
        if (k0 > row0 + 31 || row0 >= n) continue;  // every key of the tile is after this wave's rows
        // S^T tiles: key tile kt, row tile rt; lane holds keys k0 + 16 kt + 4 kb + i
        // of row row0 + 16 rt + j
        floatx4 St[2][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            half8 Ak[4];
#pragma unroll
            for (int kst = 0; kst < 4; ++kst)
                Ak[kst] = *reinterpret_cast<const half8*>(&ks[16 * kt + j][32 * kst + 8 * kb]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kst = 0; kst < 4; ++kst)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ak[kst], Qo[rt][kst], acc, 0, 0, 0);
                St[rt][kt] = acc;
            }
        }
        half8 Ap[2][2];  // P operands of the two 32-key k-steps
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int row = row0 + 16 * rt + j;
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = k0 + 16 * kt + 4 * kb + i;
                    float s = St[rt][kt][i] * a.qscale;
                    if (key > row || key >= n || row >= n) s = -INFINITY;
                    St[rt][kt][i] = s;
                    mx = fmaxf(mx, s);
                }
            mx = max_x32(max_x16(mx));
            const float mnew = fmaxf(m[rt], mx);
            // rows with nothing unmasked yet keep alpha = 1 and p = 0
            const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[rt] - mnew);
            const float mu = mnew == -INFINITY ? 0.f : mnew;
            float ps = 0.f;
            float p[4][4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[kt][i] = __builtin_amdgcn_exp2f(St[rt][kt][i] - mu);
                    ps += p[kt][i];
                }
            ps = sum_x32(sum_x16(ps));
            l[rt] = l[rt] * alpha + ps;
            m[rt] = mnew;
            // rescale the output rows 4 kb + i of the tile by their rows' alpha
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * kb + i);
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) O[rt][nt][i] *= ai;
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                Ap[rt][s2] = half8{(_Float16)p[2 * s2][0], (_Float16)p[2 * s2][1],
                                   (_Float16)p[2 * s2][2], (_Float16)p[2 * s2][3],
                                   (_Float16)p[2 * s2 + 1][0], (_Float16)p[2 * s2 + 1][1],
                                   (_Float16)p[2 * s2 + 1][2], (_Float16)p[2 * s2 + 1][3]};
        }
        // O += P V: value operand of tile nt, k-step s2: channel 16 nt + j, keys
        // k0 + 32 s2 + 4 kb + 0..3 and k0 + 32 s2 + 16 + 4 kb + 0..3
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const half4 v0 = *reinterpret_cast<const half4*>(&vt[16 * nt + j][32 * s2 + 4 * kb]);
                const half4 v1 =
                    *reinterpret_cast<const half4*>(&vt[16 * nt + j][32 * s2 + 16 + 4 * kb]);
                const half8 Bv = half8{v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                    O[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ap[rt][s2], Bv, O[rt][nt], 0, 0, 0);
            }
        }
    }
    // outputs: rows 4 kb + i of each tile, channel 16 nt + j; log-sum-exp per row
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const float linv = l[rt] > 0.f ? 1.0f / l[rt] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = row0 + 16 * rt + 4 * kb + i;
            const float li = __shfl(linv, 4 * kb + i);
            if (row < n) {
                float* o = a.out + (qbase + row) * D;
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) o[16 * nt + j] = O[rt][nt][i] * li;
            }
        }
        const int row = row0 + 16 * rt + j;
        if (kb == 0 && row < n) a.lse[qbase + row] = m[rt] + log2f(l[rt]);
    }
}

// Column sums: block (key block x of 64 keys, unit y); wavefront w owns keys
// k0 + 16 w .. + 15 and walks every query row at or after them, for each of
// the r query heads, adding exp2(s - lse_row) (the normalized probability).
template <int R>
__global__ __launch_bounds__(256) void prefill_colsum_kernel(PrefillArgs a) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = a.n;
    const int unit = blockIdx.y, b = unit / a.n_kv_heads, hkv = unit % a.n_kv_heads;
    const int kt0 = blockIdx.x * KB + 16 * wave;  // first key of this wavefront
    if (kt0 >= n) return;
    const int64_t kvbase = (int64_t)unit * n;
    const int j = lane & 15, kb = lane >> 4;
    // key operands (A of S^T): key kt0 + j, channels 32 kst + 8 kb .. + 7
    half8 Ak[4];
#pragma unroll
    for (int kst = 0; kst < 4; ++kst) {
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (kt0 + j < n)
            w = *reinterpret_cast<const uint4*>(a.k + (kvbase + kt0 + j) * D + 32 * kst + 8 * kb);
        Ak[kst] = __builtin_bit_cast(half8, w);
    }
    float cs[4] = {0.f, 0.f, 0.f, 0.f};  // keys kt0 + 4 kb + i, partial over this lane's rows
    const int qt_first = kt0 / 16, qt_end = (n + 15) / 16;
    for (int h = 0; h < R; ++h) {
        const int64_t qbase = ((int64_t)b * a.n_kv_heads * R + hkv * R + h) * n;
        for (int qt = qt_first; qt < qt_end; ++qt) {
            const int row = 16 * qt + j;
            half8 Bq[4];
#pragma unroll
            for (int kst = 0; kst < 4; ++kst) {
                uint4 w = make_uint4(0u, 0u, 0u, 0u);
                if (row < n)
                    w = *reinterpret_cast<const uint4*>(a.q + (qbase + row) * D + 32 * kst + 8 * kb);
                Bq[kst] = __builtin_bit_cast(half8, w);
            }
            const float ls = row < n ? a.lse[qbase + row] : INFINITY;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kst = 0; kst < 4; ++kst)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ak[kst], Bq[kst], acc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kt0 + 4 * kb + i;
                if (key <= row && row < n && key < n)
                    cs[i] += __builtin_amdgcn_exp2f(acc[i] * a.qscale - ls);
            }
        }
    }
    // sum over the 16 rows of the lane group (lanes j = 0..15 of each kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float x = cs[i];
        x += __shfl_xor(x, 8);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 1);
        cs[i] = x;
    }
    if (j == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kt0 + 4 * kb + i;
            if (key < n) a.acc[kvbase + key] = cs[i];
        }
    }
}

template <int R>
void launch_prefill_t(const PrefillArgs& a, int batch, hipStream_t s) {
    const unsigned units = (unsigned)(batch * a.n_kv_heads);
    const unsigned qblocks = (unsigned)((a.n + 128 / R - 1) / (128 / R));
    hipLaunchKernelGGL((prefill_fwd_kernel<R>), dim3(qblocks, units), dim3(256), 0, s, a);
    if (a.acc) {
        const unsigned kblocks = (unsigned)((a.n + KB - 1) / KB);
        hipLaunchKernelGGL((prefill_colsum_kernel<R>), dim3(kblocks, units), dim3(256), 0, s, a);
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

// Generic scaled dot-product attention forward: any head size up to 512,
// fp32 or bf16 storage, fp32 arithmetic, no matrix cores.
//
// Computes Eq. (1) of page "Attention Is All You Need/paper/es" (§3.2.1),
// softmax(Q K^T / sqrt(d_k)) V, with -inf for illegal connections (§3.2.3)
// and, given a radius, for keys outside the neighbourhood of restricted
// self-attention (§4, Table 1).
// It is the path for fp32 inputs and for head sizes the matrix-core kernel is
// not built for.
//
// Head sizes up to 8 (sdpa_fwd_generic_kernel; the pages' worked examples and
// the tiny fp32 configuration): one wave (64 lanes) per workgroup, one query
// row per lane, 64 rows per workgroup; a 1-D grid of ceil(Lq / 64) * B*H
// workgroups, the query tile index varying fastest.  Keys and values are
// staged through LDS in tiles of TK rows converted to fp32; every lane reads the
// same LDS word at a time (a broadcast, free of bank conflicts).  The softmax
// is evaluated online, tile by tile: the running maximum m and sum l per row
// are rescaled when m grows, which equals the plain softmax because a common
// shift of the scores does not change it (page "Self-Attention คืออะไร
// (แบบจับต้องได้)", section on dividing by sqrt(d_k): [100,100,100] splits
// like [0,0,0]).
//
// Head sizes 9 .. 512 (sdpa_fwd_wide_kernel; Table 3 row (A) of page
// "Attention Is All You Need/paper/es" ends at h = 1, d_k = d_v = 512): a
// whole row's q and accumulator in one lane would spill to scratch from
// d = 32 on, so G = 2 (d <= 64), 4 (d <= 128), 8 (d <= 256) or 16 (d <= 512)
// lanes share a query row, lane l holding dims 32*l .. 32*l + 31; 256 / G
// rows per 256-thread workgroup.  A score is the sum of the G lanes'
// partial dot products (log2 G xor shuffles inside the group), after which all
// G lanes hold the same score and run the same online softmax on their own
// dims.  K and V tiles (32, 16 or 8 keys) are staged as fp32 with each lane's
// chunk padded by 16 bytes, so that the G lanes' 16-byte reads of one key row
// fall in distinct banks (the other rows of the wave read the same addresses:
// broadcast), and the next tile's rows are loaded into registers while the
// current tile computes.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sdpa_kernels.h"

namespace sdpa {
namespace {

constexpr int kRows = 64;  // query rows per workgroup (= lanes)
constexpr int kTK = 16;    // keys per LDS tile

template <typename T>
__device__ inline float to_f32(T x);
template <>
__device__ inline float to_f32<float>(float x) { return x; }
template <>
__device__ inline float to_f32<__bf16>(__bf16 x) { return (float)x; }

template <typename T>
__device__ inline T from_f32(float x);
template <>
__device__ inline float from_f32<float>(float x) { return x; }
template <>
__device__ inline __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }  // nearest even

template <typename T, int DMAX>
__global__ __launch_bounds__(kRows) void sdpa_fwd_generic_kernel(
    const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
    const int32_t *__restrict__ key_lengths, int causal, int64_t radius, T *__restrict__ O,
    int H, int64_t Lq, int64_t Lk, int d_k, int d_v, float scale, uint32_t n_qtiles)
{
    __shared__ float Ks[kTK][DMAX];
    __shared__ float Vs[kTK][DMAX];

    const int lane = threadIdx.x;
    const int64_t bh = blockIdx.x / n_qtiles;
    const int64_t b = bh / H;
    const int64_t q0 = (int64_t)(blockIdx.x % n_qtiles) * kRows;
    const int64_t i = q0 + lane;           // this lane's query row
    const bool row_ok = i < Lq;

    int64_t len = Lk;
    if (key_lengths) {
        int64_t l = key_lengths[b];
        len = l < 0 ? 0 : (l > Lk ? Lk : l);
    }
    // Keys this workgroup can use: j < len and, if causal, j <= i < q0 + kRows;
    // with a radius (restricted self-attention), q0 - radius <= j <
    // q0 + kRows + radius.
    int64_t kv_end = len;
    if (causal && q0 + kRows < kv_end) kv_end = q0 + kRows;
    int64_t kv_begin = 0;
    if (radius >= 0) {
        if (q0 + kRows + radius < kv_end) kv_end = q0 + kRows + radius;
        kv_begin = q0 > radius ? q0 - radius : 0;
    }

    float q[DMAX];
    float acc[DMAX];
#pragma unroll
    for (int t = 0; t < DMAX; ++t) {
        q[t] = (row_ok && t < d_k) ? to_f32(Q[(bh * Lq + i) * d_k + t]) : 0.f;
        acc[t] = 0.f;
    }
    float m = -INFINITY;   // running maximum of the scaled scores
    float l = 0.f;         // running sum of exp(score - m)

    const T *Kh = K + bh * Lk * d_k;
    const T *Vh = V + bh * Lk * d_v;

    for (int64_t j0 = kv_begin; j0 < kv_end; j0 += kTK) {
        __syncthreads();
        // Stage rows j0 .. j0+kTK-1; rows at or beyond kv_end are zero-filled,
        // so padding contents (even NaN) never reach the arithmetic.
        for (int e = lane; e < kTK * DMAX; e += kRows) {
            const int r = e / DMAX, t = e % DMAX;
            const int64_t j = j0 + r;
            const bool in = j < kv_end;
            Ks[r][t] = (in && t < d_k) ? to_f32(Kh[j * d_k + t]) : 0.f;
            Vs[r][t] = (in && t < d_v) ? to_f32(Vh[j * d_v + t]) : 0.f;
        }
        __syncthreads();

        float s[kTK];
        float tile_max = -INFINITY;
#pragma unroll
        for (int r = 0; r < kTK; ++r) {
            const int64_t j = j0 + r;
            float dot = 0.f;
#pragma unroll
            for (int t = 0; t < DMAX; ++t) dot = fmaf(q[t], Ks[r][t], dot);
            const bool legal = j < kv_end && (!causal || j <= i) &&
                               (radius < 0 || (j >= i - radius && j <= i + radius));
            s[r] = legal ? dot * scale : -INFINITY;
            tile_max = fmaxf(tile_max, s[r]);
        }
        const float m_new = fmaxf(m, tile_max);
        // While every score seen so far is -inf, exponentiate against 0 instead
        // of -inf so that exp(-inf - (-inf)) never produces NaN.
        const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = expf(m - m_ref);
        l *= alpha;
#pragma unroll
        for (int t = 0; t < DMAX; ++t) acc[t] *= alpha;
#pragma unroll
        for (int r = 0; r < kTK; ++r) {
            const float p = expf(s[r] - m_ref);
            l += p;
#pragma unroll
            for (int t = 0; t < DMAX; ++t) acc[t] = fmaf(p, Vs[r][t], acc[t]);
        }
        m = m_new;
    }

    if (row_ok) {
        const float inv = l > 0.f ? 1.f / l : 0.f;   // no legal key: output 0
        T *o = O + (bh * Lq + i) * d_v;
#pragma unroll
        for (int t = 0; t < DMAX; ++t)
            if (t < d_v) o[t] = from_f32<T>(acc[t] * inv);
    }
}

constexpr int kWDL = 32;        // dims per lane (wide kernel)
constexpr int kWThreads = 256;  // threads per workgroup (wide kernel)

// Eight consecutive elements of a K or V row, as loaded from memory.
template <typename T>
struct Raw8;
template <>
struct Raw8<__bf16> {
    uint4 w;
    __device__ void to_f32(float *f) const
    {
        const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = __builtin_bit_cast(float, v[k] << 16);
            f[2 * k + 1] = __builtin_bit_cast(float, v[k] & 0xFFFF0000u);
        }
    }
};
template <>
struct Raw8<float> {
    uint4 w[2];
    __device__ void to_f32(float *f) const
    {
        const uint32_t v[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = __builtin_bit_cast(float, v[k]);
    }
};

// Elements t .. t+7 of row j (zeros at or beyond kv_end or d); VEC: the row
// starts are 16-byte aligned and d is a multiple of 8, so whole groups load
// as vectors.
template <typename T, bool VEC>
__device__ inline Raw8<T> load8(const T *base, int64_t j, int t, int64_t kv_end, int d)
{
    Raw8<T> r;
    const bool in = j < kv_end;
    if constexpr (VEC) {
        if (in && t < d) {
            r = *(const Raw8<T> *)(base + j * d + t);
        } else {
            r = Raw8<T>{};
        }
    } else {
        T e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) e[k] = (in && t + k < d) ? base[j * d + t + k] : (T)0.f;
        r = __builtin_bit_cast(Raw8<T>, e);
    }
    return r;
}

template <typename T, int G, bool VEC>
__global__ __launch_bounds__(kWThreads) void sdpa_fwd_wide_kernel(
    const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
    const int32_t *__restrict__ key_lengths, int causal, int64_t radius, T *__restrict__ O,
    int H, int64_t Lq, int64_t Lk, int d_k, int d_v, float scale, uint32_t n_qtiles)
{
    constexpr int DL = kWDL;
    constexpr int kRowsWG = kWThreads / G;  // query rows per workgroup
    constexpr int kTK = G >= 16 ? 8 : (G >= 4 ? 16 : 32);   // keys per LDS tile
    constexpr int kDim = G * DL;            // dims covered (>= d_k, d_v)
    constexpr int kLane = DL + 4;           // floats per lane chunk in LDS (16 B padding)
    constexpr int kRowF = G * kLane;        // floats per staged key row
    constexpr int kGroups = kTK * kDim / 8 / kWThreads;   // 8-element groups per thread, per tensor
    static_assert(kGroups * 8 * kWThreads == kTK * kDim, "whole groups per thread");
    __shared__ __attribute__((aligned(16))) float Ks[kTK * kRowF];
    __shared__ __attribute__((aligned(16))) float Vs[kTK * kRowF];

    const int tid = threadIdx.x;
    const int gl = tid % G;                 // lane within the row's group
    const int64_t bh = blockIdx.x / n_qtiles;
    const int64_t b = bh / H;
    const int64_t q0 = (int64_t)(blockIdx.x % n_qtiles) * kRowsWG;
    const int64_t i = q0 + tid / G;         // this group's query row
    const bool row_ok = i < Lq;

    int64_t len = Lk;
    if (key_lengths) {
        int64_t l = key_lengths[b];
        len = l < 0 ? 0 : (l > Lk ? Lk : l);
    }
    // Keys this workgroup can use (as in the kernel above, for kRowsWG rows).
    int64_t kv_end = len;
    if (causal && q0 + kRowsWG < kv_end) kv_end = q0 + kRowsWG;
    int64_t kv_begin = 0;
    if (radius >= 0) {
        if (q0 + kRowsWG + radius < kv_end) kv_end = q0 + kRowsWG + radius;
        kv_begin = q0 > radius ? q0 - radius : 0;
    }

    float q[DL];
    float acc[DL];
#pragma unroll
    for (int u = 0; u < DL; ++u) {
        const int t = gl * DL + u;
        q[u] = (row_ok && t < d_k) ? to_f32(Q[(bh * Lq + i) * d_k + t]) : 0.f;
        acc[u] = 0.f;
    }
    float m = -INFINITY;   // running maximum of the scaled scores
    float l = 0.f;         // running sum of exp(score - m)

    const T *Kh = K + bh * Lk * d_k;
    const T *Vh = V + bh * Lk * d_v;

    // Thread tid stages groups e = tid + kWThreads * k of each tile: key row
    // e / (kDim / 8), elements 8 * (e % (kDim / 8)) .. +7.  The next tile's
    // groups are loaded into registers while the current tile computes.
    Raw8<T> nk[kGroups], nv[kGroups];
    auto fetch = [&](int64_t j0) {
#pragma unroll
        for (int k = 0; k < kGroups; ++k) {
            const int e = tid + kWThreads * k;
            const int64_t j = j0 + e / (kDim / 8);
            const int t = 8 * (e % (kDim / 8));
            nk[k] = load8<T, VEC>(Kh, j, t, kv_end, d_k);
            nv[k] = load8<T, VEC>(Vh, j, t, kv_end, d_v);
        }
    };
    if (kv_begin < kv_end) fetch(kv_begin);

    for (int64_t j0 = kv_begin; j0 < kv_end; j0 += kTK) {
        __syncthreads();   // every thread is done with the previous tile
#pragma unroll
        for (int k = 0; k < kGroups; ++k) {
            const int e = tid + kWThreads * k;
            const int r = e / (kDim / 8), t = 8 * (e % (kDim / 8));
            const int at = r * kRowF + (t / DL) * kLane + t % DL;   // 8 elements stay in one lane chunk
            float f[8];
            nk[k].to_f32(f);
            *(float4 *)(Ks + at) = make_float4(f[0], f[1], f[2], f[3]);
            *(float4 *)(Ks + at + 4) = make_float4(f[4], f[5], f[6], f[7]);
            nv[k].to_f32(f);
            *(float4 *)(Vs + at) = make_float4(f[0], f[1], f[2], f[3]);
            *(float4 *)(Vs + at + 4) = make_float4(f[4], f[5], f[6], f[7]);
        }
        if (j0 + kTK < kv_end) fetch(j0 + kTK);
        __syncthreads();

        float s[kTK];
        float tile_max = -INFINITY;
#pragma unroll
        for (int r = 0; r < kTK; ++r) {
            const int64_t j = j0 + r;
            const float *kr = Ks + r * kRowF + gl * kLane;
            float dot = 0.f;
#pragma unroll
            for (int u = 0; u < DL; ++u) dot = fmaf(q[u], kr[u], dot);
#pragma unroll
            for (int x = 1; x < G; x <<= 1) dot += __shfl_xor(dot, x, G);
            const bool legal = j < kv_end && (!causal || j <= i) &&
                               (radius < 0 || (j >= i - radius && j <= i + radius));
            s[r] = legal ? dot * scale : -INFINITY;
            tile_max = fmaxf(tile_max, s[r]);
        }
        const float m_new = fmaxf(m, tile_max);
        const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;   // no NaN from -inf - -inf
        const float alpha = expf(m - m_ref);
        l *= alpha;
#pragma unroll
        for (int u = 0; u < DL; ++u) acc[u] *= alpha;
#pragma unroll
        for (int r = 0; r < kTK; ++r) {
            const float p = expf(s[r] - m_ref);
            l += p;
            const float *vr = Vs + r * kRowF + gl * kLane;
#pragma unroll
            for (int u = 0; u < DL; ++u) acc[u] = fmaf(p, vr[u], acc[u]);
        }
        m = m_new;
    }

    if (row_ok) {
        const float inv = l > 0.f ? 1.f / l : 0.f;   // no legal key: output 0
        T *o = O + (bh * Lq + i) * d_v;
#pragma unroll
        for (int u = 0; u < DL; ++u) {
            const int t = gl * DL + u;
            if (t < d_v) o[t] = from_f32<T>(acc[u] * inv);
        }
    }
}

template <typename T, int G>
hipError_t launch_wide(const void *Q, const void *K, const void *V, const int32_t *kl,
                       int causal, int64_t radius, void *out, int64_t B, int64_t H, int64_t Lq,
                       int64_t Lk, int d_k, int d_v, hipStream_t stream)
{
    constexpr int kRowsWG = kWThreads / G;
    const uint32_t n_qtiles = (uint32_t)((Lq + kRowsWG - 1) / kRowsWG);
    const dim3 grid((unsigned)(n_qtiles * B * H));
    const float scale = (float)(1.0 / sqrt((double)d_k));
    // whole 16-byte groups: rows 16-byte aligned and d a multiple of 8
    const bool vec = d_k % 8 == 0 && d_v % 8 == 0 && (uintptr_t)K % 16 == 0 && (uintptr_t)V % 16 == 0;
    if (vec)
        hipLaunchKernelGGL((sdpa_fwd_wide_kernel<T, G, true>), grid, dim3(kWThreads), 0, stream,
                           (const T *)Q, (const T *)K, (const T *)V, kl, causal, radius, (T *)out,
                           (int)H, Lq, Lk, d_k, d_v, scale, n_qtiles);
    else
        hipLaunchKernelGGL((sdpa_fwd_wide_kernel<T, G, false>), grid, dim3(kWThreads), 0, stream,
                           (const T *)Q, (const T *)K, (const T *)V, kl, causal, radius, (T *)out,
                           (int)H, Lq, Lk, d_k, d_v, scale, n_qtiles);
    return hipGetLastError();
}

template <typename T, int DMAX>
hipError_t launch_t(const void *Q, const void *K, const void *V, const int32_t *kl,
                    int causal, int64_t radius, void *out, int64_t B, int64_t H, int64_t Lq,
                    int64_t Lk, int d_k, int d_v, hipStream_t stream)
{
    const uint32_t n_qtiles = (uint32_t)((Lq + kRows - 1) / kRows);
    const dim3 grid((unsigned)(n_qtiles * B * H));
    const float scale = (float)(1.0 / sqrt((double)d_k));
    hipLaunchKernelGGL((sdpa_fwd_generic_kernel<T, DMAX>), grid, dim3(kRows), 0, stream,
                       (const T *)Q, (const T *)K, (const T *)V, kl, causal, radius, (T *)out,
                       (int)H, Lq, Lk, d_k, d_v, scale, n_qtiles);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_d(const void *Q, const void *K, const void *V, const int32_t *kl,
                    int causal, int64_t r, void *out, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                    int d_k, int d_v, hipStream_t stream)
{
    const int d = d_k > d_v ? d_k : d_v;
    if (d <= 8) return launch_t<T, 8>(Q, K, V, kl, causal, r, out, B, H, Lq, Lk, d_k, d_v, stream);
    if (d <= 64) return launch_wide<T, 2>(Q, K, V, kl, causal, r, out, B, H, Lq, Lk, d_k, d_v, stream);
    if (d <= 128) return launch_wide<T, 4>(Q, K, V, kl, causal, r, out, B, H, Lq, Lk, d_k, d_v, stream);
    if (d <= 256) return launch_wide<T, 8>(Q, K, V, kl, causal, r, out, B, H, Lq, Lk, d_k, d_v, stream);
    return launch_wide<T, 16>(Q, K, V, kl, causal, r, out, B, H, Lq, Lk, d_k, d_v, stream);
}

}  // namespace

hipError_t launch_generic(const void *Q, const void *K, const void *V,
                          const int32_t *key_lengths, int causal, int64_t radius, void *out,
                          int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                          int d_k, int d_v, bool is_bf16, hipStream_t stream)
{
    if (is_bf16)
        return launch_d<__bf16>(Q, K, V, key_lengths, causal, radius, out, B, H, Lq, Lk, d_k, d_v,
                                stream);
    return launch_d<float>(Q, K, V, key_lengths, causal, radius, out, B, H, Lq, Lk, d_k, d_v,
                           stream);
}

}  // namespace sdpa

// Generic scaled dot-product attention forward: any head size up to 128,
// fp32 or bf16 storage, fp32 arithmetic, no matrix cores.
//
// Computes Eq. (1) of page "Attention Is All You Need/paper/es" (§3.2.1),
// softmax(Q K^T / sqrt(d_k)) V, with -inf for illegal connections (§3.2.3)
// and, given a radius, for keys outside the neighbourhood of restricted
// self-attention (§4, Table 1).
// It is the path for fp32 inputs and for head sizes the matrix-core kernel is
// not built for.
//
// Work split: one wave (64 lanes) per workgroup, one query row per lane, 64
// rows per workgroup; a 1-D grid of ceil(Lq / 64) * B*H workgroups, the query
// tile index varying fastest.  Keys and values are
// staged through LDS in tiles of TK rows converted to fp32; every lane reads the
// same LDS word at a time (a broadcast, free of bank conflicts).  The softmax
// is evaluated online, tile by tile: the running maximum m and sum l per row
// are rescaled when m grows, which equals the plain softmax because a common
// shift of the scores does not change it (page "Self-Attention คืออะไร
// (แบบจับต้องได้)", section on dividing by sqrt(d_k): [100,100,100] splits
// like [0,0,0]).
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
    if (d <= 32) return launch_t<T, 32>(Q, K, V, kl, causal, r, out, B, H, Lq, Lk, d_k, d_v, stream);
    if (d <= 64) return launch_t<T, 64>(Q, K, V, kl, causal, r, out, B, H, Lq, Lk, d_k, d_v, stream);
    return launch_t<T, 128>(Q, K, V, kl, causal, r, out, B, H, Lq, Lk, d_k, d_v, stream);
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

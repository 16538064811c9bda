// Decode step with one new query row per head (Lq = 1), bf16, d_k = d_v = D
// with D in {64, 128}, on the vector units.
//
// What it computes: Eq. (1) of page "Attention Is All You Need/paper/es"
// (§3.2.1), softmax(q K^T / sqrt(d_k)) V for one query row q per head, with
// -inf for the padding keys j >= len_b (§3.2.3); the decoder's causal mask
// allows every cached key to the newest position, so there is no other mask.
//
// With a single query row the products are matrix-vector products: the
// matrix cores would spend 31 of their 32 query columns on nothing, so this
// kernel uses v_dot2_f32_bf16 (two bf16 products summed in fp32 per lane) for
// both of them.
//
// Layout (one wave, one "step" of kStep = 4096 / D keys):
//  * Lane = (c, j): c = lane % (D / 8) picks a 16-byte chunk of a row (8
//    dims), j = lane / (D / 8) a key.  Load instruction i (0..7) of a step
//    reads chunk c of key i * (512 / D) + j, so every instruction reads
//    512 / D whole rows (1 KiB contiguous) of K, and likewise of V, straight
//    into registers (no LDS staging).  A step is 16 loads per lane.
//  * Score of key (i, j): the lane's 8 dims against its 8 dims of q (4
//    v_dot2), summed over the D / 8 lanes of group j by DPP (row mirror,
//    half-row mirror, quad permutations): every lane of the group then holds
//    the score of each of its 8 keys.
//  * Softmax online in base 2 against a reference maximum m that moves only
//    when a step's maximum exceeds it by more than kTau (the shift cancels in
//    the final division; weights stay below 2^kTau).  The weights are rounded
//    to bf16; the row sum adds the rounded weights (the ones used in P V).
//  * P V: the lane accumulates its 8 output dims over its 8 keys, two keys at
//    a time: v_perm_b32 pairs the two keys' values of one dim, v_dot2 takes
//    them against the two weights.  At the end the partial sums of the groups
//    are added across lanes (DPP row rotation, v_permlane16_swap,
//    v_permlane32_swap).
//  * Two load sets (two steps) are in flight: the next step's rows are
//    loaded while the current one is computed.  Loads past the wave's keys
//    read 0 through the buffer descriptor's bound and cost no memory traffic.
//
// Work split: workgroup u = (head, chunk); the chunk [lo, lo + chunk) of the
// head's keys (cut to the batch's key length) is split evenly, in whole steps,
// over the NW waves (2 or 4), whose partial results (m, l, sum of weighted V)
// are merged in LDS.  With one chunk per head the workgroup writes O;
// otherwise it writes its partial result to the workspace (acc [u][D], m [u],
// l [u], floats), merged by a second kernel.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sdpa_kernels.h"
#include "sdpa_timeline.h"

namespace sdpa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kRsrcWord3 = 0x00020000;   // raw (stride 0) dword buffer access
// Cache policy of the key/value loads: non-temporal (nt; the builtin's slc
// position on gfx950).  A decode step reads each cached K/V row exactly once,
// so the rows stream through instead of being allocated in the L2 and the
// Infinity Cache.  Measured (interleaved rounds, cold caches): long decode
// -6.6 % (d = 64) and -4.6 % (d = 128), base decode -3.5 % and -6.5 %.
constexpr int kLoadStreaming = 2;
constexpr float kTau = 8.0f;             // lazy-rescale threshold, log2 units
constexpr int kLoads = 8;                // 16-byte loads of K (and of V) per lane per step
constexpr uint32_t kOnesBf16x2 = 0x3f803f80u;

// DPP controls (source lane within a row of 16 lanes)
constexpr int kQuadRev = 0x1B;           // quad_perm [3, 2, 1, 0]
constexpr int kQuadXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kRowMirror = 0x140;        // 15 - l
constexpr int kRowHalfMirror = 0x141;    // 7 - l within each half row
constexpr int kRowRor8 = 0x128;          // (l + 8) mod 16

template <int CTRL>
__device__ inline float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 0xf, 0xf, false));
}

__device__ inline float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                           c, false);
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32, nearest even
    return __builtin_bit_cast(uint32_t, v);
}

// Sum over the KC consecutive lanes of a key group (KC = 8 or 16).
template <int KC>
__device__ inline float group_sum(float v)
{
    if constexpr (KC == 16) v += dpp<kRowMirror>(v);
    v += dpp<kRowHalfMirror>(v);
    v += dpp<kQuadRev>(v);
    v += dpp<kQuadXor1>(v);
    return v;
}

// Combination of the lanes l, l + KC, l + 2 KC, ... (the same chunk in every
// key group): lane pairs at distance 8 (KC = 8 only), 16 and 32.
template <int KC, bool MAX>
__device__ inline float across_groups(float v)
{
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    if constexpr (KC == 8) v = op(v, dpp<kRowRor8>(v));
    const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                                    __builtin_bit_cast(uint32_t, v), false, false);
    v = op(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                                    __builtin_bit_cast(uint32_t, v), false, false);
    return op(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void sdpa_decode_row_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ key_lengths, uint16_t *__restrict__ O, float *__restrict__ ws,
    int H, int64_t Lk, int64_t chunk, uint32_t n_split, float scale_log2)
{
    static_assert(D == 64 || D == 128, "head sizes of the row kernel");
    static_assert(64 * NW >= D, "one thread per output dim in the merge");
    constexpr int kC = D / 8, kJ = 64 / kC, kStep = kLoads * kJ, kRowBytes = 2 * D;
    __shared__ float part[NW][D + 2];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane % kC, j = lane / kC;
    SDPA_STAMP(0);
    const uint32_t u = blockIdx.x;   // head * n_split + chunk
    const uint32_t bh = u / n_split;
    const int64_t b = bh / H;
    int64_t len = Lk;
    if (key_lengths) {
        const int64_t l = key_lengths[b];
        len = l < 0 ? 0 : (l > Lk ? Lk : l);
    }
    const int64_t lo = (int64_t)(u % n_split) * chunk;
    int64_t hi = lo + chunk < len ? lo + chunk : len;
    hi = hi < lo ? lo : hi;
    // this wave's keys [wlo, wlo + n): an even share of [lo, hi) in whole steps
    const int64_t per = ((hi - lo + NW - 1) / NW + kStep - 1) / kStep * kStep;
    const int64_t wlo = lo + wave * per;
    int64_t n = (wlo + per < hi ? wlo + per : hi) - wlo;
    n = n < 0 ? 0 : n;
    const int ns = (int)((n + kStep - 1) / kStep);

    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void *)(Q + (int64_t)bh * D), (short)0, kRowBytes, kRsrcWord3);
    const u32x4_t qc = __builtin_amdgcn_raw_buffer_load_b128(rq, (uint32_t)(c * 16), 0, 0);

    const uint16_t *Kw = K + ((int64_t)bh * Lk + wlo) * D;
    const uint16_t *Vw = V + ((int64_t)bh * Lk + wlo) * D;
    const uint32_t loff = (uint32_t)(j * kRowBytes + c * 16);
    // step s's rows into kr / vr; rows past the wave's keys read 0
    auto load = [&](int s, u32x4_t (&kr)[kLoads], u32x4_t (&vr)[kLoads]) {
        int64_t rows = n - (int64_t)s * kStep;
        rows = rows < 0 ? 0 : (rows > kStep ? kStep : rows);
        const int64_t off = rows > 0 ? (int64_t)s * kStep * D : 0;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(Kw + off), (short)0, (int)rows * kRowBytes, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(Vw + off), (short)0, (int)rows * kRowBytes, kRsrcWord3);
        // issue order = step order, so that waiting for one step's rows
        // never waits for a later step's
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            kr[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, loff + (uint32_t)(i * kJ * kRowBytes), 0, kLoadStreaming);
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            vr[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, loff + (uint32_t)(i * kJ * kRowBytes), 0, kLoadStreaming);
        __builtin_amdgcn_sched_barrier(0);
    };

    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    float m_run = -INFINITY;   // reference maximum (scaled, base 2), the same in every lane
    float l_run = 0.f;         // weight sum of the lane's key group

    auto step = [&](int s, const u32x4_t (&kr)[kLoads], const u32x4_t (&vr)[kLoads]) {
        float x[kLoads];
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            float a = dot2(kr[i].x, qc.x, 0.f);
            a = dot2(kr[i].y, qc.y, a);
            a = dot2(kr[i].z, qc.z, a);
            x[i] = dot2(kr[i].w, qc.w, a);
        }
#pragma unroll
        for (int i = 0; i < kLoads; ++i) x[i] = group_sum<kC>(x[i]);
        const int64_t k0 = (int64_t)s * kStep + j;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) x[i] = k0 + i * kJ < n ? x[i] * scale_log2 : -INFINITY;
        float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        mx = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                           __builtin_bit_cast(int, across_groups<kC, true>(mx))));
        if (mx > m_run + kTau) {
            // the first legal key finds m_run = -inf: alpha = 0 (nothing to keep)
            const float alpha = __builtin_amdgcn_exp2f(m_run - mx);
            m_run = mx;
            l_run *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] *= alpha;
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;   // no legal key yet: all weights 0
        uint32_t pp[kLoads / 2];
#pragma unroll
        for (int k = 0; k < kLoads / 2; ++k)
            pp[k] = pack_bf16x2(__builtin_amdgcn_exp2f(x[2 * k] - m_use),
                                __builtin_amdgcn_exp2f(x[2 * k + 1] - m_use));
#pragma unroll
        for (int k = 0; k < kLoads / 2; ++k) l_run = dot2(pp[k], kOnesBf16x2, l_run);
#pragma unroll
        for (int k = 0; k < kLoads / 2; ++k) {
            const uint32_t v0[4] = {vr[2 * k].x, vr[2 * k].y, vr[2 * k].z, vr[2 * k].w};
            const uint32_t v1[4] = {vr[2 * k + 1].x, vr[2 * k + 1].y, vr[2 * k + 1].z, vr[2 * k + 1].w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // (dim 2w of key 2k, of key 2k+1) and (dim 2w+1 of both)
                const uint32_t lo2 = __builtin_amdgcn_perm(v1[w], v0[w], 0x05040100u);
                const uint32_t hi2 = __builtin_amdgcn_perm(v1[w], v0[w], 0x07060302u);
                acc[2 * w] = dot2(lo2, pp[k], acc[2 * w]);
                acc[2 * w + 1] = dot2(hi2, pp[k], acc[2 * w + 1]);
            }
        }
    };

    u32x4_t ka[kLoads], va[kLoads], kb[kLoads], vb[kLoads];
    load(0, ka, va);
    load(1, kb, vb);
    for (int s = 0; s < ns; s += 2) {
        step(s, ka, va);
        if (s == 0) SDPA_STAMP(1);
        load(s + 2, ka, va);
        if (s + 1 < ns) step(s + 1, kb, vb);
        load(s + 3, kb, vb);
    }

    SDPA_STAMP(2);
    // the wave's partial result: sums over the key groups
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = across_groups<kC, false>(acc[e]);
    l_run = across_groups<kC, false>(l_run);
    if (lane < kC) {
#pragma unroll
        for (int e = 0; e < 8; ++e) part[wave][8 * c + e] = acc[e];
    }
    if (lane == 0) {
        part[wave][D] = m_run;
        part[wave][D + 1] = l_run;
    }
    __syncthreads();

    // merge of the waves: O = sum_w e^(m_w - M) acc_w / sum_w e^(m_w - M) l_w (base 2)
    const int t = threadIdx.x;
    if (t < D) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, part[w][D]);
        float num = 0.f, den = 0.f;
        if (M > -INFINITY) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float mw = part[w][D];
                const float e = mw > -INFINITY ? __builtin_amdgcn_exp2f(mw - M) : 0.f;
                num += e * part[w][t];
                den += e * part[w][D + 1];
            }
        }
        if (n_split == 1) {
            const float o = den > 0.f ? num / den : 0.f;   // no legal key: output 0
            O[(int64_t)bh * D + t] = __builtin_bit_cast(uint16_t, (__bf16)o);
        } else {
            const int64_t n_rows = (int64_t)gridDim.x;   // heads * n_split partial rows
            ws[(int64_t)u * D + t] = num;
            if (t == 0) {
                ws[n_rows * D + u] = M;
                ws[n_rows * (D + 1) + u] = den;
            }
        }
    }
    SDPA_STAMP(3);
}

template <int D, int NW>
hipError_t launch_row_d(const void *Q, const void *K, const void *V, const int32_t *key_lengths, void *out,
                        int64_t B, int64_t H, int64_t Lk, int64_t chunk, int64_t n_split, void *workspace,
                        hipStream_t stream)
{
    const int64_t n_bh = B * H;
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    hipLaunchKernelGGL((sdpa_decode_row_kernel<D, NW>), dim3((uint32_t)(n_bh * n_split)), dim3(64 * NW), 0,
                       stream, (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, key_lengths,
                       (uint16_t *)out, (float *)workspace, (int)H, Lk, chunk, (uint32_t)n_split, scale_log2);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || n_split == 1) return err;
    return launch_decode_merge((const float *)workspace, out, n_bh, 1, n_split, D, stream);
}

}  // namespace

hipError_t launch_decode_row(const void *Q, const void *K, const void *V, const int32_t *key_lengths,
                             void *out, int64_t B, int64_t H, int64_t Lk, int d, int waves, int64_t chunk,
                             int64_t n_split, void *workspace, hipStream_t stream)
{
    if (waves != 2 && waves != 4) return hipErrorInvalidValue;
    const bool two = waves == 2;
    if (d == 64)
        return two ? launch_row_d<64, 2>(Q, K, V, key_lengths, out, B, H, Lk, chunk, n_split, workspace, stream)
                   : launch_row_d<64, 4>(Q, K, V, key_lengths, out, B, H, Lk, chunk, n_split, workspace, stream);
    if (d == 128)
        return two ? launch_row_d<128, 2>(Q, K, V, key_lengths, out, B, H, Lk, chunk, n_split, workspace, stream)
                   : launch_row_d<128, 4>(Q, K, V, key_lengths, out, B, H, Lk, chunk, n_split, workspace, stream);
    return hipErrorInvalidValue;
}

}  // namespace sdpa

#ifdef SDPA_TIMELINE
// Timeline build only: the records of this file's kernel (sdpa_timeline.h).
extern "C" int sdpa_timeline_row(void *host, int64_t bytes, int clear)
{
    return sdpa::timeline_io(host, bytes, clear);
}
#endif

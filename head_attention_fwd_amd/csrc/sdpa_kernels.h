// Internal launchers of libsdpa's kernels.  Not part of the public C ABI.
//
// Every launcher assumes the host layer has validated its arguments: non-null
// pointers, sizes >= 1, B*H and the grid within the hardware limits, and the
// head dimensions within the kernel's compiled bounds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

// Any 1 <= d_k, d_v <= 512; elements are fp32 (is_bf16 = false) or bf16.
// fp32 arithmetic throughout on the vector units: one lane per query row up to
// d = 8, then 2 (d <= 64), 4 (d <= 128), 8 (d <= 256) or 16 (d <= 512) lanes per
// query row.  radius >= 0:
// restricted self-attention (|i - j| <= radius); radius < 0: no restriction.
hipError_t launch_generic(const void *Q, const void *K, const void *V,
                          const int32_t *key_lengths, int causal, int64_t radius, void *out,
                          int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                          int d_k, int d_v, bool is_bf16, hipStream_t stream);

// bf16, d_k = d_v = d with d in {16, 32, 64, 128}, on the matrix cores
// (hipErrorInvalidValue for any other d).  streaming: the inputs come from and
// the output goes to memory nobody reads soon (output stores, and for heads
// with few query tiles the Q/K/V copies, with the non-temporal cache policy);
// false when the output is read right away or the inputs were just written.
hipError_t launch_mfma(const void *Q, const void *K, const void *V,
                       const int32_t *key_lengths, int causal, void *out,
                       int64_t B, int64_t H, int64_t Lq, int64_t Lk, int d,
                       bool streaming, hipStream_t stream);

// bf16, d_k = d_v = d with d in {256, 512}, on the matrix cores (16 query rows
// per wave, v_mfma_f32_16x16x32_bf16); hipErrorInvalidValue for any other d.
// streaming: as for launch_mfma.
hipError_t launch_mfma_wide(const void *Q, const void *K, const void *V,
                            const int32_t *key_lengths, int causal, void *out,
                            int64_t B, int64_t H, int64_t Lq, int64_t Lk, int d,
                            bool streaming, hipStream_t stream);

// As launch_mfma, restricted self-attention: key j is legal for query i only
// when |i - j| <= radius (radius >= 0).
hipError_t launch_mfma_band(const void *Q, const void *K, const void *V,
                            const int32_t *key_lengths, int causal, int64_t radius, void *out,
                            int64_t B, int64_t H, int64_t Lq, int64_t Lk, int d,
                            hipStream_t stream);

// Decode step, bf16, d_k = d_v = d in {64, 128}, Lq <= 32, no causal mask.
// n_split == 0: one four-wave workgroup per head, its keys split over the
// waves and merged in LDS (workspace unused).  n_split == 1: one one-wave
// workgroup per head writes out directly (workspace unused).  n_split > 1: keys split into n_split chunks of `chunk` keys per head
// (chunk a multiple of 64, n_split * chunk >= Lk), partial results in
// `workspace` (4 * (d + 2) * B * H * n_split * Lq bytes), then merged into out
// (two kernels on `stream`).
hipError_t launch_decode(const void *Q, const void *K, const void *V, const int32_t *key_lengths,
                         void *out, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int d,
                         int64_t chunk, int64_t n_split, void *workspace, hipStream_t stream);

// Decode step with one query row per head (Lq = 1), bf16, d_k = d_v = d in
// {64, 128}, on the vector units: workgroups of `waves` (2 or 4) waves, one
// per (head, chunk of `chunk` keys), n_split chunks per head (n_split * chunk
// >= Lk).  n_split == 1: each workgroup writes its head's row of out
// (workspace unused); n_split > 1: partial results in `workspace` (4 * (d + 2)
// * B * H * n_split bytes), then merged into out (two kernels on `stream`).
hipError_t launch_decode_row(const void *Q, const void *K, const void *V, const int32_t *key_lengths,
                             void *out, int64_t B, int64_t H, int64_t Lk, int d, int waves, int64_t chunk,
                             int64_t n_split, void *workspace, hipStream_t stream);

// Merge of key-split partial results (floats in `ws`: acc [R][d], m [R], l [R]
// with R = n_bh * n_split * Lq, row (head, split, query row) at (bh * n_split
// + s) * Lq + i) into out [n_bh][Lq][d] (bf16); d in {64, 128}.
hipError_t launch_decode_merge(const float *ws, void *out, int64_t n_bh, int64_t Lq, int64_t n_split,
                               int d, hipStream_t stream);

// Projection products of multi-head attention, C = A W on the matrix cores
// (bf16, fp32 accumulation), tiles of 128 x 128 or 256 x 256 elements of C
// (chosen by the launcher from the problem size), k in steps of 32.
struct GemmSegment {
    const void *W;       // [K, N] row-major
    void *C;             // c_mode 0: [M, N] row-major; c_mode 1: [B, Hc, Lc, d], column n = head*d + t
    int64_t N;           // columns of this product (multiple of 8)
    int64_t d;           // c_mode 1: head size (multiple of 8)
    int64_t c_elems;     // elements of C
    int n_tiles;         // set by launch_proj_gemm
};
// Up to three products that share A, their output columns side by side.
struct GemmSegments {
    GemmSegment seg[3];
    int count;
    uint32_t n_ntiles;   // set by launch_proj_gemm
};
struct GemmShape {
    int64_t M, K;        // rows of A and C; K a multiple of 32
    uint32_t n_mtiles;   // set by launch_proj_gemm
    int64_t La, Ha, da;  // a_mode 1: A(m, k) = heads[b][k / da][i][k % da], m = b*La + i (da % 32 == 0)
    int64_t a_elems;     // elements of A
    int64_t Lc, Hc;      // c_mode 1: m = b*Lc + i, Hc heads
};
// a_mode 0: A row-major [M, K]; a_mode 1: the head gather above.  c_mode as in
// GemmSegment.  Every buffer below 2 GiB - 1 MiB.
hipError_t launch_proj_gemm(const void *A, int a_mode, const GemmShape &shape,
                            const GemmSegments &segs, int c_mode, hipStream_t stream);

}  // namespace sdpa

// Internal launchers of libsdpa's kernels.  Not part of the public C ABI.
//
// Every launcher assumes the host layer has validated its arguments: non-null
// pointers, sizes >= 1, B*H and the grid within the hardware limits, and the
// head dimensions within the kernel's compiled bounds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

// Any 1 <= d_k, d_v <= 128; elements are fp32 (is_bf16 = false) or bf16.
// fp32 arithmetic throughout; one lane per query row.  radius >= 0: restricted
// self-attention (|i - j| <= radius); radius < 0: no restriction.
hipError_t launch_generic(const void *Q, const void *K, const void *V,
                          const int32_t *key_lengths, int causal, int64_t radius, void *out,
                          int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                          int d_k, int d_v, bool is_bf16, hipStream_t stream);

// bf16, d_k = d_v = d with d in {32, 64, 128}, on the matrix cores
// (hipErrorInvalidValue for any other d).
hipError_t launch_mfma(const void *Q, const void *K, const void *V,
                       const int32_t *key_lengths, int causal, void *out,
                       int64_t B, int64_t H, int64_t Lq, int64_t Lk, int d,
                       hipStream_t stream);

// As launch_mfma, restricted self-attention: key j is legal for query i only
// when |i - j| <= radius (radius >= 0).
hipError_t launch_mfma_band(const void *Q, const void *K, const void *V,
                            const int32_t *key_lengths, int causal, int64_t radius, void *out,
                            int64_t B, int64_t H, int64_t Lq, int64_t Lk, int d,
                            hipStream_t stream);

// bf16, d_k = d_v = 64, Lq <= 32, no causal mask: keys split into n_split chunks
// of `chunk` keys per head (chunk a multiple of 64, n_split * chunk >= Lk),
// partial results in `workspace` (4 * 66 * B * H * n_split * Lq bytes), then
// merged into out.  Two kernels on `stream`.
hipError_t launch_split_mfma_d64(const void *Q, const void *K, const void *V,
                                 const int32_t *key_lengths, void *out, int64_t B, int64_t H,
                                 int64_t Lq, int64_t Lk, int64_t chunk, int64_t n_split,
                                 void *workspace, hipStream_t stream);

}  // namespace sdpa

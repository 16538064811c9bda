// libsdpa C ABI: argument validation, kernel choice and launch.
//
// The declarations, argument meaning, layouts and error behaviour are in
// include/sdpa.h.  Validation happens entirely on the host before any HIP call,
// so an invalid call never touches the device or the output buffer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <initializer_list>

#include "sdpa.h"
#include "sdpa_kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxHeadDim = 128;
constexpr int64_t kMaxDim = INT32_MAX;
// Workgroups of a 1-D launch: grid size in work-items must fit in 32 bits.
constexpr int64_t kMaxWorkgroups = (int64_t)1 << 24;

bool overlaps(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes)
{
    if (!a || !b || a_bytes <= 0 || b_bytes <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

// n = x * y * z * w with overflow detection (all factors >= 0).
bool mul_ok(int64_t &n, std::initializer_list<int64_t> f)
{
    n = 1;
    for (int64_t x : f) {
        if (x != 0 && n > INT64_MAX / x) return false;
        n *= x;
    }
    return true;
}

}  // namespace

extern "C" {

const char *sdpa_status_str(sdpa_status s)
{
    switch (s) {
    case SDPA_OK: return "success";
    case SDPA_ERR_NULL_POINTER: return "a required pointer (Q, K, V or out) is NULL";
    case SDPA_ERR_BAD_SHAPE: return "invalid shape: a size is negative or exceeds the limits";
    case SDPA_ERR_UNSUPPORTED: return "unsupported dtype or head dimension";
    case SDPA_ERR_ALIAS: return "out overlaps an input buffer";
    case SDPA_ERR_HIP: return "a HIP runtime call failed (see sdpa_last_hip_error)";
    }
    return "unknown sdpa_status";
}

int sdpa_last_hip_error(void) { return g_last_hip_error; }

sdpa_status sdpa_forward(const void *Q, const void *K, const void *V,
                         const int32_t *key_lengths, int causal, void *out,
                         int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                         int64_t d_k, int64_t d_v, sdpa_dtype dtype, void *stream)
{
    if (B < 0 || H < 0 || Lq < 0 || Lk < 0 || d_k < 1 || d_v < 1) return SDPA_ERR_BAD_SHAPE;
    if (dtype != SDPA_F32 && dtype != SDPA_BF16) return SDPA_ERR_UNSUPPORTED;
    if (d_k > kMaxHeadDim || d_v > kMaxHeadDim) return SDPA_ERR_UNSUPPORTED;
    if (B > kMaxDim || H > kMaxDim || Lq > kMaxDim || Lk > kMaxDim) return SDPA_ERR_BAD_SHAPE;
    if (B == 0 || H == 0 || Lq == 0) return SDPA_OK;   // empty output: nothing to write

    const int64_t elem = dtype == SDPA_BF16 ? 2 : 4;
    int64_t nq, nk, nv, no;
    if (!mul_ok(nq, {B, H, Lq, d_k, elem}) || !mul_ok(nk, {B, H, Lk, d_k, elem}) ||
        !mul_ok(nv, {B, H, Lk, d_v, elem}) || !mul_ok(no, {B, H, Lq, d_v, elem}))
        return SDPA_ERR_BAD_SHAPE;
    if (B * H > kMaxDim) return SDPA_ERR_BAD_SHAPE;
    // Both kernels use at most ceil(Lq / 64) workgroups per head.
    if (((Lq + 63) / 64) > kMaxWorkgroups / (B * H)) return SDPA_ERR_BAD_SHAPE;

    if (!Q || !out || (Lk > 0 && (!K || !V))) return SDPA_ERR_NULL_POINTER;
    if (overlaps(out, no, Q, nq) || overlaps(out, no, K, nk) || overlaps(out, no, V, nv) ||
        overlaps(out, no, key_lengths, 4 * B))
        return SDPA_ERR_ALIAS;

    hipStream_t s = (hipStream_t)stream;
    hipError_t err;
    // Lk == 0 needs no special case: both kernels then stage no key tile and
    // write 0 for every row (no legal connection).
    if (dtype == SDPA_BF16 && d_k == 64 && d_v == 64) {
        err = sdpa::launch_mfma_d64(Q, K, V, key_lengths, causal ? 1 : 0, out, B, H, Lq, Lk, s);
    } else {
        err = sdpa::launch_generic(Q, K, V, key_lengths, causal ? 1 : 0, out, B, H, Lq, Lk,
                                   (int)d_k, (int)d_v, dtype == SDPA_BF16, s);
    }
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return SDPA_ERR_HIP;
    }
    return SDPA_OK;
}

}  // extern "C"

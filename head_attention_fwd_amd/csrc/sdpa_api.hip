// libsdpa C ABI: argument validation, kernel choice and launch.
//
// The declarations, argument meaning, layouts and error behaviour are in
// include/sdpa.h.  Validation happens entirely on the host before any HIP call,
// so an invalid call never touches the device or the output buffer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string.h>

#include <initializer_list>
#include <mutex>

#include "sdpa.h"
#include "sdpa_kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

// The C ABI declares enum parameters, but a caller may pass any integer there;
// in C++ an enum object holding a value outside its enumerators' range may not
// be read as the enum, so the entry points take its bytes as an int first.
static_assert(sizeof(sdpa_dtype) == sizeof(int) && sizeof(sdpa_status) == sizeof(int),
              "enums of the C ABI are int-sized");
template <class E>
int enum_value(const E &e)
{
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}

constexpr int64_t kMaxHeadDim = 512;
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

sdpa_status hip_status(hipError_t err)
{
    if (err == hipSuccess) return SDPA_OK;
    g_last_hip_error = (int)err;
    return SDPA_ERR_HIP;
}

// Size checks shared by every entry point (no pointers involved).
sdpa_status check_sizes(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d_k, int64_t d_v,
                        int dtype)
{
    if (B < 0 || H < 0 || Lq < 0 || Lk < 0 || d_k < 1 || d_v < 1) return SDPA_ERR_BAD_SHAPE;
    if (dtype != SDPA_F32 && dtype != SDPA_BF16) return SDPA_ERR_UNSUPPORTED;
    if (d_k > kMaxHeadDim || d_v > kMaxHeadDim) return SDPA_ERR_UNSUPPORTED;
    if (B > kMaxDim || H > kMaxDim || Lq > kMaxDim || Lk > kMaxDim) return SDPA_ERR_BAD_SHAPE;
    if (B == 0 || H == 0 || Lq == 0) return SDPA_OK;   // empty output: nothing to write
    const int64_t elem = dtype == SDPA_BF16 ? 2 : 4;
    int64_t n;
    if (!mul_ok(n, {B, H, Lq, d_k, elem}) || !mul_ok(n, {B, H, Lk, d_k, elem}) ||
        !mul_ok(n, {B, H, Lk, d_v, elem}) || !mul_ok(n, {B, H, Lq, d_v, elem}))
        return SDPA_ERR_BAD_SHAPE;
    if (B * H > kMaxDim) return SDPA_ERR_BAD_SHAPE;
    // Every kernel uses at most ceil(Lq / 16) workgroups per head (the wide
    // kernel at d > 256: 16 query rows per workgroup).
    if (((Lq + 15) / 16) > kMaxWorkgroups / (B * H)) return SDPA_ERR_BAD_SHAPE;
    return SDPA_OK;
}

struct Sizes {
    int64_t nq = 0, nk = 0, nv = 0, no = 0;   // bytes of Q, K, V, out
    bool empty = false;
};

// Everything sdpa_forward checks before any HIP call.
sdpa_status validate(const void *Q, const void *K, const void *V, const int32_t *key_lengths,
                     const void *out, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d_k,
                     int64_t d_v, int dtype, Sizes &z)
{
    const sdpa_status st = check_sizes(B, H, Lq, Lk, d_k, d_v, dtype);
    if (st != SDPA_OK) return st;
    if (B == 0 || H == 0 || Lq == 0) {
        z.empty = true;
        return SDPA_OK;
    }
    const int64_t elem = dtype == SDPA_BF16 ? 2 : 4;
    mul_ok(z.nq, {B, H, Lq, d_k, elem});
    mul_ok(z.nk, {B, H, Lk, d_k, elem});
    mul_ok(z.nv, {B, H, Lk, d_v, elem});
    mul_ok(z.no, {B, H, Lq, d_v, elem});
    if (!Q || !out || (Lk > 0 && (!K || !V))) return SDPA_ERR_NULL_POINTER;
    if (overlaps(out, z.no, Q, z.nq) || overlaps(out, z.no, K, z.nk) || overlaps(out, z.no, V, z.nv) ||
        overlaps(out, z.no, key_lengths, 4 * B))
        return SDPA_ERR_ALIAS;
    return SDPA_OK;
}

// radius < 0: unrestricted attention; radius >= 0: keys within radius of the
// query row only (restricted self-attention).
sdpa_status forward_kernels(const void *Q, const void *K, const void *V, const int32_t *key_lengths,
                            int causal, void *out, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                            int64_t d_k, int64_t d_v, int dtype, hipStream_t s,
                            int64_t radius = -1, bool streaming = true)
{
    // A radius that reaches every (query, key) pair restricts nothing: the
    // largest |i - j| is max(Lq, Lk) - 1.  Then the unrestricted kernels run
    // (the same result as sdpa_forward, bit for bit).
    if (radius >= Lq - 1 && radius >= Lk - 1) radius = -1;
    // Lk == 0 needs no special case: both kernels then stage no key tile and
    // write 0 for every row (no legal connection).
    if (dtype == SDPA_BF16 && d_k == d_v && (d_k == 16 || d_k == 32 || d_k == 64 || d_k == 128)) {
        if (radius >= 0)
            return hip_status(sdpa::launch_mfma_band(Q, K, V, key_lengths, causal ? 1 : 0, radius, out,
                                                     B, H, Lq, Lk, (int)d_k, s));
        return hip_status(sdpa::launch_mfma(Q, K, V, key_lengths, causal ? 1 : 0, out, B, H, Lq, Lk,
                                            (int)d_k, streaming, s));
    }
    if (dtype == SDPA_BF16 && d_k == d_v && (d_k == 256 || d_k == 512) && radius < 0)
        return hip_status(sdpa::launch_mfma_wide(Q, K, V, key_lengths, causal ? 1 : 0, out, B, H, Lq, Lk,
                                                 (int)d_k, streaming, s));
    return hip_status(sdpa::launch_generic(Q, K, V, key_lengths, causal ? 1 : 0, radius, out, B, H,
                                           Lq, Lk, (int)d_k, (int)d_v, dtype == SDPA_BF16, s));
}

// The dedicated paths of sdpa_decode: bf16, d_k = d_v in {64, 128}, at most 32
// query rows; a single query row takes the vector-unit kernel, more rows the
// matrix-core one (a 32-row wave per chunk of keys).
bool split_applies(int64_t Lq, int64_t d_k, int64_t d_v, int dtype)
{
    return dtype == SDPA_BF16 && d_k == d_v && (d_k == 64 || d_k == 128) && Lq >= 1 && Lq <= 32;
}

// Chunks per head of the matrix-core decode kernels (2 to 32 query rows).  With
// many heads (at least kWgHeads = 256: four waves per head then give every CU a
// few waves), n_split = 0: each head's keys are split
// over the four waves of one workgroup and merged in LDS.  Otherwise enough
// chunks for about 1536 one-wave workgroups (three per CU, two rounds), at
// least two 64-key tiles per chunk, merged by a second kernel (n_split = 1:
// one chunk covers the head, no merge).  chunk is a multiple of 64;
// n_split * chunk >= Lk.
struct SplitPlan {
    int64_t chunk, n_split;
};
SplitPlan split_plan(int64_t n_bh, int64_t Lk)
{
    constexpr int64_t kWgHeads = 256, kTarget = 1536, kTile = 64, kMinChunk = 2 * kTile;
    if (n_bh >= kWgHeads) return SplitPlan{Lk, 0};
    int64_t want = (kTarget + n_bh - 1) / n_bh;
    const int64_t most = (Lk + kMinChunk - 1) / kMinChunk;
    if (want > most) want = most;
    if (want < 1) want = 1;
    int64_t chunk = (Lk + want - 1) / want;
    chunk = (chunk + kTile - 1) / kTile * kTile;
    if (chunk < kTile) chunk = kTile;
    return SplitPlan{chunk, (Lk + chunk - 1) / chunk > 0 ? (Lk + chunk - 1) / chunk : 1};
}

// Plan of the single-row kernel (steps of 4096 / d keys).  With many heads (at
// least 256) one chunk covers each head; otherwise chunks of four waves with at
// least two steps per wave, enough of them for about 2048 waves (two per
// SIMD), merged by a second kernel.  A head in one chunk takes two waves when
// it has at most four steps of keys, else four.  chunk is a whole number of
// steps per wave; n_split * chunk >= Lk.
struct DecodePlan {
    bool row;        // single-row kernel (else the matrix-core decode kernels)
    int waves;       // single-row kernel: waves per workgroup
    SplitPlan sp;
};
DecodePlan row_plan(int64_t n_bh, int64_t Lk, int64_t d)
{
    constexpr int64_t kWgHeads = 256, kTargetWaves = 2048, kNw = 4;
    const int64_t step = 4096 / d, steps = (Lk + step - 1) / step;
    const DecodePlan whole{true, steps <= 4 ? 2 : 4, SplitPlan{Lk, 1}};
    if (n_bh >= kWgHeads) return whole;
    int64_t spw = (n_bh * steps + kTargetWaves - 1) / kTargetWaves;
    spw = spw < 2 ? 2 : spw;
    const int64_t n_split = (steps + kNw * spw - 1) / (kNw * spw);
    if (n_split <= 1) return whole;
    int64_t cs = (steps + n_split - 1) / n_split;   // steps per chunk, a multiple of kNw
    cs = (cs + kNw - 1) / kNw * kNw;
    return DecodePlan{true, (int)kNw, SplitPlan{cs * step, (steps + cs - 1) / cs}};
}

// The plan of one sdpa_decode call on a dedicated path.
DecodePlan decode_plan(int64_t n_bh, int64_t Lq, int64_t Lk, int64_t d)
{
    if (Lq == 1) return row_plan(n_bh, Lk, d);
    return DecodePlan{false, 0, split_plan(n_bh, Lk)};
}

// Partial results (fp32 acc [d_v], m and l per split and query row); none
// when one chunk covers each head.
int64_t split_workspace_bytes(int64_t n_bh, int64_t Lq, int64_t d_v, const SplitPlan &sp)
{
    return sp.n_split <= 1 ? 0 : 4 * (d_v + 2) * n_bh * sp.n_split * Lq;
}

sdpa_status launch_decode_plan(const DecodePlan &dp, const void *Q, const void *K, const void *V,
                               const int32_t *key_lengths, void *out, int64_t B, int64_t H, int64_t Lq,
                               int64_t Lk, int d, void *workspace, hipStream_t s)
{
    if (dp.row)
        return hip_status(sdpa::launch_decode_row(Q, K, V, key_lengths, out, B, H, Lk, d, dp.waves,
                                                  dp.sp.chunk, dp.sp.n_split, workspace, s));
    return hip_status(sdpa::launch_decode(Q, K, V, key_lengths, out, B, H, Lq, Lk, d, dp.sp.chunk,
                                          dp.sp.n_split, workspace, s));
}

// ---- device scratch of sdpa_decode_noalloc
//
// The key-split partial results of sdpa_decode_noalloc live in this array: one
// copy per device (each GPU the library runs on holds it until the process
// ends), so the entry point allocates nothing.  In host code `scratch` is only
// a host-side stand-in; its device address is looked up once per device with
// hipGetSymbolAddress and only that address is passed to kernels.
constexpr int64_t kScratchBytes = SDPA_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device (null: not looked up)

// The device address of `scratch` on device `dev`, looked up with that device
// current on the first call for it.
hipError_t device_scratch(int dev, void **ptr)
{
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        hipError_t err = hipGetDevice(&cur);
        if (err != hipSuccess) return err;
        if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess) return err;
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (err == hipSuccess) err = back;
        }
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

// ---- multi-head attention: projections around the attention (§3.2.2)

// Largest buffer a projection product addresses (32-bit offsets, with room for
// the out-of-range marker).
constexpr int64_t kMaxGemmBytes = ((int64_t)1 << 31) - ((int64_t)1 << 20);

struct MhPlan {
    int64_t q_bytes, k_bytes, v_bytes, a_bytes;   // head-major Q, K, V, attention output
    int64_t q_off, k_off, v_off, a_off, total;    // workspace offsets (256-byte aligned)
    int64_t x_q_bytes, x_kv_bytes, out_bytes, wq_bytes, wk_bytes, wv_bytes, wo_bytes;
};

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

sdpa_status mh_plan(int64_t B, int64_t Lq, int64_t Lk, int64_t d_model, int64_t h, int64_t d_k,
                    int64_t d_v, int dtype, MhPlan &p)
{
    if (B < 0 || Lq < 0 || Lk < 0 || d_model < 1 || h < 1 || d_k < 1 || d_v < 1)
        return SDPA_ERR_BAD_SHAPE;
    if (dtype != SDPA_BF16) return SDPA_ERR_UNSUPPORTED;
    if (d_k > kMaxHeadDim || d_v > kMaxHeadDim || d_model % 32 != 0 || d_k % 8 != 0 ||
        d_v % 32 != 0)
        return SDPA_ERR_UNSUPPORTED;
    if (B > kMaxDim || Lq > kMaxDim || Lk > kMaxDim || d_model > kMaxDim || h > kMaxDim)
        return SDPA_ERR_BAD_SHAPE;
    const sdpa_status st = check_sizes(B, h, Lq, Lk, d_k, d_v, dtype);
    if (st != SDPA_OK) return st;
    bool ok = mul_ok(p.q_bytes, {B, h, Lq, d_k, 2}) && mul_ok(p.k_bytes, {B, h, Lk, d_k, 2}) &&
              mul_ok(p.v_bytes, {B, h, Lk, d_v, 2}) && mul_ok(p.a_bytes, {B, h, Lq, d_v, 2}) &&
              mul_ok(p.x_q_bytes, {B, Lq, d_model, 2}) && mul_ok(p.x_kv_bytes, {B, Lk, d_model, 2}) &&
              mul_ok(p.wq_bytes, {d_model, h, d_k, 2}) && mul_ok(p.wv_bytes, {d_model, h, d_v, 2});
    if (!ok) return SDPA_ERR_BAD_SHAPE;
    p.out_bytes = p.x_q_bytes;
    p.wk_bytes = p.wq_bytes;
    p.wo_bytes = p.wv_bytes;
    for (int64_t n : {p.q_bytes, p.k_bytes, p.v_bytes, p.a_bytes, p.x_q_bytes, p.x_kv_bytes,
                      p.wq_bytes, p.wv_bytes})
        if (n > kMaxGemmBytes) return SDPA_ERR_BAD_SHAPE;
    p.q_off = 0;
    p.k_off = align256(p.q_off + p.q_bytes);
    p.v_off = align256(p.k_off + p.k_bytes);
    p.a_off = align256(p.v_off + p.v_bytes);
    p.total = align256(p.a_off + p.a_bytes);
    // projection grids (128 x 128 tiles at most): row tiles times at most 3
    // products' column tiles
    const int64_t mt = (B * (Lq > Lk ? Lq : Lk) + 127) / 128;
    const int64_t nt = 3 * ((h * (d_k > d_v ? d_k : d_v) + 127) / 128) + (d_model + 127) / 128;
    if (mt > 0 && nt > kMaxWorkgroups / mt) return SDPA_ERR_BAD_SHAPE;
    return SDPA_OK;
}

sdpa::GemmSegment segment(const void *W, void *C, int64_t N, int64_t d, int64_t c_elems)
{
    sdpa::GemmSegment sg;
    sg.W = W;
    sg.C = C;
    sg.N = N;
    sg.d = d;
    sg.c_elems = c_elems;
    sg.n_tiles = 0;   // set by the launcher
    return sg;
}

}  // namespace

extern "C" {

const char *sdpa_status_str(sdpa_status status)
{
    switch (enum_value(status)) {
    case SDPA_OK: return "success";
    case SDPA_ERR_NULL_POINTER: return "a required pointer (Q, K, V or out) is NULL";
    case SDPA_ERR_BAD_SHAPE: return "invalid shape: a size is negative or exceeds the limits";
    case SDPA_ERR_UNSUPPORTED: return "unsupported dtype or head dimension";
    case SDPA_ERR_ALIAS: return "out overlaps an input buffer";
    case SDPA_ERR_HIP: return "a HIP runtime call failed (see sdpa_last_hip_error)";
    case SDPA_ERR_WORKSPACE: return "the workspace is missing, too small, or overlaps another buffer";
    case SDPA_ERR_SCRATCH_LIMIT:
        return "the call needs more scratch than the library's static device scratch holds "
               "(sdpa_decode_noalloc: see SDPA_DECODE_NOALLOC_SCRATCH_BYTES; use sdpa_decode)";
    }
    return "unknown sdpa_status";
}

int sdpa_last_hip_error(void) { return g_last_hip_error; }

sdpa_status sdpa_forward(const void *Q, const void *K, const void *V,
                         const int32_t *key_lengths, int causal, void *out,
                         int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                         int64_t d_k, int64_t d_v, sdpa_dtype dtype, void *stream)
{
    const int dt = enum_value(dtype);
    Sizes z;
    const sdpa_status st = validate(Q, K, V, key_lengths, out, B, H, Lq, Lk, d_k, d_v, dt, z);
    if (st != SDPA_OK || z.empty) return st;
    return forward_kernels(Q, K, V, key_lengths, causal, out, B, H, Lq, Lk, d_k, d_v, dt,
                           (hipStream_t)stream);
}

int64_t sdpa_multihead_workspace_bytes(int64_t B, int64_t Lq, int64_t Lk, int64_t d_model,
                                       int64_t h, int64_t d_k, int64_t d_v, sdpa_dtype dtype)
{
    const int dt = enum_value(dtype);
    MhPlan p;
    if (mh_plan(B, Lq, Lk, d_model, h, d_k, d_v, dt, p) != SDPA_OK) return -1;
    return p.total;
}

sdpa_status sdpa_multihead_forward(const void *Xq, const void *Xkv, const void *Wq, const void *Wk,
                                   const void *Wv, const void *Wo, const int32_t *key_lengths,
                                   int causal, void *out, int64_t B, int64_t Lq, int64_t Lk,
                                   int64_t d_model, int64_t h, int64_t d_k, int64_t d_v,
                                   sdpa_dtype dtype, void *workspace, int64_t workspace_bytes,
                                   void *stream)
{
    const int dt = enum_value(dtype);
    MhPlan p;
    const sdpa_status st = mh_plan(B, Lq, Lk, d_model, h, d_k, d_v, dt, p);
    if (st != SDPA_OK) return st;
    if (B == 0 || Lq == 0) return SDPA_OK;   // empty output
    if (!Xq || !Wq || !Wk || !Wv || !Wo || !out || (Lk > 0 && !Xkv)) return SDPA_ERR_NULL_POINTER;
    if (overlaps(out, p.out_bytes, Xq, p.x_q_bytes) || overlaps(out, p.out_bytes, Xkv, p.x_kv_bytes) ||
        overlaps(out, p.out_bytes, Wq, p.wq_bytes) || overlaps(out, p.out_bytes, Wk, p.wk_bytes) ||
        overlaps(out, p.out_bytes, Wv, p.wv_bytes) || overlaps(out, p.out_bytes, Wo, p.wo_bytes) ||
        overlaps(out, p.out_bytes, key_lengths, 4 * B))
        return SDPA_ERR_ALIAS;
    if (!workspace || workspace_bytes < p.total) return SDPA_ERR_WORKSPACE;
    if (overlaps(workspace, p.total, Xq, p.x_q_bytes) || overlaps(workspace, p.total, Xkv, p.x_kv_bytes) ||
        overlaps(workspace, p.total, Wq, p.wq_bytes) || overlaps(workspace, p.total, Wk, p.wk_bytes) ||
        overlaps(workspace, p.total, Wv, p.wv_bytes) || overlaps(workspace, p.total, Wo, p.wo_bytes) ||
        overlaps(workspace, p.total, out, p.out_bytes) ||
        overlaps(workspace, p.total, key_lengths, 4 * B))
        return SDPA_ERR_WORKSPACE;

    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    void *Qh = ws + p.q_off, *Kh = ws + p.k_off, *Vh = ws + p.v_off, *Ah = ws + p.a_off;

    // 1. Q W_i^Q, K W_i^K, V W_i^V for every head, into [B, h, L, d]; one launch
    //    when queries, keys and values come from the same sequence.
    sdpa::GemmShape sq{};
    sq.K = d_model;
    sq.M = B * Lq;

    sq.Lc = Lq;
    sq.Hc = h;
    sdpa::GemmSegments gq{};
    gq.seg[0] = segment(Wq, Qh, h * d_k, d_k, p.q_bytes / 2);
    gq.count = 1;
    const bool self_attn = Xkv == Xq && Lk == Lq;
    if (self_attn) {
        gq.seg[1] = segment(Wk, Kh, h * d_k, d_k, p.k_bytes / 2);
        gq.seg[2] = segment(Wv, Vh, h * d_v, d_v, p.v_bytes / 2);
        gq.count = 3;
    }
    sdpa_status r = hip_status(sdpa::launch_proj_gemm(Xq, 0, sq, gq, 1, s));
    if (r != SDPA_OK) return r;
    if (!self_attn && Lk > 0) {
        sdpa::GemmShape sk = sq;
        sk.M = B * Lk;
        sk.Lc = Lk;
        sdpa::GemmSegments gk{};
        gk.seg[0] = segment(Wk, Kh, h * d_k, d_k, p.k_bytes / 2);
        gk.seg[1] = segment(Wv, Vh, h * d_v, d_v, p.v_bytes / 2);
        gk.count = 2;
        r = hip_status(sdpa::launch_proj_gemm(Xkv, 0, sk, gk, 1, s));
        if (r != SDPA_OK) return r;
    }

    // 2. head_i = Attention(...) for every head (Eq. (1) with the masks).
    // the heads were just written by the projection and the output projection
    // reads the result next: no streaming cache policy
    r = forward_kernels(Qh, Kh, Vh, key_lengths, causal, Ah, B, h, Lq, Lk, d_k, d_v, SDPA_BF16, s,
                        -1, false);
    if (r != SDPA_OK) return r;

    // 3. Concat(head_1, ..., head_h) W^O, the concatenation read in place.
    sdpa::GemmShape so{};
    so.M = B * Lq;
    so.K = h * d_v;
    so.La = Lq;
    so.Ha = h;
    so.da = d_v;
    so.a_elems = p.a_bytes / 2;
    sdpa::GemmSegments go{};
    go.seg[0] = segment(Wo, out, d_model, d_model, p.out_bytes / 2);
    go.count = 1;
    return hip_status(sdpa::launch_proj_gemm(Ah, 1, so, go, 0, s));
}

sdpa_status sdpa_forward_restricted(const void *Q, const void *K, const void *V,
                                    const int32_t *key_lengths, int causal, int64_t radius,
                                    void *out, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                                    int64_t d_k, int64_t d_v, sdpa_dtype dtype, void *stream)
{
    const int dt = enum_value(dtype);
    if (radius < 0) return SDPA_ERR_BAD_SHAPE;
    Sizes z;
    const sdpa_status st = validate(Q, K, V, key_lengths, out, B, H, Lq, Lk, d_k, d_v, dt, z);
    if (st != SDPA_OK || z.empty) return st;
    return forward_kernels(Q, K, V, key_lengths, causal, out, B, H, Lq, Lk, d_k, d_v, dt,
                           (hipStream_t)stream, radius);
}

int64_t sdpa_decode_workspace_bytes(int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                                    int64_t d_k, int64_t d_v, sdpa_dtype dtype)
{
    const int dt = enum_value(dtype);
    const sdpa_status st = check_sizes(B, H, Lq, Lk, d_k, d_v, dt);
    if (st != SDPA_OK) return -1;
    if (B == 0 || H == 0 || Lq == 0) return 0;
    if (!split_applies(Lq, d_k, d_v, dt)) return 0;
    return split_workspace_bytes(B * H, Lq, d_v, decode_plan(B * H, Lq, Lk, d_k).sp);
}

sdpa_status sdpa_decode(const void *Q, const void *K, const void *V,
                        const int32_t *key_lengths, void *out,
                        int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                        int64_t d_k, int64_t d_v, sdpa_dtype dtype,
                        void *workspace, int64_t workspace_bytes, void *stream)
{
    const int dt = enum_value(dtype);
    Sizes z;
    const sdpa_status st = validate(Q, K, V, key_lengths, out, B, H, Lq, Lk, d_k, d_v, dt, z);
    if (st != SDPA_OK || z.empty) return st;
    hipStream_t s = (hipStream_t)stream;
    if (!split_applies(Lq, d_k, d_v, dt))
        return forward_kernels(Q, K, V, key_lengths, 0, out, B, H, Lq, Lk, d_k, d_v, dt, s);

    const DecodePlan dp = decode_plan(B * H, Lq, Lk, d_k);
    const SplitPlan &sp = dp.sp;
    const int64_t need = split_workspace_bytes(B * H, Lq, d_v, sp);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return SDPA_ERR_WORKSPACE;
        if (overlaps(workspace, need, Q, z.nq) || overlaps(workspace, need, K, z.nk) ||
            overlaps(workspace, need, V, z.nv) || overlaps(workspace, need, out, z.no) ||
            overlaps(workspace, need, key_lengths, 4 * B))
            return SDPA_ERR_WORKSPACE;
    }
    if (B * H * sp.n_split > kMaxWorkgroups || B * H * Lq > kMaxWorkgroups) return SDPA_ERR_BAD_SHAPE;
    return launch_decode_plan(dp, Q, K, V, key_lengths, out, B, H, Lq, Lk, (int)d_k,
                              need > 0 ? workspace : nullptr, s);
}

sdpa_status sdpa_decode_noalloc(const void *Q, const void *K, const void *V,
                                const int32_t *key_lengths, void *out,
                                int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                                int64_t d_k, int64_t d_v, sdpa_dtype dtype, void *stream)
{
    const int dt = enum_value(dtype);
    Sizes z;
    const sdpa_status st = validate(Q, K, V, key_lengths, out, B, H, Lq, Lk, d_k, d_v, dt, z);
    if (st != SDPA_OK || z.empty) return st;
    hipStream_t s = (hipStream_t)stream;
    if (!split_applies(Lq, d_k, d_v, dt))
        return forward_kernels(Q, K, V, key_lengths, 0, out, B, H, Lq, Lk, d_k, d_v, dt, s);
    const DecodePlan dp = decode_plan(B * H, Lq, Lk, d_k);
    const SplitPlan &sp = dp.sp;
    const int64_t need = split_workspace_bytes(B * H, Lq, d_v, sp);
    if (need > kScratchBytes) return SDPA_ERR_SCRATCH_LIMIT;
    if (B * H * sp.n_split > kMaxWorkgroups || B * H * Lq > kMaxWorkgroups) return SDPA_ERR_BAD_SHAPE;
    void *ws = nullptr;
    if (need > 0) {
        int dev = -1;
        hipError_t err = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
        if (err == hipSuccess) err = device_scratch(dev, &ws);
        if (err != hipSuccess) return hip_status(err);
    }
    return launch_decode_plan(dp, Q, K, V, key_lengths, out, B, H, Lq, Lk, (int)d_k, ws, s);
}

}  // extern "C"

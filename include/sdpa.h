/*
 * sdpa.h -- C ABI of libsdpa: multi-head scaled dot-product attention, forward
 * pass, on an AMD Instinct MI355X (gfx950).
 *
 * The operation (page "Attention Is All You Need/paper/es", §3.2.1, Eq. (1);
 * §3.2.2 for the h heads; §3.2.3 for the mask):
 *
 *   out[b,h,i,:] = sum_j P[b,h,i,j] * V[b,h,j,:]
 *   P[b,h,i,:]   = softmax_j( Q[b,h,i,:] . K[b,h,j,:] / sqrt(d_k)  +  M[b,i,j] )
 *
 * with M[b,i,j] = -inf for an illegal connection and 0 otherwise.  Key j is
 * illegal for query i of batch entry b when
 *   j >= len_b            (key padding; len_b = clamp(key_lengths[b], 0, Lk),
 *                          or Lk when key_lengths is NULL), or
 *   causal && j > i       (a decoder position may use the positions up to and
 *                          including its own, §3.2.3; top-left aligned when
 *                          Lq != Lk).
 * A query row with no legal key gets out = 0.  The scale 1/sqrt(d_k) is fixed
 * by the method and is not a parameter.  There is no dropout in this pass.
 *
 * Uses covered by the same call (§3.2.3): encoder self-attention (causal = 0,
 * Lq = Lk), decoder causal self-attention (causal = 1), encoder-decoder
 * cross-attention (queries from the decoder, Lq != Lk allowed, key_lengths for
 * the encoder's padding).
 *
 * Layout.  Q [B,H,Lq,d_k], K [B,H,Lk,d_k], V [B,H,Lk,d_v], out [B,H,Lq,d_v]:
 * device pointers to contiguous row-major arrays of the element type `dtype`
 * (the same type for all four).  key_lengths: device pointer to int32[B], or
 * NULL.  Offsets are computed in 64 bits.
 *
 * Arithmetic.  SDPA_BF16 on the matrix cores (head sizes below): bf16
 * products with fp32 accumulation, fp32 softmax, the weights rounded to bf16
 * (nearest even) before the product with V, output rounded to bf16 (nearest
 * even).  Other SDPA_BF16 head sizes: fp32 arithmetic on the bf16 inputs,
 * output rounded to bf16.  SDPA_F32: fp32 throughout.  Results are
 * deterministic run to run.
 *
 * Supported sizes.  SDPA_BF16: 1 <= d_k, d_v <= 512 (d_k = d_v in {16, 32, 64,
 * 128, 256, 512} runs on the matrix cores: the head sizes of the base and big
 * models, §3.2.2, and of Table 3 row (A) at d_model = 512, down to its last
 * row, h = 1, d_k = d_v = 512; restricted attention at 256 and 512 runs on the
 * fp32 vector units).  SDPA_F32: 1 <= d_k, d_v <= 512.
 * B*H <= 2^31 - 1,
 * Lq, Lk <= 2^31 - 1.  B, H, Lq or Lk equal to 0 is an empty call (SDPA_OK,
 * nothing launched).
 *
 * Ownership and concurrency.  The caller owns every buffer; the library
 * allocates and frees nothing, keeps no per-call state and never synchronises.
 * The call enqueues its kernel on `stream` (a hipStream_t; NULL is the null
 * stream) and returns; the output is valid once that stream reaches the
 * kernel.  `out` must not overlap Q, K, V or key_lengths.
 *
 * Errors.  No exception crosses this interface.  Argument errors are detected
 * on the host before any HIP call and leave `out` untouched.  key_lengths
 * values live on the device and are not checked on the host: the kernel
 * clamps them to [0, Lk].
 */
#ifndef SDPA_H_
#define SDPA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sdpa_status {
    SDPA_OK = 0,
    SDPA_ERR_NULL_POINTER = 1,   /* Q, K, V or out is NULL (with a non-empty shape) */
    SDPA_ERR_BAD_SHAPE = 2,      /* a size is negative, or a product overflows the limits */
    SDPA_ERR_UNSUPPORTED = 3,    /* (dtype, d_k, d_v) combination not built */
    SDPA_ERR_ALIAS = 4,          /* out overlaps Q, K, V or key_lengths */
    SDPA_ERR_HIP = 5,            /* a HIP call failed; see sdpa_last_hip_error() */
    SDPA_ERR_WORKSPACE = 6,      /* sdpa_decode: workspace NULL, too small, or overlapping */
    SDPA_ERR_SCRATCH_LIMIT = 7   /* sdpa_decode_noalloc: needs more than its static scratch */
} sdpa_status;

typedef enum sdpa_dtype {
    SDPA_F32 = 0,
    SDPA_BF16 = 1
} sdpa_dtype;

/*
 * Attention forward (Eq. (1) with the mask above) over B batch entries and H
 * heads.  Arguments:
 *   Q, K, V      device inputs, layouts above;
 *   key_lengths  device int32[B] key lengths, or NULL for "all Lk keys";
 *   causal       0: no causal mask; nonzero: key j illegal for query i if j > i;
 *   out          device output [B,H,Lq,d_v], written completely;
 *   B, H, Lq, Lk, d_k, d_v   sizes;
 *   dtype        element type of Q, K, V and out;
 *   stream       hipStream_t to launch on (NULL = null stream).
 * Returns SDPA_OK after a successful enqueue, or an error code.
 */
sdpa_status sdpa_forward(const void *Q, const void *K, const void *V,
                         const int32_t *key_lengths, int causal, void *out,
                         int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                         int64_t d_k, int64_t d_v, sdpa_dtype dtype, void *stream);

/*
 * Restricted self-attention (page "Attention Is All You Need/paper/es", §4 and
 * Table 1: each output position considers only a neighbourhood of size r of
 * the sequence centred on it; work O(r n d) per layer instead of O(n^2 d)).
 * The neighbourhood is given by its radius: key j is additionally illegal for
 * query i when |i - j| > radius, i.e. r = 2 * radius + 1 positions (fewer at
 * the ends of the sequence).  Positions i and j are compared as in the causal
 * mask (top-left aligned when Lq != Lk).  Every other argument, the layout,
 * the arithmetic, the ownership rules and the errors are those of
 * sdpa_forward; with radius >= max(Lq, Lk) - 1 the result is exactly
 * sdpa_forward's.  Only the key tiles that meet some row's neighbourhood are
 * read.
 *   radius       >= 0 (SDPA_ERR_BAD_SHAPE otherwise, before any HIP call).
 */
sdpa_status sdpa_forward_restricted(const void *Q, const void *K, const void *V,
                                    const int32_t *key_lengths, int causal, int64_t radius,
                                    void *out, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                                    int64_t d_k, int64_t d_v, sdpa_dtype dtype, void *stream);

/*
 * Multi-head attention with its projections (page "Attention Is All You
 * Need/paper/es", §3.2.2):
 *
 *   out = MultiHead(Q, K, V) = Concat(head_1, ..., head_h) W^O,
 *   head_i = Attention(Q W_i^Q, K W_i^K, V W_i^V),
 *
 * Attention being the operation of sdpa_forward (scale 1/sqrt(d_k), the
 * padding mask from key_lengths and, if causal, the causal mask).  Q is the
 * sequence the queries come from, K = V the sequence the keys and values come
 * from: the same buffer for encoder or decoder self-attention (Xkv == Xq and
 * Lk == Lq), the encoder output for encoder-decoder attention (§3.2.3).
 *   Xq        device [B, Lq, d_model];
 *   Xkv       device [B, Lk, d_model] (may equal Xq);
 *   Wq, Wk    device [d_model, h * d_k]: W_i^Q (W_i^K) in R^{d_model x d_k} is
 *             columns i*d_k .. i*d_k + d_k - 1;
 *   Wv        device [d_model, h * d_v], W_i^V likewise;
 *   Wo        device [h * d_v, d_model] = W^O: row i*d_v + t multiplies
 *             component t of head i in the concatenation;
 *   out       device [B, Lq, d_model], written completely;
 *   workspace device scratch of at least sdpa_multihead_workspace_bytes(...)
 *             bytes (the projected heads and the attention output, bf16),
 *             owned by the caller; its contents on entry do not matter.
 * All arrays contiguous row-major, dtype SDPA_BF16 only: bf16 products with
 * fp32 accumulation, the projected heads and the attention output rounded to
 * bf16 (nearest even), the result rounded to bf16.  No bias terms (the pages'
 * projections are matrices).  Supported: d_model % 32 == 0, d_k % 8 == 0,
 * d_v % 32 == 0, d_k, d_v <= 512, every array and each projected tensor below
 * 2 GiB - 1 MiB (SDPA_ERR_UNSUPPORTED / SDPA_ERR_BAD_SHAPE otherwise).
 * Errors as sdpa_forward, plus SDPA_ERR_WORKSPACE (missing, too small, or
 * overlapping another buffer); out must not overlap an input.  Four kernels
 * (three when Xkv == Xq) are enqueued on `stream`; calls that share a
 * workspace must be ordered on one stream.  B == 0 or Lq == 0: SDPA_OK,
 * nothing launched.
 */
sdpa_status sdpa_multihead_forward(const void *Xq, const void *Xkv, const void *Wq,
                                   const void *Wk, const void *Wv, const void *Wo,
                                   const int32_t *key_lengths, int causal, void *out,
                                   int64_t B, int64_t Lq, int64_t Lk, int64_t d_model,
                                   int64_t h, int64_t d_k, int64_t d_v, sdpa_dtype dtype,
                                   void *workspace, int64_t workspace_bytes, void *stream);

/* Workspace bytes sdpa_multihead_forward needs for these sizes, or -1 when it
 * would reject them (no pointers are involved). */
int64_t sdpa_multihead_workspace_bytes(int64_t B, int64_t Lq, int64_t Lk, int64_t d_model,
                                       int64_t h, int64_t d_k, int64_t d_v, sdpa_dtype dtype);

/*
 * Decode-step attention: the same result as sdpa_forward with causal = 0, for
 * the case of a few query rows per head against a long key/value cache (the
 * new positions of an autoregressive decoder, page "Attention Is All You
 * Need/paper/es" §3.1 and §3.2.3: each output position attends to all the
 * positions generated so far, given by key_lengths[b], the cache length
 * including the new positions).
 *
 * For bf16 with d_k = d_v in {64, 128} and 1 <= Lq <= 32 the keys of every
 * (b, h) are split into chunks that run in parallel (one query row: dot
 * products on the vector units; 2 to 32 rows: the matrix cores).  When a
 * head's keys span several chunks, each chunk writes its partial result (per
 * query row: reference maximum m, weight sum l and the unnormalised weighted
 * sum of V) to `workspace`, and a second kernel merges the chunks:
 * O = sum_c e^(m_c - M) acc_c / sum_c e^(m_c - M) l_c with M = max_c m_c
 * (base 2 in the kernel; a chunk without legal keys contributes nothing; no
 * legal key at all gives 0); with one chunk per head (many heads or a short
 * cache) one kernel writes O and no workspace is used.  Any other (dtype, d_k,
 * d_v, Lq) runs the sdpa_forward kernels and needs no workspace.
 *
 * Arguments as for sdpa_forward (no causal flag), plus
 *   workspace        device scratch of at least sdpa_decode_workspace_bytes()
 *                    bytes (may be NULL when that is 0); owned by the caller,
 *                    contents on entry irrelevant, overwritten; must not
 *                    overlap Q, K, V, key_lengths or out;
 *   workspace_bytes  its size.
 * Two calls may share a workspace only if they run in stream order.
 * Returns SDPA_OK after the enqueue (one or two kernels on `stream`), or an error code;
 * SDPA_ERR_WORKSPACE if the workspace is needed and is NULL, too small or
 * overlapping.  Arithmetic and rounding as for sdpa_forward (the merge is fp32);
 * results are deterministic run to run.
 */
sdpa_status sdpa_decode(const void *Q, const void *K, const void *V,
                        const int32_t *key_lengths, void *out,
                        int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                        int64_t d_k, int64_t d_v, sdpa_dtype dtype,
                        void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Bytes of workspace sdpa_decode needs for these sizes: 0 when it runs the
 * sdpa_forward kernels or one chunk covers each head, otherwise
 * 4 * (d_v + 2) * B * H * Lq * n_chunks, where n_chunks depends on B * H, Lk,
 * d_k and whether Lq is 1.  Returns -1 for sizes sdpa_decode would reject with
 * SDPA_ERR_BAD_SHAPE or SDPA_ERR_UNSUPPORTED.
 */
int64_t sdpa_decode_workspace_bytes(int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                                    int64_t d_k, int64_t d_v, sdpa_dtype dtype);

/*
 * sdpa_decode without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same result as
 * sdpa_decode (same kernels, same chunking); the key-split partial results go
 * to a static device array of the library (SDPA_DECODE_NOALLOC_SCRATCH_BYTES
 * bytes, one copy per device, held until the process ends), whose device
 * address is looked up on the first call on each device (the device of
 * `stream`, or the current device for the null stream).  The call makes no
 * hipMalloc, hipFree or other allocating call.
 *
 * Arguments, layouts, arithmetic and errors as for sdpa_decode, plus
 * SDPA_ERR_SCRATCH_LIMIT (checked on the host before any HIP call) when the
 * split path would need more than SDPA_DECODE_NOALLOC_SCRATCH_BYTES of partial
 * results (4 * (d_v + 2) * B * H * Lq * n_chunks bytes, as
 * sdpa_decode_workspace_bytes reports); shapes outside the split path need no
 * scratch.  Every call on one device shares that device's array: calls that
 * may overlap in time on one device (two streams, two host threads without
 * stream order) race and give undefined results.  Nothing in the array needs
 * to start at zero (each call writes every partial result it reads).
 */
#define SDPA_DECODE_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)

sdpa_status sdpa_decode_noalloc(const void *Q, const void *K, const void *V,
                                const int32_t *key_lengths, void *out,
                                int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                                int64_t d_k, int64_t d_v, sdpa_dtype dtype, void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *sdpa_status_str(sdpa_status status);

/* The hipError_t value behind the calling thread's last SDPA_ERR_HIP (0 if none). */
int sdpa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_H_ */

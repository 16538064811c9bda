// Scaled dot-product attention forward on the gfx950 matrix cores for wide
// heads: bf16 inputs, d_k = d_v = D with D in {256, 512}, fp32 accumulation
// (v_mfma_f32_16x16x32_bf16).
//
// What it computes: Eq. (1) of page "Attention Is All You Need/paper/es"
// (§3.2.1), softmax(Q K^T / sqrt(d_k)) V per head, with -inf for illegal
// connections before the softmax (§3.2.3): keys j >= len_b (padding) and, when
// causal, keys j > i.  Table 3 row (A) of the same page ends at h = 1 with
// d_k = d_v = 512; both products stay dense contractions at that width, so
// they run on the matrix cores like the narrower heads.
//
// Design (one workgroup = 4 waves = 64 query rows of one (b, h), 16 rows per
// wave; keys in tiles of 32, two 16-key blocks each):
//
//  * At D = 512 a wave of 32 query rows would need 256 accumulator registers
//    per lane for O alone, so a wave takes 16 rows and the 16x16x32 MFMA: O^T
//    then needs D/4 registers per lane and the wave's Q, held in registers as
//    the B operand of the score product for the whole launch, another D/4
//    (256 at D = 512: one wave per SIMD).
//  * Scores are formed transposed, S^T = K Q^T, per 16-key block: A = 16 keys
//    x 32 dims (from LDS), B = 32 dims x 16 queries.  In the accumulator lane l
//    holds query l % 16 and keys 4(l/16) .. 4(l/16)+3 of the block.
//  * Both operands of one MFMA list the 32 contraction indices in the same
//    (lane group, element) order, so any fixed assignment of indices to those
//    slots gives the same sum.  Element e of lane group g is taken as index
//    4g + e (e < 4) and 16 + 4g + (e - 4) (e >= 4): the scores of a tile's two
//    16-key blocks that a lane holds are then, rounded to bf16, exactly its B
//    operand of O^T += V^T P^T over the tile's 32 keys, and P never leaves
//    registers.  In the score product the slots of lane group g are the 8
//    consecutive dims 8g .. 8g+7 of each 32-dim step (one 16-byte read).
//  * V^T (A operand, 16 dims x 32 keys) is read from row-major V in LDS with
//    ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
//    i % 4 of the 4-element rows addressed by lanes 4e + i / 4 (e = 0..3), so
//    lanes 4e + j addressing dims 4j .. 4j+3 of key row k0 + e hand lane i the
//    4 keys k0 .. k0+3 of dim i.
//  * K and V rows sit in LDS as in HBM with their 16-byte chunk indices
//    XORed by the row: K rows by r mod 16 (the 16 K rows that 16 lanes read
//    at one chunk, and any 8 consecutive of them, land on distinct positions),
//    V rows by f(r) = 2 (r mod 8) + (r / 8 mod 2), which keeps bit 0 of the
//    chunk index apart from its higher bits (the 4 V rows x 2 adjacent chunks
//    that 16 lanes read in a transposing read land on 8 distinct positions
//    modulo 128 bytes).  The counters show no LDS bank conflicts.  Two buffers: the copy of tile t+1 (HBM
//    straight into LDS, buffer_load ... lds) runs while tile t is multiplied;
//    one barrier per tile.  The copy's buffer descriptor ends at the key
//    length, so rows past it read as 0.
//  * The LDS operand reads of both products run kPF MFMA steps ahead of their
//    use, with scheduling fences between steps so that the compiler does not
//    hoist more of them (at D = 512 the registers are already full).  Each
//    K or V byte read from LDS feeds 16 multiply-adds (one per query row of
//    the wave), so the products are bound by LDS bandwidth at about half the
//    matrix-core rate.
//  * The row maximum over a row's four lane groups uses v_permlane16_swap and
//    v_permlane32_swap (no LDS traffic).
//  * Output through LDS: after the last tile each wave writes its 16 x D tile
//    into a freed tile buffer in the accumulator layout and reads it back row
//    by row, so every store writes whole rows (1 KiB contiguous).  Storing the
//    accumulator layout directly put 32 bytes of 16 rows in each instruction;
//    the staged form took the d = 512, h = 1 encoder launch from 28.2 to
//    25.1 us.
//  * Softmax online in base 2: p = exp2(s log2(e)/sqrt(d_k) - m), with m a
//    reference maximum of the row in the same units, moved to the row's
//    current maximum only when that exceeds m by more than kTau (so p stays
//    below 2^kTau, harmless in fp32 and bf16); the common shift cancels in the
//    final division by the row sum.  After the first tile the rescale of the
//    accumulator (a wave-uniform branch) is rarely taken.  The row
//    sum adds the bf16-rounded weights, i.e. the weights used in P V.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sdpa_kernels.h"
#include "sdpa_timeline.h"

namespace sdpa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kBM = 16 * kWaves;        // query rows per workgroup
constexpr int kBN = 32;                 // keys per tile
constexpr int kRsrcWord3 = 0x00020000;  // raw (stride 0) dword buffer access
// Output stores non-temporal (nt; the builtin's slc position on gfx950): O is
// written once and not read by the launch (Table 3 row (A) encoder, d = 512:
// -3.7 % on cold inputs).
constexpr int kStoreStreaming = 2;
// K/V copies non-temporal when a head has at most this many query tiles (each
// K/V row copied into LDS by at most four workgroups at nearly the same time):
// the d = 512 encoder -4.6 %.
constexpr int kStreamQueryTiles = 4;
constexpr int kPF = 2;                  // LDS operand reads issued this many MFMA steps ahead
constexpr float kTau = 8.0f;            // lazy-rescale threshold, log2 units

// Chunk swizzle of V row r (see the header comment).
__device__ inline int chunk_xor(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

__device__ inline uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32, nearest even
    return __builtin_bit_cast(uint32_t, v);
}

__device__ inline u32x2_t lds_read_tr(const uint16_t *p)
{
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)p));
}

__device__ inline u32x4_t lds_read_b128(const char *p)
{
    return *(const __attribute__((address_space(3))) u32x4_t *)(
        (__attribute__((address_space(3))) const void *)p);
}

__device__ inline f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// One wave-wide HBM -> LDS copy: lane L's 16 bytes at byte offset voff of the
// buffer land at LDS address dst + 16 L (LDS base in M0).  Inline assembly, so
// that the compiler neither tracks it (it would wait for every copy in flight
// before each LDS read) nor reorders LDS accesses across it; the kernel waits
// for its copies itself (vmcnt(0) before each barrier).  Nothing else in this
// kernel uses M0 on gfx950.
// STREAM: the non-temporal cache policy (nt).
template <bool STREAM = false>
__device__ inline void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc, const uint16_t *dst, uint32_t voff)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)dst);
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                     :: "s"(m0), "v"(voff), "s"(rsrc) : "memory");
    else
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(m0), "v"(voff), "s"(rsrc) : "memory");
}

// Maximum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups holding one
// query row): v_permlane16_swap then v_permlane32_swap, no LDS traffic.
__device__ inline float max_across_groups(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    x = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}

// s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);

// Waves per SIMD: D = 512 takes all 256 VGPRs and 128 KiB of LDS (one
// workgroup per CU); D = 256 fits two workgroups per CU (64 KiB of LDS each).
// OUT_NT: output stores non-temporal (not when the caller reads the output right
// away); copies_nt: K/V copies non-temporal (few query tiles per head, and not
// when the caller has just written the inputs).
template <int D, bool OUT_NT = true>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(512 / D, 512 / D)))
void sdpa_fwd_mfma_wide_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
                               const uint16_t *__restrict__ V, const int32_t *__restrict__ key_lengths,
                               int causal, uint16_t *__restrict__ O, int H, int64_t Lq, int64_t Lk,
                               float scale_log2, uint32_t n_qtiles, uint32_t n_bh, int copies_nt)
{
    static_assert(D == 256 || D == 512, "wide heads only");
    constexpr int kRowBytes = 2 * D;
    constexpr int kChunks = D / 8;                      // 16-byte chunks per row
    constexpr int kTileElems = kBN * D;
    constexpr int kSteps = D / 32;                      // 32-dim steps of the score product
    constexpr int kDB = D / 16;                         // 16-dim blocks of the output
    constexpr int kRowsPerSlice = 512 / D;              // rows per 1 KiB copy
    constexpr int kSlicesPerWave = kTileElems / 512 / kWaves;
    __shared__ __attribute__((aligned(16))) uint16_t lds[4 * kTileElems];   // K0 V0 K1 V1

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;      // query of the wave (accumulator column)
    const int grp = lane >> 4;      // lane group
    SDPA_STAMP(0);

    // Work order: causal grids take the longest query tiles first; otherwise
    // each XCD (blockIdx % 8) takes a run of consecutive items, so the query
    // tiles of one head share an L2.
    const uint32_t w = blockIdx.x;
    uint32_t bh, qt;
    if (causal) {
        bh = w % n_bh;
        qt = n_qtiles - 1 - w / n_bh;
    } else {
        const uint32_t n_items = n_qtiles * n_bh;
        const uint32_t item = (n_items & 7) == 0 ? (w & 7) * (n_items >> 3) + (w >> 3) : w;
        bh = item / n_qtiles;
        qt = item % n_qtiles;
    }
    const int64_t b = bh / H;
    const int64_t q0 = (int64_t)qt * kBM;
    const int64_t q0w = q0 + 16 * wave;     // first row of this wave
    const int64_t qrow = q0w + col;         // this lane's query row

    int64_t len = Lk;
    if (key_lengths) {
        const int64_t l = key_lengths[b];
        len = l < 0 ? 0 : (l > Lk ? Lk : l);
    }
    int64_t kv_end = len;
    if (causal && q0 + kBM < kv_end) kv_end = q0 + kBM;
    const int n_tiles = (int)((kv_end + kBN - 1) / kBN);

    // Q operand: the lane's query row, dims 32s + 8 grp .. +7 of every step s;
    // rows past Lq read 0.
    u32x4_t qf[kSteps];
    {
        int64_t rows = Lq - q0w;
        rows = rows < 0 ? 0 : (rows > 16 ? 16 : rows);
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(Q + ((int64_t)bh * Lq + q0w) * D), (short)0, (int)rows * kRowBytes, kRsrcWord3);
        const uint32_t qoff = (uint32_t)(col * kRowBytes + 16 * grp);
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
            qf[s] = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + 64 * s, 0, 0);
    }

    const uint16_t *Kh = K + (int64_t)bh * Lk * D;
    const uint16_t *Vh = V + (int64_t)bh * Lk * D;
    // Copy offsets: lane L of slice j fills LDS row pos, physical chunk pc,
    // which holds the row's chunk pc ^ chunk_xor(pos).
    uint32_t coff[kSlicesPerWave];
    int cpos[kSlicesPerWave];
#pragma unroll
    for (int j = 0; j < kSlicesPerWave; ++j) {
        const int pos = kRowsPerSlice * (wave * kSlicesPerWave + j) + lane / kChunks;
        const int pc = lane % kChunks;
        cpos[j] = pos;
        coff[j] = (uint32_t)(pos * kRowBytes + ((pc ^ (pos & 15)) << 4));   // K: XOR with r mod 16
    }
    auto issue = [&](int t) {
        const int64_t kv0 = (int64_t)t * kBN;
        int64_t rows = len - kv0;
        rows = rows < 0 ? 0 : (rows > kBN ? kBN : rows);
        const int nbytes = (int)rows * kRowBytes;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void *)(Kh + kv0 * D), (short)0, nbytes, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void *)(Vh + kv0 * D), (short)0, nbytes, kRsrcWord3);
        uint16_t *kb = lds + (t & 1) * 2 * kTileElems;
        if (copies_nt) {
#pragma unroll
            for (int j = 0; j < kSlicesPerWave; ++j) {
                copy_to_lds<true>(rk, kb + (wave * kSlicesPerWave + j) * 512, coff[j]);
                // V: XOR with chunk_xor(r) instead of r mod 16
                const uint32_t vo = coff[j] ^ (uint32_t)(((cpos[j] & 15) ^ chunk_xor(cpos[j])) << 4);
                copy_to_lds<true>(rv, kb + kTileElems + (wave * kSlicesPerWave + j) * 512, vo);
            }
        } else {
#pragma unroll
            for (int j = 0; j < kSlicesPerWave; ++j) {
                copy_to_lds(rk, kb + (wave * kSlicesPerWave + j) * 512, coff[j]);
                const uint32_t vo = coff[j] ^ (uint32_t)(((cpos[j] & 15) ^ chunk_xor(cpos[j])) << 4);
                copy_to_lds(rv, kb + kTileElems + (wave * kSlicesPerWave + j) * 512, vo);
            }
        }
    };

    // LDS operand offsets (bytes).  K, step s (dims 32s .. 32s+31): lane
    // 16 grp + col reads 16 bytes, chunk 4s + grp of row col (and col + 16 for
    // the second block).  The row's XOR splits into bits 0..1 (a per-lane
    // constant) and bits 2..3, which permute the four steps s = 4i .. 4i+3:
    // kofs[s % 4] + 256 (s / 4) is the address.
    const int kx = col;                                                // rows col and col + 16
    uint32_t kofs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        kofs[j] = (uint32_t)(col * kRowBytes + 16 * (grp ^ (kx & 3)) + 64 * (j ^ (kx >> 2)));
    // V, block db (dims 16 db .. 16 db + 15): lane 16 grp + 4e + j addresses
    // key row 4 grp + e (+16 for keys 16 .. 31), dims 16 db + 4j, i.e. chunk
    // 2 db + j/2, half j % 2; the XOR's bit 0 is a per-lane constant, its bits
    // 1..3 permute the eight blocks db = 8i .. 8i+7: vofs[db % 8] + 256 (db / 8).
    const int vrow = 4 * grp + ((lane >> 2) & 3);
    const int vj = lane & 3;
    const int vx = chunk_xor(vrow);                                    // rows vrow and vrow + 16
    const uint32_t vbase = (uint32_t)(vrow * kRowBytes + 8 * (vj & 1) + ((((vj >> 1) ^ (vx & 1))) << 4));
    uint32_t vofs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) vofs[j] = vbase + (uint32_t)(32 * (j ^ ((vx >> 1) & 7)));

    f32x4_t o[kDB];
#pragma unroll
    for (int i = 0; i < kDB; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // reference maximum (scaled, base 2), same in the 4 lane groups
    float l_run = 0.f;         // this lane's share of the row sum

    if (n_tiles > 0) issue(0);
    for (int t = 0; t < n_tiles; ++t) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
        if (t == 0) SDPA_STAMP(1);
        if (t + 1 < n_tiles) issue(t + 1);
        const char *kb = (const char *)(lds + (t & 1) * 2 * kTileElems);
        const char *vb = kb + 2 * kTileElems;

        // S^T of the two 16-key blocks; K operands read kPF steps ahead
        auto kread = [&](int s, u32x4_t &ra, u32x4_t &rb) {
            const char *p = kb + kofs[s & 3] + 256 * (s >> 2);
            ra = lds_read_b128(p);
            rb = lds_read_b128(p + 16 * kRowBytes);
        };
        f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;
        u32x4_t ka[kPF + 1], kc[kPF + 1];
#pragma unroll
        for (int s = 0; s < kPF; ++s) kread(s, ka[s], kc[s]);
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            if (s + kPF < kSteps) kread(s + kPF, ka[(s + kPF) % (kPF + 1)], kc[(s + kPF) % (kPF + 1)]);
            s0 = mfma16(ka[s % (kPF + 1)], qf[s], s0);
            s1 = mfma16(kc[s % (kPF + 1)], qf[s], s1);
            __builtin_amdgcn_sched_barrier(0);
        }

        // masks, row maximum, weights
        const int64_t kv0 = (int64_t)t * kBN;
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t k0 = kv0 + 4 * grp + j, k1 = k0 + 16;
            const bool ok0 = k0 < len && (!causal || k0 <= qrow);
            const bool ok1 = k1 < len && (!causal || k1 <= qrow);
            x[j] = ok0 ? s0[j] * scale_log2 : -INFINITY;
            x[4 + j] = ok1 ? s1[j] * scale_log2 : -INFINITY;
        }
        float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        mx = max_across_groups(mx);
        const bool grow = mx > m_run + kTau;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            // a row's first legal key has m_run = -inf: alpha = 0 (nothing to keep)
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;
            m_run = grow ? mx : m_run;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < kDB; ++i) o[i] *= alpha;
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;   // no legal key yet: all weights 0
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pk[i] = pack_bf16x2(__builtin_amdgcn_exp2f(x[2 * i] - m_use),
                                __builtin_amdgcn_exp2f(x[2 * i + 1] - m_use));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            l_run += __builtin_bit_cast(float, pk[i] << 16) + __builtin_bit_cast(float, pk[i] & 0xffff0000u);
        const u32x4_t pb = u32x4_t{pk[0], pk[1], pk[2], pk[3]};

        // O^T += V^T P^T; V operands read kPF blocks ahead
        auto vread = [&](int db) {
            const char *p = vb + vofs[db & 7] + 256 * (db >> 3);
            const u32x2_t a0 = lds_read_tr((const uint16_t *)p);
            const u32x2_t a1 = lds_read_tr((const uint16_t *)(p + 16 * kRowBytes));
            return u32x4_t{a0.x, a0.y, a1.x, a1.y};
        };
        u32x4_t va[kPF + 1];
#pragma unroll
        for (int i = 0; i < kPF; ++i) va[i] = vread(i);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
            if (db + kPF < kDB) va[(db + kPF) % (kPF + 1)] = vread(db + kPF);
            o[db] = mfma16(va[db % (kPF + 1)], pb, o[db]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    SDPA_STAMP(2);
    // Row sum over the 4 lane groups; a row with no legal key gets 0.
    float l = l_run + __shfl_xor(l_run, 16);
    l += __shfl_xor(l, 32);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    int64_t rows = Lq - q0w;
    rows = rows < 0 ? 0 : (rows > 16 ? 16 : rows);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(O + ((int64_t)bh * Lq + q0w) * D), (short)0, (int)rows * kRowBytes, kRsrcWord3);
    // The wave's 16 x D output tile goes through LDS so that every store
    // writes whole rows (1 KiB contiguous per instruction): written in the
    // accumulator layout (lane: row col, 8-byte piece grp % 2 of 16-byte chunk
    // 2 db + grp / 2), read back row by row; chunks XORed by the row mod 16.
    // The barrier makes sure every wave is done with the last tile's buffers.
    constexpr int kC = D / 8, kRps = 512 / D;
    __syncthreads();
    char *stage = (char *)(lds + wave * 16 * D);
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
        const u32x2_t v = u32x2_t{pack_bf16x2(o[db][0] * inv, o[db][1] * inv),
                                  pack_bf16x2(o[db][2] * inv, o[db][3] * inv)};
        const int c = 2 * db + (grp >> 1);
        *(u32x2_t *)(stage + col * kRowBytes + ((c ^ col) << 4) + 8 * (grp & 1)) = v;
    }
#pragma unroll
    for (int i = 0; i < 16 / kRps; ++i) {
        const int r = kRps * i + lane / kC, c = lane % kC;
        const u32x4_t v = *(const u32x4_t *)(stage + r * kRowBytes + ((c ^ (r & 15)) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, (uint32_t)(r * kRowBytes + c * 16), 0,
                                               OUT_NT ? kStoreStreaming : 0);
    }
    SDPA_STAMP(3);
}

template <int D>
hipError_t launch_wide_d(const void *Q, const void *K, const void *V, const int32_t *key_lengths,
                         int causal, void *out, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                         bool streaming, hipStream_t stream)
{
    const uint32_t n_qtiles = (uint32_t)((Lq + kBM - 1) / kBM);
    const uint32_t n_bh = (uint32_t)(B * H);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const int copies_nt = streaming && n_qtiles <= kStreamQueryTiles;
    if (streaming)
        hipLaunchKernelGGL((sdpa_fwd_mfma_wide_kernel<D, true>), dim3(n_qtiles * n_bh), dim3(kWaves * 64), 0,
                           stream, (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V,
                           key_lengths, causal, (uint16_t *)out, (int)H, Lq, Lk, scale_log2, n_qtiles, n_bh,
                           copies_nt);
    else
        hipLaunchKernelGGL((sdpa_fwd_mfma_wide_kernel<D, false>), dim3(n_qtiles * n_bh), dim3(kWaves * 64), 0,
                           stream, (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V,
                           key_lengths, causal, (uint16_t *)out, (int)H, Lq, Lk, scale_log2, n_qtiles, n_bh,
                           copies_nt);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_wide(const void *Q, const void *K, const void *V, const int32_t *key_lengths,
                            int causal, void *out, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int d,
                            bool streaming, hipStream_t stream)
{
    if (d == 256) return launch_wide_d<256>(Q, K, V, key_lengths, causal, out, B, H, Lq, Lk, streaming, stream);
    if (d == 512) return launch_wide_d<512>(Q, K, V, key_lengths, causal, out, B, H, Lq, Lk, streaming, stream);
    return hipErrorInvalidValue;
}

}  // namespace sdpa

#ifdef SDPA_TIMELINE
// Timeline build only: the records of this file's kernel (sdpa_timeline.h).
extern "C" int sdpa_timeline_wide(void *host, int64_t bytes, int clear)
{
    return sdpa::timeline_io(host, bytes, clear);
}
#endif

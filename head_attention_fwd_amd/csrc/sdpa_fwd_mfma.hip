// Scaled dot-product attention forward for bf16 inputs with d_k = d_v = D,
// D in {16, 32, 64, 128}, on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation).
//
// What it computes: Eq. (1) of page "Attention Is All You Need/paper/es"
// (§3.2.1), softmax(Q K^T / sqrt(d_k)) V per head (§3.2.2: d_k = d_v = 64 in
// the base and big models; Table 3 row (A) varies the head count at fixed
// d_model = 512, i.e. d_k = 128, 32 and 16), with -inf for illegal connections before the
// softmax (§3.2.3): keys j >= len_b (padding) and, when causal, keys j > i.
// Both products are dense contractions ("highly optimised matrix multiplication
// code", §3.2.1), so they run on the matrix cores; the Lq x Lk score matrix
// never leaves registers.
//
// Design (one workgroup = NW waves = 32*NW query rows of one (b, h); keys in
// tiles of 32*NB, processed as NB blocks of 32):
//
//  * Scores are formed transposed, S^T = K Q^T, one 32x32 block per MFMA
//    chain: A = 32 keys x 16 dims (from LDS), B = 16 dims x 32 queries (the
//    wave's Q rows, loaded once into registers).  In the accumulator layout a
//    lane then holds 16 scores of ONE query (lane % 32), and the other half of
//    the wave holds the other 16 keys of the same query.  The row maximum is an
//    in-lane reduction plus one exchange with lane ^ 32; the row sum needs no
//    exchange until the epilogue.
//  * The weights P^T (bf16) are exactly the B operand of the second product,
//    O^T += V^T P^T (A = 32 dims x 16 keys from LDS): no LDS round trip for P.
//    For that the 32 key rows of a score block are fed to the first MFMA in
//    the order pi(m) = m with bits 2 and 3 swapped; then lane half g of the
//    accumulator holds, in registers r = 8h..8h+7, the 8 consecutive keys
//    16h + 8g + (r % 8), which is what the second MFMA expects of its B operand.
//  * The output accumulator O^T also holds one query per lane, so the online
//    rescaling factor exp(m_old - m_new) is a per-lane scalar.
//  * K and V are staged in LDS row-major, exactly as they sit in HBM (K rows
//    stored in pi order), with 16-byte chunks XOR-swizzled by the row so that
//    the operand reads of a wave are free of bank conflicts.  The V^T operand
//    is read with ds_read_b64_tr_b16, which transposes 16-bit elements across
//    each group of 16 lanes: lane i receives element i % 4 of the 4-element
//    rows addressed by lanes 4e + i / 4 (e = 0..3), so two such reads give a
//    lane 8 consecutive keys of one dim.  A ring of three LDS buffers: tiles
//    t+1 and t+2 are being copied from HBM into LDS (asynchronously, without
//    registers) while tile t is multiplied, one barrier per tile.
//  * Softmax in base 2: p = exp2(s * log2(e)/sqrt(d_k) - m), with m tracked in
//    the same scaled units; exp2 is v_exp_f32.  A row's reference maximum m
//    is moved (to the row's current maximum) only when that maximum exceeds m
//    by more than kTau; otherwise p stays below 2^kTau, harmless in fp32 and
//    bf16.  The result is the same softmax, and after the first tiles the
//    rescale of the accumulator is almost never taken.  The row sum adds the bf16-rounded weights
//    (v_dot2c_f32_bf16 against 1), i.e. exactly the weights used in P.V.
//  * Software pipeline inside a tile: while a wave evaluates the softmax of
//    block b on the VALU, the matrix core works on S of block b+1 and on P.V
//    of block b-1 (the MFMA and VALU instructions share one issue port, so the
//    wave needs independent matrix work in its instruction stream to keep both
//    units busy).  P.V of block b-1 is issued before block b's rescale check,
//    so a rare move of the reference maximum only rescales the accumulator.
//  * Tiles after the first compute no row maximum: a row's weights are taken
//    against its reference maximum, and only when they sum past 2^20 (rare)
//    does the row recompute them against the block maximum.  Only the first
//    tile computes block maxima (restricted attention: every tile outside
//    the fully legal middle range); tiles crossing the causal diagonal or the
//    padding end apply masks.  Tiles entirely beyond the key length are never
//    loaded.
//  * Work order: one query tile per workgroup, each XCD on its own run of
//    heads so the workgroups streaming one head's K/V share an L2; causal
//    grids dispatch the longest query tiles first (greedy longest-first over
//    the workgroup slots, which the hardware dispatcher fills in order), a
//    few heads at a time per XCD.  Launches with per-entry key lengths whose
//    workgroups are all resident at once instead deal their query tiles to
//    the XCDs and CUs balanced over the entries' key lengths (balanced_item).
//  * Cache policy: output stores non-temporal (O is not read again by the
//    launch); on heads with few query tiles the Q/K/V copies too.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sdpa_kernels.h"
#include "sdpa_timeline.h"

namespace sdpa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kTau = 8.0f;          // lazy-rescale threshold, log2 units

// Shape of the kernels (each value measured on MI355X against its neighbours).
constexpr int kWaves = 4;              // waves per workgroup (32 query rows each); d = 16: 2
constexpr int kKeyBlocks = 2;          // 32-key blocks per LDS tile at d = 32 (d = 64, 128: 1)
constexpr int kSplitKeyBlocks = 1;     // 32-key blocks per LDS tile of the key-split kernel
constexpr int kCausalHeadGroup = 4;    // causal order: heads per group on an XCD
constexpr int kStreamQueryTiles = 4;   // K/V copies non-temporal up to this many query tiles per head
constexpr int kBalancedMaxTiles = 32;  // balanced order up to this many key tiles per entry
constexpr int kCUs = 256;              // compute units of an MI355X (8 XCDs of 32)
// Run-time flags of the forward kernel, set by the launcher.
constexpr int kFlagCopiesNt = 1;       // Q/K/V copies non-temporal
constexpr int kFlagBalanced = 2;       // work order balanced over the entries' key lengths
constexpr int kWavesPerSimd128 = 2;    // register budget of the forward kernel at d = 128 ...
constexpr int kWavesPerSimd128Long = 3;   // ... and of its form for long key ranges
constexpr int kLongKeys128 = 1024;     // d = 128 launches with more keys take the long form
constexpr int kBandKeyBlocks64 = 1;    // restricted attention, d = 64: 32-key tiles (finer band edges)
// Waves per SIMD the register budget is set for, by head size: D = 128 needs
// 64 accumulator and 32 Q-operand registers (2 waves; 3 for long key ranges,
// 168 VGPRs), D = 32 and D = 16 fit 4; D = 64 with 32-key tiles (one score
// block in flight) fits 4 as well.
template <int D, int NB = 2, bool BAND = false>
struct Occupancy {
    static constexpr int kWaves = D >= 128 ? (BAND ? 2 : kWavesPerSimd128) : (D >= 64 ? (NB == 1 ? 4 : 3) : 4);
};

// 16-byte chunk swizzles of a row of D bf16 values (D/8 chunks), XORed into
// the chunk index.  The LDS serves 64 banks of 4 bytes per cycle: 16 lanes of
// a 16-byte read, 32 lanes of an 8-byte one.  K (and Q) rows: the 16 rows that
// the 16 lanes of one cycle read get distinct bank ranges.  D = 128: rows of
// 256 bytes all start at bank 0, so 16 rows need 16 distinct chunk positions
// (row mod 16).  D = 64: two rows per 256 bytes; injective on any 8
// consecutive rows and on the 8 even or 8 odd rows of any 16 consecutive rows.
// D = 32, four rows per 256 bytes: rows r and r + 4 differ.  D = 16, eight rows
// per 256 bytes: rows r and r + 8 differ.
template <int D>
__device__ inline int swz(int row)
{
    // D = 16: rows of 32 bytes (two chunks); rows r and r + 8 swap chunks
    return D >= 128 ? row & 15 : (D >= 64 ? (row ^ (row >> 3)) & 7 : (D >= 32 ? (row >> 2) & 3 : (row >> 3) & 1));
}

// V rows: the 4 rows that one 16-lane group of ds_read_b64_tr_b16 touches (32
// bytes, two chunks, of each) get disjoint bank ranges, and so do the two
// groups of one cycle.  D = 128: each row's 64-byte quarter q moves to quarter
// q ^ (row mod 4), so 4 rows x 64 bytes cover all 64 banks.  D = 64: chunk
// pairs XOR (row mod 4) * 2 (two rows per 256 bytes).  D = 32: the two 16-dim
// halves of a row stay apart.
template <int D>
__device__ inline int swz_v(int row)
{
    return D >= 128 ? (row & 3) << 2 : (D >= 64 ? (row & 3) << 1 : (D >= 32 ? (row & 1) << 1 : 0));
}

// Key row order fed to the score MFMA: swap bits 2 and 3 (an involution).
__device__ inline int pi32(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

__device__ inline uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32, nearest even
    return __builtin_bit_cast(uint32_t, v);
}

__device__ inline bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ inline u32x4_t as_u32x4(bf16x8_t v) { return __builtin_bit_cast(u32x4_t, v); }

// Transposing LDS read (see the header comment for the lane mapping).
__device__ inline u32x2_t ds_read_tr16_b64(const uint16_t *p)
{
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)p));
}

// max / sum over the two lanes l and l ^ 32 (v_permlane32_swap, no LDS traffic)
__device__ inline float max_across_halves(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ inline float sum_across_halves(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ inline f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Wait states between the last MFMA writing the accumulator and a read of it
// inside inline assembly, which the compiler's hazard tracking does not see
// through (more than the 32x32 XDL write -> VALU read requirement).
__device__ inline void acc_read_fence() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory"); }

// Buffer resource word 3 for raw (unswizzled, stride 0) dword access on CDNA.
constexpr int kBufferRsrcWord3 = 0x00020000;
// Cache policy of the output stores: non-temporal (the nt bit, the builtin's
// slc position on gfx950).  O is written once and not read again by the launch,
// so its lines are streamed out instead of being kept in the L2 and the
// Infinity Cache beside the K/V rows that other workgroups still read.
// Measured on cold-input launches: base encoder -7 to -10 %, big cross 0 to
// -6 %, the long causal launch within +-0.5 %.
constexpr int kStoreStreaming = 2;

// One wave-wide HBM -> LDS copy: lane L's 16 bytes at byte offset voff of the
// buffer land at LDS address dst + 16*L (buffer_load_dwordx4 ... lds, LDS base
// in M0).  Issued as inline assembly so that the compiler does not track it:
// its conservative tracking of such copies made it wait for every copy in
// flight before any LDS read, which would serialize the prefetch.  The kernel
// therefore orders these copies itself (wait_vmem_keep before each barrier).
// M0 is written here and nowhere else in this kernel (nothing else in it uses
// M0 on gfx950), so it is not declared clobbered (it is a reserved register).
// STREAM: the non-temporal cache policy (nt), for rows that few workgroups read.
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

// K/V tile loads go straight from HBM into LDS (buffer_load_dwordx4 ... lds): no
// staging registers, no LDS store instructions.  One such instruction moves
// 64 lanes x 16 B = 1 KiB = 512/D rows of a tile into LDS at consecutive
// addresses (lane L -> byte 16*L of the slice), so the LDS layout is chosen by
// which global 16-byte chunk each lane fetches: with C = D/8 chunks per row,
// lane L fills LDS row (512/D)*slice + L/C, physical chunk L % C.  The buffer
// descriptor of each tile starts at the tile's first row and covers only the
// rows below the key length; the hardware returns 0 for reads past that bound,
// which zero-fills padded rows.
template <int NW, int BN, int D>
struct TileLoader {
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kChunks = D / 8;                   // 16-byte chunks per row
    static constexpr int kRowsPerSlice = 512 / D;           // rows per 1 KiB copy
    static constexpr int kSlices = BN * D / 512;            // 1 KiB slices per K (or V) tile
    static constexpr int kPerWave = kSlices / NW;
    static_assert(kSlices % NW == 0, "every wave issues the same number of copies");
    static constexpr int kLoadsPerTile = 2 * kPerWave;      // per wave: K and V slices
    uint32_t koff[kPerWave], voff[kPerWave];               // byte offsets within the tile
    int slice0;

    __device__ inline void init(int wave, int lane)
    {
        slice0 = wave * kPerWave;
#pragma unroll
        for (int j = 0; j < kPerWave; ++j) {
            const int pos = kRowsPerSlice * (slice0 + j) + lane / kChunks;   // LDS row filled by this lane
            const int pc = lane % kChunks;                    // physical chunk
            const int kr = (pos & ~31) | pi32(pos & 31);      // K row stored at LDS row pos
            koff[j] = (uint32_t)(kr * kRowBytes + ((pc ^ swz<D>(pos)) << 4));
            voff[j] = (uint32_t)(pos * kRowBytes + ((pc ^ swz_v<D>(pos)) << 4));
        }
    }

    // Issue the asynchronous copies of rows kv0 .. kv0+BN-1 (rows >= valid read 0);
    // stream (wave-uniform): with the non-temporal cache policy.
    __device__ inline void issue(const uint16_t *Kh, const uint16_t *Vh, int64_t kv0,
                                 int64_t valid, uint16_t *Ks, uint16_t *Vs, bool stream = false) const
    {
        int64_t rows = valid - kv0;
        rows = rows < 0 ? 0 : (rows > BN ? BN : rows);
        const int nbytes = (int)rows * kRowBytes;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void *)(Kh + kv0 * D), (short)0, nbytes, kBufferRsrcWord3);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void *)(Vh + kv0 * D), (short)0, nbytes, kBufferRsrcWord3);
        if (stream) {
#pragma unroll
            for (int j = 0; j < kPerWave; ++j) {
                copy_to_lds<true>(rk, Ks + (slice0 + j) * 512, koff[j]);
                copy_to_lds<true>(rv, Vs + (slice0 + j) * 512, voff[j]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < kPerWave; ++j) {
                copy_to_lds(rk, Ks + (slice0 + j) * 512, koff[j]);
                copy_to_lds(rv, Vs + (slice0 + j) * 512, voff[j]);
            }
        }
    }
};

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt left at their maxima: at most n
// of this wave's memory operations are still outstanding (vector memory loads
// complete in issue order, so the oldest copies have landed).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
template <int N>
__device__ inline void wait_vmem_keep() { __builtin_amdgcn_s_waitcnt(waitcnt_vm(N)); }
// s_waitcnt lgkmcnt(0) with vmcnt and expcnt left at their maxima.
constexpr int kWaitLds0 = 15 | (3 << 14) | (7 << 4);

// Per-wave state of the forward pass and the work on one key tile.  BAND:
// restricted self-attention, keys within `radius` of the query row only.
template <int NW, int NB, int D, bool BAND = false>
struct Attn {
    static constexpr int kD = D;                 // d_k = d_v
    static constexpr int kRowBytes = 2 * D;      // one K or V row in HBM and LDS
    static constexpr int kKB = D / 16;           // 16-dim chunks of the score contraction
    // 32-dim blocks of the output.  D = 16: one block whose dims 16..31 are not
    // head dims: their V^T rows are read from the neighbouring LDS row (an
    // MFMA output row depends only on its own A row, so they never mix into
    // dims 0..15) and they are never stored.
    static constexpr int kDB = (D + 31) / 32;
    static constexpr int kLdsPad = D < 32 ? 32 : 0;   // elements: those reads past the last row stay in LDS
    static constexpr int BM = 32 * NW;
    static constexpr int BN = 32 * NB;
    static constexpr int kTileElems = BN * kD;   // bf16 elements per K (or V) tile
    static constexpr int kBuffers = 3;                  // LDS ring: tiles t, t+1 read, t+2 landing
    static constexpr int kBufStride = 2 * kTileElems;   // K tile, then V tile, per buffer
    // Q is staged in buffer 2 before tile 2 arrives when each wave's 32 Q rows
    // fit exactly where its own share of tile 2's copies will land; otherwise
    // (D = 128 with 32-key tiles) the Q operand is loaded straight into
    // registers.
    static constexpr bool kQViaLds = 2 * BN / NW >= 32;
    static_assert(D == 16 || D == 32 || D == 64 || D == 128, "head sizes with a matrix-core layout");

    uint16_t *kbuf[kBuffers], *vbuf[kBuffers];   // LDS tile buffers
    const uint16_t *Kh, *Vh;
    int64_t len;                     // legal keys of this batch entry (clamped)
    int64_t q0w;                     // first query row of this wave (wave-uniform)
    int l32;                         // this lane's query row is q0w + l32
    int causal;
    int n_tiles;
    int64_t qrel;                    // BAND: q0w relative to the first key of the range
    int64_t radius;                  // BAND: neighbourhood radius
    bool kv_stream = false;          // K/V copies non-temporal (few query tiles per head)
    float scale_log2;
    int g;                           // lane half

    TileLoader<NW, BN, D> ld;
    bf16x8_t qf[kKB];                // Q^T operand (B of S^T = K Q^T)
    int wave;                        // wave index in the workgroup (uniform)
    int koff[2][kKB];                // LDS byte offsets of K reads (blocks of even/odd parity)
    int voff[kDB];                   // LDS byte offsets of V transposing reads
    f32x16_t acc[kDB];               // O^T: dims 32*db + 8*(r/4) + 4*g + r%4, this lane's query row
    float m_run, l_run;

    // S^T block bk of the tile in buffer Ks.
    __device__ __forceinline__ f32x16_t scores(const uint16_t *Ks, int bk) const
    {
        f32x16_t s;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
            const u32x4_t a = *(const u32x4_t *)((const char *)Ks + koff[bk & 1][kb] + (bk >> 1) * 64 * kRowBytes);
            s = mfma32(as_bf16x8(a), qf[kb], s);
        }
        return s;
    }

    // acc += V^T P^T for block bk (its two 16-key slabs kk = 2*bk, 2*bk + 1).
    // zero: the accumulator is known to be 0 (the first product of the key
    // loop; a constant after unrolling), so the first MFMA starts from 0
    // instead of reading it.
    __device__ __forceinline__ void pv(const uint16_t *Vs, int bk, const bf16x8_t *p, bool zero = false)
    {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kk = 2 * bk + h;
#pragma unroll
            for (int db = 0; db < kDB; ++db) {
                const char *vb = (const char *)Vs + voff[db];
                const u32x2_t lo = ds_read_tr16_b64((const uint16_t *)(vb + (16 * kk) * kRowBytes));
                const u32x2_t hi = ds_read_tr16_b64((const uint16_t *)(vb + (16 * kk + 4) * kRowBytes));
                const u32x4_t a = {lo[0], lo[1], hi[0], hi[1]};
                acc[db] = mfma32(as_bf16x8(a), p[h], (zero && h == 0) ? f32x16_t{} : acc[db]);
            }
        }
    }

    // Row maximum of a block (scaled, log2 units), both lane halves combined.
    __device__ __forceinline__ float block_max(const f32x16_t &s) const
    {
        float mx = fmaxf(s[0], s[1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[r]);
        return max_across_halves(mx) * scale_log2;
    }

    // Multiply what was accumulated relative to the old reference maximum by
    // alpha: the accumulator, the row sum and (if given) weights not yet
    // multiplied by V (re-rounded to bf16).
    __device__ __forceinline__ void scale_pending(float alpha, bf16x8_t *pending)
    {
        l_run *= alpha;
        // In-place multiplies (tied operands): the accumulator keeps its
        // registers across this rarely taken path, so the common path needs no
        // copies where the two paths join.
        acc_read_fence();
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                asm volatile("v_mul_f32 %0, %0, %1" : "+v"(acc[db][i]) : "v"(alpha));
        if (pending) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4_t w = as_u32x4(pending[h]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float lo = __builtin_bit_cast(float, w[i] << 16) * alpha;
                    const float hi = __builtin_bit_cast(float, w[i] & 0xFFFF0000u) * alpha;
                    w[i] = pack_bf16x2(lo, hi);
                }
                pending[h] = as_bf16x8(w);
            }
        }
    }

    // Move the reference maximum of the rows whose block maximum grew by more
    // than kTau over it, rescaling what was accumulated against the old one.
    // fresh: no legal key has been seen yet (the key loop's first block; a
    // constant after unrolling), so the accumulator and the row sum are 0 and
    // the reference maximum is simply the block maximum.
    __device__ __forceinline__ void rescale_if_needed(float mxs, bool fresh = false)
    {
        if (fresh) {
            m_run = mxs;
            return;
        }
        const bool grow = mxs > m_run + kTau;    // false while mxs is -inf
        if (__builtin_expect(__any(grow), 0)) {
            // Keep this a real branch: after the first blocks it is rarely taken,
            // and if-converted it would cost dozens of multiplies per block.
            asm volatile("" ::: "memory");
            const float m_new = grow ? mxs : m_run;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            m_run = m_new;
            scale_pending(alpha, nullptr);
        }
    }

    // Weights of one block relative to the reference maximum, packed as the two
    // B operands of the P.V product.  Returns this lane's sum of the
    // bf16-rounded weights (the ones used in P.V).
    __device__ __forceinline__ float weights(const f32x16_t &s, bf16x8_t *p) const
    {
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;   // all -inf so far
        const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
        float sum = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4_t w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * h + 2 * i], scale_log2, -m_use));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * h + 2 * i + 1], scale_log2, -m_use));
                // The packed word is summed as a scalar: hipcc 7.2 passed the
                // first word to every dot2 when given elements of a vector.
                const uint32_t pk = pack_bf16x2(p0, p1);
                sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), ones, sum, false);
                w[i] = pk;
            }
            p[h] = as_bf16x8(w);
        }
        return sum;
    }

    // Scheduling of one straight-line stretch of a fully legal tile (block b's
    // weights on the VALU; S of block b+1 or of the next tile's block 0, and
    // P.V of block b-1, on the matrix core): the compiler would otherwise issue
    // the stretch's MFMAs back to back and leave the wave without matrix work
    // while its VALU runs.  The LDS reads go first, then each MFMA is followed
    // by a group of VALU instructions.  Masks: 0x100 LDS read, 0x008 MFMA,
    // 0x002 VALU.
    __device__ __forceinline__ static void mfma_then_valu(int n)
    {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < n) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
            }
    }

    __device__ __forceinline__ static void interleave_stretch(int b)
    {
        if (b == 0) {
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);    // K reads of S
            mfma_then_valu(4);
        } else {
            __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);   // V reads of P.V, K reads of S
            mfma_then_valu(8);
        }
    }

    // Block b of a fully legal tile (every row holds a finite reference
    // maximum), after its weights were taken against the reference (bsum = this
    // lane's part of the row's block sum, 16 of its 32 keys): only if either
    // half of a row's block sum passes kSumMax (a score grew by more than
    // log2(kSumMax / 16) over the reference) does that row move its reference
    // to the block maximum and recompute the block.  The decision is taken per
    // row, for both lane halves l32 and l32 + 32 together: they feed the same
    // P.V products and share the row sum, so they must keep one reference.
    // P.V of block b-1 is already issued, so moving a reference only rescales
    // the accumulator and the row sum.
    __device__ __forceinline__ void finish_max_free(const f32x16_t &s, bf16x8_t *p, float bsum)
    {
        constexpr float kSumMax = 1048576.0f;   // 2^20
        const bool over = !(bsum <= kSumMax);
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(over) != 0, 0)) {
            asm volatile("" ::: "memory");   // keep the rare path a real branch
            // the row's decision: this lane's half or the other (lane l32 ^ 32)
            const uint32_t o = over ? 1u : 0u;
            const auto both = __builtin_amdgcn_permlane32_swap(o, o, false, false);
            const bool grow = ((uint32_t)both[0] | (uint32_t)both[1]) != 0;
            const float mxs = block_max(s);
            if (grow) {
                scale_pending(__builtin_amdgcn_exp2f(m_run - mxs), nullptr);
                m_run = mxs;
            }
            const float redo = weights(s, p);
            bsum = grow ? redo : bsum;
        }
        l_run += bsum;
    }

    // A fully legal tile after the first, software-pipelined across tiles: S of
    // its block 0 was computed by the previous tile (s_io in); while block b's
    // weights run on the VALU, the matrix core has S of block b+1 (for the last
    // block: S of the next tile's block 0, from Knext, into s_io) and P.V of
    // block b-1.  The next tile's K is in LDS: every wave waited for all its
    // copies before this tile's barrier.  When there is no next tile the buffer
    // holds older data and that result is not used.
    __device__ __forceinline__ void tile_blocks_full(const uint16_t *Ks, const uint16_t *Vs,
                                                     const uint16_t *Knext, f32x16_t &s_io)
    {
        f32x16_t s[NB];
        bf16x8_t p[NB][2];
        s[0] = s_io;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b + 1 < NB) s[b + 1] = scores(Ks, b + 1);
            else s_io = scores(Knext, 0);
            const float bsum = weights(s[b], p[b]);   // no block maximum
            if (b > 0) pv(Vs, b - 1, p[b - 1]);
            interleave_stretch(b);   // in the same straight-line stretch as the above
            finish_max_free(s[b], p[b], bsum);
        }
        pv(Vs, NB - 1, p[NB - 1]);
    }

    // Any other tile (the first, one crossing the causal diagonal or the
    // padding end, one beyond this wave's rows) block by block, with masks
    // (key kv0 + 32*b + 16*(r/8) + 8*g + r%8 is legal iff that offset < lim)
    // and, unless MAXFREE, block maxima.  On the first tile the block maxima
    // set every row's reference maximum (key 0 is legal for every row when
    // len > 0).  A block with no legal key for any row of the wave
    // contributes exactly 0.  Decisions are per row, so a row's result
    // depends on its own legal keys only.
    // FIRST: the first tile of the key loop (the accumulator and the row sum
    // are still 0: its first block sets the reference maxima without scaling,
    // and its first product starts from 0).
    // MAXFREE: a later tile of the unrestricted kernel (every row met key 0
    // in tile 0, so its reference maximum is finite): no block maxima, the
    // weights are taken against the reference as on the fully legal tiles,
    // masked keys give exp2(-inf) = 0.
    template <bool FIRST = false, bool MAXFREE = false>
    __device__ __forceinline__ void tile_blocks_masked(const uint16_t *Ks, const uint16_t *Vs, int lim,
                                                       int lo = 0)
    {
        f32x16_t s[NB];
        bf16x8_t p[NB][2];
        s[0] = scores(Ks, 0);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            // the per-register part is a constant compared with lim - 8g - 32b
            const int lim_g = lim - 8 * g - 32 * b;
            if constexpr (BAND) {
                // BAND: keys below offset lo are out of the row's neighbourhood too
                const int lo_g = lo - 8 * g - 32 * b;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 16 * (r >> 3) + (r & 7);
                    if (off >= lim_g || off < lo_g) s[b][r] = -INFINITY;
                }
            } else if (__builtin_amdgcn_ballot_w64(lim_g < 24) != 0) {
                // some lane's last legal key offset is below 23 (else the
                // block is fully legal for the wave: no per-element masks)
                asm volatile("" ::: "memory");
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (16 * (r >> 3) + (r & 7) >= lim_g) s[b][r] = -INFINITY;
            }
            if constexpr (MAXFREE) {
                if (b > 0) pv(Vs, b - 1, p[b - 1]);
                if (b + 1 < NB) s[b + 1] = scores(Ks, b + 1);
                const float bsum = weights(s[b], p[b]);
                finish_max_free(s[b], p[b], bsum);
            } else {
                const float mxs = block_max(s[b]);
                if (b > 0) pv(Vs, b - 1, p[b - 1], FIRST && b == 1);
                rescale_if_needed(mxs, FIRST && b == 0);
                if (b + 1 < NB) s[b + 1] = scores(Ks, b + 1);
                l_run += weights(s[b], p[b]);
            }
        }
        pv(Vs, NB - 1, p[NB - 1], FIRST && NB == 1);
    }

    // Issue the copies of tile u into buffer u % kBuffers.
    __device__ __forceinline__ void prefetch(int u, uint16_t *kb, uint16_t *vb)
    {
        ld.issue(Kh, Vh, (int64_t)u * BN, len, kb, vb, kv_stream);
    }

    // Q^T as the B operand of the score MFMA, from where the prologue staged it
    // in buffer 2: the lane's query row l32, dims 16*kb + 8*g .. +7 (logical
    // chunk 2*kb + g, stored at chunk (2*kb + g) ^ swz(l32)).  Without LDS
    // staging the prologue has loaded qf straight from HBM.
    __device__ __forceinline__ void read_q()
    {
        if constexpr (kQViaLds) {
            const uint16_t *row = D < 32 ? kbuf[2] + (32 * wave + l32) * kD
                                         : (l32 < 16 ? kbuf[2] : vbuf[2]) + (16 * wave + (l32 & 15)) * kD;
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb)
                qf[kb] = *(const bf16x8_t *)(row + (((2 * kb + g) ^ swz<D>(l32)) << 3));
        }
    }

    // Start of tile t, the same for every wave and every kind of tile (one
    // barrier per tile).  Before the barrier each wave waits for all its copies
    // in flight, tiles t and t+1 (and Q at t = 0); after it, tiles t and t+1
    // are in LDS for every wave and every wave is done with tile t-1, whose
    // buffer takes tile t+2.  At t = 0 the wave first reads its Q rows, which
    // lie where its own copies of tile 2 land.  With Q staged in LDS (and
    // outside the band kernel, whose ring may start at tile 1, and the
    // one-wave key-split kernel, where the peeled tile raised the spilled
    // SGPRs from 78 to 116 at d = 128) tile 0 waits for Q and tile 0 only: tile 1's
    // copies, issued last, may still be in flight (vector memory loads
    // complete in issue order), so a workgroup starts computing after two
    // thirds of its first burst of loads.
    static constexpr bool kFirstWaitOne = kQViaLds && !BAND && NW > 1;
    __device__ __forceinline__ void tile_begin(int t, uint16_t *knext, uint16_t *vnext)
    {
        if (kFirstWaitOne && t == 0 && n_tiles > 1)
            wait_vmem_keep<TileLoader<NW, BN, D>::kLoadsPerTile>();
        else
            wait_vmem_keep<0>();
        __syncthreads();
        if (t == 0) {
            SDPA_STAMP(1);
            read_q();
            __builtin_amdgcn_s_waitcnt(kWaitLds0);
        }
        if (t + 2 < n_tiles) prefetch(t + 2, knext, vnext);
    }

    // A fully legal tile after the first, in LDS buffer BUF = t % 3.
    // Instantiated per buffer so that every LDS operand address is a per-lane
    // register plus an immediate offset.
    template <int BUF>
    __device__ __forceinline__ void tile_full(int t, f32x16_t &s_io)
    {
        tile_begin(t, kbuf[(BUF + 2) % 3], vbuf[(BUF + 2) % 3]);
        tile_blocks_full(kbuf[BUF], vbuf[BUF], kbuf[(BUF + 1) % 3], s_io);
    }

    // Tile 0 of the unrestricted kernel: every wave has keys in it (key 0 is
    // legal for every row when the tile exists), so there is no early exit,
    // and the accumulator is still 0.
    __device__ __forceinline__ void tile_first()
    {
        tile_begin(0, kbuf[2], vbuf[2]);
        int64_t lim64 = len;
        const int64_t causal_lim = q0w + l32 + 1;
        if (causal && causal_lim < lim64) lim64 = causal_lim;
        const int lim = (int)(lim64 < 0 ? 0 : (lim64 > BN ? BN : lim64));
        tile_blocks_masked<true>(kbuf[0], vbuf[0], lim);
    }

    // Any other tile, with the buffer chosen at run time (FIRST: tile 0, whose
    // blocks start from a zero accumulator).
    template <bool FIRST = false, bool MAXFREE = false>
    __device__ __forceinline__ void tile_any(int t)
    {
        const int buf = t % 3;
        const int nxt = (t + 2) % 3;
        tile_begin(t, kbuf[0] + nxt * kBufStride, vbuf[0] + nxt * kBufStride);
        const int64_t kv0 = (int64_t)t * BN;
        if constexpr (BAND) {
            // Rows qrel .. qrel+31 (relative to the range's first key) may use
            // keys qrel - radius .. qrel + 31 + radius (and, if causal, up to
            // their own row); a wave with none in this tile has nothing to do.
            if (kv0 + BN - 1 < qrel - radius || kv0 > qrel + 31 + radius || (causal && kv0 > qrel + 31))
                return;
            int64_t lim64 = len - kv0;
            const int64_t band_lim = (qrel - kv0) + l32 + radius + 1;
            if (band_lim < lim64) lim64 = band_lim;
            const int64_t causal_lim = (qrel - kv0) + l32 + 1;
            if (causal && causal_lim < lim64) lim64 = causal_lim;
            const int lim = (int)(lim64 < 0 ? 0 : (lim64 > BN ? BN : lim64));
            const int64_t lo64 = (qrel - kv0) + l32 - radius;
            const int lo = (int)(lo64 < 0 ? 0 : (lo64 > BN ? BN : lo64));
            tile_blocks_masked<FIRST>(kbuf[0] + buf * kBufStride, vbuf[0] + buf * kBufStride, lim, lo);
            return;
        }
        // A wave whose rows all precede the tile's first key has nothing to do.
        if (causal && kv0 > q0w + 31) return;
        // Keys this lane may use in the tile: below the key length and, if
        // causal, up to its own row.
        int64_t lim64 = len - kv0;
        const int64_t causal_lim = (q0w - kv0) + l32 + 1;
        if (causal && causal_lim < lim64) lim64 = causal_lim;
        const int lim = (int)(lim64 < 0 ? 0 : (lim64 > BN ? BN : lim64));
        tile_blocks_masked<FIRST, MAXFREE>(kbuf[0] + buf * kBufStride, vbuf[0] + buf * kBufStride, lim);
    }

    // All key tiles: the first, then the fully legal ones in a loop unrolled
    // over the buffer ring (no per-tile branch on the tile kind), then the
    // rest.  Every wave passes the same number of barriers (one per tile); the
    // waves of a workgroup may switch between the phases at different tiles.
    __device__ __forceinline__ void run()
    {
        if constexpr (BAND) {
            run_band();
            return;
        }
        if (n_tiles == 0) return;
        // Tiles 1 .. n_full-1 are fully legal for every row of this wave.
        int64_t n_full = len / BN;
        if (causal) {
            const int64_t diag = (q0w + 1) / BN;   // (t+1)*BN - 1 <= q0w
            if (diag < n_full) n_full = diag;
        }
        // Three phases, each with its own copy of the code, so that the
        // accumulators stay in place from one phase to the next (one loop over
        // both kinds of tile made the register allocator copy them at every
        // masked tile).
        if constexpr (NW == 1) {
            // the one-wave key-split kernel keeps a single loop: with the
            // phases, its d = 128 form got an accumulation register as an
            // operand of the rescale's inline multiplies (rejected by the
            // assembler)
            for (int t = 0; t < n_tiles;) {
                if (t == 1 && n_full > 1) {
                    f32x16_t s_io = scores(kbuf[1], 0);   // tile 1 landed before tile 0's barrier
                    for (; t + 2 < n_full; t += 3) {
                        tile_full<1>(t, s_io);
                        tile_full<2>(t + 1, s_io);
                        tile_full<0>(t + 2, s_io);
                    }
                    if (t < n_full) tile_full<1>(t++, s_io);
                    if (t < n_full) tile_full<2>(t++, s_io);
                } else {
                    tile_any(t++);
                }
            }
            return;
        }
        tile_first();
        int t = 1;
        if (n_full > 1) {
            if constexpr (kFirstWaitOne) {
                // tile 1 is in LDS for every wave after its own barrier; each
                // later tile has landed at the barrier before its own
                tile_begin(1, kbuf[0], vbuf[0]);
                f32x16_t s_io = scores(kbuf[1], 0);
                tile_blocks_full(kbuf[1], vbuf[1], kbuf[2], s_io);
                for (t = 2; t + 2 < n_full; t += 3) {
                    tile_full<2>(t, s_io);
                    tile_full<0>(t + 1, s_io);
                    tile_full<1>(t + 2, s_io);
                }
                if (t < n_full) tile_full<2>(t++, s_io);
                if (t < n_full) tile_full<0>(t++, s_io);
            } else {
                f32x16_t s_io = scores(kbuf[1], 0);   // tile 1 landed before tile 0's barrier
                for (; t + 2 < n_full; t += 3) {
                    tile_full<1>(t, s_io);
                    tile_full<2>(t + 1, s_io);
                    tile_full<0>(t + 2, s_io);
                }
                if (t < n_full) tile_full<1>(t++, s_io);
                if (t < n_full) tile_full<2>(t++, s_io);
            }
        }
        for (; t < n_tiles; ++t) tile_any<false, true>(t);   // reference maxima finite since tile 0
    }

    // BAND: the fully legal tiles of this wave form the middle range
    // [f_lo, f_hi): every key of such a tile lies within every row's
    // neighbourhood (and below the key length, and not after the row if
    // causal), and every row has met a legal key in an earlier tile, so its
    // reference maximum is finite as the max-free path requires.  The tiles
    // before and after go block by block with masks.
    __device__ __forceinline__ void run_band()
    {
        if (n_tiles == 0) return;
        // first tile start >= qrel + 32 - radius: every row's lowest legal key
        // (qrel + l32 - radius) lies before it
        const int64_t lo_key = qrel + 32 - radius;
        int64_t f_lo = lo_key <= 0 ? 1 : (lo_key + BN - 1) / BN;
        if (f_lo < 1) f_lo = 1;
        int64_t f_hi = len / BN;
        const int64_t up = (qrel + radius + 1) / BN;   // (t+1)*BN - 1 <= qrel + radius
        if (up < f_hi) f_hi = up;
        if (causal) {
            const int64_t diag = (qrel + 1) / BN;
            if (diag < f_hi) f_hi = diag;
        }
        // In phases, as in run(): the masked tiles before the ring, the ring,
        // the masked tiles after it.
        const bool ring = f_hi > f_lo;
        const int64_t ring_lo = ring ? f_lo : n_tiles;
        tile_any<true>(0);    // f_lo >= 1
        int t = 1;
        for (; t < ring_lo && t < n_tiles; ++t) tile_any(t);
        if (ring && t == f_lo) {
            // tile f_lo landed before tile f_lo-1's barrier; enter the ring at
            // its phase
            f32x16_t s_io = scores(kbuf[0] + (t % 3) * kBufStride, 0);
            if (t % 3 == 2) tile_full<2>(t++, s_io);
            if (t % 3 == 0 && t < f_hi) tile_full<0>(t++, s_io);
            for (; t + 2 < f_hi; t += 3) {
                tile_full<1>(t, s_io);
                tile_full<2>(t + 1, s_io);
                tile_full<0>(t + 2, s_io);
            }
            if (t < f_hi) tile_full<1>(t++, s_io);
            if (t < f_hi) tile_full<2>(t++, s_io);
        }
        for (; t < n_tiles; ++t) tile_any(t);
    }
};

// Key-split mode (several query rows against a long key range, split over
// workgroups): the workgroup takes keys [kv_lo, kv_lo + chunk) of its head and,
// instead of O, writes its partial result for each query row i of split u =
// bh * n_split + s: acc[u][i][0..63] = sum_j w_ij v_j, m[u][i] = the reference
// maximum m_i (log2 units of the scaled scores), l[u][i] = sum_j w_ij, with
// w_ij = exp2(s_ij - m_i) rounded to bf16 (the weights used in the product).
// Partial results for any reference combine exactly (log-sum-exp merge).
struct SplitOut {
    float *acc, *m, *l;
    int64_t chunk;       // keys per split, a multiple of the key tile
    uint32_t n_split;    // splits per head
};

// One query tile (BM rows of head bh) against keys [kv_lo, kv_hi): load Q,
// stream the key tiles, store O (or, with SPLIT, the partial result).
// OUT_NT: output stores non-temporal; copies_nt: Q/K/V copies non-temporal
// (the launcher sets it for heads with few query tiles).  A caller that reads
// the output right away (the multi-head path's output projection) or whose
// inputs were just written (its Q/K/V projections) takes neither: there the
// lines are worth keeping (multi-head base encoder step +2.3 % with them).
// OUT_NT is a template parameter: as a run-time flag it cost 1 % on the base
// encoder.
template <int NW, int NB, int D, bool SPLIT, bool BAND = false, bool OUT_NT = true>
__device__ __forceinline__ void attend_query_tile(
    uint16_t *const *kbuf, uint16_t *const *vbuf, const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const int32_t *__restrict__ key_lengths, int causal,
    uint16_t *__restrict__ O, int H, int64_t Lq, int64_t Lk, float scale_log2,
    uint32_t bh, uint32_t qt, int wave, int lane, int64_t kv_lo, int64_t kv_hi, const SplitOut &so, uint32_t u,
    int64_t radius = 0, bool copies_nt = false, int64_t len_known = -1)
{
    using A = Attn<NW, NB, D, BAND>;
    constexpr int BM = A::BM;
    constexpr int BN = A::BN;
    constexpr int kD = D, kRowBytes = A::kRowBytes, kKB = A::kKB, kDB = A::kDB;
    SDPA_STAMP(0);
    const int g = lane >> 5;      // lane half
    const int l32 = lane & 31;
    const int64_t b = bh / H;
    const int64_t q0 = (int64_t)qt * BM;

    A st;
#pragma unroll
    for (int i = 0; i < A::kBuffers; ++i) { st.kbuf[i] = kbuf[i]; st.vbuf[i] = vbuf[i]; }
    st.causal = causal;
    st.kv_stream = copies_nt;
    st.scale_log2 = scale_log2;
    st.g = g;
    st.q0w = q0 + 32 * wave;
    st.l32 = l32;
    int64_t len = Lk;
    if (len_known >= 0) {
        len = len_known;                 // read (and clamped) by the caller
    } else if (key_lengths) {
        const int64_t l = key_lengths[b];
        len = l < 0 ? 0 : (l > Lk ? Lk : l);
    }
    if constexpr (BAND) {
        // The workgroup's rows q0 .. q0+BM-1 use keys from q0 - radius on.
        kv_lo = q0 > radius ? q0 - radius : 0;
        st.radius = radius;
        st.qrel = st.q0w - kv_lo;
    }
    // Legal keys of this workgroup's range, counted from kv_lo (the causal
    // mask is only used with kv_lo = 0 or, BAND, through qrel).
    len = (len < kv_hi ? len : kv_hi) - kv_lo;
    len = len < 0 ? 0 : len;
    st.len = len;
    int64_t kv_end = len;                        // keys the workgroup needs
    if constexpr (BAND) {
        const int64_t q_end = q0 - kv_lo + BM;   // one past the last row, relative
        if (q_end + radius < kv_end) kv_end = q_end + radius;
        if (causal && q_end < kv_end) kv_end = q_end;
    } else {
        if (causal && q0 + BM < kv_end) kv_end = q0 + BM;
    }
    st.n_tiles = (int)((kv_end + BN - 1) / BN);

    st.Kh = K + ((int64_t)bh * Lk + kv_lo) * kD;
    st.Vh = V + ((int64_t)bh * Lk + kv_lo) * kD;

    // Rows of this wave present in Q / O; buffer descriptors bounded to them make
    // reads past Lq return 0 and writes past Lq vanish.
    int64_t rows_here = Lq - st.q0w;
    rows_here = rows_here < 0 ? 0 : (rows_here > 32 ? 32 : rows_here);
    const int64_t tile_base = ((int64_t)bh * Lq + st.q0w) * kD;   // wave-uniform
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(Q + tile_base), (short)0, (int)rows_here * kRowBytes, kBufferRsrcWord3);

    st.wave = wave;

    // LDS byte offsets of this lane's operand reads.
    //  K (A of S^T): row pos = 32*bk + l32, dims 16*kb + 8*g .. +7; swz(pos)
    //  depends on bk only through its parity, so blocks bk and bk + 2 share
    //  offsets up to a constant.
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
            const int pos = bk * 32 + l32;
            st.koff[bk][kb] = 2 * (pos * kD + (((2 * kb + g) ^ swz<D>(pos)) << 3));
        }
    //  V (A of O^T, transposing read): in 16-lane group G, lane i addresses row
    //  i/4 of a 4-row slab and dims 4*(i%4) .. +3 of the 16-dim slab
    //  32*db + 16*(G%2); slab rows are 16*kk + 8*g + 4*h.
    {
        const int i = lane & 15;
        const int G1 = (lane >> 4) & 1;
        const int row = 8 * g + (i >> 2);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
            const int col = 32 * db + 16 * G1 + 4 * (i & 3);
            st.voff[db] = 2 * (row * kD + ((((col >> 3) ^ swz_v<D>(row))) << 3) + (col & 7));
        }
    }

#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.acc[db][i] = 0.f;
    st.m_run = -INFINITY;         // reference max of scaled scores (log2 units)
    st.l_run = 0.f;               // this lane's part of the running sum

    st.ld.init(wave, lane);
    if (st.n_tiles > 0) {
        if constexpr (A::kQViaLds) {
            // This wave's 32 Q rows into buffer 2 (rows 0-15 where its share of
            // tile 2's K rows lands, rows 16-31 where its V rows land; D = 16:
            // all 32 in its K share, 32 rows of 128 keys), 512/D rows per copy,
            // chunks swizzled by the row.
            constexpr int kRps = 512 / D, kC = D / 8;
#pragma unroll
            for (int sl = 0; sl < 32 / kRps; ++sl) {
                const int qrow = kRps * sl + lane / kC;
                const int r0 = kRps * sl;                    // first Q row of this copy
                const uint16_t *dst = D < 32 ? st.kbuf[2] + 32 * wave * kD
                                             : (r0 < 16 ? st.kbuf[2] : st.vbuf[2]) + (16 * wave + (r0 & 15)) * kD;
                const uint32_t voff = (uint32_t)(qrow * kRowBytes + (((lane % kC) ^ swz<D>(qrow)) << 4));
                // Q rows are read by this workgroup only: on the short launches
                // non-temporal too (big cross -2.4 %; on long launches no gain)
                if (copies_nt) copy_to_lds<true>(rq, dst, voff);
                else copy_to_lds(rq, dst, voff);
            }
        } else {
            // Q^T operand straight into registers: lane (l32, g) holds row l32,
            // dims 16*kb + 8*g .. +7.  Compiler-visible loads, so the compiler
            // puts a wait for them before the first read of qf (the register
            // file has no interlock on a load's destination); the tile copies
            // it does not see are issued after them and complete later, so
            // that wait never ends early.
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb)
                st.qf[kb] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(
                    rq, (uint32_t)(l32 * kRowBytes + (kb * 16 + g * 8) * 2), 0, 0));
        }
        // then the first tiles
        st.prefetch(0, st.kbuf[0], st.vbuf[0]);
    }
    if (st.n_tiles > 1) st.prefetch(1, st.kbuf[1], st.vbuf[1]);
    if constexpr (!A::kQViaLds) {
        // Read qf once here so that the compiler's wait for the Q loads sits
        // before the tile loop: it waits for the first tiles too, which the
        // first barrier waits for anyway, instead of draining the copies in
        // flight on every tile.
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) asm volatile("" ::"v"(st.qf[kb]));
    }

    st.run();
    SDPA_STAMP(2);

    // ---- epilogue: O = acc / l, rounded to bf16
    acc_read_fence();
    const float l_tot = sum_across_halves(st.l_run);
    if constexpr (SPLIT) {
        // The partial result, rows below Lq only (bounded descriptors drop the rest).
        const int64_t row0 = (int64_t)u * Lq + st.q0w;
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(so.acc + row0 * kD), (short)0, (int)rows_here * kD * 4, kBufferRsrcWord3);
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int rq4 = 0; rq4 < 4; ++rq4) {
                // Built as a float vector first: hipcc 7.2 stored the first
                // slice for every rq4 when given bit-cast elements directly.
                const f32x4_t w = {st.acc[db][4 * rq4 + 0], st.acc[db][4 * rq4 + 1],
                                   st.acc[db][4 * rq4 + 2], st.acc[db][4 * rq4 + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4_t, w), ra, (uint32_t)((l32 * kD + db * 32 + rq4 * 8 + g * 4) * 4), 0, 0);
            }
        if (g == 0) {
            const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(so.m + row0), (short)0, (int)rows_here * 4, kBufferRsrcWord3);
            const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(so.l + row0), (short)0, (int)rows_here * 4, kBufferRsrcWord3);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, st.m_run), rm,
                                                  (uint32_t)(l32 * 4), 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, l_tot), rl,
                                                  (uint32_t)(l32 * 4), 0, 0);
        }
        SDPA_STAMP(3);
        return;
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;   // no legal key: output 0
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(O + tile_base), (short)0, (int)rows_here * kRowBytes, kBufferRsrcWord3);
    // The wave's 32 x D output tile goes through LDS so that every store
    // instruction writes 512/D whole rows (1 KiB contiguous): written in the
    // accumulator layout (lane: row l32, 8-byte pieces of 16-byte chunk
    // 4*db + rq4), read back as row (512/D)*i + lane/(D/8), chunk lane%(D/8).
    // Chunks are XOR-swizzled by the row (D = 32: rows r and r + 4 share banks,
    // so by r/4).  The barrier makes sure every wave is done with the tile
    // buffers this reuses (no copies are in flight after the last tile); the
    // waves' stages (32 * D elements each) fit in the three buffers.
    static_assert(NW * 32 * kD <= A::kBuffers * A::kBufStride, "output stage fits in LDS");
    __syncthreads();
    uint16_t *stage = kbuf[0] + wave * 32 * kD;
    constexpr int kC = kD / 8, kRps = 512 / kD;
    auto oswz = [](int r) { return kD >= 64 ? r & 7 : (kD >= 32 ? (r >> 2) & 3 : 0); };
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int rq4 = 0; rq4 < 4; ++rq4) {
            if (32 * db + 8 * rq4 >= kD) continue;   // D = 16: dims 16..31 are not output
            u32x2_t w;
            w[0] = pack_bf16x2(st.acc[db][4 * rq4 + 0] * inv, st.acc[db][4 * rq4 + 1] * inv);
            w[1] = pack_bf16x2(st.acc[db][4 * rq4 + 2] * inv, st.acc[db][4 * rq4 + 3] * inv);
            const int c = 4 * db + rq4;
            *(u32x2_t *)((char *)stage + l32 * kRowBytes + ((c ^ oswz(l32)) << 4) + 8 * g) = w;
        }
    // the lane index recomputed (mbcnt) rather than kept live across the key
    // loop: at d = 128 keeping it cost a spilled register
    const int lane_o = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    // one branch for the whole stage (the cache policy is an immediate)
#pragma unroll
    for (int i = 0; i < 32 / kRps; ++i) {
        const int r = kRps * i + lane_o / kC, c = lane_o % kC;
        const u32x4_t w = *(const u32x4_t *)((const char *)stage + r * kRowBytes + ((c ^ oswz(r)) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(w, ro, (uint32_t)(r * kRowBytes + c * 16), 0,
                                               OUT_NT ? kStoreStreaming : 0);
    }
    SDPA_STAMP(3);
}

// Balanced order of a launch with per-entry key lengths (at most 64 entries, a
// multiple of 8 (entry, head) pairs, at most kBalancedMaxTiles key tiles per
// entry).  The query tiles of a pair cost about the entry's count of key tiles
// (causal: the later query tile more; both grow with the length).  Every wave
// ranks the entries by that count (longest first, ties by index; one ballot
// per count), then reads its query tile off a fixed plan: pairs in rank order
// are dealt to the 8 XCDs in a snake (0..7, 7..0, ...), and within an XCD its
// query tiles, longest first, fill rounds of 32 dispatch positions (one per
// CU), every other round reversed, so that the workgroups a CU runs at once
// add up to about the same work.  The hardware starts workgroup w on XCD
// w % 8 and an XCD's workgroups in order of w / 8; the order affects speed
// only (every query tile is taken exactly once).  Measured before it was
// built, by permuting the entries' lengths on the host to the same effect:
// base encoder -10.5 %, big cross -10 %, d = 128 encoder -13 %.  Returns the
// entry's key length, clamped to [0, Lk].
__device__ inline int64_t balanced_item(uint32_t w, uint32_t n_qtiles, uint32_t n_bh, int H,
                                        const int32_t *__restrict__ key_lengths, int64_t Lk, int BN,
                                        int lane, int wave, int *s_len, int causal, uint32_t &bh,
                                        uint32_t &qt)
{
    const int B = (int)(n_bh / (uint32_t)H);
    // Wave 0 reads the lengths and hands them to the other waves through LDS:
    // every workgroup of the launch reads the same two cache lines at its
    // start, and one read per workgroup instead of one per wave keeps that
    // burst of requests to one L2 channel short.
    if (wave == 0 && lane < B) {
        const int64_t l = key_lengths[lane];
        s_len[lane] = (int)(l < 0 ? 0 : (l > Lk ? Lk : l));
    }
    __syncthreads();
    int len = 0;
    int t = -1;                                   // key tiles of entry `lane` (-1: no such entry)
    if (lane < B) {
        len = s_len[lane];
        t = (len + BN - 1) / BN;
    }
    const int T = (int)((Lk + BN - 1) / BN);
    uint32_t rank = 0, above = 0;
    for (int c = T; c >= 0; --c) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(t == c);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        rank = t == c ? above + below : rank;     // a select, no branch
        above += (uint32_t)__builtin_popcountll(m);
    }
    const uint32_t x = w & 7, j = w >> 3;                     // XCD, position in it
    const uint32_t nx = n_qtiles * (n_bh >> 3);               // query tiles per XCD
    const uint32_t r = j >> 5, p = j & 31;                    // round, position in it
    const uint32_t s = nx - 32 * r < 32 ? nx - 32 * r : 32;   // positions in this round
    const uint32_t i = 32 * r + ((r & 1) ? s - 1 - p : p);    // rank of the tile in the XCD
    const uint32_t u = i / n_qtiles;                          // rank of its pair in the XCD
    qt = i % n_qtiles;
    if (causal) qt = n_qtiles - 1 - qt;                       // the pair's longest tile first
    const uint32_t k = 8 * u + ((u & 1) ? 7 - x : x);         // global rank of the pair
    const uint32_t e = k / (uint32_t)H;                       // rank of its entry
    const uint64_t mb = __builtin_amdgcn_ballot_w64(t >= 0 && rank == e);
    const int b = mb ? (int)__builtin_ctzll(mb) : 0;   // exactly one lane has rank e
    bh = (uint32_t)b * (uint32_t)H + k % (uint32_t)H;
    return (int64_t)__builtin_amdgcn_readlane(len, b);
}

// Work decomposition: one query tile (qt, head bh) per workgroup.  The
// hardware hands workgroup w to XCD w % 8 and, within an XCD, starts
// workgroups in order of w as slots free up.
//  * Non-causal: item (w % 8) * (T / 8) + w / 8 when 8 divides the item count
//    T, numbered head-major: each XCD works on a contiguous run of heads, and
//    the workgroups streaming the same K/V rows share that XCD's L2.
//  * Causal: a query tile's work grows with qt, so the tiles go out longest
//    first (qt descending), which fills the slots greedily longest-first and
//    leaves only short tiles for the end of the grid.  When 8 divides the head
//    count each XCD takes its own run of heads; when a head's K and V reach
//    1 MiB, in groups of kCausalHeadGroup heads one after the other,
//    longest first within a group: fewer heads in flight keep more of their
//    K/V rows in the XCD's L2 (on 8 heads of 8192 keys per XCD: 4 at a time
//    fetched 550 MiB per launch into L2, all 8 at once 1188 MiB, one at a time
//    196 MiB but with the long tiles of the last head starting late).  Short
//    heads fit the L2 together, and taking all of them at once balances best.
template <int NW, int NB, int D, int WAVES = Occupancy<D, NB>::kWaves, bool OUT_NT = true>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(WAVES, WAVES))) void sdpa_fwd_mfma_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const int32_t *__restrict__ key_lengths, int causal,
    uint16_t *__restrict__ O, int H, int64_t Lq, int64_t Lk, float scale_log2,
    uint32_t n_qtiles, uint32_t n_bh, int flags)
{
    using A = Attn<NW, NB, D>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[A::kBuffers * A::kBufStride + A::kLdsPad];
    __shared__ int s_len[64];        // the entries' key lengths (balanced order only)
    uint16_t *kbuf[A::kBuffers], *vbuf[A::kBuffers];
#pragma unroll
    for (int i = 0; i < A::kBuffers; ++i) {
        kbuf[i] = lds + i * A::kBufStride;
        vbuf[i] = kbuf[i] + A::kTileElems;
    }

    const int lane = threadIdx.x & 63;
    // wave index as a scalar (it is uniform across the wave)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const uint32_t w = blockIdx.x;
    uint32_t bh, qt;
    int64_t len_known = -1;
    if (flags & kFlagBalanced) {
        len_known = balanced_item(w, n_qtiles, n_bh, H, key_lengths, Lk, A::BN, lane, wave, s_len, causal,
                                  bh, qt);
    } else if (causal) {
        if ((n_bh & 7) == 0) {
            const uint32_t hx = n_bh >> 3, j = w >> 3;   // heads per XCD, position in the XCD
            // groups of G heads in turn, longest tiles first within a group,
            // once a head's K and V reach 1 MiB (smaller ones share the L2
            // anyway, and all heads at once balance better)
            const bool big = (uint64_t)Lk * (4 * D) >= (1u << 20);
            const uint32_t G = (big && hx % kCausalHeadGroup == 0) ? kCausalHeadGroup : hx;
            const uint32_t grp = j / (G * n_qtiles), r = j % (G * n_qtiles);
            bh = (w & 7) * hx + grp * G + r % G;
            qt = n_qtiles - 1 - r / G;
        } else {
            bh = w % n_bh;
            qt = n_qtiles - 1 - w / n_bh;
        }
    } else {
        const uint32_t n_items = n_qtiles * n_bh;
        const uint32_t item = (n_items & 7) == 0 ? (w & 7) * (n_items >> 3) + (w >> 3) : w;
        bh = item / n_qtiles;
        qt = item % n_qtiles;
    }
    attend_query_tile<NW, NB, D, false, false, OUT_NT>(kbuf, vbuf, Q, K, V, key_lengths, causal, O, H,
                                                    Lq, Lk, scale_log2, bh, qt, wave, lane, 0, Lk,
                                                    SplitOut{}, 0, 0, (flags & kFlagCopiesNt) != 0,
                                                    len_known);
}


// Restricted self-attention: every workgroup covers about BM + 2 * radius
// keys, so the work is even and the non-causal order (head-major runs per XCD)
// is used.
template <int NW, int NB, int D>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(Occupancy<D, NB, true>::kWaves, Occupancy<D, NB, true>::kWaves))) void sdpa_fwd_mfma_band_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const int32_t *__restrict__ key_lengths, int causal,
    int64_t radius, uint16_t *__restrict__ O, int H, int64_t Lq, int64_t Lk, float scale_log2,
    uint32_t n_qtiles, uint32_t n_bh)
{
    using A = Attn<NW, NB, D, true>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[A::kBuffers * A::kBufStride + A::kLdsPad];
    uint16_t *kbuf[A::kBuffers], *vbuf[A::kBuffers];
#pragma unroll
    for (int i = 0; i < A::kBuffers; ++i) {
        kbuf[i] = lds + i * A::kBufStride;
        vbuf[i] = kbuf[i] + A::kTileElems;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t w = blockIdx.x;
    const uint32_t n_items = n_qtiles * n_bh;
    const uint32_t item = (n_items & 7) == 0 ? (w & 7) * (n_items >> 3) + (w >> 3) : w;
    attend_query_tile<NW, NB, D, false, true>(kbuf, vbuf, Q, K, V, key_lengths, causal, O, H, Lq, Lk,
                                              scale_log2, item / n_qtiles, item % n_qtiles, wave, lane,
                                              0, Lk, SplitOut{}, 0, radius);
}


// Key-split kernel: one wave per workgroup, 32 query rows (Lq <= 32) against
// one chunk of keys; workgroup w takes split s = w % n_split of head
// bh = w / n_split and writes its partial result (SplitOut), or, with one
// chunk per head (SPLIT = false), O itself.  No causal mask.
template <int D, bool SPLIT>
__global__ __launch_bounds__(64) void sdpa_split_mfma_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const int32_t *__restrict__ key_lengths, uint16_t *__restrict__ O,
    int H, int64_t Lq, int64_t Lk, float scale_log2, SplitOut so)
{
    // One wave, 32-key tiles: 24 KiB of LDS at d = 64 (six workgroups per CU
    // keep the cache streaming), 48 KiB at d = 128.
    constexpr int NW = 1, NB = kSplitKeyBlocks;
    using A = Attn<NW, NB, D>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[A::kBuffers * A::kBufStride + A::kLdsPad];
    uint16_t *kbuf[A::kBuffers], *vbuf[A::kBuffers];
#pragma unroll
    for (int i = 0; i < A::kBuffers; ++i) {
        kbuf[i] = lds + i * A::kBufStride;
        vbuf[i] = kbuf[i] + A::kTileElems;
    }
    const int lane = threadIdx.x & 63;
    const uint32_t u = blockIdx.x;
    const uint32_t bh = u / so.n_split;
    const int64_t kv_lo = (int64_t)(u % so.n_split) * so.chunk;
    int64_t kv_hi = kv_lo + so.chunk;
    kv_hi = kv_hi < Lk ? kv_hi : Lk;
    attend_query_tile<NW, NB, D, SPLIT>(kbuf, vbuf, Q, K, V, key_lengths, 0, O, H, Lq, Lk,
                                        scale_log2, bh, 0, 0, lane, kv_lo, kv_hi, so, u);
}

// Decode step with the keys of one head split over the four waves of one
// workgroup (many heads: no partial results leave the workgroup).  Wave w takes
// keys [w c, (w + 1) c) of its head (c = the head's key length over four, in
// whole 32-key tiles) with a two-buffer ring of its own in LDS, then writes its
// partial result (reference maximum m, weight sum l, unnormalised sum of
// weighted V rows, all per query row) into that LDS space; after a barrier the
// workgroup merges them:
//   O = sum_w e^(m_w - M) acc_w / sum_w e^(m_w - M) l_w,   M = max_w m_w
// (base 2 in the kernel; a wave without keys contributes nothing; no key at
// all gives 0).  Lq <= 32 rows, no causal mask.
constexpr int kDecodeWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kDecodeWaves) void sdpa_decode_wg_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const int32_t *__restrict__ key_lengths,
    uint16_t *__restrict__ O, int H, int64_t Lq, int64_t Lk, float scale_log2)
{
    constexpr int NW = kDecodeWaves, BN = 32;
    using A = Attn<1, 1, D>;
    constexpr int kD = D, kRowBytes = A::kRowBytes, kKB = A::kKB, kDB = A::kDB;
    constexpr int kWaveLds = 2 * A::kBufStride;           // two K+V tile buffers per wave
    static_assert(32 * kD * 4 + 2 * 32 * 4 <= 2 * kWaveLds, "a wave's partial result fits its LDS");
    constexpr int kCopies = 2 * A::kBufStride / 1024;       // copy instructions per tile (K and V)
    __shared__ __attribute__((aligned(16))) uint16_t lds[NW * kWaveLds];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    SDPA_STAMP(0);
    const uint32_t bh = blockIdx.x;
    const int64_t b = bh / H;
    int64_t len = Lk;
    if (key_lengths) {
        const int64_t l = key_lengths[b];
        len = l < 0 ? 0 : (l > Lk ? Lk : l);
    }
    const int64_t c = ((len + NW - 1) / NW + BN - 1) / BN * BN;
    const int64_t kv_lo = wave * c;
    int64_t n = (kv_lo + c < len ? kv_lo + c : len) - kv_lo;
    n = n < 0 ? 0 : n;
    const int nt = (int)((n + BN - 1) / BN);

    A st;
    st.causal = 0;
    st.scale_log2 = scale_log2;
    st.g = g;
    st.q0w = 0;
    st.l32 = l32;
    st.wave = 0;
    st.len = n;
    st.n_tiles = nt;
    st.Kh = K + ((int64_t)bh * Lk + kv_lo) * kD;
    st.Vh = V + ((int64_t)bh * Lk + kv_lo) * kD;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
            const int pos = bk * 32 + l32;
            st.koff[bk][kb] = 2 * (pos * kD + (((2 * kb + g) ^ swz<D>(pos)) << 3));
        }
    {
        const int i = lane & 15;
        const int G1 = (lane >> 4) & 1;
        const int row = 8 * g + (i >> 2);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
            const int col = 32 * db + 16 * G1 + 4 * (i & 3);
            st.voff[db] = 2 * (row * kD + ((((col >> 3) ^ swz_v<D>(row))) << 3) + (col & 7));
        }
    }
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.acc[db][i] = 0.f;
    st.m_run = -INFINITY;
    st.l_run = 0.f;
    st.ld.init(0, lane);

    uint16_t *const mine = lds + wave * kWaveLds;
    uint16_t *kb[2] = {mine, mine + A::kBufStride};
    uint16_t *vb[2] = {mine + A::kTileElems, mine + A::kBufStride + A::kTileElems};
    int64_t rows_here = Lq < 32 ? Lq : 32;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(Q + (int64_t)bh * Lq * kD), (short)0, (int)rows_here * kRowBytes, kBufferRsrcWord3);
    if (nt > 0) st.ld.issue(st.Kh, st.Vh, 0, n, kb[0], vb[0]);
    if (nt > 1) st.ld.issue(st.Kh, st.Vh, BN, n, kb[1], vb[1]);
#pragma unroll
    for (int kb2 = 0; kb2 < kKB; ++kb2)
        st.qf[kb2] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(
            rq, (uint32_t)(l32 * kRowBytes + (kb2 * 16 + g * 8) * 2), 0, 0));
#pragma unroll
    for (int kb2 = 0; kb2 < kKB; ++kb2) asm volatile("" ::"v"(st.qf[kb2]));
    for (int t = 0; t < nt; ++t) {
        // this wave's copies of tile t have landed (those of tile t+1 may not)
        if (t + 1 < nt) wait_vmem_keep<kCopies>();
        else wait_vmem_keep<0>();
        if (t == 0) SDPA_STAMP(1);
        const int64_t rem = n - (int64_t)t * BN;
        st.tile_blocks_masked(kb[t & 1], vb[t & 1], (int)(rem < BN ? rem : BN));
        // the tile's operands are in registers (the products consumed them):
        // its buffer takes tile t+2
        if (t + 2 < nt) st.ld.issue(st.Kh, st.Vh, (int64_t)(t + 2) * BN, n, kb[t & 1], vb[t & 1]);
    }

    SDPA_STAMP(2);
    // this wave's partial result into its own LDS space: acc [32 rows][D], m [32], l [32]
    acc_read_fence();
    const float l_tot = sum_across_halves(st.l_run);
    float *part = (float *)mine;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            part[l32 * kD + 32 * db + 8 * (r >> 2) + 4 * g + (r & 3)] = st.acc[db][r];
    if (g == 0) {
        part[32 * kD + l32] = st.m_run;
        part[32 * kD + 32 + l32] = l_tot;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < rows_here * kD; idx += 64 * NW) {
        const int i = idx / kD, d = idx % kD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, ((const float *)(lds + w * kWaveLds))[32 * kD + i]);
        float num = 0.f, den = 0.f;
        if (M > -INFINITY) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float *pw = (const float *)(lds + w * kWaveLds);
                const float mw = pw[32 * kD + i];
                const float e = mw > -INFINITY ? __builtin_amdgcn_exp2f(mw - M) : 0.f;
                num += e * pw[i * kD + d];
                den += e * pw[32 * kD + 32 + i];
            }
        }
        const float o = den > 0.f ? num / den : 0.f;
        O[((int64_t)bh * Lq + i) * kD + d] = __builtin_bit_cast(uint16_t, (__bf16)o);
    }
    SDPA_STAMP(3);
}

// Merge of the split partial results: block = one wave for row i of head bh
// (block bh * Lq + i); lane t handles output dims t, t + 64, ...  Lane s of
// each group of 64 splits loads that split's m and l (all loads of a group at
// once); with M = max_s m_s and w_s = exp2(m_s - M) (0 for a split without
// legal keys):
//   O = sum_s w_s acc_s / sum_s w_s l_s   (0 if no split has a key).
__device__ inline float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ inline float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

template <int D>
__global__ __launch_bounds__(64) void sdpa_split_merge_kernel(
    const float *__restrict__ acc, const float *__restrict__ m, const float *__restrict__ l,
    uint16_t *__restrict__ O, int64_t Lq, uint32_t n_split)
{
    constexpr int kD = D, kPer = D / 64;   // output dims per lane
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;                 // bh * Lq + i
    const int64_t bh = row / Lq, i = row % Lq;
    const int64_t u0 = bh * n_split;
    float M = -INFINITY;
    for (uint32_t s0 = 0; s0 < n_split; s0 += 64)
        if (s0 + t < n_split) M = fmaxf(M, m[(u0 + s0 + t) * Lq + i]);
    M = wave_max(M);
    float num[kPer], den = 0.f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) num[e] = 0.f;
    if (M > -INFINITY) {
        for (uint32_t s0 = 0; s0 < n_split; s0 += 64) {
            float w = 0.f;
            if (s0 + t < n_split) {
                const int64_t r = (u0 + s0 + t) * Lq + i;
                const float ms = m[r];
                if (ms > -INFINITY) {
                    w = __builtin_amdgcn_exp2f(ms - M);
                    den += w * l[r];
                }
            }
            const uint32_t n = n_split - s0 < 64 ? n_split - s0 : 64;
            const float *a = acc + ((u0 + s0) * Lq + i) * kD + t;
            for (uint32_t t0 = 0; t0 < n; t0 += 8) {   // 8 independent loads in flight per dim
                float x[8][kPer];
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int e = 0; e < kPer; ++e)
                        x[j][e] = t0 + j < n ? a[(int64_t)(t0 + j) * Lq * kD + 64 * e] : 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float wj = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), (t0 + j) & 63));
#pragma unroll
                    for (int e = 0; e < kPer; ++e) num[e] += wj * x[j][e];
                }
            }
        }
        den = wave_sum(den);
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const float o = den > 0.f ? num[e] / den : 0.f;
        O[row * kD + t + 64 * e] = __builtin_bit_cast(uint16_t, (__bf16)o);
    }
}

template <int D>
hipError_t launch_decode_d(const void *Q, const void *K, const void *V, const int32_t *key_lengths,
                           void *out, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t chunk,
                           int64_t n_split, void *workspace, hipStream_t stream)
{
    const int64_t n_bh = B * H;
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    if (n_split == 0) {
        // Many heads: the keys of each head split over the four waves of its
        // workgroup, merged in LDS.
        hipLaunchKernelGGL((sdpa_decode_wg_kernel<D>), dim3((uint32_t)n_bh), dim3(64 * kDecodeWaves), 0,
                           stream, (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V,
                           key_lengths, (uint16_t *)out, (int)H, Lq, Lk, scale_log2);
        return hipGetLastError();
    }
    if (n_split == 1) {
        // One chunk per head: each one-wave workgroup writes O itself; no
        // partial results, no merge.
        const SplitOut whole{nullptr, nullptr, nullptr, Lk, 1u};
        hipLaunchKernelGGL((sdpa_split_mfma_kernel<D, false>), dim3((uint32_t)n_bh), dim3(64), 0, stream,
                           (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, key_lengths,
                           (uint16_t *)out, (int)H, Lq, Lk, scale_log2, whole);
        return hipGetLastError();
    }
    const int64_t n_rows = n_bh * n_split * Lq;
    float *ws = (float *)workspace;
    const SplitOut so{ws, ws + n_rows * D, ws + n_rows * (D + 1), chunk, (uint32_t)n_split};
    hipLaunchKernelGGL((sdpa_split_mfma_kernel<D, true>), dim3((uint32_t)(n_bh * n_split)), dim3(64), 0,
                       stream, (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, key_lengths,
                       nullptr, (int)H, Lq, Lk, scale_log2, so);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_decode_merge(ws, out, n_bh, Lq, n_split, D, stream);
}

template <int D>
hipError_t launch_merge_d(const float *ws, void *out, int64_t n_bh, int64_t Lq, int64_t n_split,
                          hipStream_t stream)
{
    const int64_t n_rows = n_bh * n_split * Lq;
    hipLaunchKernelGGL((sdpa_split_merge_kernel<D>), dim3((uint32_t)(n_bh * Lq)), dim3(64), 0, stream,
                       ws, ws + n_rows * D, ws + n_rows * (D + 1), (uint16_t *)out, Lq, (uint32_t)n_split);
    return hipGetLastError();
}

template <int NW, int NB, int D, int WAVES>
hipError_t launch_fwd(const void *Q, const void *K, const void *V, const int32_t *key_lengths, int causal,
                      void *out, int64_t H, int64_t Lq, int64_t Lk, float scale_log2, uint32_t n_qtiles,
                      uint32_t n_bh, bool streaming, hipStream_t stream)
{
    // Each K/V row is copied once per query tile of its head: with few of them
    // the rows stream through the caches (non-temporal copies).
    int flags = (streaming && n_qtiles <= kStreamQueryTiles) ? kFlagCopiesNt : 0;
    // Balanced order: launches with per-entry key lengths whose workgroups
    // are all resident at once (with more, the hardware balances by handing
    // free slots to the next workgroups, and the per-workgroup ranking only
    // costs: d = 32 encoder +9 %, d = 16 +5 %).
    const int64_t B = n_bh / H;
    const int64_t slots = (int64_t)kCUs * (4 * WAVES / NW);
    if (key_lengths && B <= 64 && (n_bh & 7) == 0 &&
        (Lk + 32 * NB - 1) / (32 * NB) <= kBalancedMaxTiles && (int64_t)n_qtiles * n_bh <= slots)
        flags |= kFlagBalanced;
    if (streaming)
        hipLaunchKernelGGL((sdpa_fwd_mfma_kernel<NW, NB, D, WAVES, true>), dim3(n_qtiles * n_bh), dim3(NW * 64),
                           0, stream, (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, key_lengths,
                           causal, (uint16_t *)out, (int)H, Lq, Lk, scale_log2, n_qtiles, n_bh, flags);
    else
        hipLaunchKernelGGL((sdpa_fwd_mfma_kernel<NW, NB, D, WAVES, false>), dim3(n_qtiles * n_bh), dim3(NW * 64),
                           0, stream, (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, key_lengths,
                           causal, (uint16_t *)out, (int)H, Lq, Lk, scale_log2, n_qtiles, n_bh, flags);
    return hipGetLastError();
}

template <int D>
hipError_t launch_mfma_d(const void *Q, const void *K, const void *V, const int32_t *key_lengths,
                         int causal, void *out, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                         bool streaming, hipStream_t stream)
{
    // D = 16: 2-wave workgroups (64 query rows) with 64-key tiles, so that each
    // wave copies one whole 1 KiB slice and, at 12 KiB of LDS and 86 VGPRs, a CU
    // holds 10 of them (2560 slots; 4-wave workgroups with 128-key tiles: 1024).
    constexpr int NW = D <= 16 ? 2 : kWaves;
    // D = 128: 32-key tiles, so that the three-buffer ring stays at 48 KiB.
    // D = 64: 32-key tiles at four waves per SIMD (24 KiB of LDS, 115 VGPRs),
    // so that every query tile of the base model's launches is resident at
    // once (causal: the tiles that cross the diagonal are also half as long).
    // Against 64-key tiles at three waves per SIMD (148 VGPRs, 48 KiB): base
    // encoder -4 %, big cross -2 % (once the stores and the short launches'
    // copies were non-temporal), long causal -0.7 to -0.9 %, its multi-head
    // step -1.5 %.
    constexpr int NB = D >= 64 ? 1 : (D >= 32 ? kKeyBlocks : 2);
    constexpr int BM = 32 * NW;
    const uint32_t n_qtiles = (uint32_t)((Lq + BM - 1) / BM);
    const uint32_t n_bh = (uint32_t)(B * H);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    if constexpr (D == 128) {
        // Long key ranges: a register budget of three waves per SIMD (168
        // VGPRs), long causal 496 -> 480 us; short launches keep two (19.1
        // against 19.7 us on the h = 4 encoder).
        if (Lk > kLongKeys128)
            return launch_fwd<NW, NB, D, kWavesPerSimd128Long>(Q, K, V, key_lengths, causal, out, H, Lq, Lk,
                                                               scale_log2, n_qtiles, n_bh, streaming, stream);
    }
    return launch_fwd<NW, NB, D, Occupancy<D, NB>::kWaves>(Q, K, V, key_lengths, causal, out, H, Lq, Lk,
                                                           scale_log2, n_qtiles, n_bh, streaming, stream);
}

template <int D>
hipError_t launch_mfma_band_d(const void *Q, const void *K, const void *V, const int32_t *key_lengths,
                              int causal, int64_t radius, void *out, int64_t B, int64_t H, int64_t Lq,
                              int64_t Lk, hipStream_t stream)
{
    constexpr int NW = kWaves;
    constexpr int NB = D >= 128 ? 1 : (D == 64 ? kBandKeyBlocks64 : (D >= 32 ? kKeyBlocks : 4));
    constexpr int BM = 32 * NW;
    const uint32_t n_qtiles = (uint32_t)((Lq + BM - 1) / BM);
    const uint32_t n_bh = (uint32_t)(B * H);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    hipLaunchKernelGGL((sdpa_fwd_mfma_band_kernel<NW, NB, D>), dim3(n_qtiles * n_bh),
                       dim3(NW * 64), 0, stream, (const uint16_t *)Q, (const uint16_t *)K,
                       (const uint16_t *)V, key_lengths, causal, radius, (uint16_t *)out, (int)H, Lq,
                       Lk, scale_log2, n_qtiles, n_bh);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_band(const void *Q, const void *K, const void *V, const int32_t *key_lengths,
                            int causal, int64_t radius, void *out, int64_t B, int64_t H, int64_t Lq,
                            int64_t Lk, int d, hipStream_t stream)
{
    switch (d) {
    case 16: return launch_mfma_band_d<16>(Q, K, V, key_lengths, causal, radius, out, B, H, Lq, Lk, stream);
    case 32: return launch_mfma_band_d<32>(Q, K, V, key_lengths, causal, radius, out, B, H, Lq, Lk, stream);
    case 64: return launch_mfma_band_d<64>(Q, K, V, key_lengths, causal, radius, out, B, H, Lq, Lk, stream);
    case 128: return launch_mfma_band_d<128>(Q, K, V, key_lengths, causal, radius, out, B, H, Lq, Lk, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mfma(const void *Q, const void *K, const void *V, const int32_t *key_lengths,
                       int causal, void *out, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int d,
                       bool streaming, hipStream_t stream)
{
    switch (d) {
    case 16: return launch_mfma_d<16>(Q, K, V, key_lengths, causal, out, B, H, Lq, Lk, streaming, stream);
    case 32: return launch_mfma_d<32>(Q, K, V, key_lengths, causal, out, B, H, Lq, Lk, streaming, stream);
    case 64: return launch_mfma_d<64>(Q, K, V, key_lengths, causal, out, B, H, Lq, Lk, streaming, stream);
    case 128: return launch_mfma_d<128>(Q, K, V, key_lengths, causal, out, B, H, Lq, Lk, streaming, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_merge(const float *ws, void *out, int64_t n_bh, int64_t Lq, int64_t n_split,
                               int d, hipStream_t stream)
{
    if (d == 64) return launch_merge_d<64>(ws, out, n_bh, Lq, n_split, stream);
    if (d == 128) return launch_merge_d<128>(ws, out, n_bh, Lq, n_split, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const void *Q, const void *K, const void *V, const int32_t *key_lengths,
                         void *out, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int d,
                         int64_t chunk, int64_t n_split, void *workspace, hipStream_t stream)
{
    switch (d) {
    case 64: return launch_decode_d<64>(Q, K, V, key_lengths, out, B, H, Lq, Lk, chunk, n_split, workspace, stream);
    case 128: return launch_decode_d<128>(Q, K, V, key_lengths, out, B, H, Lq, Lk, chunk, n_split, workspace, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace sdpa

#ifdef SDPA_TIMELINE
// Timeline build only: the records of this file's kernels (sdpa_timeline.h).
extern "C" int sdpa_timeline_fwd(void *host, int64_t bytes, int clear)
{
    return sdpa::timeline_io(host, bytes, clear);
}
#endif

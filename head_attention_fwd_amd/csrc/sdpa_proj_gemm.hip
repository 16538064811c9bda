// Projections of multi-head attention on the gfx950 matrix cores:
//
//   MultiHead(Q, K, V) = Concat(head_1, ..., head_h) W^O,
//   head_i = Attention(Q W_i^Q, K W_i^K, V W_i^V)
//
// (page "Attention Is All You Need/paper/es", §3.2.2).  Both kinds of
// projection are one product C[M, N] = A[M, K] W[K, N] over the M = B * L
// positions of a sequence, bf16 inputs, fp32 accumulation, bf16 result:
//
//  * input projections: A = the sequence [B, L, d_model] (row-major), W = the
//    h matrices W_i of one kind side by side, [d_model, h * d] (W_i in columns
//    i*d .. i*d + d - 1), and C written straight into the head-major layout
//    [B, h, L, d] that the attention kernels read (column n = i*d + t of C is
//    component t of head i).  Up to three such products that share A (Q, K and
//    V of self-attention) run as one launch, the output columns of the three
//    laid side by side;
//  * output projection: A = Concat(head_1, ..., head_h), read from the
//    attention's head-major output [B, h, L, d_v] (column k = i*d_v + t of the
//    concatenation is component t of head i), W = W^O [h * d_v, d_model], and
//    C = the result [B, L, d_model], row-major.
//
// Design (one workgroup = 4 waves and a 128 x 128 tile of C, or 8 waves and a
// 256 x 256 tile; k in steps of 32):
//  * Computed transposed, C^T = W^T A^T, one 32 x 32 block per MFMA chain
//    (v_mfma_f32_32x32x16_bf16): A operand = 32 columns n of W x 16 k, read
//    from a W tile kept as it sits in HBM ([k][n], n contiguous) with
//    ds_read_b64_tr_b16, which transposes 16-bit elements across 16 lanes; B
//    operand = 16 k x 32 rows m of A, read from an A tile kept as in HBM ([m][k]).
//    In the accumulator a lane holds one row m and, per block, 16 columns n in
//    runs of 4, so the result leaves through LDS as whole 128-byte rows.
//  * The waves form a 2 x GN grid over the tile, each wave WM x WN blocks
//    (2 x 2 or 4 x 2): WM * WN MFMAs per 16-k step, each W operand used WM
//    times and each A operand WN times.
//  * HBM -> LDS copies without registers (buffer_load ... lds), 16-byte chunks
//    XOR-swizzled by the row so that the operand reads are free of bank
//    conflicts; a ring of three buffers with two tiles in flight and one
//    barrier per tile, the k loop unrolled over the ring.  48 KiB of LDS
//    (three workgroups per CU) or 128 KiB (one; its output stage is the
//    largest part).
//  * Bounded buffer descriptors: rows of A past M read 0, stores past M or past
//    a product's N are dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sdpa_kernels.h"

constexpr int kBigTileWavesN = 4;   // waves along n in the large tile (8 waves, 256 x 256)
constexpr int kBigTileCount = 1024; // large tiles once a product has this many 256 x 128 tiles (else 128 x 128)

namespace sdpa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int BK = 32;
constexpr int kBuffers = 3;

// Tile shape: the waves form a 2 x GN grid (m x n), each wave WM x WN blocks of
// 32 x 32; the workgroup tile is BM x BN = 64*WM x 32*GN*WN.
template <int WM, int WN, int GN>
struct Tile {
    static constexpr int kWaves = 2 * GN;
    static constexpr int BM = 64 * WM, BN = 32 * GN * WN;
    static constexpr int kATileElems = BM * BK;     // [BM m][32 k]: 64-byte rows
    static constexpr int kWTileElems = BK * BN;     // [32 k][BN n]: 2*BN-byte rows
    static constexpr int kBufElems = kATileElems + kWTileElems;
    static constexpr int kASlices = kATileElems * 2 / 1024;   // 1 KiB copies per tile
    static constexpr int kWSlices = kWTileElems * 2 / 1024;
    static constexpr int kAPerWave = kASlices / kWaves, kWPerWave = kWSlices / kWaves;
    static constexpr int kCopiesPerWave = kAPerWave + kWPerWave;
    static constexpr int kWRowsPerSlice = 1024 / (2 * BN);
    static constexpr int kWChunks = BN / 8;         // 16-byte chunks per W row
    static constexpr int kStageElems = kWaves * 32 * WM * 32 * WN;   // output stage
    static constexpr int kLdsElems = kBuffers * kBufElems > kStageElems ? kBuffers * kBufElems : kStageElems;
    static_assert(kASlices % kWaves == 0 && kWSlices % kWaves == 0, "even copy split");
};

constexpr uint32_t kNoOffset = 0x7FFFFFF0u;     // past every descriptor bound: read 0 / store dropped
constexpr int kBufferRsrcWord3 = 0x00020000;

__device__ inline uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};   // nearest even
    return __builtin_bit_cast(uint32_t, v);
}
__device__ inline bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ inline u32x2_t ds_read_tr16_b64(const uint16_t *p)
{
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)p));
}
__device__ inline f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One wave-wide HBM -> LDS copy: lane L's 16 bytes at byte offset voff of the
// buffer land at LDS address dst + 16*L.  Inline assembly, untracked by the
// compiler: the kernel waits for these copies itself (vmcnt) before the barrier
// that publishes a tile.
__device__ inline void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc, const uint16_t *dst, uint32_t voff)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)dst);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(voff), "s"(rsrc) : "memory");
}

// s_waitcnt vmcnt(n), expcnt and lgkmcnt left at their maxima.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Chunk swizzles.  A tile rows (64 bytes, 4 chunks): rows r and r + 4 share
// banks, so the chunk index is XORed with (r / 4) % 4.  W tile rows (256 bytes):
// the 4 rows one transposing read touches get disjoint chunk pairs.
__device__ inline int swz_a(int row) { return (row >> 2) & 3; }
__device__ inline int swz_w(int row) { return (row & 3) << 1; }

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0,
                                             (int)(bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes)),
                                             kBufferRsrcWord3);
}

template <int AMODE, int CMODE, int WM, int WN, int GN>
__global__ __launch_bounds__(2 * GN * 64)
__attribute__((amdgpu_waves_per_eu(WM * WN > 4 ? 2 : 3, WM * WN > 4 ? 2 : 3)))
void proj_gemm_kernel(const uint16_t *__restrict__ A, GemmShape sh, GemmSegments segs)
{
    using T = Tile<WM, WN, GN>;
    constexpr int BM = T::BM, BN = T::BN, kATileElems = T::kATileElems, kBufElems = T::kBufElems;
    __shared__ __attribute__((aligned(16))) uint16_t lds[T::kLdsElems];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;      // the wave's part: 32*WM x 32*WN

    // Tile of this workgroup: each XCD (workgroup w goes to XCD w % 8) takes a
    // contiguous run of items, n fastest, so the workgroups reading one row
    // block of A share that XCD's L2.
    const uint32_t w = blockIdx.x;
    const uint32_t n_items = sh.n_mtiles * segs.n_ntiles;
    const uint32_t item = (n_items & 7) == 0 ? (w & 7) * (n_items >> 3) + (w >> 3) : w;
    const int64_t m0 = (int64_t)(item / segs.n_ntiles) * BM;
    int nt = (int)(item % segs.n_ntiles);
    int s = 0;
    while (s + 1 < segs.count && nt >= segs.seg[s].n_tiles) nt -= segs.seg[s++].n_tiles;
    const GemmSegment seg = segs.seg[s];
    const uint16_t *Wg = (const uint16_t *)seg.W;
    const int64_t n0 = (int64_t)nt * BN;
    const int64_t M = sh.M, K = sh.K, N = seg.N;

    // ---- copy offsets (fixed per lane; tiles move the descriptor base)
    // A tile: copy j of this wave fills rows 16*slice .. +15 (slice = kAPerWave*wave
    // + j), lane L -> row 16*slice + L/4, physical chunk L%4 (logical chunk
    // L%4 ^ swz_a(row)).
    uint32_t aoff[T::kAPerWave];
#pragma unroll
    for (int j = 0; j < T::kAPerWave; ++j) {
        const int row = 16 * (T::kAPerWave * wave + j) + (lane >> 2);
        const int lc = (lane & 3) ^ swz_a(row);
        const int64_t m = m0 + row;
        if constexpr (AMODE == 0) {
            aoff[j] = (uint32_t)((row * K + lc * 8) * 2);    // relative to A + m0*K + k0
        } else {
            // A(m, k) = heads[b][k / d][i][k % d], m = b * L + i: the row's
            // element offset in head 0, relative to the tile's head and k
            const int64_t b = m / sh.La, i = m % sh.La;
            const int64_t row_base = (b * sh.Ha * sh.La + i) * sh.da;
            aoff[j] = m < M ? (uint32_t)((row_base + lc * 8) * 2) : kNoOffset;
        }
    }
    // W tile: copy j of this wave fills rows R*slice .. +R-1 (k; R = 1024 / (2*BN)
    // rows per copy), lane L -> row R*slice + L/C, physical chunk L%C (C = BN/8
    // chunks per row; logical chunk L%C ^ swz_w(row)).
    uint32_t woff[T::kWPerWave];
#pragma unroll
    for (int j = 0; j < T::kWPerWave; ++j) {
        const int row = T::kWRowsPerSlice * (T::kWPerWave * wave + j) + lane / T::kWChunks;
        const int lc = (lane % T::kWChunks) ^ swz_w(row);
        woff[j] = (uint32_t)((row * N + lc * 8) * 2);          // relative to W + k0*N + n0
    }

    const int n_k = (int)((K + BK - 1) / BK);
    auto issue = [&](int t, int buf) {
        const int64_t k0 = (int64_t)t * BK;
        uint16_t *As = lds + buf * kBufElems;
        uint16_t *Ws = As + kATileElems;
        __amdgpu_buffer_rsrc_t ra;
        if constexpr (AMODE == 0) {
            const int64_t base = m0 * K + k0;
            ra = rsrc(A + base, (M * K - base) * 2);
        } else {
            // the 32 k of a tile lie in one head (d % 32 == 0)
            const int64_t head = k0 / sh.da, t0 = k0 % sh.da;
            const int64_t base = head * sh.La * sh.da + t0;
            ra = rsrc(A + base, sh.a_elems * 2 - base * 2);
        }
        const int64_t wbase = k0 * N + n0;
        const __amdgpu_buffer_rsrc_t rw = rsrc(Wg + wbase, (K * N - wbase) * 2);
#pragma unroll
        for (int j = 0; j < T::kAPerWave; ++j) copy_to_lds(ra, As + (T::kAPerWave * wave + j) * 512, aoff[j]);
#pragma unroll
        for (int j = 0; j < T::kWPerWave; ++j) copy_to_lds(rw, Ws + (T::kWPerWave * wave + j) * 512, woff[j]);
    };

    // ---- operand read offsets (bytes within a tile)
    // B operand (A^T): row 32*WM*wm + 32*mb + l32, logical chunk 2*kk + g.
    int boff[WM][2];
#pragma unroll
    for (int mb = 0; mb < WM; ++mb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int row = 32 * WM * wm + 32 * mb + l32;
            boff[mb][kk] = row * 64 + (((2 * kk + g) ^ swz_a(row)) << 4);
        }
    // A operand (W^T), transposing read: in 16-lane group G, lane i addresses
    // row 8*g + i/4 (+4 for the second read, +16*kk per 16-k step) and the 4
    // columns 32*nb' + 16*(G%2) + 4*(i%4) of the tile, nb' = WN*wn + nb; lane l
    // then holds column 32*nb' + l%32 at k = 16*kk + 8*g .. +7.
    int voff[WN];
    {
        const int i = lane & 15, G1 = (lane >> 4) & 1;
        const int row = 8 * g + (i >> 2);
#pragma unroll
        for (int nb = 0; nb < WN; ++nb) {
            const int col = 32 * (WN * wn + nb) + 16 * G1 + 4 * (i & 3);
            voff[nb] = 2 * (row * BN + ((((col >> 3) ^ swz_w(row))) << 3) + (col & 7));
        }
    }

    f32x16_t acc[WN][WM];
#pragma unroll
    for (int nb = 0; nb < WN; ++nb)
#pragma unroll
        for (int mb = 0; mb < WM; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.f;

    // One k-tile in LDS buffer BUF = t % 3 (instantiated per buffer, so that
    // every LDS operand address is a register plus an immediate).
    auto tile = [&](int t, auto buf_tag) {
        constexpr int BUF = decltype(buf_tag)::value;
        // Tile t has landed once at most tile t+1's copies are outstanding; the
        // barrier publishes it and retires every wave's reads of tile t-1, whose
        // buffer takes tile t+2.
        if (t + 1 < n_k) __builtin_amdgcn_s_waitcnt(waitcnt_vm(T::kCopiesPerWave));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();
        if (t + 2 < n_k) issue(t + 2, (BUF + 2) % kBuffers);
        const char *As = (const char *)(lds + BUF * kBufElems);
        const char *Ws = As + kATileElems * 2;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8_t bop[WM], aop[WN];
#pragma unroll
            for (int mb = 0; mb < WM; ++mb) bop[mb] = as_bf16x8(*(const u32x4_t *)(As + boff[mb][kk]));
#pragma unroll
            for (int nb = 0; nb < WN; ++nb) {
                const char *vb = Ws + voff[nb] + 16 * kk * BN * 2;
                const u32x2_t lo = ds_read_tr16_b64((const uint16_t *)vb);
                const u32x2_t hi = ds_read_tr16_b64((const uint16_t *)(vb + 4 * BN * 2));
                const u32x4_t a = {lo[0], lo[1], hi[0], hi[1]};
                aop[nb] = as_bf16x8(a);
            }
#pragma unroll
            for (int nb = 0; nb < WN; ++nb)
#pragma unroll
                for (int mb = 0; mb < WM; ++mb) acc[nb][mb] = mfma32(aop[nb], bop[mb], acc[nb][mb]);
        }
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using B2 = std::integral_constant<int, 2>;

    issue(0, 0);
    if (n_k > 1) issue(1, 1);
    // Unrolled over the ring (a branch on t % 3 per tile made the register
    // allocator copy the accumulators at every join: 6x slower).
    int t = 0;
    for (; t + 2 < n_k; t += 3) {
        tile(t, B0{});
        tile(t + 1, B1{});
        tile(t + 2, B2{});
    }
    if (t < n_k) tile(t++, B0{});
    if (t < n_k) tile(t++, B1{});

    // ---- epilogue: the wave's quarter through LDS (rows m of 64*WN bytes, chunks
    // XOR-swizzled by the row within each group of 8), then 16-byte stores of
    // whole chunks, 64 / (4*WN) rows per store.
    constexpr int kSC = 4 * WN;                   // 16-byte chunks per staged row
    constexpr int kSRows = 64 / kSC;              // rows per store instruction
    __syncthreads();                  // every wave is done with the tile buffers
    uint16_t *stage = lds + wave * (32 * WM) * (32 * WN);
#pragma unroll
    for (int nb = 0; nb < WN; ++nb)
#pragma unroll
        for (int mb = 0; mb < WM; ++mb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // acc[nb][mb][4q .. 4q+3]: row 32*mb + l32, columns 32*nb + 8*q + 4*g .. +3
                const int row = 32 * mb + l32;
                const int c = 4 * nb + q;
                u32x2_t v;
                v[0] = pack_bf16x2(acc[nb][mb][4 * q + 0], acc[nb][mb][4 * q + 1]);
                v[1] = pack_bf16x2(acc[nb][mb][4 * q + 2], acc[nb][mb][4 * q + 3]);
                *(u32x2_t *)((char *)stage + row * (16 * kSC) + ((c ^ (row & 7)) << 4) + 8 * g) = v;
            }
    const __amdgpu_buffer_rsrc_t rc = rsrc(seg.C, seg.c_elems * 2);
#pragma unroll
    for (int it = 0; it < 32 * WM / kSRows; ++it) {
        const int row = kSRows * it + lane / kSC, c = lane % kSC;
        const u32x4_t v = *(const u32x4_t *)((const char *)stage + row * (16 * kSC) + ((c ^ (row & 7)) << 4));
        const int64_t m = m0 + 32 * WM * wm + row;
        const int64_t n = n0 + 32 * WN * wn + 8 * c;
        uint32_t off = kNoOffset;
        if (m < M && n < N) {
            if constexpr (CMODE == 0) {
                off = (uint32_t)((m * N + n) * 2);
            } else {
                const int64_t b = m / sh.Lc, i = m % sh.Lc;
                const int64_t head = n / seg.d, tt = n % seg.d;
                off = (uint32_t)((((b * sh.Hc + head) * sh.Lc + i) * seg.d + tt) * 2);
            }
        }
        __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, 0);
    }
}

// Tile counts of one shape, then the launch.
template <int WM, int WN, int GN>
hipError_t launch_shape(const void *A, int a_mode, GemmShape shape, GemmSegments segs,
                        int c_mode, hipStream_t stream)
{
    using T = Tile<WM, WN, GN>;
    constexpr int kWaves = T::kWaves;
    shape.n_mtiles = (uint32_t)((shape.M + T::BM - 1) / T::BM);
    segs.n_ntiles = 0;
    for (int i = 0; i < segs.count; ++i) {
        segs.seg[i].n_tiles = (int)((segs.seg[i].N + T::BN - 1) / T::BN);
        segs.n_ntiles += (uint32_t)segs.seg[i].n_tiles;
    }
    const uint32_t grid = shape.n_mtiles * segs.n_ntiles;
    if (grid == 0) return hipSuccess;
    if (a_mode == 0 && c_mode == 1)
        hipLaunchKernelGGL((proj_gemm_kernel<0, 1, WM, WN, GN>), dim3(grid), dim3(kWaves * 64), 0, stream,
                           (const uint16_t *)A, shape, segs);
    else if (a_mode == 1 && c_mode == 0)
        hipLaunchKernelGGL((proj_gemm_kernel<1, 0, WM, WN, GN>), dim3(grid), dim3(kWaves * 64), 0, stream,
                           (const uint16_t *)A, shape, segs);
    else if (a_mode == 0 && c_mode == 0)
        hipLaunchKernelGGL((proj_gemm_kernel<0, 0, WM, WN, GN>), dim3(grid), dim3(kWaves * 64), 0, stream,
                           (const uint16_t *)A, shape, segs);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

// Tile shape by problem size: once there would be at least 1024 tiles of
// 256 x 128, one 8-wave workgroup per CU on 256 x 256 tiles (each wave 4 x 2
// blocks: 0.75 KiB of LDS reads per MFMA instead of 1 KiB, and each A and W
// tile copied into LDS serves twice the columns); smaller products keep
// 128 x 128 tiles (three 4-wave workgroups per CU, more tiles to spread).
// Measured on MI355X: 32768 x 1024 x 3072 took 251 us on 128 x 128 tiles,
// 224 us on 256 x 128 (4 waves) and 209 us on 256 x 256 (8 waves);
// 16384 x 512 x 1536 (768 tiles of 256 x 128) 36.4 us on 128 x 128 tiles
// against 38.1 us on 256 x 128.
hipError_t launch_proj_gemm(const void *A, int a_mode, const GemmShape &shape,
                            const GemmSegments &segs, int c_mode, hipStream_t stream)
{
    int64_t big_tiles = 0;
    for (int i = 0; i < segs.count; ++i) big_tiles += (segs.seg[i].N + 127) / 128;
    big_tiles *= (shape.M + 255) / 256;
    if (big_tiles >= kBigTileCount)
        return launch_shape<4, 2, kBigTileWavesN>(A, a_mode, shape, segs, c_mode, stream);
    return launch_shape<2, 2, 2>(A, a_mode, shape, segs, c_mode, stream);
}

}  // namespace sdpa

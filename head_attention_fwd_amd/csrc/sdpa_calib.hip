// Calibration kernels for the measurement of the attention kernels (built into
// libsdpa_calib.so, separate from libsdpa; bench.py --overlap-probe).  Not part
// of the attention path.
//
// Overlap probe: how much of a matrix-core stream and a vector-ALU stream run
// at the same time when they come from different waves on one SIMD.  One
// workgroup of 8 waves per CU (two waves per SIMD): waves 0-3 issue
// v_mfma_f32_32x32x16_bf16 on four independent accumulators, waves 4-7 issue
// independent fp32 FMAs, 8 per MFMA (the ratio of the d = 64 softmax's VALU
// instructions to its MFMAs).  Launched with the matrix stream only, the
// vector stream only, or both; the accumulators of the matrix stream live in
// ordinary VGPRs (mode 0) or in the accumulation registers (mode 1).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int MODE, bool DO_M, bool DO_V>
__global__ __launch_bounds__(512) void overlap_probe_kernel(float *out, int iters)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float r = 0.f;
    if (wave < 4) {
        if (DO_M) {
            bf16x8_t a, b;
            for (int i = 0; i < 8; ++i) {
                a[i] = (__bf16)(0.001f * (lane + i));
                b[i] = (__bf16)(0.002f * (lane - i));
            }
            f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
            for (int it = 0; it < iters; ++it) {
                if constexpr (MODE == 0) {
                    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
                    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
                    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
                    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
                } else {
                    // each accumulator is read again four MFMAs later, far more
                    // than the dependency distance the matrix core needs
                    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c0) : "v"(a), "v"(b));
                    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c1) : "v"(a), "v"(b));
                    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c2) : "v"(a), "v"(b));
                    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c3) : "v"(a), "v"(b));
                }
            }
            if constexpr (MODE != 0) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
            for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
        }
    } else if (DO_V) {
        float x[16];
        for (int i = 0; i < 16; ++i) x[i] = 1.0f + 1e-6f * (lane + i);
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int i = 0; i < 16; ++i) x[i] = __builtin_fmaf(x[i], 0.9999f, 1e-7f);
        }
        for (int i = 0; i < 16; ++i) r += x[i];
    }
    out[blockIdx.x * 512 + threadIdx.x] = r;
}

template <int MODE, bool M, bool V>
hipError_t launch(float *out, int n_wg, int iters, hipStream_t s)
{
    hipLaunchKernelGGL((overlap_probe_kernel<MODE, M, V>), dim3(n_wg), dim3(512), 0, s, out, iters);
    return hipGetLastError();
}

}  // namespace

extern "C" {

// which: 0 matrix stream only, 1 vector stream only, 2 both; mode: 0 VGPR
// accumulators, 1 accumulation registers.  out: device float[n_wg * 512].
// Returns a hipError_t (0 on success); the launch goes on `stream`.
int sdpa_calib_overlap(int mode, int which, float *out, int n_wg, int iters, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    if (!out || n_wg < 1 || iters < 1 || mode < 0 || mode > 1 || which < 0 || which > 2)
        return (int)hipErrorInvalidValue;
    if (mode == 0)
        return (int)(which == 0 ? launch<0, true, false>(out, n_wg, iters, s)
                                : which == 1 ? launch<0, false, true>(out, n_wg, iters, s)
                                             : launch<0, true, true>(out, n_wg, iters, s));
    return (int)(which == 0 ? launch<1, true, false>(out, n_wg, iters, s)
                            : which == 1 ? launch<1, false, true>(out, n_wg, iters, s)
                                         : launch<1, true, true>(out, n_wg, iters, s));
}

}  // extern "C"

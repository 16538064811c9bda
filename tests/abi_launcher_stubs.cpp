// Test infrastructure: stand-ins for libsdpa's kernel launchers, so that the
// host layer (head_attention_fwd_amd/csrc/sdpa_api.hip: argument checks,
// planning, the scratch lookup) can be built alone with host sanitizers and
// driven by the CPU tests.  Every stand-in counts its call and returns an
// error; the tests require that no call reached one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdpa_kernels.h"

namespace {
int g_launches = 0;
hipError_t counted()
{
    ++g_launches;
    return hipErrorInvalidDeviceFunction;
}
}  // namespace

namespace sdpa {

hipError_t launch_generic(const void *, const void *, const void *, const int32_t *, int, int64_t,
                          void *, int64_t, int64_t, int64_t, int64_t, int, int, bool, hipStream_t)
{
    return counted();
}
hipError_t launch_mfma(const void *, const void *, const void *, const int32_t *, int, void *,
                       int64_t, int64_t, int64_t, int64_t, int, bool, hipStream_t)
{
    return counted();
}
hipError_t launch_mfma_wide(const void *, const void *, const void *, const int32_t *, int, void *,
                            int64_t, int64_t, int64_t, int64_t, int, bool, hipStream_t)
{
    return counted();
}
hipError_t launch_mfma_band(const void *, const void *, const void *, const int32_t *, int, int64_t,
                            void *, int64_t, int64_t, int64_t, int64_t, int, hipStream_t)
{
    return counted();
}
hipError_t launch_decode(const void *, const void *, const void *, const int32_t *, void *, int64_t,
                         int64_t, int64_t, int64_t, int, int64_t, int64_t, void *, hipStream_t)
{
    return counted();
}
hipError_t launch_decode_row(const void *, const void *, const void *, const int32_t *, void *, int64_t,
                             int64_t, int64_t, int, int, int64_t, int64_t, void *, hipStream_t)
{
    return counted();
}
hipError_t launch_decode_merge(const float *, void *, int64_t, int64_t, int64_t, int, hipStream_t)
{
    return counted();
}
hipError_t launch_proj_gemm(const void *, int, const GemmShape &, const GemmSegments &, int, hipStream_t)
{
    return counted();
}

}  // namespace sdpa

extern "C" int sdpa_test_stub_launches(void) { return g_launches; }

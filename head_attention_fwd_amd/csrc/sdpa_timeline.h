// Per-workgroup timeline of a launch, for the timeline build of the library
// (libsdpa_timeline.so, compiled with SDPA_TIMELINE; the normal build compiles
// every stamp out).
//
// Lane 0 of wave 0 of workgroup w writes the GPU's 100 MHz real-time counter
// (s_memrealtime, one clock for the whole device) at four points of the
// workgroup's life into slot [w][e]:
//   e = 0  entry
//   e = 1  the first key tile (or step) in registers / LDS and usable
//   e = 2  the last key tile done
//   e = 3  output stores issued
// Each instrumented source has its own buffer (kTimelineWorkgroups x 4 records)
// and its own reader; a launch overwrites the records of its workgroups.  The
// stamps wait for the wave's outstanding scalar and LDS operations
// (s_memrealtime returns through the scalar data path), so the timeline build
// runs slightly slower than the normal one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

constexpr int kTimelineEvents = 4;
constexpr uint32_t kTimelineWorkgroups = 1u << 16;
constexpr int64_t kTimelineBytes = (int64_t)sizeof(unsigned long long) * kTimelineWorkgroups * kTimelineEvents;

}  // namespace sdpa

#ifdef SDPA_TIMELINE

namespace sdpa {
namespace {
__device__ unsigned long long g_timeline[kTimelineWorkgroups * kTimelineEvents];

// clear != 0: set every record to 0; else copy the first `bytes` bytes of the
// records to host memory.  Returns a hipError_t.
inline int timeline_io(void *host, int64_t bytes, int clear)
{
    if (clear) {
        void *p = nullptr;
        hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(g_timeline));
        if (err == hipSuccess) err = hipMemset(p, 0, (size_t)kTimelineBytes);
        return (int)err;
    }
    if (!host || bytes < 0 || bytes > kTimelineBytes) return (int)hipErrorInvalidValue;
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_timeline), (size_t)bytes, 0, hipMemcpyDeviceToHost);
}
}  // namespace
}  // namespace sdpa

#define SDPA_STAMP(e)                                                                                  \
    do {                                                                                               \
        if (threadIdx.x == 0 && blockIdx.x < ::sdpa::kTimelineWorkgroups)                              \
            ::sdpa::g_timeline[(size_t)blockIdx.x * ::sdpa::kTimelineEvents + (e)] =                   \
                __builtin_amdgcn_s_memrealtime();                                                      \
    } while (0)

#else

#define SDPA_STAMP(e) ((void)0)

#endif

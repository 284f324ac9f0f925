// Stand-ins for the HIP runtime and the kernel launchers, for the sanitizer build of
// the library's host code (planner and C ABI): the host-only paths the test program takes
// make no HIP call, and each stand-in counts any call that happens anyway and fails
// it, so the test program can check that none did.
#include <hip/hip_runtime.h>

#include "rpa_launch.h"

int g_hip_calls = 0;

namespace {
hipError_t called() {
    ++g_hip_calls;
    return hipErrorNotSupported;
}
}  // namespace

const char* hipGetErrorString(hipError_t) { return "stand-in: no HIP runtime in the sanitizer build"; }
hipError_t hipStreamSynchronize(hipStream_t) { return called(); }
hipError_t hipEventCreate(hipEvent_t*) { return called(); }
hipError_t hipEventSynchronize(hipEvent_t) { return called(); }
hipError_t hipEventElapsedTime(float*, hipEvent_t, hipEvent_t) { return called(); }
hipError_t hipHostMalloc(void**, size_t, unsigned int) { return called(); }
hipError_t hipHostFree(void*) { return called(); }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { return called(); }

namespace rpa {
hipError_t launch_wide(const LaunchAttn&, hipStream_t, hipEvent_t, hipEvent_t) { return called(); }
hipError_t launch_narrow(const LaunchAttn&, hipStream_t, hipEvent_t, hipEvent_t) { return called(); }
hipError_t launch_mixed(const LaunchAttn&, hipStream_t, hipEvent_t, hipEvent_t) { return called(); }
hipError_t launch_narrow_valu(const LaunchAttn&, int, hipStream_t, hipEvent_t, hipEvent_t) { return called(); }
hipError_t launch_merge(const MergeArgs&, bool, hipStream_t) { return called(); }
hipError_t launch_append(const AppendArgs&, hipStream_t) { return called(); }
hipError_t launch_clear(int32_t*, int64_t, hipStream_t) { return called(); }
hipError_t static_scratch(void**) { return called(); }
}  // namespace rpa

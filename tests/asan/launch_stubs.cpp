// Host-only stand-ins for the kernel launchers and the three HIP runtime calls
// that api.cpp makes, so that api.cpp (argument checks, launch planning,
// workspace layout, the page allocator) can be built with AddressSanitizer by
// g++ and driven by the ABI tests on a machine without a GPU. Each launcher
// only counts its calls; spa_test_launch_count() lets a test check that a
// failing call enqueued nothing.
#include <hip/hip_runtime.h>

#include "../../sparse_paged_attention_amd/csrc/spa_internal.h"

static int g_launches = 0;

extern "C" int spa_test_launch_count(void) { return g_launches; }

extern "C" hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
extern "C" hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

namespace spa {
hipError_t scratch_area(void** ptr, size_t* bytes) {
  *ptr = reinterpret_cast<void*>(uintptr_t(0x2000));   // never dereferenced on the host
  *bytes = kScratchBytes;
  return hipSuccess;
}
hipError_t launch_append(const PoolArgs&, const BatchArgs&, const uint16_t*, const uint16_t*, const HeadList*,
                         hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_write(const PoolArgs&, const int32_t*, int64_t, int64_t, const uint16_t*, const uint16_t*,
                        const HeadList*, int32_t, int32_t, int32_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_summary(const PoolArgs&, const BatchArgs&, const HeadList&, const int32_t*, int32_t,
                          hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_select(const PoolArgs&, const BatchArgs&, const HeadList&, int32_t, const uint16_t*,
                         const int32_t*, int32_t, int32_t*, int32_t*, int32_t*, int32_t*, float*, int32_t,
                         const uint16_t*, const uint16_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_attn(const PoolArgs&, const BatchArgs&, const AttnPlan&, int32_t, const uint16_t*,
                       const int32_t*, const int32_t*, const int32_t*, const int32_t*, float*, float*, float*,
                       float*, const uint16_t*, const uint16_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace spa

// The read probe lives in its own kernel file; a stand-in keeps the export list whole.
extern "C" int spa_probe_read_chunks(const void*, size_t, const int32_t*, int32_t, int32_t, uint32_t*,
                                     hipStream_t) {
  ++g_launches;
  return 0;
}

// Host-only stand-ins for the HIP runtime calls and the kernel launches that
// pkv_host.cpp makes, so the host layer can be built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer and driven without a GPU.
// Host memory stands for device memory: a "device" copy is a memcpy, and a
// launch only counts itself (the driver checks that calls refused on the
// host launch nothing).
#include <cstring>

#include "pkv_internal.h"

int g_launches = 0;

extern "C" {
const char* hipGetErrorString(hipError_t) { return "stub HIP runtime"; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipHostGetDevicePointer(void** dev, void* host, unsigned int) {
  *dev = host;
  return hipSuccess;
}
}

namespace pkv {
static hipError_t count() {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_kv_write(const CacheDesc&, const void*, const void*, const int64_t*, int64_t,
                           hipStream_t) { return count(); }
hipError_t launch_block_copy(const CacheDesc&, const int64_t*, int64_t, hipStream_t) { return count(); }
hipError_t launch_block_swap(const CacheDesc&, char*, const int64_t*, int64_t, bool, hipStream_t) {
  return count();
}
hipError_t launch_read_slices(const CacheDesc&, const int64_t*, int64_t, int, uint32_t*,
                              hipStream_t) { return count(); }
hipError_t launch_decode_rows(const CacheDesc&, const AttnDesc& a, hipStream_t) {
  // the stream decode's ranges live in the workspace the host laid out
  if (a.stream_waves > 0 && a.stream_acc) a.stream_acc[0] = 0.f;
  return count();
}
hipError_t launch_prefill_rows(const CacheDesc&, const AttnDesc&, hipStream_t) { return count(); }
hipError_t launch_mixed_rows(const CacheDesc&, const AttnDesc&, hipStream_t) { return count(); }
bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }
int decode_stream_slots(int, int, int) { return 2048; }
int device_cus() { return 256; }
static char g_scratch[kNoAllocScratchBytes];
hipError_t noalloc_scratch(char** ptr) {
  *ptr = g_scratch;
  return hipSuccess;
}
}  // namespace pkv

// Host-only stand-in for the HIP runtime calls that the library's host code makes, so that
// code can be built with AddressSanitizer and UndefinedBehaviorSanitizer and driven on a
// machine without a GPU.
//
// "Device" buffers are plain host allocations.  Copies and fills act on them directly, so
// the sanitizer checks every extent the library computes for them.  Kernel launches are
// recorded and checked against the launch limits of the hardware, and nothing runs.  Kernel
// registration is accepted and ignored.  One stream (the null stream) and no devices
// beyond device 0 exist.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstring>
#include <vector>

#include "sim_runtime.h"

namespace {

struct Config {
  dim3 grid, block;
  size_t shmem;
  hipStream_t stream;
};

std::vector<sim::Launch> g_launches;
std::vector<Config> g_configs;  // pushed by the <<<...>>> form, popped by the launch stub
hipError_t g_last = hipSuccess;
int g_bad = 0;

// A static pool of events: the library keeps its timing events for the life of the process.
constexpr int kEvents = 4096;
unsigned char g_event_pool[kEvents];
int g_events_used = 0;

bool dim_ok(const dim3& d, uint32_t max_y_z) { return d.x >= 1 && d.y >= 1 && d.z >= 1 && d.y <= max_y_z && d.z <= max_y_z; }

hipError_t record(const void* fn, dim3 grid, dim3 block, size_t shmem) {
  sim::Launch L{fn, grid, block, shmem, true};
  const uint64_t threads = (uint64_t)block.x * block.y * block.z;
  // per dimension the work-item count (blocks x threads) is a 32-bit quantity
  const bool ok = dim_ok(grid, 65535u) && dim_ok(block, 1024u) && threads <= 1024 &&
                  (uint64_t)grid.x * block.x <= 0xFFFFFFFFull && (uint64_t)grid.y * block.y <= 0xFFFFFFFFull &&
                  (uint64_t)grid.z * block.z <= 0xFFFFFFFFull && shmem <= 160 * 1024;
  L.ok = ok;
  g_launches.push_back(L);
  if (!ok) {
    ++g_bad;
    g_last = hipErrorInvalidConfiguration;
    return hipErrorInvalidConfiguration;
  }
  return hipSuccess;
}

}  // namespace

namespace sim {
size_t launches() { return g_launches.size(); }
const Launch& launch(size_t i) { return g_launches[i]; }
int bad_launches() { return g_bad; }
}  // namespace sim

extern "C" {

void** __hipRegisterFatBinary(const void*) {
  static void* handle = nullptr;
  return &handle;
}
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterFunction(void**, const void*, char*, const char*, unsigned int, void*, void*, dim3*, dim3*, int*) {}
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}

hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t shmem, hipStream_t stream) {
  g_configs.push_back(Config{grid, block, shmem, stream});
  return hipSuccess;
}
hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* shmem, hipStream_t* stream) {
  if (g_configs.empty()) return hipErrorInvalidConfiguration;
  const Config c = g_configs.back();
  g_configs.pop_back();
  *grid = c.grid;
  *block = c.block;
  *shmem = c.shmem;
  *stream = c.stream;
  return hipSuccess;
}

hipError_t hipLaunchKernel(const void* fn, dim3 grid, dim3 block, void**, size_t shmem, hipStream_t) {
  return record(fn, grid, block, shmem);
}
hipError_t hipExtLaunchKernel(const void* fn, dim3 grid, dim3 block, void**, size_t shmem, hipStream_t, hipEvent_t,
                              hipEvent_t, int) {
  return record(fn, grid, block, shmem);
}

hipError_t hipGetLastError(void) {
  const hipError_t e = g_last;
  g_last = hipSuccess;
  return e;
}
hipError_t hipGetDevice(int* device) {
  if (!device) return hipErrorInvalidValue;
  *device = 0;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** ptr, const void* symbol) {
  if (!ptr || !symbol) return hipErrorInvalidSymbol;
  *ptr = const_cast<void*>(symbol);  // the host copy of the variable stands for it
  return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  if (n && (!dst || !src)) return hipErrorInvalidValue;
  if (n) std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipMemsetAsync(void* dst, int value, size_t n, hipStream_t) {
  if (n && !dst) return hipErrorInvalidValue;
  if (n) std::memset(dst, value, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned) {
  if (!event) return hipErrorInvalidValue;
  if (g_events_used == kEvents) return hipErrorOutOfMemory;
  *event = reinterpret_cast<hipEvent_t>(&g_event_pool[g_events_used++]);
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  if (!ms) return hipErrorInvalidValue;
  *ms = 0.001f;
  return hipSuccess;
}

}  // extern "C"

// The forward for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid it): qlora_linear_fwd with its workspace taken
// from a fixed array that the library holds on each device, instead of a caller's buffer.
//
// The array holds what a workspace holds: the arrival counters of the split reductions in
// its first QLORA_WS_COUNTER_BYTES (zero between calls; zeroed once at set-up), then the
// FP32 partials and the BF16 adapter intermediate of the call.  Calls whose workspace need
// exceeds its size are refused before anything is launched.  Every call on a device shares
// that device's array, so calls that overlap on one device (two streams at once) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qlora_host.h"

namespace {

constexpr size_t kScratchBytes = QLORA_NOALLOC_SCRATCH_BYTES;

// Device memory for the calls of this entry point; each device holds its own copy until the
// process ends.  Host code reaches it only through the address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {nullptr};

// The device address of `scratch` on the current device.  The first call on a device looks
// it up (with that device current) and zeroes its counter head on `stream`; later calls
// return the kept address.
void* scratch_on_current_device(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    if (qlora::launch_zero_words(static_cast<unsigned int*>(ptr), (int64_t)(QLORA_WS_COUNTER_BYTES / 4), stream) !=
        hipSuccess)
      return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int qlora_linear_fwd_noalloc(const qlora_nf4dq_t* Wq, const uint16_t* X, int64_t M, const uint16_t* A,
                                        const uint16_t* B, int32_t r, float alpha, uint16_t* Y, uint16_t* T_save,
                                        hipStream_t stream) {
  int st = qlora::fwd_validate(Wq, X, M, A, B, r, alpha, Y);
  if (st) return st;
  if (qlora::fwd_workspace_bytes(M, Wq->d_out, Wq->d_in, r, Wq->dq_format) > kScratchBytes)
    return QLORA_ERR_SCRATCH;
  void* ws = scratch_on_current_device(stream);
  if (!ws) return QLORA_ERR_HIP;
  qlora::TimingOff no_events;  // timing events would be created (allocated) on first use
  return qlora::fwd_enqueue(Wq, X, M, A, B, r, alpha, Y, T_save, ws, stream);
}

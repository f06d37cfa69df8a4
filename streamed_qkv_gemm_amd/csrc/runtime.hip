// Host-side HIP runtime calls the C-ABI layer needs besides kernel launches: the
// error text of a status, the asynchronous copies that move packed K/V blocks
// between pinned host memory and device staging buffers, the events that order
// those copies, on a stream of their own, against the kernels, and the device
// scratch of the allocation-free Q-recompute entry point.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace sqg {

// One chunk of recomputed bf16 Q for callers that cannot allocate: a file-scope device
// array that each GPU the library runs on holds until the process ends.  Host code never
// uses the array's name as an address (on the host it is a stand-in, not device memory):
// the device address comes from hipGetSymbolAddress, looked up once per device with that
// device current.
__device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int scratch_for_current_device(void** ptr) {
  int dev = 0;
  hipError_t r = hipGetDevice(&dev);
  if (r != hipSuccess) return (int)r;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r != hipSuccess) return (int)r;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

const char* hip_error_text(int err) { return hipGetErrorString((hipError_t)err); }

int copy_async(void* dst, const void* src, int64_t bytes, CopyKind kind, void* stream) {
  if (bytes <= 0) return 0;
  const hipMemcpyKind k = kind == kHostToDevice ? hipMemcpyHostToDevice : hipMemcpyDeviceToHost;
  return (int)hipMemcpyAsync(dst, src, (size_t)bytes, k, (hipStream_t)stream);
}

int event_create(void** ev) {
  hipEvent_t e = nullptr;
  const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
  *ev = r == hipSuccess ? static_cast<void*>(e) : nullptr;
  return (int)r;
}

int event_destroy(void* ev) { return ev ? (int)hipEventDestroy(static_cast<hipEvent_t>(ev)) : 0; }

int event_record(void* ev, void* stream) {
  return (int)hipEventRecord(static_cast<hipEvent_t>(ev), static_cast<hipStream_t>(stream));
}

int stream_wait_event(void* stream, void* ev) {
  return (int)hipStreamWaitEvent(static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(ev), 0);
}

}  // namespace sqg

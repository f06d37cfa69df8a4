// Host-side HIP runtime calls the C-ABI layer needs besides kernel launches: the
// error text of a status, the asynchronous copies that move packed K/V blocks
// between pinned host memory and device staging buffers, and the events that order
// those copies, on a stream of their own, against the kernels.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace sqg {

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

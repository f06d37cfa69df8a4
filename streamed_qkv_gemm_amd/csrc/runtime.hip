// Host-side HIP runtime calls the C-ABI layer needs besides kernel launches: the
// error text of a status and the asynchronous copies that move packed K/V blocks
// between pinned host memory and device staging buffers.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace sqg {

const char* hip_error_text(int err) { return hipGetErrorString((hipError_t)err); }

int copy_async(void* dst, const void* src, int64_t bytes, CopyKind kind, void* stream) {
  if (bytes <= 0) return 0;
  const hipMemcpyKind k = kind == kHostToDevice ? hipMemcpyHostToDevice : hipMemcpyDeviceToHost;
  return (int)hipMemcpyAsync(dst, src, (size_t)bytes, k, (hipStream_t)stream);
}

}  // namespace sqg

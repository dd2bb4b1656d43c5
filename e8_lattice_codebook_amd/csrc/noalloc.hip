// glq_e8rht_linear_noalloc: the E8RHTLinear forward with its workspace in a
// file-scope device array instead of a caller's buffer, for callers that cannot
// allocate (code under graph capture, serving loops, harnesses that forbid
// hipMalloc).  Nothing here allocates: the array is part of the library's code
// object, one copy per device, reserved when the library is loaded on that device.
#include <atomic>

#include "internal.h"

namespace {

// the workspace of every call on this device; its address on each device is looked
// up once and kept (the name itself is a host-side stand-in, never a device address)
__device__ __attribute__((aligned(256))) unsigned char scratch[GLQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];

// the device address of this device's `scratch`, or NULL when it cannot be had
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  // threads racing on a device's first call each look the same address up
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" glq_status glq_e8rht_linear_noalloc(const glq_layer* layer, const void* x, glq_dtype x_dt, int64_t B,
                                               void* y, glq_dtype y_dt, hipStream_t stream) {
  if (!layer) return GLQ_ERR_NULL;
  if (B < 1) return GLQ_ERR_SHAPE;
  const size_t need = glq_e8rht_linear_workspace_bytes(layer, B);
  if (need > size_t(GLQ_NOALLOC_SCRATCH_BYTES)) return GLQ_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (!ws) return GLQ_ERR_HIP;
  // the linear validates everything else before it launches anything; its workspace
  // is plain scratch (no initial contents), so what an earlier call left is harmless
  return glq_e8rht_linear(layer, x, x_dt, B, y, y_dt, ws, size_t(GLQ_NOALLOC_SCRATCH_BYTES), stream);
}

namespace glq {
GLQ_DEBUG_COUNTER(debug_violations_noalloc)
}  // namespace glq

// ssd_forward without an allocation or a workspace argument: the stage-1
// outputs g and dt_t (the only scratch the forward pass needs) live in a
// fixed device array of this library, one copy per GPU, instead of in a
// caller-provided workspace.  For callers that cannot allocate device
// memory (code under graph capture, tight serving loops).
//
// The array's address is taken once per device, with that device current,
// and kept; kernels receive that address, never the array's host-side name.
// Every call on a GPU shares that GPU's array: calls that overlap in time on
// one GPU (different streams, or different host threads without ordering)
// race on it.  Nothing in it needs to start at zero: stage 1 writes every
// element stages 2 and 3 read.
#include "ssd_device.h"
#include "ssd_host.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

// Device address of `scratch` on each device, taken on first use.
struct ScratchAddress {
  std::atomic<uintptr_t> slot[kMaxDevices];
};
ScratchAddress g_scratch;

// The device address of this device's scratch array, or 0 on failure.
uintptr_t scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  uintptr_t p = dev < kMaxDevices ? g_scratch.slot[dev].load(std::memory_order_acquire) : 0;
  if (p != 0) return p;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
    clear_launch_error();
    return 0;
  }
  p = reinterpret_cast<uintptr_t>(ptr);
  if (dev < kMaxDevices) g_scratch.slot[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

int launch_forward_noalloc(const void* x, const float* dt, const float* A, const void* B,
                           const void* C, const float* D, const float* init_state, void* y,
                           float* states, float* final_state, bool bf16_in, bool bf16_out,
                           const Shape& s, void* stream) {
  const size_t n = (size_t)s.batch * (size_t)s.nheads * (size_t)s.seqlen;
  if (2 * sizeof(float) * n > kNoallocScratchBytes) return (int)hipErrorInvalidValue;
  const uintptr_t base = scratch_address();
  if (base == 0) return (int)hipErrorInvalidSymbol;
  float* g = reinterpret_cast<float*>(base);
  float* dt_t = g + n;
  int err = launch_chunk_cumsum(dt, A, g, dt_t, s, stream);
  if (err == 0)
    err = launch_state_and_out(x, B, C, dt_t, g, D, init_state, states, final_state, y, bf16_in,
                               bf16_out, s, stream);
  return err;
}

}  // namespace ssd

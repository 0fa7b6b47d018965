// moe_layer_forward_noalloc: the layer call for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  Its workspace is a fixed array in the library's
// own device memory instead of a caller buffer; everything else is
// moe_layer_forward, kernels included.
//
// The array is a file-scope __device__ variable: every GPU the library runs on
// holds its own copy (MOE_NOALLOC_SCRATCH_BYTES) until the process ends.  In
// host code its name is not a device address, so the address is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// only that pointer is ever handed to kernels.  No call here allocates or
// frees anything.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte units");

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of this device's copy of `scratch`, or nullptr (with
// *err set) when it cannot be resolved.
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !p) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

MOE_API int moe_layer_forward_noalloc(const moe_dims* dims, const void* x, int x_dtype, int32_t T,
                                      const float* w_router, const float* bias,
                                      const void* const* expert_table, float* out, uint32_t flags,
                                      float rms_eps, int32_t* stats, void* stream) {
  // size checks first: moe_workspace_bytes validates the dims, and a call
  // too large for the array is refused before any HIP call
  if (T < 1) return MOE_EINVAL;
  const size_t need = moe_workspace_bytes(dims, T);
  if (need == 0) {
    // invalid dims: let the layer call's own validation name the error
    return moe_layer_forward(dims, x, x_dtype, T, w_router, bias, expert_table, out, flags,
                             rms_eps, stats, nullptr, 0, stream);
  }
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ENOSPC;
  hipError_t err = hipSuccess;
  void* ws = scratch_on_current_device(&err);
  if (!ws) {
    (void)hipGetLastError();  // reported through the status and moe_strerror instead
    return moe::hip_error_status(err);
  }
  return moe_layer_forward(dims, x, x_dtype, T, w_router, bias, expert_table, out, flags, rms_eps,
                           stats, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

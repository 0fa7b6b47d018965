// Phase trace of the kernels' workgroups: measurement, not part of the layer.
//
// Built into lib/libmoe_trace.so only (the build defines MOE_PHASE_TRACE);
// in libmoe.so every mark below compiles to nothing.  A traced workgroup
// keeps, in registers, the device's 100 MHz clock (s_memrealtime: one counter
// for the whole chip, so workgroups can be placed on one time line) at its
// start, at up to five points named by the kernel, and at its end, and its
// first thread writes them, with the compute unit it ran on and a tag, into
// the record of its workgroup index (modulo kTraceBlocks) in a device array of
// its source file.  moe_trace_read (include/moe.h) copies a kernel's records
// out.  Records persist until a later launch of the same kernel overwrites
// them or moe_trace_reset clears them.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

constexpr int kTraceBlocks = 32768;  // records per traced kernel
constexpr int kTraceWords = 8;       // start, points 1..5, end, (compute unit << 8) | tag

#ifdef MOE_PHASE_TRACE
constexpr bool kTrace = true;
struct BlockTrace {
  unsigned long long t[kTraceWords - 1] = {};
  __device__ __forceinline__ void start() { t[0] = __builtin_amdgcn_s_memrealtime(); }
  __device__ __forceinline__ void mark(int i) { t[i] = __builtin_amdgcn_s_memrealtime(); }
  // the workgroup's first thread writes the record (every thread may call)
  __device__ __forceinline__ void store(unsigned long long* arr, int slot, unsigned block,
                                        int tag) {
    if (threadIdx.x != 0) return;
    unsigned long long* r =
        arr + ((size_t)slot * kTraceBlocks + block % kTraceBlocks) * kTraceWords;
    const unsigned long long end = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < kTraceWords - 2; ++i) r[i] = t[i];
    r[kTraceWords - 2] = end;
    r[kTraceWords - 1] = ((unsigned long long)__smid() << 8) | (unsigned)tag;
  }
};
// One array per source file (device globals are not shared across files
// here), with its copy-out and reset for the host.
#define MOE_TRACE_STORAGE(name, slots)                                                      \
  __device__ unsigned long long name[(slots) * kTraceBlocks * kTraceWords];                \
  static hipError_t name##_read(int slot, void* dst, size_t bytes) {                        \
    if (slot < 0 || slot >= (slots) ||                                                     \
        bytes > sizeof(unsigned long long) * kTraceBlocks * kTraceWords)                   \
      return hipErrorInvalidValue;                                                         \
    return hipMemcpyFromSymbol(dst, HIP_SYMBOL(name), bytes,                               \
                               (size_t)slot * kTraceBlocks * kTraceWords * 8,              \
                               hipMemcpyDeviceToHost);                                     \
  }                                                                                        \
  static hipError_t name##_reset() {                                                        \
    void* p = nullptr;                                                                     \
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(name));                              \
    if (e == hipSuccess) e = hipMemset(p, 0, sizeof(name));                                \
    return e;                                                                              \
  }
#else
constexpr bool kTrace = false;
struct BlockTrace {
  __device__ __forceinline__ void start() {}
  __device__ __forceinline__ void mark(int) {}
  __device__ __forceinline__ void store(unsigned long long*, int, unsigned, int) {}
};
#define MOE_TRACE_STORAGE(name, slots)                                                      \
  constexpr unsigned long long* name = nullptr;                                            \
  static hipError_t name##_read(int, void*, size_t) { return hipErrorNotSupported; }        \
  static hipError_t name##_reset() { return hipErrorNotSupported; }
#endif

// Marks of code that some callers trace and others do not.
struct NoMarks {
  __device__ __forceinline__ void mark(int) {}
};

// Host side, one per source file that holds traced kernels.
// ffn_gemv.hip: 0 gate/up of the single-token kernel family, 1 k_route_small,
// 2 k_down_combine_t1; ffn_mfma.hip: 0 thin gate/up, 1 thin down, 2 mixed
// gate/up, 3 mixed down; route.hip: 0 the router front end.
hipError_t trace_read_gemv(int slot, void* dst, size_t bytes);
hipError_t trace_read_mfma(int slot, void* dst, size_t bytes);
hipError_t trace_read_route(int slot, void* dst, size_t bytes);
hipError_t trace_reset_gemv();
hipError_t trace_reset_mfma();
hipError_t trace_reset_route();

}  // namespace moe

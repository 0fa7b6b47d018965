// A plain streaming read: the reference for what share of the HBM peak a
// read-only kernel reaches on this device, next to which the expert kernels'
// achieved bandwidth is read.  It does no layer arithmetic.
//
// Every lane reads 16-byte pieces with non-temporal loads, eight in flight,
// over a grid-strided range, and folds them into one word with XOR; a word is
// stored only if it equals a key no input has (so the loads cannot be
// dropped and nothing is written in practice).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_internal.h"

namespace moe {

typedef unsigned pv4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const pv4u* g_pv4u_ptr;

constexpr uint32_t kProbeKey = 0x9E3779B9u;

__global__ __launch_bounds__(256) void k_read_probe(const uint8_t* __restrict__ buf, size_t n16,
                                                    uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    pv4u v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = __builtin_nontemporal_load((g_pv4u_ptr)(buf + 16 * (i + j * stride)));
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < n16; i += stride) {
    const pv4u v = __builtin_nontemporal_load((g_pv4u_ptr)(buf + 16 * i));
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kProbeKey) sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                             hipStream_t s) {
  return launch(8, k_read_probe, dim3(blocks), dim3(256), s, static_cast<const uint8_t*>(buf),
                bytes / 16, sink);
}

}  // namespace moe

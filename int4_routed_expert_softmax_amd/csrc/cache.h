// HBM slot cache for expert blobs whose home is host memory (or any memory the
// device can read): placement of a call's union experts into slots, on the
// device, and the copy of the missed blobs into their slots.  Internal; the
// entry point is moe_layer_forward_cached (include/moe.h).
#pragma once

#include "moe_internal.h"

namespace moe {

// Cache state, in caller memory, zero-filled once (= every slot empty):
//   CacheHeader (32 B)
//   | slot_of[E]   int32: slot + 1 of a resident expert, 0 = not resident
//   | expert_of[S] int32: expert + 1 a slot holds, 0 = empty
//   | stamp[S]     uint32: clock value of the slot's last use
struct CacheHeader {
  uint32_t clock;        // calls so far
  uint32_t hits, misses; // union experts found resident / copied in, over all calls
  uint32_t last_hits, last_misses;
  uint32_t pad[3];
};
static_assert(sizeof(CacheHeader) == 32, "header layout is part of the ABI");

inline size_t cache_state_bytes(int E, int S) {
  return sizeof(CacheHeader) + 4 * (size_t)E + 8 * (size_t)S;
}

// Largest slot count the placement block handles (one thread per slot); no
// more slots than experts are ever useful, and E <= 1024.
constexpr int kMaxSlots = 1024;

struct CacheArgs {
  uint8_t* state;
  int E, S;
  uint8_t* slots;            // S slots of blob_bytes each
  size_t blob_bytes;
  const uint8_t* const* home;  // [E] every expert's blob where it lives
  const int32_t* uniq;       // this call's union (ascending ids) and its size
  const int32_t* n_uniq;
  DownPlan* plan;            // [U] blob pointers rewritten to the slots
  const uint8_t** eff;       // [E] this call's expert table (union entries written)
  const uint8_t** fill_src;  // [min(E, T k)] blobs to copy in, and their slots
  uint8_t** fill_dst;
  int32_t* n_fill;
  int32_t* hit;              // [U] 1: union position u was resident, 0: copied in by this call
};

// Part `part` of nparts of the copy of blob m (m < *n_fill) from its home into
// its slot, by one whole workgroup: 16 bytes per load, four loads in flight
// per thread.
__device__ __forceinline__ void fill_part(const uint8_t* const* fill_src, uint8_t* const* fill_dst,
                                          const int32_t* n_fill, size_t blob_bytes, int m,
                                          int part, int nparts) {
  if (m >= *n_fill) return;
  const uint4* src = reinterpret_cast<const uint4*>(fill_src[m]);
  uint4* dst = reinterpret_cast<uint4*>(fill_dst[m]);
  const size_t n16 = blob_bytes / 16;
  const size_t per = (n16 + nparts - 1) / nparts;
  const size_t beg = (size_t)part * per;
  const size_t end = beg + per < n16 ? beg + per : n16;
  const size_t nt = blockDim.x;
  for (size_t i = beg + threadIdx.x; i < end; i += 4 * nt) {
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i + (size_t)j * nt < end) v[j] = src[i + (size_t)j * nt];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i + (size_t)j * nt < end) dst[i + (size_t)j * nt] = v[j];
  }
}

hipError_t launch_cache_place(const CacheArgs& a, hipStream_t s);
// max_fill: an upper bound on the number of misses (the union's capacity).
hipError_t launch_cache_fill(const CacheArgs& a, int max_fill, hipStream_t s);
// The cache's hits' gate/up (single-token kernel, one block per row block,
// union position and token group, positions with L.hit[u] == 1 only) in one
// launch with the copies of its misses, so the hits compute while the misses
// are in flight; the misses' gate/up follows in a launch of its own.
hipError_t launch_gateup_fill(const ExpertList& L, int max_experts, int d, int f, Digits xd,
                              Digits ad, int token_groups, const CacheArgs& a, int max_fill,
                              hipStream_t s);

}  // namespace moe

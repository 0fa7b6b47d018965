// HBM slot cache in front of the experts' home memory: the union of a call is
// placed into slots (hits keep theirs, misses take the least recently used
// slots, ties to the lower slot), the missed blobs are copied in, and the
// expert kernels then read every union expert from HBM.  The call's routing
// decides what moves, as in the pages' token path (route, then union, then
// place) — colibri 技术解读, "引擎结构：一个 C 文件，五步 token 路径"; where an
// expert's bytes live decides only the speed — README 工作原理 ›
// 绝不为同一次磁盘读取等待两遍.
#include "cache.h"

namespace moe {

// One block of 1024 threads; thread s < S owns slot s.  Hits take this call's
// clock first, so they rank above every other slot and, with S >= U, the
// M = misses lowest-ranked slots (by last use, then slot index) are never a
// hit's.  Miss m (in ascending expert order) takes the slot of rank m.  No
// global location is read after this kernel writes it.
__global__ __launch_bounds__(1024) void k_cache_place(CacheArgs a) {
  __shared__ uint32_t s_st[kMaxSlots];
  __shared__ uint64_t s_key[kMaxSlots];
  __shared__ int32_t s_victim[kSmallPicks];
  __shared__ int32_t s_miss_e[kSmallPicks];
  __shared__ int32_t s_slot[kSmallPicks];  // >= 0: the hit's slot; < 0: -1 - miss rank
  __shared__ int s_hits, s_misses;
  CacheHeader* hdr = reinterpret_cast<CacheHeader*>(a.state);
  int32_t* slot_of = reinterpret_cast<int32_t*>(a.state + sizeof(CacheHeader));
  int32_t* expert_of = slot_of + a.E;
  uint32_t* stamp = reinterpret_cast<uint32_t*>(expert_of + a.S);
  const int t = threadIdx.x, S = a.S;
  const uint32_t clock = hdr->clock + 1;
  const int U = *a.n_uniq;

  if (t < S) s_st[t] = stamp[t];
  __syncthreads();
  if (t < 64) {
    // wave 0: one union position per lane (U <= 64)
    const bool in = t < U;
    const int e = in ? a.uniq[t] : 0;
    // a slot number outside [1, S] (a state not zero-filled) counts as absent
    const int s1r = in ? slot_of[e] : 0;
    const int s1 = (s1r >= 1 && s1r <= S) ? s1r : 0;
    const bool hit = in && s1 != 0, miss = in && s1 == 0;
    const uint64_t mm = __ballot(miss), hm = __ballot(hit);
    if (hit) {
      s_st[s1 - 1] = clock;
      s_slot[t] = s1 - 1;
    }
    if (miss) {
      const int m = __popcll(mm & ((1ull << t) - 1ull));
      s_miss_e[m] = e;
      s_slot[t] = -1 - m;
    }
    if (t == 0) {
      s_hits = __popcll(hm);
      s_misses = __popcll(mm);
    }
  }
  __syncthreads();
  if (t < S) s_key[t] = ((uint64_t)s_st[t] << 32) | (uint32_t)t;
  __syncthreads();
  const int M = s_misses;
  if (t < S) {
    const uint64_t key = s_key[t];
    int rank = 0;
    for (int j = 0; j < S; ++j) rank += s_key[j] < key;
    if (rank < M) s_victim[rank] = t;
  }
  __syncthreads();
  if (t < M) {
    const int v = s_victim[t], e = s_miss_e[t];
    const int old = expert_of[v];
    if (old >= 1 && old <= a.E) slot_of[old - 1] = 0;  // an evicted expert is never a miss
    expert_of[v] = e + 1;
    slot_of[e] = v + 1;
    s_st[v] = clock;
    a.fill_src[t] = a.home[e];
    a.fill_dst[t] = a.slots + (size_t)v * a.blob_bytes;
  }
  __syncthreads();
  if (t < S) stamp[t] = s_st[t];
  if (t < U) {
    const int sl = s_slot[t] >= 0 ? s_slot[t] : s_victim[-1 - s_slot[t]];
    const uint8_t* p = a.slots + (size_t)sl * a.blob_bytes;
    a.eff[a.uniq[t]] = p;
    a.plan[t].blob = p;
    a.hit[t] = s_slot[t] >= 0 ? 1 : 0;
  }
  if (t == 0) {
    hdr->clock = clock;
    hdr->hits += s_hits;
    hdr->misses += M;
    hdr->last_hits = s_hits;
    hdr->last_misses = M;
    *a.n_fill = M;
  }
}

// Copies blob m = blockIdx.y (m < *n_fill) from its home into its slot,
// grid.x blocks sharing a blob.
constexpr int kFillBlocks = 512;

__global__ __launch_bounds__(256) void k_cache_fill(CacheArgs a) {
  fill_part(a.fill_src, a.fill_dst, a.n_fill, a.blob_bytes, blockIdx.y, blockIdx.x, gridDim.x);
}

hipError_t launch_cache_place(const CacheArgs& a, hipStream_t s) {
  if (a.S < 1 || a.S > kMaxSlots) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_cache_place, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cache_fill(const CacheArgs& a, int max_fill, hipStream_t s) {
  if (max_fill < 1 || a.blob_bytes % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_cache_fill, dim3(kFillBlocks, max_fill), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe

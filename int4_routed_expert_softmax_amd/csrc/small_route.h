// Top-k and union of a small batch (at most kSmallBatch tokens and
// kSmallPicks picks) by the waves of one workgroup, from the batch's complete
// logits, and the publication of the result.  Used by the single-token
// gate/up blocks (which need the routing before their first weight load) and
// by the one-block routing kernel of small batches.  Every user computes a
// token's choice with the same code, so all agree bit for bit.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cstdint>

#include "device_util.h"
#include "moe_internal.h"
#include "select.h"
#include "trace.h"

namespace moe {

// Routing of a small batch, recomputed by every gate/up block.
struct SmallRoute {
  int32_t idx[kSmallPicks];
  float w[kSmallPicks];
  int32_t uniq[kSmallPicks];
  int32_t offsets[kSmallPicks + 1];
  int32_t rows[kSmallPicks];
  alignas(16) int32_t sorted[kSmallPicks];
  int32_t n;
  // per token, the best k of each 64-expert group (logit, id)
  double cz[kSmallBatch][64];
  int32_t ce[kSmallBatch][64];
};

// Top-k of a small batch by the block's waves (G * K2 <= 64, G = groups of
// 64 experts, K2 = k rounded up to a power of two).  Stage 1: the best K2 of
// every group of every token, one wave per group, stored as runs of K2 with
// odd groups reversed.  Stage 2: one wave per token merges its runs; lanes
// 0..k-1 are the token's top k (its best k are among its groups' best K2).
template <int K2, typename Marks>
__device__ __forceinline__ void small_topk(const RouteOut& ro, SmallRoute& sr, int wave,
                                           int nwaves, Marks* tr) {
  const int T = ro.T, E = ro.E, k = ro.k;
  const int lane = threadIdx.x & 63;
  const int G = (E + 63) / 64;
  const int ntask = T * G;
  auto zload = [&](int task) {
    const int t = task / G, e = (task - t * G) * 64 + lane;
    return e < E ? ro.z[(size_t)t * E + e] : -INFINITY;
  };
  // the next task's logits are requested before the current one is sorted
  double znext = wave < ntask ? zload(wave) : -INFINITY;
  for (int task = wave; task < ntask; task += nwaves) {
    const int t = task / G, g = task - t * G;
    const int e = g * 64 + lane;
    double z = znext;
    if (task + nwaves < ntask) znext = zload(task + nwaves);
    int id = e < E ? e : INT_MAX;
    wave_best<K2>(z, id);
    if (lane < K2) {
      const int at = g * K2 + ((g & 1) ? K2 - 1 - lane : lane);
      sr.cz[t][at] = z;
      sr.ce[t][at] = id;
    }
  }
  __syncthreads();
  if (tr) tr->mark(1);
  int span = K2;
  while (span < G * K2) span *= 2;
  for (int t = wave; t < T; t += nwaves) {
    double z = lane < G * K2 ? sr.cz[t][lane] : -INFINITY;
    int id = lane < G * K2 ? sr.ce[t][lane] : INT_MAX;
    merge_runs<K2, K2>(z, id, span);
    // k <= E puts k real experts first; the clamp only keeps a table lookup
    // in bounds should that ever fail
    topk_emit(z, (unsigned)id < (unsigned)E ? id : 0, k, sr.idx + t * k, sr.w + t * k);
  }
}

// Top-k and batch union of a small batch (T <= kSmallBatch, T * k <=
// kSmallPicks) from its complete logits ro.z, into sr, by the block's nwaves
// waves (every thread of the block takes part).
// Trace points (tr): 1 per-group sorts done, 2 merges done, 3 union done.
template <typename Marks = NoMarks>
__device__ __forceinline__ void small_route(const RouteOut& ro, SmallRoute& sr, int wave,
                                            int nwaves, Marks* tr = nullptr) {
  const int T = ro.T, E = ro.E, k = ro.k;
  const int G = (E + 63) / 64;
  const int K2 = k <= 1 ? 1 : 1 << (32 - __builtin_clz(k - 1));
  if (G * K2 <= 64) {
    switch (K2) {
      case 1: small_topk<1>(ro, sr, wave, nwaves, tr); break;
      case 2: small_topk<2>(ro, sr, wave, nwaves, tr); break;
      case 4: small_topk<4>(ro, sr, wave, nwaves, tr); break;
      case 8: small_topk<8>(ro, sr, wave, nwaves, tr); break;
      case 16: small_topk<16>(ro, sr, wave, nwaves, tr); break;
      default: small_topk<32>(ro, sr, wave, nwaves, tr); break;
    }
  } else {
    for (int t = wave; t < T; t += nwaves) wave_topk(ro.z + (size_t)t * E, E, k, sr.idx + t * k, sr.w + t * k);
  }
  __syncthreads();
  if (tr) tr->mark(2);
  if (wave == 0) wave_union_small(sr.idx, T * k, E, sr.uniq, &sr.n, sr.offsets, sr.rows, sr.sorted);
  __syncthreads();
  if (tr) tr->mark(3);
}

// Writes a small batch's routing (ids, weights, union, slot lists, stats and,
// with ro.plan, the down plan from the expert table tab).  Every thread of
// the block calls it; nthreads = block size.
__device__ __forceinline__ void publish_small_route(const RouteOut& ro, const SmallRoute& sr,
                                                    const uint8_t* const* tab, int nthreads) {
  const int E = ro.E, n = ro.T * ro.k;
  const int cap = min(E, n);
  for (int i = threadIdx.x; i < n; i += nthreads) {
    ro.idx[i] = sr.idx[i];
    ro.w[i] = sr.w[i];
    ro.rows[i] = sr.rows[i];
  }
  for (int i = threadIdx.x; i <= cap; i += nthreads) {
    ro.offsets[i] = sr.offsets[i];
    if (i < cap) ro.uniq[i] = sr.uniq[i];
  }
  if (threadIdx.x == 0) *ro.n_uniq = sr.n;
  if (ro.plan && threadIdx.x < sr.n) {
    const int i = threadIdx.x, beg = sr.offsets[i], cnt = sr.offsets[i + 1] - beg;
    DownPlan pl;
    pl.blob = tab[sr.uniq[i]];
    pl.n = cnt;
#pragma unroll
    for (int j = 0; j < kSmallBatch; ++j) pl.slot[j] = j < cnt ? sr.rows[beg + j] : 0;
    pl.pad = 0;
    ro.plan[i] = pl;
  }
  if (ro.stats) {
    if (threadIdx.x == 0) ro.stats[0] = sr.n;
    for (int e = threadIdx.x; e < E; e += nthreads) ro.stats[1 + e] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < sr.n; i += nthreads)
      ro.stats[1 + sr.uniq[i]] = sr.offsets[i + 1] - sr.offsets[i];
  }
}

}  // namespace moe

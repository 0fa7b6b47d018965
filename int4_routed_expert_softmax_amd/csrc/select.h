// Device code shared by the routing kernels and the gate/up kernel (which
// recomputes top-k and the union for small batches): wave-level top-k with
// renormalised softmax weights, and the batch union of a block.
//
// The router picks 8 of 256 routed experts per token and layer, and the picks
// of a batch are merged so each distinct expert is read once (colibri 技术解读
// (linlog.top), "MoE 的稀疏性" and "引擎结构：一个 C 文件，五步 token 路径";
// colibrì README (简体中文), 工作原理 › 绝不为同一次磁盘读取等待两遍).
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cstdint>
#include <type_traits>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- top-k
// Selection order: larger logit first, equal logits -> lower expert id.
// e == INT_MAX marks "no candidate", ranked after everything.
// (Bitwise, not short-circuit, so it compiles to compares and selects.)
__device__ __forceinline__ bool ranks_before(double bz, int be, double az, int ae) {
  return (be != INT_MAX) & ((ae == INT_MAX) | (bz > az) | ((bz == az) & (be < ae)));
}

template <int kCtrl>
__device__ __forceinline__ void argmax_step(double& z, int& e) {
  const long long b = __double_as_longlong(z);
  const int hi = dpp_i<kCtrl>((int)(b >> 32));
  const int lo = dpp_i<kCtrl>((int)b);
  const int oe = dpp_i<kCtrl>(e);
  const double oz = __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
  if (ranks_before(oz, oe, z, e)) {
    z = oz;
    e = oe;
  }
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  const int lo = __builtin_amdgcn_readlane((int)b, l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Wave-wide best (z, e) under ranks_before, the same in every lane: a DPP
// butterfly inside each row of 16 lanes, then the four row winners in order.
__device__ __forceinline__ void wave_argmax(double& z, int& e) {
  argmax_step<kDppXor1>(z, e);
  argmax_step<kDppXor2>(z, e);
  argmax_step<kDppHalfMirror>(z, e);
  argmax_step<kDppMirror>(z, e);
  double bz = readlane_f64(z, 0);
  int be = __builtin_amdgcn_readlane(e, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const double cz = readlane_f64(z, 16 * r);
    const int ce = __builtin_amdgcn_readlane(e, 16 * r);
    if (ranks_before(cz, ce, bz, be)) {
      bz = cz;
      be = ce;
    }
  }
  z = bz;
  e = be;
}

// Lanes 0..k-1 hold the chosen (logit, id) pairs in selection order: write
// the ids and the renormalised softmax weights exp(z_j - z_0) / sum over the
// chosen of exp(z_j' - z_0) (fp64, rounded once to fp32).
__device__ __forceinline__ void topk_emit(double my_z, int my_e, int k, int32_t* idx_out,
                                          float* w_out) {
  const int lane = threadIdx.x & 63;
  const double z0 = readlane_f64(my_z, 0);
  const double p = lane < k ? exp(my_z - z0) : 0.0;
  const double den = wave_sum(p);
  if (lane < k) {
    idx_out[lane] = my_e;
    w_out[lane] = (float)(p / den);
  }
}

// ---------------------------------------------------------------- bitonic
// The value of lane ^ J: DPP inside a row of 16 lanes (J = 4 as a quad
// reversal followed by a half-row mirror: i ^ 3 ^ 7 = i ^ 4), a cross-lane
// permute across rows.
template <int J>
__device__ __forceinline__ int lane_xor(int v) {
  if constexpr (J == 1) return dpp_i<kDppXor1>(v);
  else if constexpr (J == 2) return dpp_i<kDppXor2>(v);
  else if constexpr (J == 4) return dpp_i<kDppHalfMirror>(dpp_i<kDppXor3>(v));
  else if constexpr (J == 8) return dpp_i<kDppRor8>(v);
  else return __shfl_xor(v, J, 64);
}

// Selection order without branches: larger logit first, equal logits ->
// lower id.  Padding is (-inf, INT_MAX), which every real pair precedes.
__device__ __forceinline__ bool goes_first(double bz, int be, double az, int ae) {
  return (bz > az) | ((bz == az) & (be < ae));
}

// One compare-exchange of a bitonic network: this lane and lane ^ J keep the
// earlier (keep_first) or the later of their two pairs.  Two padding pairs
// are equal, so exchanging them changes nothing.
template <int J>
__device__ __forceinline__ void bitonic_step(double& z, int& e, bool keep_first) {
  const long long b = __double_as_longlong(z);
  const int hi = lane_xor<J>((int)(b >> 32));
  const int lo = lane_xor<J>((int)b);
  const int oe = lane_xor<J>(e);
  const double oz = __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
  const bool take = goes_first(oz, oe, z, e) == keep_first;
  z = take ? oz : z;
  e = take ? oe : e;
}

// Keep, in both lanes, the earlier of this lane's pair and lane ^ J's.
template <int J>
__device__ __forceinline__ void keep_earlier(double& z, int& e) {
  const long long b = __double_as_longlong(z);
  const int hi = lane_xor<J>((int)(b >> 32));
  const int lo = lane_xor<J>((int)b);
  const int oe = lane_xor<J>(e);
  const double oz = __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
  const bool take = goes_first(oz, oe, z, e);
  z = take ? oz : z;
  e = take ? oe : e;
}

// Half-cleaner steps J, J/2, ..., 1 of Batcher's bitonic network; blocks of
// DIR lanes alternate direction (lanes with bit DIR clear put the earlier
// pair first).
template <int J, int DIR>
__device__ __forceinline__ void half_clean(double& z, int& e) {
  if constexpr (J >= 1) {
    const int lane = threadIdx.x & 63;
    bitonic_step<J>(z, e, ((lane & J) == 0) == ((lane & DIR) == 0));
    half_clean<J / 2, DIR>(z, e);
  }
}

// Bitonic sort of every run of K2 lanes (stages S = 2 .. K2), directions
// alternating from run to run.
template <int S, int K2>
__device__ __forceinline__ void sort_runs(double& z, int& e) {
  if constexpr (S <= K2) {
    half_clean<S / 2, S>(z, e);
    sort_runs<S * 2, K2>(z, e);
  }
}

// Bitonic top-k merge levels L, 2L, ... below `span`: runs of K2 lanes, L
// apart, sorted in opposite directions; keeping the earlier of lanes i and
// i ^ L leaves the best K2 of each pair of runs as a bitonic sequence, which
// the half-cleaner re-sorts, directions now alternating over 2L lanes.
template <int L, int K2>
__device__ __forceinline__ void merge_runs(double& z, int& e, int span) {
  if constexpr (L <= 32) {
    if (L < span) {
      keep_earlier<L>(z, e);
      half_clean<K2 / 2, 2 * L>(z, e);
      merge_runs<2 * L, K2>(z, e, span);
    }
  }
}

// The best K2 (a power of two) of the wave's 64 (logit, id) pairs, one per
// lane, into lanes 0..K2-1 in selection order.  Ids must be distinct apart
// from the (-inf, INT_MAX) padding.
template <int K2>
__device__ __forceinline__ void wave_best(double& z, int& e) {
  sort_runs<2, K2>(z, e);
  merge_runs<K2, K2>(z, e, 64);
}

constexpr int kMaxPerLane = 16;  // E <= 1024
constexpr int kMaxK = 32;
constexpr int kMaxE = 1024;

// One wave picks the top k of the E logits zt[] of one token (slot order =
// selection order) and their renormalised softmax weights: softmax over all E
// restricted to the chosen ids and renormalised equals
// exp(z_j - z_0) / sum_j' exp(z_j' - z_0) over the chosen logits, z_0 the
// largest (fp64).  Lane l holds the logits of experts l, l+64, ... (MPER of
// them, E <= 64 * MPER); each of the k rounds takes every lane's best
// remaining logit and a DPP arg-max across the wave.  Every lane must be
// active.
template <int MPER>
__device__ __forceinline__ void wave_topk_n(const double* zt, int E, int k, int32_t* idx_out,
                                            float* w_out) {
  const int lane = threadIdx.x & 63;
  double v[MPER];
#pragma unroll
  for (int m = 0; m < MPER; ++m) {
    const int e = lane + 64 * m;
    v[m] = e < E ? zt[e] : 0.0;
  }
  uint32_t taken = 0;
  double my_z = 0.0;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    double bz = 0.0;
    int be = INT_MAX;
#pragma unroll
    for (int m = 0; m < MPER; ++m) {
      const int e = lane + 64 * m;
      if (e < E && !((taken >> m) & 1u) && (be == INT_MAX || v[m] > bz)) {
        bz = v[m];
        be = e;
      }
    }
    wave_argmax(bz, be);
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_z = bz;
      my_e = be;
    }
  }
  topk_emit(my_z, my_e, k, idx_out, w_out);
}

__device__ __forceinline__ void wave_topk(const double* zt, int E, int k, int32_t* idx_out,
                                          float* w_out) {
  if (E <= 64) wave_topk_n<1>(zt, E, k, idx_out, w_out);
  else if (E <= 128) wave_topk_n<2>(zt, E, k, idx_out, w_out);
  else if (E <= 256) wave_topk_n<4>(zt, E, k, idx_out, w_out);
  else if (E <= 512) wave_topk_n<8>(zt, E, k, idx_out, w_out);
  else wave_topk_n<16>(zt, E, k, idx_out, w_out);
}

// Batch union of n <= 64 picks by one wave.  Lane l holds pick l (slot l,
// expert idx[l]); its key id * 64 + l orders picks by expert, then slot
// (= token order).  A pick's rank among all keys is its position in rows; the
// first pick of each expert opens a union entry.  uniq/offsets as
// union_body; cnt_out[u] = picks of uniq[u].  s_sorted: 64 ints of scratch
// LDS, 16-byte aligned.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}
__device__ __forceinline__ void wave_union_small(const int32_t* idx, int n, int E, int32_t* uniq,
                                                 int32_t* n_uniq, int32_t* offsets, int32_t* rows,
                                                 int32_t* s_sorted) {
  const int lane = threadIdx.x & 63;
  const bool valid = lane < n;
  const int id = valid ? idx[lane] : 0;
  const int key = valid ? id * 64 + lane : INT_MAX;
  // rank = keys below this one: every lane reads all 64 keys from LDS (the
  // same address in every lane: broadcast reads), 64 independent compares
  s_sorted[lane] = key;
  wave_lds_sync();
  // (keys past n are INT_MAX: reading a few past n changes no rank)
  int rank = 0;
  auto count = [&](auto nk) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < decltype(nk)::value; j += 4) {
      const int4 kk = *reinterpret_cast<const int4*>(s_sorted + j);
      rank += (kk.x < key) + (kk.y < key) + (kk.z < key) + (kk.w < key);
    }
  };
  if (n <= 16) count(std::integral_constant<int, 16>());
  else count(std::integral_constant<int, 64>());
  wave_lds_sync();
  if (valid) {
    rows[rank] = lane;
    s_sorted[rank] = id;
  }
  wave_lds_sync();
  // lane r now looks at sorted position r
  const int sid = valid ? s_sorted[lane] : 0;
  const int prev = (valid && lane > 0) ? s_sorted[lane - 1] : -1;
  const bool first = valid && sid != prev;
  const uint64_t fm = __ballot(first);
  const int U = __popcll(fm);
  if (first) {
    const int u = __popcll(fm & ((1ull << lane) - 1ull));
    uniq[u] = sid;
    offsets[u] = lane;
  }
  // offsets[U .. cap] = n and uniq[U .. cap - 1] = -1.  offsets has cap + 1
  // <= 65 entries, one more than the wave has lanes: lane l writes entry
  // l + 1 and lane 0 entry U (U itself can be 64, every pick a different
  // expert).
  const int cap = min(E, n);
  if (lane >= U && lane < cap) {
    offsets[lane + 1] = n;
    uniq[lane] = -1;
  }
  if (lane == 0) {
    offsets[U] = n;
    *n_uniq = U;
  }
}

// ---------------------------------------------------------------- union
// cnt[e] by LDS histogram, offsets by an exclusive scan, uniq by a scan over
// the non-empty flags.  Slots are placed in ascending token order without
// relying on the order of atomics: tokens are taken 64 at a time, each expert
// gets a 64-bit mask of the tokens of the block that picked it, and a slot's
// rank inside the block is the popcount of the mask bits below its token.
struct UnionLds {
  int cnt[kMaxE], off[kMaxE], cur[kMaxE];
  uint32_t mlo[kMaxE], mhi[kMaxE];
  int wave_a[16], wave_b[16];
};

// Exclusive block scan of two ints at once over NTH threads.
template <int NTH>
__device__ __forceinline__ void block_scan2(int a, int b, int& ea, int& eb, int& ta, int& tb,
                                            UnionLds& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int ia = a, ib = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int na = __shfl_up(ia, o, 64), nb = __shfl_up(ib, o, 64);
    if (lane >= o) {
      ia += na;
      ib += nb;
    }
  }
  if (lane == 63) {
    sm.wave_a[wave] = ia;
    sm.wave_b[wave] = ib;
  }
  __syncthreads();
  int ba = 0, bb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int i = 0; i < NTH / 64; ++i) {
    const int wa = sm.wave_a[i], wb = sm.wave_b[i];
    if (i < wave) {
      ba += wa;
      bb += wb;
    }
    sa += wa;
    sb += wb;
  }
  __syncthreads();
  ea = ba + ia - a;
  eb = bb + ib - b;
  ta = sa;
  tb = sb;
}

template <int NTH>
__device__ void union_body(const int32_t* idx, int T, int E, int k, int32_t* uniq,
                           int32_t* n_uniq, int32_t* offsets, int32_t* rows, int32_t* stats,
                           UnionLds& sm) {
  const int tid = threadIdx.x;
  const int n = T * k;
  const int cap = min(E, n);
  for (int e = tid; e < kMaxE; e += NTH) {
    sm.cnt[e] = 0;
    sm.cur[e] = 0;
    sm.mlo[e] = 0;
    sm.mhi[e] = 0;
  }
  __syncthreads();
  for (int i = tid; i < n; i += NTH) {
    const int e = idx[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&sm.cnt[e], 1);  // ids outside [0, E) are ignored
  }
  __syncthreads();
  // each thread owns a contiguous run of experts
  const int ept = (E + NTH - 1) / NTH;
  const int e0 = min(E, tid * ept), e1 = min(E, e0 + ept);
  int csum = 0, nz = 0;
  for (int e = e0; e < e1; ++e) {
    csum += sm.cnt[e];
    nz += sm.cnt[e] > 0;
  }
  int off, pos, tot_slots, U;
  block_scan2<NTH>(csum, nz, off, pos, tot_slots, U, sm);
  for (int e = e0; e < e1; ++e) {
    const int c = sm.cnt[e];
    sm.off[e] = off;
    if (c > 0) {
      uniq[pos] = e;
      offsets[pos] = off;
      ++pos;
    }
    if (stats) stats[1 + e] = c;
    off += c;
  }
  for (int u = U + tid; u <= cap; u += NTH) {
    offsets[u] = tot_slots;
    if (u < cap) uniq[u] = -1;
  }
  if (tid == 0) {
    *n_uniq = U;
    if (stats) stats[0] = U;
  }
  __syncthreads();
  for (int t0 = 0; t0 < T; t0 += 64) {
    const int ne = min(64, T - t0) * k;
    for (int i = tid; i < ne; i += NTH) {
      const int e = idx[t0 * k + i];
      const int tl = i / k;
      if ((unsigned)e < (unsigned)E) atomicOr(tl < 32 ? &sm.mlo[e] : &sm.mhi[e], 1u << (tl & 31));
    }
    __syncthreads();
    for (int i = tid; i < ne; i += NTH) {
      const int e = idx[t0 * k + i];
      if ((unsigned)e >= (unsigned)E) continue;
      const int tl = i / k;
      const uint32_t lo = sm.mlo[e], hi = sm.mhi[e];
      const int r = tl < 32 ? __popc(lo & ((1u << tl) - 1u))
                            : __popc(lo) + __popc(hi & ((1u << (tl - 32)) - 1u));
      rows[sm.off[e] + sm.cur[e] + r] = t0 * k + i;
    }
    __syncthreads();
    for (int e = tid; e < E; e += NTH) {
      sm.cur[e] += __popc(sm.mlo[e]) + __popc(sm.mhi[e]);
      sm.mlo[e] = 0;
      sm.mhi[e] = 0;
    }
    __syncthreads();
  }
}

}  // namespace moe

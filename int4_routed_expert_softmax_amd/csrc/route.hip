// Router (fp64 logits, top-k, renormalised softmax weights), batch union,
// RMSNorm and activation digit split for the gfx950 MoE layer.
//
// The router picks 8 of 256 routed experts per token and layer and the picks
// of a batch are merged so each distinct expert is read once (colibri 技术解读
// (linlog.top), "MoE 的稀疏性" and "引擎结构：一个 C 文件，五步 token 路径";
// colibrì README (简体中文), 工作原理 › 绝不为同一次磁盘读取等待两遍).
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cstdint>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- RMSNorm
// xn[t][i] = h[t][i] * r, r = 1 / sqrt(mean(h^2) + eps), mean and root in
// fp64, the product rounded once to f32.  One workgroup per token.
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ h,
                                                 float* __restrict__ xn, int d, float eps) {
  const int t = blockIdx.x;
  const float* ht = h + (size_t)t * d;
  double ss = 0.0;
  for (int i = threadIdx.x; i < d; i += 256) ss += (double)ht[i] * (double)ht[i];
  ss = wave_sum(ss);
  __shared__ double part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double tot = (part[0] + part[1]) + (part[2] + part[3]);
  const double r = 1.0 / sqrt(tot / d + (double)eps);
  for (int i = threadIdx.x; i < d; i += 256) xn[(size_t)t * d + i] = (float)((double)ht[i] * r);
}

// ---------------------------------------------------------------- logits
// z[t][e] = sum_i x[t][i] * Wr[e][i] + b[e] in fp64.  A fp32 x fp32 product has
// at most 48 significant bits, so every product is exact in fp64 and only the
// (fp64) summation order differs from a sequential sum: ~1e-16 relative, far
// below the gap between neighbouring logits.  One workgroup per (expert,
// block of TB tokens); the router row is read once per token block.
template <int TB>
__global__ __launch_bounds__(256) void k_logits(const void* __restrict__ x, int x_bf16, int T,
                                                int d, int E, const float* __restrict__ Wr,
                                                const float* __restrict__ bias,
                                                double* __restrict__ z) {
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * TB;
  const int nt = min(TB, T - t0);
  const float4* w4 = reinterpret_cast<const float4*>(Wr + (size_t)e * d);
  double acc[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) acc[j] = 0.0;
  const int n4 = d >> 2;
  for (int i = threadIdx.x; i < n4; i += 256) {
    const float4 w = w4[i];
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      if (j < nt) {
        float4 v;
        if (x_bf16) {
          const uint2 b = reinterpret_cast<const uint2*>(
              static_cast<const uint16_t*>(x) + (size_t)(t0 + j) * d)[i];
          v.x = __uint_as_float(b.x << 16);
          v.y = __uint_as_float(b.x & 0xFFFF0000u);
          v.z = __uint_as_float(b.y << 16);
          v.w = __uint_as_float(b.y & 0xFFFF0000u);
        } else {
          v = reinterpret_cast<const float4*>(static_cast<const float*>(x) + (size_t)(t0 + j) * d)[i];
        }
        acc[j] += (double)w.x * (double)v.x;
        acc[j] += (double)w.y * (double)v.y;
        acc[j] += (double)w.z * (double)v.z;
        acc[j] += (double)w.w * (double)v.w;
      }
    }
  }
  __shared__ double part[TB][4];
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const double s = wave_sum(acc[j]);
    if ((threadIdx.x & 63) == 0) part[j][threadIdx.x >> 6] = s;
  }
  __syncthreads();
  if (threadIdx.x < nt) {
    const int j = threadIdx.x;
    const double s = (part[j][0] + part[j][1]) + (part[j][2] + part[j][3]);
    z[(size_t)(t0 + j) * E + e] = s + (bias ? (double)bias[e] : 0.0);
  }
}

// ---------------------------------------------------------------- top-k
// One wave per token.  Lane l holds the logits of experts l, l+64, ...; k
// rounds of a wave arg-max pick the largest remaining logit, ties to the lower
// id.  Weights: softmax over all experts restricted to the chosen ones and
// renormalised, which equals exp(z_j - z_0) / sum_j' exp(z_j' - z_0) over the
// chosen logits (z_0 the largest), computed in fp64.
constexpr int kMaxPerLane = 16;  // E <= 1024
constexpr int kMaxK = 32;

__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ z, int T, int E, int k,
                                              int32_t* __restrict__ idx, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const double* zt = z + (size_t)t * E;
  double v[kMaxPerLane];
#pragma unroll
  for (int m = 0; m < kMaxPerLane; ++m) {
    const int e = lane + 64 * m;
    v[m] = e < E ? zt[e] : -DBL_MAX;
  }
  uint32_t taken = 0;
  double my_z = 0.0;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    double bz = -DBL_MAX;
    int be = INT_MAX;
#pragma unroll
    for (int m = 0; m < kMaxPerLane; ++m) {
      const int e = lane + 64 * m;
      if (e < E && !(taken >> m & 1u) && (v[m] > bz || be == INT_MAX)) {
        bz = v[m];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double oz = __shfl_xor(bz, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (oe != INT_MAX && (be == INT_MAX || oz > bz || (oz == bz && oe < be))) {
        bz = oz;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_z = bz;
      my_e = be;
    }
  }
  const double z0 = __shfl(my_z, 0, 64);
  const double p = lane < k ? exp(my_z - z0) : 0.0;
  const double den = wave_sum(p);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = (float)(p / den);
  }
}

// ---------------------------------------------------------------- union
// One workgroup of 1024 threads.  cnt[e] by LDS histogram, offsets by an
// exclusive scan, uniq by a scan over the non-empty flags.  Slots are placed
// in ascending token order without relying on atomic ordering: tokens are
// taken 64 at a time, each expert gets a 64-bit mask of the tokens of the
// block that picked it, and a slot's rank inside the block is the popcount of
// the mask bits below its token.
constexpr int kUnionThreads = 1024;
constexpr int kMaxE = 1024;

__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < kUnionThreads / 64; ++i) {
    const int s = s_wave[i];
    if (i < wave) base += s;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return base + inc - v;
}

__global__ __launch_bounds__(kUnionThreads) void k_union(const int32_t* __restrict__ idx, int T,
                                                          int E, int k, int32_t* __restrict__ uniq,
                                                          int32_t* __restrict__ n_uniq,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ rows,
                                                          int32_t* __restrict__ stats) {
  __shared__ int s_cnt[kMaxE], s_off[kMaxE], s_cur[kMaxE];
  __shared__ uint32_t s_mlo[kMaxE], s_mhi[kMaxE];
  __shared__ int s_wave[kUnionThreads / 64];
  const int tid = threadIdx.x;
  const int n = T * k;
  const int cap = min(E, n);
  for (int e = tid; e < kMaxE; e += kUnionThreads) {
    s_cnt[e] = 0;
    s_cur[e] = 0;
    s_mlo[e] = 0;
    s_mhi[e] = 0;
  }
  __syncthreads();
  for (int i = tid; i < n; i += kUnionThreads) {
    const int e = idx[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);  // ids outside [0, E) are ignored
  }
  __syncthreads();
  const int c = tid < E ? s_cnt[tid] : 0;
  int tot_slots, U;
  const int off = block_exclusive_scan(c, s_wave, tot_slots);
  const int pos = block_exclusive_scan(c > 0 ? 1 : 0, s_wave, U);
  if (tid < E) {
    s_off[tid] = off;
    if (c > 0) {
      uniq[pos] = tid;
      offsets[pos] = off;
    }
    if (stats) stats[1 + tid] = c;
  }
  for (int u = U + tid; u <= cap; u += kUnionThreads) {
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
    for (int i = tid; i < ne; i += kUnionThreads) {
      const int e = idx[t0 * k + i];
      const int tl = i / k;
      if ((unsigned)e < (unsigned)E) atomicOr(tl < 32 ? &s_mlo[e] : &s_mhi[e], 1u << (tl & 31));
    }
    __syncthreads();
    for (int i = tid; i < ne; i += kUnionThreads) {
      const int e = idx[t0 * k + i];
      if ((unsigned)e >= (unsigned)E) continue;
      const int tl = i / k;
      const uint32_t lo = s_mlo[e], hi = s_mhi[e];
      const int r = tl < 32 ? __popc(lo & ((1u << tl) - 1u))
                            : __popc(lo) + __popc(hi & ((1u << (tl - 32)) - 1u));
      rows[s_off[e] + s_cur[e] + r] = t0 * k + i;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kUnionThreads) {
      s_cur[e] += __popc(s_mlo[e]) + __popc(s_mhi[e]);
      s_mlo[e] = 0;
      s_mhi[e] = 0;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- digit split
// One wave per (row, 64-column group); gather[r] (if given) selects the source
// row of output row r.
__global__ __launch_bounds__(256) void k_digitize(const void* __restrict__ x, int x_bf16,
                                                  const int32_t* __restrict__ gather, int rows,
                                                  int K, Digits out) {
  const int lane = threadIdx.x & 63;
  const int ng = K / kGroup;
  const int nch = K / kChunk;
  const long items = (long)rows * ng;
  for (long it = (long)blockIdx.x * 4 + (threadIdx.x >> 6); it < items; it += (long)gridDim.x * 4) {
    const int r = (int)(it / ng), g = (int)(it % ng);
    const int src = gather ? gather[r] : r;
    const size_t i = (size_t)src * K + (size_t)g * kGroup + lane;
    const float v = x_bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(x)[i] << 16)
                           : static_cast<const float*>(x)[i];
    digitize_group(v, lane, g, out.q + (size_t)r * nch * kChunkDigitBytes,
                   out.sx + (size_t)r * nch, out.sc + (size_t)r * ng);
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_rmsnorm(const float* h, float* xn, int T, int d, float eps, hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(T), dim3(256), 0, s, h, xn, d, eps);
  return hipGetLastError();
}

hipError_t launch_logits(const void* x, int x_bf16, int T, int d, int E, const float* Wr,
                         const float* bias, double* z, hipStream_t s) {
  if (T <= 1) {
    hipLaunchKernelGGL(k_logits<1>, dim3(E, T), dim3(256), 0, s, x, x_bf16, T, d, E, Wr, bias, z);
  } else {
    hipLaunchKernelGGL(k_logits<8>, dim3(E, (T + 7) / 8), dim3(256), 0, s, x, x_bf16, T, d, E, Wr,
                       bias, z);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const double* z, int T, int E, int k, int32_t* idx, float* w,
                       hipStream_t s) {
  hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, s, z, T, E, k, idx, w);
  return hipGetLastError();
}

hipError_t launch_union(const int32_t* idx, int T, int E, int k, int32_t* uniq, int32_t* n_uniq,
                        int32_t* offsets, int32_t* rows, int32_t* stats, hipStream_t s) {
  hipLaunchKernelGGL(k_union, dim3(1), dim3(kUnionThreads), 0, s, idx, T, E, k, uniq, n_uniq,
                     offsets, rows, stats);
  return hipGetLastError();
}

hipError_t launch_digitize(const void* x, int x_bf16, const int32_t* gather, int rows, int K,
                           Digits out, hipStream_t s) {
  const long items = (long)rows * (K / kGroup);
  const long blocks = (items + 3) / 4;
  const int grid = (int)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(k_digitize, dim3(grid), dim3(256), 0, s, x, x_bf16, gather, rows, K, out);
  return hipGetLastError();
}

}  // namespace moe

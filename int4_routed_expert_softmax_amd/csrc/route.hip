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
#include "select.h"

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
// below the gap between neighbouring logits.
//
// Batches of more than kSmallBatch tokens: a block = kLogTok tokens x 256
// experts x one of kLogSplit column ranges, one thread per expert.  Router
// columns pass through LDS (64 at a time, rows padded against bank
// conflicts) and each x value is widened to fp64 once per block; thread e
// writes zp[s][t][e], the partial sum over range s.  k_topk adds the ranges
// and the bias in a fixed order, so the result does not depend on scheduling.
constexpr int kLogTok = 16;
constexpr int kLogCols = 64;

__global__ __launch_bounds__(256) void k_logits(const void* __restrict__ x, int x_bf16, int T,
                                                int d, int E, const float* __restrict__ Wr,
                                                double* __restrict__ zp) {
  __shared__ float s_w[256][kLogCols + 1];
  __shared__ __attribute__((aligned(16))) double s_x[kLogCols][kLogTok];
  const int t = threadIdx.x;
  const int t0 = blockIdx.x * kLogTok;
  const int nt = min(kLogTok, T - t0);
  const int split = blockIdx.y;
  const int e0 = blockIdx.z * 256;
  const int e = e0 + t;
  const int nchunk = d / kLogCols;
  const int c_begin = split * nchunk / kLogSplit, c_end = (split + 1) * nchunk / kLogSplit;
  double acc[kLogTok];
#pragma unroll
  for (int j = 0; j < kLogTok; ++j) acc[j] = 0.0;
  for (int c = c_begin; c < c_end; ++c) {
    const int col0 = c * kLogCols;
    // 256 rows x 16 float4 of the router, coalesced along each row
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int q = i * 256 + t, row = q >> 4, c4 = q & 15;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e0 + row < E)
        v = *reinterpret_cast<const float4*>(Wr + (size_t)(e0 + row) * d + col0 + 4 * c4);
      s_w[row][4 * c4] = v.x;
      s_w[row][4 * c4 + 1] = v.y;
      s_w[row][4 * c4 + 2] = v.z;
      s_w[row][4 * c4 + 3] = v.w;
    }
    // kLogTok tokens x 64 columns of x, widened to fp64, stored [column][token]
#pragma unroll
    for (int i = 0; i < kLogTok * kLogCols / 256; ++i) {
      const int q = i * 256 + t, tok = q / kLogCols, col = q % kLogCols;
      double v = 0.0;
      if (tok < nt) {
        const size_t at = (size_t)(t0 + tok) * d + col0 + col;
        v = x_bf16 ? (double)__uint_as_float((uint32_t)static_cast<const uint16_t*>(x)[at] << 16)
                   : (double)static_cast<const float*>(x)[at];
      }
      s_x[col][tok] = v;
    }
    __syncthreads();
#pragma unroll 4
    for (int col = 0; col < kLogCols; ++col) {
      const double w = (double)s_w[t][col];
#pragma unroll
      for (int j = 0; j < kLogTok; ++j) acc[j] += w * s_x[col][j];
    }
    __syncthreads();
  }
  if (e < E) {
    for (int j = 0; j < nt; ++j) zp[((size_t)split * T + t0 + j) * E + e] = acc[j];
  }
}

// ---------------------------------------------------------------- top-k
// One wave per token.  With nsplit > 1 the logits are the fixed-order sum of
// the per-range partials plus the bias, formed in LDS first.
__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ z, int nsplit,
                                              const float* __restrict__ bias, int T, int E, int k,
                                              int32_t* __restrict__ idx, float* __restrict__ w) {
  __shared__ double s_z[4][kMaxE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const double* zt = z + (size_t)t * E;
  if (nsplit > 1) {
    for (int e = lane; e < E; e += 64) {
      double v = 0.0;
      for (int s = 0; s < nsplit; ++s) v += z[((size_t)s * T + t) * E + e];
      s_z[wave][e] = v + (bias ? (double)bias[e] : 0.0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    zt = s_z[wave];
  }
  wave_topk(zt, E, k, idx + (size_t)t * k, w + (size_t)t * k);
}

// ---------------------------------------------------------------- union
constexpr int kUnionThreads = 1024;

__global__ __launch_bounds__(kUnionThreads) void k_union(const int32_t* __restrict__ idx, int T,
                                                          int E, int k, int32_t* __restrict__ uniq,
                                                          int32_t* __restrict__ n_uniq,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ rows,
                                                          int32_t* __restrict__ stats) {
  __shared__ UnionLds sm;
  union_body<kUnionThreads>(idx, T, E, k, uniq, n_uniq, offsets, rows, stats, sm);
}

// ---------------------------------------------------------------- router front end
// For batches of up to kSmallBatch tokens, one launch computes every logit and
// the activations' digit form: one workgroup per expert computes that
// expert's logits for every token, and extra workgroups after them make the
// digit split in parallel (RMSNorm first if asked, recomputed in the same
// order in every workgroup so all agree bit for bit).  Top-k and the union
// run at the start of the next kernel (the gate/up projection), which needs
// them first; nothing here waits on another workgroup.
template <int TB>
__global__ __launch_bounds__(256) void k_router_front(RouterArgs a) {
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, d = a.d, E = a.E;
  __shared__ double part[TB][4];
  __shared__ double s_r[TB];

  auto xval = [&](int t, size_t i) -> float {
    return a.x_bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(a.x)[(size_t)t * d + i] << 16)
                    : static_cast<const float*>(a.x)[(size_t)t * d + i];
  };
  auto xval4 = [&](int t, int i4) -> float4 {
    if (a.x_bf16) {
      const uint2 b = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.x) + (size_t)t * d)[i4];
      return make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
                         __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u));
    }
    return reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + (size_t)t * d)[i4];
  };
  // Rows of up to 8192 columns stay in registers (8 float4 per thread): the
  // router row is requested before the RMSNorm reduction so the two overlap,
  // and a single token's x is read once.
  constexpr int kReg = 8;
  const int n4 = d >> 2;
  const bool in_regs = n4 <= 256 * kReg;
  float4 wr[kReg], xr[kReg];
  if (in_regs) {
#pragma unroll
    for (int m = 0; m < kReg; ++m) {
      const int i4 = tid + 256 * m;
      if (e < E && i4 < n4) wr[m] = reinterpret_cast<const float4*>(a.Wr + (size_t)e * d)[i4];
      if (TB == 1 && i4 < n4) xr[m] = xval4(0, i4);
    }
  }
  if (a.prenorm) {
    // r_t = 1 / sqrt(mean(h_t^2) + eps) in fp64
    double ss[TB];
#pragma unroll
    for (int j = 0; j < TB; ++j) ss[j] = 0.0;
    if (TB == 1 && in_regs) {
#pragma unroll
      for (int m = 0; m < kReg; ++m) {
        if (tid + 256 * m < n4) {
          const float4 v = xr[m];
          ss[0] += (double)v.x * (double)v.x;
          ss[0] += (double)v.y * (double)v.y;
          ss[0] += (double)v.z * (double)v.z;
          ss[0] += (double)v.w * (double)v.w;
        }
      }
    } else {
      for (int i = tid; i < d; i += 256)
#pragma unroll
        for (int j = 0; j < TB; ++j)
          if (j < T) {
            const double h = xval(j, i);
            ss[j] += h * h;
          }
    }
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const double sj = wave_sum(ss[j]);
      if (lane == 0) part[j][wave] = sj;
    }
    __syncthreads();
    if (tid < T) {
      const double tot = (part[tid][0] + part[tid][1]) + (part[tid][2] + part[tid][3]);
      s_r[tid] = 1.0 / sqrt(tot / d + (double)a.eps);
    }
    __syncthreads();
  }
  // the value the router and the experts see: x, or RMSNorm(x) rounded to f32
  auto norm = [&](int t, float v) -> float { return a.prenorm ? (float)((double)v * s_r[t]) : v; };
  auto xin = [&](int t, size_t i) -> float { return norm(t, xval(t, i)); };

  if (e >= E) {
    // workgroups past the last expert: the digit split, one wave per 64
    // columns of a token
    const int nb = d / 64, nch = d / kChunk, ng = d / kXGroup;
    for (int it = (e - E) * 4 + wave; it < T * nb; it += (gridDim.x - E) * 4) {
      const int t = it / nb, col = (it % nb) * 64 + lane;
      digitize32(xin(t, col), col, true, a.xd.q + (size_t)t * nch * kChunkDigitBytes,
                 a.xd.sx + (size_t)t * ng, a.xd.sc + (size_t)t * ng);
    }
    return;
  }
  double acc[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) acc[j] = 0.0;
  if (in_regs) {
#pragma unroll
    for (int m = 0; m < kReg; ++m) {
      const int i4 = tid + 256 * m;
      if (i4 < n4) {
        const float4 w = wr[m];
#pragma unroll
        for (int j = 0; j < TB; ++j) {
          if (j < T) {
            const float4 v = TB == 1 ? xr[m] : xval4(j, i4);
            acc[j] += (double)w.x * (double)norm(j, v.x);
            acc[j] += (double)w.y * (double)norm(j, v.y);
            acc[j] += (double)w.z * (double)norm(j, v.z);
            acc[j] += (double)w.w * (double)norm(j, v.w);
          }
        }
      }
    }
  } else {
    const float4* w4 = reinterpret_cast<const float4*>(a.Wr + (size_t)e * d);
    for (int i = tid; i < n4; i += 256) {
      const float4 w = w4[i];
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        if (j < T) {
          acc[j] += (double)w.x * (double)xin(j, 4 * i);
          acc[j] += (double)w.y * (double)xin(j, 4 * i + 1);
          acc[j] += (double)w.z * (double)xin(j, 4 * i + 2);
          acc[j] += (double)w.w * (double)xin(j, 4 * i + 3);
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const double sj = wave_sum(acc[j]);
    if (lane == 0) part[j][wave] = sj;
  }
  __syncthreads();
  if (tid < T) {
    const double sj = (part[tid][0] + part[tid][1]) + (part[tid][2] + part[tid][3]);
    a.z[(size_t)tid * E + e] = sj + (a.bias ? (double)a.bias[e] : 0.0);
  }
}

// ---------------------------------------------------------------- digit split
// One wave per 64 columns of a row; gather[r] (if given) selects the source
// row of output row r.
__global__ __launch_bounds__(256) void k_digitize(const void* __restrict__ x, int x_bf16,
                                                  const int32_t* __restrict__ gather, int rows,
                                                  int K, Digits out) {
  const int lane = threadIdx.x & 63;
  const int nb = K / 64, nch = K / kChunk, ng = K / kXGroup;
  const long items = (long)rows * nb;
  for (long it = (long)blockIdx.x * 4 + (threadIdx.x >> 6); it < items; it += (long)gridDim.x * 4) {
    const int r = (int)(it / nb), col = (int)(it % nb) * 64 + lane;
    const int src = gather ? gather[r] : r;
    const size_t i = (size_t)src * K + col;
    const float v = x_bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(x)[i] << 16)
                           : static_cast<const float*>(x)[i];
    digitize32(v, col, true, out.q + (size_t)r * nch * kChunkDigitBytes, out.sx + (size_t)r * ng,
               out.sc + (size_t)r * ng);
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_rmsnorm(const float* h, float* xn, int T, int d, float eps, hipStream_t s) {
  return launch(0, k_rmsnorm, dim3(T), dim3(256), s, h, xn, d, eps);
}

hipError_t launch_logits(const void* x, int x_bf16, int T, int d, int E, const float* Wr,
                         double* zp, hipStream_t s) {
  const dim3 grid((T + kLogTok - 1) / kLogTok, kLogSplit, (E + 255) / 256);
  return launch(1, k_logits, grid, dim3(256), s, x, x_bf16, T, d, E, Wr, zp);
}

hipError_t launch_topk(const double* z, int nsplit, const float* bias, int T, int E, int k,
                       int32_t* idx, float* w, hipStream_t s) {
  return launch(2, k_topk, dim3((T + 3) / 4), dim3(256), s, z, nsplit, bias, T, E, k, idx, w);
}

hipError_t launch_union(const int32_t* idx, int T, int E, int k, int32_t* uniq, int32_t* n_uniq,
                        int32_t* offsets, int32_t* rows, int32_t* stats, hipStream_t s) {
  return launch(3, k_union, dim3(1), dim3(kUnionThreads), s, idx, T, E, k, uniq, n_uniq, offsets,
                rows, stats);
}

hipError_t launch_router_front(const RouterArgs& a, hipStream_t s) {
  const int dig_blocks = a.xd.q ? (a.T * (a.d / 64) + 3) / 4 : 0;
  const dim3 grid(a.E + dig_blocks);
  if (a.T <= 1) return launch(1, k_router_front<1>, grid, dim3(256), s, a);
  if (a.T <= 2) return launch(1, k_router_front<2>, grid, dim3(256), s, a);
  if (a.T <= 4) return launch(1, k_router_front<4>, grid, dim3(256), s, a);
  return launch(1, k_router_front<8>, grid, dim3(256), s, a);
}

hipError_t launch_digitize(const void* x, int x_bf16, const int32_t* gather, int rows, int K,
                           Digits out, hipStream_t s) {
  const long items = (long)rows * (K / kGroup);
  const long blocks = (items + 3) / 4;
  const int grid = (int)(blocks < 4096 ? blocks : 4096);
  return launch(4, k_digitize, dim3(grid), dim3(256), s, x, x_bf16, gather, rows, K, out);
}

}  // namespace moe

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
#include "pack.h"
#include "select.h"
#include "trace.h"

namespace moe {

MOE_TRACE_STORAGE(g_trace_route, 1)
hipError_t trace_read_route(int slot, void* dst, size_t bytes) {
  return g_trace_route_read(slot, dst, bytes);
}
hipError_t trace_reset_route() { return g_trace_route_reset(); }

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
// Batches past the small-batch limits: a fp64 GEMM on the matrix cores
// (v_mfma_f64_16x16x4_f64: exact fp64 products, fp64 sums).  A block = 32
// tokens x 64 experts x one of kLogSplit column ranges, 4 waves of 16
// experts x 32 tokens.  64-column chunks of x and of the router rows are
// widened to fp64 into LDS, transposed to [column][token|expert] (so a lane's
// MFMA operand is one 8-byte read), with the next chunk already loaded into
// registers.  zp[s][t][e] is the partial sum over range s; k_topk adds the
// ranges and the bias in a fixed order, so the result does not depend on
// scheduling.
constexpr int kLgT = 32;
constexpr int kLgE = 64;
constexpr int kLgC = 64;

typedef double f64x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_logits(const void* __restrict__ x, int x_bf16, int T,
                                                int d, int E, const float* __restrict__ Wr,
                                                double* __restrict__ zp) {
  __shared__ double s_x[kLgC][kLgT + 1];
  __shared__ double s_w[kLgC][kLgE + 1];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // workgroup F runs on XCD F % 8: every workgroup of column range F % 8
  // shares one L2, which then fetches that range of x and of the router rows
  // once for all its token and expert blocks
  static_assert(kLogSplit == kXcds, "one column range per XCD");
  const int F = blockIdx.x, split = F % kLogSplit, q = F / kLogSplit;
  const int ntb = (T + kLgT - 1) / kLgT;
  const int t0 = (q % ntb) * kLgT;
  const int nt = min(kLgT, T - t0);
  const int e0 = (q / ntb) * kLgE;
  const int nchunk = d / kLgC;
  const int c_begin = split * nchunk / kLogSplit, c_end = (split + 1) * nchunk / kLogSplit;

  // staging: x value q = i * 256 + t is token q / 64, column q % 64; router
  // value q is expert q / 64, column q % 64 (coalesced along the columns)
  constexpr int kXPer = kLgT * kLgC / 256, kWPer = kLgE * kLgC / 256;
  float xv[kXPer], wv[kWPer];
  auto fetch = [&](int c) {
    const int col0 = c * kLgC;
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int q = i * 256 + t, tok = q / kLgC, col = q % kLgC;
      float v = 0.0f;
      if (tok < nt) {
        const size_t at = (size_t)(t0 + tok) * d + col0 + col;
        v = x_bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(x)[at] << 16)
                   : static_cast<const float*>(x)[at];
      }
      xv[i] = v;
    }
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
      const int q = i * 256 + t, ex = q / kLgC, col = q % kLgC;
      wv[i] = e0 + ex < E ? Wr[(size_t)(e0 + ex) * d + col0 + col] : 0.0f;
    }
  };

  f64x4 acc[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
  if (c_begin < c_end) fetch(c_begin);
  for (int c = c_begin; c < c_end; ++c) {
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int q = i * 256 + t;
      s_x[q % kLgC][q / kLgC] = (double)xv[i];
    }
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
      const int q = i * 256 + t;
      s_w[q % kLgC][q / kLgC] = (double)wv[i];
    }
    __syncthreads();
    if (c + 1 < c_end) fetch(c + 1);
    // lane l: A = x[token 16 mt + l % 16][column k], B = Wr[expert 16 w + l % 16][column k],
    // k = 4 ks + l / 16
#pragma unroll
    for (int ks = 0; ks < kLgC / 4; ++ks) {
      const int k = 4 * ks + (lane >> 4);
      const double b = s_w[k][16 * wave + (lane & 15)];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f64_16x16x4f64(s_x[k][16 * mt + (lane & 15)], b, acc[mt], 0, 0, 0);
    }
    __syncthreads();
  }
  // lane l, element i: token 16 mt + l / 16 + 4 i, expert 16 w + l % 16
  const int e = e0 + 16 * wave + (lane & 15);
  if (e < E) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * mt + (lane >> 4) + 4 * i;
        if (tok < nt) zp[((size_t)split * T + t0 + tok) * E + e] = acc[mt][i];
      }
  }
}

// ---------------------------------------------------------------- top-k
// One wave per token.  With nsplit > 1 the logits are the fixed-order sum of
// the per-range partials plus the bias, formed in LDS first.
// Bitonic top-k of one token by one wave, when every group of 64 experts'
// best K2 (k rounded up to a power of two) fit in the wave together (G K2 <=
// 64): each group is sorted into a run of its best K2 (odd groups reversed)
// in LDS, then the runs are merged pairwise, keeping the better half, down
// to the best K2.  cz, ce: this wave's 64-entry LDS scratch.
template <int K2>
__device__ __forceinline__ void wave_topk_bitonic(const double* zt, int E, int k, int32_t* idx_out,
                                                  float* w_out, double* cz, int* ce) {
  const int lane = threadIdx.x & 63;
  const int G = (E + 63) / 64;
  for (int g = 0; g < G; ++g) {
    const int e = g * 64 + lane;
    double z = e < E ? zt[e] : -INFINITY;
    int id = e < E ? e : INT_MAX;
    wave_best<K2>(z, id);
    if (lane < K2) {
      const int at = g * K2 + ((g & 1) ? K2 - 1 - lane : lane);
      cz[at] = z;
      ce[at] = id;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int span = K2;
  while (span < G * K2) span *= 2;
  double z = lane < G * K2 ? cz[lane] : -INFINITY;
  int id = lane < G * K2 ? ce[lane] : INT_MAX;
  merge_runs<K2, K2>(z, id, span);
  // k <= E puts k real experts first; the clamp only keeps a lookup in bounds
  topk_emit(z, (unsigned)id < (unsigned)E ? id : 0, k, idx_out, w_out);
}

// One token per wave, kTopkWaves waves per block.
constexpr int kTopkWaves = 1;
__global__ __launch_bounds__(64 * kTopkWaves) void k_topk(const double* __restrict__ z, int nsplit,
                                                          const float* __restrict__ bias, int T,
                                                          int E, int k, int32_t* __restrict__ idx,
                                                          float* __restrict__ w) {
  __shared__ double s_z[kTopkWaves][kMaxE];
  __shared__ double s_cz[kTopkWaves][64];
  __shared__ int s_ce[kTopkWaves][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkWaves + wave;
  if (t >= T) return;
  const double* zt = z + (size_t)t * E;
  if (nsplit > 1) {
    // the kLogSplit partial sums of two experts are requested before any is
    // added (then added in range order, as before)
#pragma unroll 2
    for (int e = lane; e < E; e += 64) {
      double p[kLogSplit];
#pragma unroll
      for (int s = 0; s < kLogSplit; ++s) p[s] = z[((size_t)s * T + t) * E + e];
      const double b = bias ? (double)bias[e] : 0.0;
      double v = 0.0;
#pragma unroll
      for (int s = 0; s < kLogSplit; ++s) v += p[s];
      s_z[wave][e] = v + b;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    zt = s_z[wave];
  }
  const int G = (E + 63) / 64;
  const int K2 = k <= 1 ? 1 : 1 << (32 - __builtin_clz(k - 1));
  int32_t* io = idx + (size_t)t * k;
  float* wo = w + (size_t)t * k;
  if (G * K2 <= 64) {
    double* cz = s_cz[wave];
    int* ce = s_ce[wave];
    switch (K2) {
      case 1: wave_topk_bitonic<1>(zt, E, k, io, wo, cz, ce); break;
      case 2: wave_topk_bitonic<2>(zt, E, k, io, wo, cz, ce); break;
      case 4: wave_topk_bitonic<4>(zt, E, k, io, wo, cz, ce); break;
      case 8: wave_topk_bitonic<8>(zt, E, k, io, wo, cz, ce); break;
      case 16: wave_topk_bitonic<16>(zt, E, k, io, wo, cz, ce); break;
      default: wave_topk_bitonic<32>(zt, E, k, io, wo, cz, ce); break;
    }
  } else {
    wave_topk(zt, E, k, io, wo);
  }
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
// For small batches, one launch computes every logit (bias added) and, for the
// GEMV path, the activations' digit form: one workgroup per expert computes
// that expert's logits for every token, and extra workgroups after them make
// the digit split in parallel (RMSNorm first if asked, recomputed in the same
// order in every workgroup so all agree bit for bit).  Top-k and the union
// run next in one workgroup: at the start of the gate/up kernel (GEMV path)
// or in k_route_small (grouped GEMM); nothing here waits on another
// workgroup.
// Router front end blocks: kRF threads, kRFW waves.  A token's logit is the
// same sum for any batch size: thread tid takes float4 columns tid + kRF m,
// then a wave reduction and sum_waves over the waves.
constexpr int kRF = 512;
constexpr int kRFW = kRF / 64;
static_assert(kRFW == 8, "sum_waves adds 8 wave sums");
__device__ __forceinline__ double sum_waves(const double (&p)[kRFW]) {
  return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

// Waves per row of the x pack: all 8 of a workgroup, one row per workgroup
// (an eighth of a 6144-column row per wave): the pack workgroups share
// compute units with the logit workgroups, and with 2 waves per row (4 rows a
// workgroup) they finished after the logits (8 tokens: 7.4-8 us against 6).
__host__ __device__ inline int rf_pack_waves(int) { return 8; }
__host__ __device__ inline int rf_pack_blocks(int rows) {
  const int rpb = kRFW / rf_pack_waves(rows);
  return (rows + rpb - 1) / rpb;
}

// Returns the workgroup's kind (trace tag): 1 logits, 2 x pack, 3 digit split.
template <int TB>
__device__ __forceinline__ int router_front_body(const RouterArgs& a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, d = a.d, E = a.E;
  // workgroups [0, E tsplit): the logits of expert bx % E for tokens t0 ..
  // t0 + Tl - 1 (tsplit > 1 only without RMSNorm or digit split); the others
  // are numbered as if tsplit were 1
  const int nlog = E * a.tsplit, bx = blockIdx.x;
  const int e = bx < nlog ? bx % E : bx - nlog + E;
  const int t0 = bx < nlog ? (bx / E) * TB : 0;
  const int Tl = bx < nlog ? min(TB, T - t0) : T;
  const int gx = (int)gridDim.x - nlog + E;
  // the last rf_pack_blocks workgroups pack the rows for the grouped GEMM,
  // alongside the logits, each row by rf_pack_waves waves
  const int pack_blocks = a.px.dst ? rf_pack_blocks(a.px.rows) : 0;
  if (pack_blocks) {
    const int pb = gx - pack_blocks;
    if (e >= pb) {
      __shared__ float s_m[kRFW];
      const int nw = rf_pack_waves(a.px.rows);
      const int r = (e - pb) * (kRFW / nw) + wave / nw;
      if (a.px.i8) {
        // int8 groups need no row-wide maximum: no barrier
        if (r < a.px.rows) pack_row_i8(a.px, r, lane, wave % nw, nw);
      } else {
        pack_row_split(a.px, r < a.px.rows ? r : -1, wave % nw, nw, s_m, wave, lane);
      }
      return 2;
    }
  }
  __shared__ double part[TB][kRFW];
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
  // Rows of up to 8192 columns stay in registers (4 float4 per thread): the
  // router row is requested before the RMSNorm reduction so the two overlap,
  // and a single token's x is read once.
  constexpr int kReg = 8192 / 4 / kRF;
  const int n4 = d >> 2;
  const bool in_regs = n4 <= kRF * kReg;
  float4 wr[kReg], xr[kReg];
  if (in_regs) {
#pragma unroll
    for (int m = 0; m < kReg; ++m) {
      const int i4 = tid + kRF * m;
      if (e < E && i4 < n4) wr[m] = reinterpret_cast<const float4*>(a.Wr + (size_t)e * d)[i4];
      if (TB == 1 && i4 < n4) xr[m] = xval4(t0, i4);
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
        if (tid + kRF * m < n4) {
          const float4 v = xr[m];
          ss[0] += (double)v.x * (double)v.x;
          ss[0] += (double)v.y * (double)v.y;
          ss[0] += (double)v.z * (double)v.z;
          ss[0] += (double)v.w * (double)v.w;
        }
      }
    } else {
      // the same partition and order as above (float4 i4 = tid + kRF m, its
      // four values in turn), so a token's sum does not depend on the batch.
      // Every row is read unconditionally (rows past the batch repeat the
      // last one and their sums are never used), so the loads of all rows
      // are in flight together.
      for (int i4 = tid; i4 < n4; i4 += kRF)
#pragma unroll
        for (int j = 0; j < TB; ++j) {
          const float4 v = xval4(TB == 1 ? 0 : (j < T ? j : T - 1), i4);
          ss[j] += (double)v.x * (double)v.x;
          ss[j] += (double)v.y * (double)v.y;
          ss[j] += (double)v.z * (double)v.z;
          ss[j] += (double)v.w * (double)v.w;
        }
    }
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const double sj = wave_sum(ss[j]);
      if (lane == 0) part[j][wave] = sj;
    }
    __syncthreads();
    if (tid < T) {
      const double tot = sum_waves(part[tid]);
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
    for (int it = (e - E) * kRFW + wave; it < T * nb;
         it += (gx - E - pack_blocks) * kRFW) {
      const int t = it / nb, col = (it % nb) * 64 + lane;
      if (a.i8)
        digitize64_i8(xin(t, col), col, true, a.xd.q + (size_t)t * nch * kChunkDigitBytes,
                      a.xd.sx + (size_t)t * ng, a.xd.sc + (size_t)t * ng);
      else
        digitize32(xin(t, col), col, true, a.xd.q + (size_t)t * nch * kChunkDigitBytes,
                   a.xd.sx + (size_t)t * ng, a.xd.sc + (size_t)t * ng);
    }
    return 3;
  }
  double acc[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) acc[j] = 0.0;
  if (in_regs) {
#pragma unroll
    for (int m = 0; m < kReg; ++m) {
      const int i4 = tid + kRF * m;
      if (i4 < n4) {
        const float4 w = wr[m];
#pragma unroll
        for (int j = 0; j < TB; ++j) {
          // unconditional loads (rows past the batch repeat the last one,
          // their sums are never stored): all rows' loads go out together
          const int jj = t0 + (TB == 1 ? 0 : (j < Tl ? j : Tl - 1));
          const float4 v = TB == 1 ? xr[m] : xval4(jj, i4);
          acc[j] += (double)w.x * (double)norm(jj, v.x);
          acc[j] += (double)w.y * (double)norm(jj, v.y);
          acc[j] += (double)w.z * (double)norm(jj, v.z);
          acc[j] += (double)w.w * (double)norm(jj, v.w);
        }
      }
    }
  } else {
    const float4* w4 = reinterpret_cast<const float4*>(a.Wr + (size_t)e * d);
    for (int i = tid; i < n4; i += kRF) {
      const float4 w = w4[i];
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        if (j < Tl) {
          acc[j] += (double)w.x * (double)xin(t0 + j, 4 * i);
          acc[j] += (double)w.y * (double)xin(t0 + j, 4 * i + 1);
          acc[j] += (double)w.z * (double)xin(t0 + j, 4 * i + 2);
          acc[j] += (double)w.w * (double)xin(t0 + j, 4 * i + 3);
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
  if (tid < Tl) {
    const double sj = sum_waves(part[tid]);
    a.z[(size_t)(t0 + tid) * E + e] = sj + (a.bias ? (double)a.bias[e] : 0.0);
  }
  return 1;
}

template <int TB>
__global__ __launch_bounds__(kRF) void k_router_front(RouterArgs a) {
  BlockTrace tr;
  tr.start();
  const int tag = router_front_body<TB>(a);
  tr.store(g_trace_route, 0, blockIdx.x, tag);
}

// ---------------------------------------------------------------- digit split
// One wave per 64 columns of a row; gather[r] (if given) selects the source
// row of output row r.  i8: integer activations (int8 per 64 columns).
__global__ __launch_bounds__(256) void k_digitize(const void* __restrict__ x, int x_bf16,
                                                  const int32_t* __restrict__ gather, int rows,
                                                  int K, Digits out, int i8) {
  const int lane = threadIdx.x & 63;
  const int nb = K / 64, nch = K / kChunk, ng = K / kXGroup;
  const long items = (long)rows * nb;
  for (long it = (long)blockIdx.x * 4 + (threadIdx.x >> 6); it < items; it += (long)gridDim.x * 4) {
    const int r = (int)(it / nb), col = (int)(it % nb) * 64 + lane;
    const int src = gather ? gather[r] : r;
    const size_t i = (size_t)src * K + col;
    const float v = x_bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(x)[i] << 16)
                           : static_cast<const float*>(x)[i];
    if (i8)
      digitize64_i8(v, col, true, out.q + (size_t)r * nch * kChunkDigitBytes,
                    out.sx + (size_t)r * ng, out.sc + (size_t)r * ng);
    else
      digitize32(v, col, true, out.q + (size_t)r * nch * kChunkDigitBytes,
                 out.sx + (size_t)r * ng, out.sc + (size_t)r * ng);
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_rmsnorm(const float* h, float* xn, int T, int d, float eps, hipStream_t s) {
  return launch(0, k_rmsnorm, dim3(T), dim3(256), s, h, xn, d, eps);
}

hipError_t launch_logits(const void* x, int x_bf16, int T, int d, int E, const float* Wr,
                         double* zp, hipStream_t s) {
  const dim3 grid((unsigned)(kLogSplit * ((T + kLgT - 1) / kLgT) * ((E + kLgE - 1) / kLgE)));
  return launch(1, k_logits, grid, dim3(256), s, x, x_bf16, T, d, E, Wr, zp);
}

hipError_t launch_topk(const double* z, int nsplit, const float* bias, int T, int E, int k,
                       int32_t* idx, float* w, hipStream_t s) {
  if (nsplit != 1 && nsplit != kLogSplit) return hipErrorInvalidValue;
  return launch(2, k_topk, dim3((T + kTopkWaves - 1) / kTopkWaves), dim3(64 * kTopkWaves), s, z,
                nsplit, bias, T, E, k, idx, w);
}

hipError_t launch_union(const int32_t* idx, int T, int E, int k, int32_t* uniq, int32_t* n_uniq,
                        int32_t* offsets, int32_t* rows, int32_t* stats, hipStream_t s) {
  return launch(3, k_union, dim3(1), dim3(kUnionThreads), s, idx, T, E, k, uniq, n_uniq, offsets,
                rows, stats);
}

hipError_t launch_router_front(const RouterArgs& a_in, hipStream_t s) {
  RouterArgs a = a_in;
  const int dig_blocks = a.xd.q ? (a.T * (a.d / 64) + kRFW - 1) / kRFW : 0;
  if (a.px.dst && (a.px.K % 8 != 0 || a.px.rows < 1 || (a.px.i8 && a.px.K % 512 != 0)))
    return hipErrorInvalidValue;
  const int pack_blocks = a.px.dst ? rf_pack_blocks(a.px.rows) : 0;
  // without RMSNorm and digit split (the grouped GEMM's small batches), 5 to
  // 8 tokens take two workgroups per expert, each over its own tokens
  a.tsplit = (!dig_blocks && !a.prenorm && a.T > 4) ? 2 : 1;
  const dim3 grid(a.E * a.tsplit + dig_blocks + pack_blocks);
  if (a.T <= 1) return launch(1, k_router_front<1>, grid, dim3(kRF), s, a);
  if (a.T <= 2) return launch(1, k_router_front<2>, grid, dim3(kRF), s, a);
  if (a.T <= 4 || a.tsplit == 2) return launch(1, k_router_front<4>, grid, dim3(kRF), s, a);
  return launch(1, k_router_front<8>, grid, dim3(kRF), s, a);
}

hipError_t launch_digitize(const void* x, int x_bf16, const int32_t* gather, int rows, int K,
                           Digits out, hipStream_t s, int i8) {
  const long items = (long)rows * (K / kGroup);
  const long blocks = (items + 3) / 4;
  const int grid = (int)(blocks < 4096 ? blocks : 4096);
  return launch(4, k_digitize, dim3(grid), dim3(256), s, x, x_bf16, gather, rows, K, out, i8);
}

}  // namespace moe

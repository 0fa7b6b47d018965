// Expert FFN for decode-sized batches: fused int4 dequant GEMVs on gfx950.
//
// Each chosen expert runs its feed-forward computation once per batch over all
// tokens that picked it (colibri 技术解读 (linlog.top), "集群模式与开放问题清单";
// batch union: colibrì README (简体中文), 工作原理 › 绝不为同一次磁盘读取等待两遍).
// The expert is y = Wd (silu(Wg x) * (Wu x)) on signed int4 weights with one
// fp16 scale per 64 inputs.
//
// HBM-bound design: every lane streams its rows' 4-bit codes with coalesced
// 16-byte loads (64 lanes cover 1 KB of a row per instruction), applies the
// fp16 group scale in registers and the wave reduces each row across lanes.
// The int4 x activation products are exact integer dot products
// (v_dot4_i32_i8 on the activation's three int8 digit planes), so one weight
// costs about 1.3 VALU operations — well inside the ~2.6 per weight that the
// chip's vector rate allows at full HBM bandwidth.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {

constexpr int kRowsPerWave = 16;
constexpr int kWaves = 4;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;  // = kGroup: one group of a per block

struct ExpertRef {
  const uint8_t* blob;
  int beg, n;
};

__device__ __forceinline__ ExpertRef expert_ref(const ExpertList& L, int u) {
  ExpertRef r;
  if (L.single) {
    r.blob = L.single;
    r.beg = 0;
    r.n = L.single_n;
  } else {
    r.blob = L.table[L.uniq[u]];
    r.beg = L.offsets[u];
    r.n = L.offsets[u + 1] - r.beg;
  }
  return r;
}

__device__ __forceinline__ int slot_of(const ExpertList& L, const ExpertRef& x, int i) {
  return L.single ? i : L.list[x.beg + i];
}

// Gate/up: block (rb, u) computes rows [64 rb, 64 rb + 64) of gate and up of
// union expert u for all its tokens, forms a = silu(g) * u and stores that
// 64-wide group of a in digit form, ready for the down projection.
// CPL = 16-byte code chunks per lane per pass (d = 6144 -> 192 chunks -> 3,
// one pass); NT = tokens whose digits a lane holds in registers at a time.
template <int CPL, int NT>
__global__ __launch_bounds__(256) void k_gateup(ExpertList L, int d, int f, Digits xd, Digits ad) {
  const int u = blockIdx.y;
  if (!L.single && u >= *L.n_uniq) return;
  const ExpertRef ex = expert_ref(L, u);
  const int rb = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = d / kChunk, ngx = d / kGroup;
  const size_t fd = (size_t)f * d;
  const uint8_t* gcode = ex.blob;
  const uint8_t* ucode = ex.blob + fd / 2;
  const _Float16* gsc = reinterpret_cast<const _Float16*>(ex.blob + 3 * fd / 2);
  const _Float16* usc = gsc + fd / kGroup;
  const int r0 = rb * kRowsPerBlock + wave * kRowsPerWave;
  __shared__ float s_g[NT][kRowsPerBlock], s_u[NT][kRowsPerBlock];

  for (int t0 = 0; t0 < ex.n; t0 += NT) {
    const int nt = min(NT, ex.n - t0);
    int xrow[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) xrow[j] = j < nt ? slot_of(L, ex, t0 + j) / L.kdiv : 0;
    for (int c0 = 0; c0 < nch; c0 += 64 * CPL) {
      ChunkDigits xdig[CPL][NT];
      int xs[CPL][NT];
      float xc[CPL][NT];
      bool act[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = c0 + lane + 64 * i;
        act[i] = c < nch;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          if (act[i] && j < nt) {
            xdig[i][j] = load_chunk_digits(xd.q + ((size_t)xrow[j] * nch + c) * kChunkDigitBytes);
            xs[i][j] = xd.sx[(size_t)xrow[j] * nch + c];
            xc[i][j] = xd.sc[(size_t)xrow[j] * ngx + c / 2];
          } else {
            xdig[i][j] = ChunkDigits{};
            xs[i][j] = 0;
            xc[i][j] = 0.0f;
          }
        }
      }
#pragma unroll 2
      for (int rr = 0; rr < kRowsPerWave; ++rr) {
        const size_t r = (size_t)(r0 + rr);
        uint4 wg[CPL], wu[CPL];
        float sg[CPL], su[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = c0 + lane + 64 * i;
          if (act[i]) {
            wg[i] = *reinterpret_cast<const uint4*>(gcode + r * (d / 2) + (size_t)c * 16);
            wu[i] = *reinterpret_cast<const uint4*>(ucode + r * (d / 2) + (size_t)c * 16);
            sg[i] = f16_to_f32(gsc + r * ngx + c / 2);
            su[i] = f16_to_f32(usc + r * ngx + c / 2);
          }
        }
        float ag[NT], au[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) ag[j] = au[j] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          if (!act[i]) continue;
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const int pg = chunk_dot(wg[i], xdig[i][j]) - 8 * xs[i][j];
            const int pu = chunk_dot(wu[i], xdig[i][j]) - 8 * xs[i][j];
            ag[j] += (float)pg * (sg[i] * xc[i][j]);
            au[j] += (float)pu * (su[i] * xc[i][j]);
          }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const float g = wave_sum(ag[j]);
          const float uu = wave_sum(au[j]);
          if (lane == 0) {
            const int row = wave * kRowsPerWave + rr;
            s_g[j][row] = c0 == 0 ? g : s_g[j][row] + g;
            s_u[j][row] = c0 == 0 ? uu : s_u[j][row] + uu;
          }
        }
      }
    }
    __syncthreads();
    for (int j = wave; j < nt; j += kWaves) {
      const int slot = slot_of(L, ex, t0 + j);
      const int nca = f / kChunk, nga = f / kGroup;
      const float a = silu(s_g[j][lane]) * s_u[j][lane];
      digitize_group(a, lane, rb, ad.q + (size_t)slot * nca * kChunkDigitBytes,
                     ad.sx + (size_t)slot * nca, ad.sc + (size_t)slot * nga);
    }
    __syncthreads();
  }
}

// Down: block (rb, u) computes rows [64 rb, 64 rb + 64) of y = Wd a for every
// token of union expert u; y is indexed by slot.
template <int CPL, int NT>
__global__ __launch_bounds__(256) void k_down(ExpertList L, int d, int f, Digits ad,
                                              float* __restrict__ y) {
  const int u = blockIdx.y;
  if (!L.single && u >= *L.n_uniq) return;
  const ExpertRef ex = expert_ref(L, u);
  const int rb = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = f / kChunk, nga = f / kGroup;
  const size_t fd = (size_t)f * d;
  const uint8_t* dcode = ex.blob + fd;
  const _Float16* dsc = reinterpret_cast<const _Float16*>(ex.blob + 3 * fd / 2) + 2 * (fd / kGroup);
  const int r0 = rb * kRowsPerBlock + wave * kRowsPerWave;
  __shared__ float s_y[NT][kRowsPerBlock];

  for (int t0 = 0; t0 < ex.n; t0 += NT) {
    const int nt = min(NT, ex.n - t0);
    int slot[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) slot[j] = j < nt ? slot_of(L, ex, t0 + j) : 0;
    for (int c0 = 0; c0 < nch; c0 += 64 * CPL) {
      ChunkDigits adig[CPL][NT];
      int as[CPL][NT];
      float ac[CPL][NT];
      bool act[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = c0 + lane + 64 * i;
        act[i] = c < nch;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          if (act[i] && j < nt) {
            adig[i][j] = load_chunk_digits(ad.q + ((size_t)slot[j] * nch + c) * kChunkDigitBytes);
            as[i][j] = ad.sx[(size_t)slot[j] * nch + c];
            ac[i][j] = ad.sc[(size_t)slot[j] * nga + c / 2];
          } else {
            adig[i][j] = ChunkDigits{};
            as[i][j] = 0;
            ac[i][j] = 0.0f;
          }
        }
      }
#pragma unroll 8
      for (int rr = 0; rr < kRowsPerWave; ++rr) {
        const size_t r = (size_t)(r0 + rr);
        uint4 wd[CPL];
        float sd[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = c0 + lane + 64 * i;
          if (act[i]) {
            wd[i] = *reinterpret_cast<const uint4*>(dcode + r * (f / 2) + (size_t)c * 16);
            sd[i] = f16_to_f32(dsc + r * nga + c / 2);
          }
        }
        float acc[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          if (!act[i]) continue;
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const int p = chunk_dot(wd[i], adig[i][j]) - 8 * as[i][j];
            acc[j] += (float)p * (sd[i] * ac[i][j]);
          }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const float sum = wave_sum(acc[j]);
          if (lane == 0) {
            const int row = wave * kRowsPerWave + rr;
            s_y[j][row] = c0 == 0 ? sum : s_y[j][row] + sum;
          }
        }
      }
    }
    __syncthreads();
    for (int j = wave; j < nt; j += kWaves) y[(size_t)slot[j] * d + rb * kRowsPerBlock + lane] = s_y[j][lane];
    __syncthreads();
  }
}

// out[t][c] = (x[t][c] if resid) + sum_j w[t][j] * y[t*k + j][c], ascending j.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const float* __restrict__ w, const float* resid,
                                                 float* out, int d, int k) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  float acc = 0.0f;
  for (int j = 0; j < k; ++j) acc += w[(size_t)t * k + j] * y[((size_t)t * k + j) * d + c];
  if (resid) acc = resid[(size_t)t * d + c] + acc;
  out[(size_t)t * d + c] = acc;
}

hipError_t launch_gateup(const ExpertList& L, int max_experts, int d, int f, Digits xd, Digits ad,
                         hipStream_t s) {
  const dim3 grid(f / kRowsPerBlock, max_experts);
  hipLaunchKernelGGL((k_gateup<3, 1>), grid, dim3(256), 0, s, L, d, f, xd, ad);
  return hipGetLastError();
}

hipError_t launch_down(const ExpertList& L, int max_experts, int d, int f, Digits ad, float* y,
                       hipStream_t s) {
  const dim3 grid(d / kRowsPerBlock, max_experts);
  hipLaunchKernelGGL((k_down<1, 1>), grid, dim3(256), 0, s, L, d, f, ad, y);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y, const float* w, const float* resid, float* out, int T,
                          int d, int k, hipStream_t s) {
  hipLaunchKernelGGL(k_combine, dim3((d + 255) / 256, T), dim3(256), 0, s, y, w, resid, out, d, k);
  return hipGetLastError();
}

}  // namespace moe

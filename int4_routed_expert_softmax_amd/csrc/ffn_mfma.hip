// Expert FFN for multi-token batches (prefill, batched verification): a
// grouped GEMM on the MFMA units.
//
// Each chosen expert runs its feed-forward computation once per batch over all
// of its tokens, so its bytes are read once (colibri 技术解读 (linlog.top),
// "集群模式与开放问题清单"; colibrì README (简体中文), 工作原理 › 绝不为同一次磁盘读取等待两遍).
//
// Operands of v_mfma_f32_16x16x32_f16 (fp32 accumulate):
//  - B (weights): a wave owns 64 weight rows.  Their int4 codes arrive in
//    512-column stages through wave-private LDS (coalesced 256-byte row
//    pieces, prefetched one stage ahead into registers) and are dequantised in
//    registers: a code becomes the fp16 number 1032 + q (one AND/OR per two
//    codes), 1032 is subtracted exactly, and the product with the group's fp16
//    scale is rounded once to fp16.
//  - A (activations): rows in fp16 scaled by a power of two per row (k_pack)
//    and read straight from L2; the row's power of two multiplies the result.
// A 32-bit word of 8 codes splits into fp16 pairs (column j, column j + 4),
// so k_pack stores each block of 8 columns in that order: position p holds
// column (p >> 1) + 4 (p & 1).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4* g_u32x4_ptr;

constexpr int kNt = 4;                               // 16-row N-tiles per wave
constexpr int kWaveRows = kNt * 16;                  // weight rows per wave
constexpr int kGWaves = 4;                           // waves per block
constexpr int kStageCols = 512;                      // columns per LDS stage
constexpr int kStageBytes = kStageCols / 2;          // code bytes per row per stage
constexpr int kStagePieces = kWaveRows * kStageBytes / 16 / 64;  // 16-byte loads per lane
constexpr int kLdsStride = kStageBytes + 8;          // padded LDS row (bytes)
constexpr int kPackExp = 14;                         // packed |value| < 2^14

__device__ __forceinline__ int slot_of_col(int e) { return 2 * (e & 3) + (e >> 2); }

__device__ __forceinline__ u32x4 nt_load16(const uint8_t* p) {
  return __builtin_nontemporal_load((g_u32x4_ptr)(p));
}

// 8 codes (a 32-bit word, column j in bits 4j..4j+3) times one fp16 scale ->
// 8 fp16 weights in slot order (col 0, 4, 1, 5, 2, 6, 3, 7).
__device__ __forceinline__ f16x8 dequant8(uint32_t w, f16x2 s2) {
  const uint32_t v = w ^ 0x88888888u;  // offset binary: q + 8
  const f16x2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t h = ((v >> (4 * j)) & 0x000F000Fu) | 0x64006400u;  // 1024 + q + 8
    const f16x2 q = __builtin_bit_cast(f16x2, h) - off;               // exact
    const f16x2 ws = q * s2;                                          // one rounding
    r[2 * j] = ws[0];
    r[2 * j + 1] = ws[1];
  }
  return r;
}

// Index of the last entry of the ascending prefix p[0..n] that is <= j.
__device__ __forceinline__ int find_bucket(const int32_t* p, int n, int j) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p[mid] <= j) lo = mid;
    else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------- packing
// One wave per row: max |v| over the row, then fp16(v * 2^(14 - e)) with
// max|v| < 2^e, columns permuted within blocks of 8; unit[r] = 2^(e - 14).
// With mbo set, the last block instead writes the union's M-block prefix:
// mbo[u] = sum over u' < u of ceil(count(u') / mblock), u = 0..U.
struct PackArgs {
  const void* src;
  int src_bf16, K, rows;
  const int32_t* gather;  // source row of row r (nullptr: r)
  _Float16* dst;          // [rows][K]
  float* unit;            // [rows]
  const int32_t* offsets;
  const int32_t* n_uniq;
  int32_t* mbo;
  int mblock;
};

__device__ __forceinline__ void load8(const void* src, int bf16, size_t i, float (&v)[8]) {
  if (bf16) {
    const uint4 b = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + i);
    const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + i);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + i + 4);
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w;
    v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
  }
}

__global__ __launch_bounds__(256) void k_pack(PackArgs p) {
  if (p.mbo && blockIdx.x == gridDim.x - 1) {
    __shared__ int s_tot[4];
    const int U = *p.n_uniq, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = 4 * t + i;
      c[i] = u < U ? (p.offsets[u + 1] - p.offsets[u] + p.mblock - 1) / p.mblock : 0;
      sum += c[i];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int nb = __shfl_up(incl, o, 64);
      if (lane >= o) incl += nb;
    }
    if (lane == 63) s_tot[wave] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < wave; ++w) run += s_tot[w];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = 4 * t + i;
      if (u < U) p.mbo[u] = run;
      run += c[i];
    }
    if (t == 0) p.mbo[U] = s_tot[0] + s_tot[1] + s_tot[2] + s_tot[3];
    return;
  }
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= p.rows) return;
  const int lane = threadIdx.x & 63;
  const size_t src_row = p.gather ? (size_t)p.gather[r] : (size_t)r;
  const size_t base = src_row * p.K;
  float m = 0.0f;
  for (int c = lane * 8; c < p.K; c += 512) {
    float v[8];
    load8(p.src, p.src_bf16, base + c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  }
  m = wave_max(m);
  int e = 0;
  if (m > 0.0f) frexpf(m, &e);  // m < 2^e
  const float up = m > 0.0f ? ldexpf(1.0f, kPackExp - e) : 1.0f;
  _Float16* drow = p.dst + (size_t)r * p.K;
  for (int c = lane * 8; c < p.K; c += 512) {
    float v[8];
    load8(p.src, p.src_bf16, base + c, v);
    f16x8 h;
#pragma unroll
    for (int j = 0; j < 8; ++j) h[slot_of_col(j)] = (_Float16)(v[j] * up);
    *reinterpret_cast<f16x8*>(drow + c) = h;
  }
  if (lane == 0) p.unit[r] = m > 0.0f ? ldexpf(1.0f, e - kPackExp) : 1.0f;
}

// ---------------------------------------------------------------- projection
enum { kGateUp = 0, kDown = 1 };

struct GemmArgs {
  ExpertList L;
  const int32_t* mbo;  // union M-block prefix (unused for a single expert)
  int d, f;
  const _Float16* a;   // packed A rows
  const float* unit;   // their units
  float* out;          // gate/up: silu(g) * u [slots][f]; down: y [slots][d]
};

// One block: 4 independent waves (no block-wide barrier), each owning 64
// weight rows (gate/up: 32 rows of gate and the same 32 rows of up), times one
// M-block of up to 16 * MW tokens of one expert.
template <int MODE, int MW>
__global__ __launch_bounds__(64 * kGWaves) void k_gemm(GemmArgs g) {
  constexpr int MB = 16 * MW;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wv = blockIdx.x * kGWaves + wave;
  const int d = g.d, f = g.f;
  const int K = MODE == kGateUp ? d : f;
  const int nwaves = MODE == kGateUp ? f / 32 : d / kWaveRows;
  if (wv >= nwaves) return;

  const ExpertList& L = g.L;
  int off, cnt, tok0;
  const uint8_t* blob;
  if (L.single) {
    off = 0;
    cnt = L.single_n;
    tok0 = blockIdx.y * MB;
    if (tok0 >= cnt) return;
    blob = L.single;
  } else {
    const int U = *L.n_uniq;
    const int j = blockIdx.y;
    if (j >= g.mbo[U]) return;
    const int u = find_bucket(g.mbo, U, j);
    off = L.offsets[u];
    cnt = L.offsets[u + 1] - off;
    tok0 = (j - g.mbo[u]) * MB;
    blob = L.table[L.uniq[u]];
  }
  const int ntok = min(MB, cnt - tok0);
  const int nmt = (ntok + 15) >> 4;
  const int n = lane & 15, kg = lane >> 4;

  // A rows of this lane (row n of every M-tile); rows past the expert's last
  // token repeat its last token and are dropped in the epilogue
  uint32_t arow[MW];
#pragma unroll
  for (int mt = 0; mt < MW; ++mt) {
    const int i = min(tok0 + 16 * mt + n, cnt - 1);
    int r = i;
    if (!L.single) {
      const int slot = L.list[off + i];
      r = MODE == kGateUp ? slot / L.kdiv : slot;
    }
    arow[mt] = (uint32_t)r * (uint32_t)K;
  }

  // weight rows: LDS rows 0..31 and 32..63 come from two base pointers
  const size_t fd = (size_t)f * d;
  const int ng = K / 64;
  const _Float16* sbase = reinterpret_cast<const _Float16*>(blob + 3 * (fd / 2));
  const uint8_t *c0, *c1;
  const _Float16 *s0, *s1;
  if (MODE == kGateUp) {
    c0 = blob + (size_t)(32 * wv) * (K / 2);
    c1 = c0 + fd / 2;
    s0 = sbase + (size_t)(32 * wv) * ng;
    s1 = s0 + fd / 64;
  } else {
    c0 = blob + fd + (size_t)(64 * wv) * (K / 2);
    c1 = c0 + (size_t)32 * (K / 2);
    s0 = sbase + 2 * (fd / 64) + (size_t)(64 * wv) * ng;
    s1 = s0 + (size_t)32 * ng;
  }

  __shared__ __attribute__((aligned(16))) uint8_t s_codes[kGWaves * kWaveRows * kLdsStride];
  uint8_t* s_b = s_codes + wave * kWaveRows * kLdsStride;

  // stage prefetch: piece p = lane + 64 i covers LDS row p / 16 (i < 8: base
  // c0, rows 4 i + lane / 16) and 16 bytes at (p % 16) * 16 of the stage
  const uint32_t lrow = lane >> 4, lpiece = lane & 15;
  const uint32_t lane_off = lrow * (uint32_t)(K / 2) + lpiece * 16u;
  const int nst = (K + kStageCols - 1) / kStageCols;
  u32x4 pre[kStagePieces];
  uint4 spre[kNt];  // 8 fp16 scales per tile
  auto fetch = [&](int st) {
    const uint32_t so = (uint32_t)st * kStageBytes;
    const bool full = (st + 1) * kStageCols <= K;
    const bool piece_ok = full || so + lpiece * 16u < (uint32_t)(K / 2);
#pragma unroll
    for (int i = 0; i < kStagePieces; ++i) {
      const uint8_t* cb = i < kStagePieces / 2 ? c0 : c1;
      const uint32_t ro = (uint32_t)(4 * (i % (kStagePieces / 2))) * (uint32_t)(K / 2);
      pre[i] = piece_ok ? nt_load16(cb + ro + so + lane_off) : u32x4{0u, 0u, 0u, 0u};
    }
    // scales of rows 16 nt + n, groups 8 st .. 8 st + 7
#pragma unroll
    for (int nt = 0; nt < kNt; ++nt) {
      const _Float16* sr = (nt < 2 ? s0 : s1) + (size_t)(16 * (nt & 1) + n) * ng;
      if ((ng & 7) == 0) {
        spre[nt] = *reinterpret_cast<const uint4*>(sr + 8 * st);
      } else {
        uint16_t h[8];
#pragma unroll
        for (int gg = 0; gg < 8; ++gg)
          h[gg] = __builtin_bit_cast(uint16_t, sr[min(8 * st + gg, ng - 1)]);
        spre[nt] = make_uint4(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16,
                              h[4] | (uint32_t)h[5] << 16, h[6] | (uint32_t)h[7] << 16);
      }
    }
  };

  f32x4 acc[MW][kNt];
#pragma unroll
  for (int mt = 0; mt < MW; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNt; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto kblock = [&](int st, int kb, const uint4 (&sc)[kNt]) {
    f16x8 b[kNt];
#pragma unroll
    for (int nt = 0; nt < kNt; ++nt) {
      const uint32_t w =
          *reinterpret_cast<const uint32_t*>(s_b + (16 * nt + n) * kLdsStride + kb * 16 + 4 * kg);
      const int gg = kb >> 1;
      const uint32_t word = (gg >> 1) == 0 ? sc[nt].x : (gg >> 1) == 1 ? sc[nt].y
                            : (gg >> 1) == 2 ? sc[nt].z : sc[nt].w;
      const uint32_t h = (gg & 1) ? word >> 16 : word & 0xFFFFu;
      b[nt] = dequant8(w, __builtin_bit_cast(f16x2, h | h << 16));
    }
    const uint32_t col = (uint32_t)(st * kStageCols + kb * 32 + 8 * kg);
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) {
      if (mt < nmt) {
        const f16x8 av = *reinterpret_cast<const f16x8*>(g.a + arow[mt] + col);
#pragma unroll
        for (int nt = 0; nt < kNt; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b[nt], acc[mt][nt], 0, 0, 0);
      }
    }
  };

  fetch(0);
  for (int st = 0; st < nst; ++st) {
#pragma unroll
    for (int i = 0; i < kStagePieces; ++i) {
      const int p = lane + 64 * i;
      uint8_t* dst = s_b + (p >> 4) * kLdsStride + (p & 15) * 16;
      *reinterpret_cast<uint2*>(dst) = make_uint2(pre[i].x, pre[i].y);
      *reinterpret_cast<uint2*>(dst + 8) = make_uint2(pre[i].z, pre[i].w);
    }
    uint4 sc[kNt];
#pragma unroll
    for (int nt = 0; nt < kNt; ++nt) sc[nt] = spre[nt];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (st + 1 < nst) fetch(st + 1);
    const int nkb = min(kStageCols, K - st * kStageCols) / 32;
    if (nkb == kStageCols / 32) {
#pragma unroll
      for (int kb = 0; kb < kStageCols / 32; ++kb) kblock(st, kb, sc);
    } else {
      for (int kb = 0; kb < nkb; ++kb) kblock(st, kb, sc);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // epilogue: lane (n, kg) holds, per tile, tokens 4 kg + i of the M-tile for
  // weight row 16 nt + n
#pragma unroll
  for (int mt = 0; mt < MW; ++mt) {
    if (mt >= nmt) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tok0 + 16 * mt + 4 * kg + i;
      if (t >= cnt) continue;
      const int slot = L.single ? t : L.list[off + t];
      if (MODE == kGateUp) {
        const int xr = L.single ? t : slot / L.kdiv;
        const float us = g.unit[xr];
        float* orow = g.out + (size_t)slot * f + 32 * wv;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float gv = acc[mt][h][i] * us, uv = acc[mt][h + 2][i] * us;
          orow[16 * h + n] = silu(gv) * uv;
        }
      } else {
        const float us = g.unit[slot];
        float* orow = g.out + (size_t)slot * d + kWaveRows * wv;
#pragma unroll
        for (int nt = 0; nt < kNt; ++nt) orow[16 * nt + n] = acc[mt][nt][i] * us;
      }
    }
  }
}

// ---------------------------------------------------------------- launchers

constexpr int kMfmaMW = 4;
constexpr int kMBlock = 16 * kMfmaMW;

int mfma_mblock() { return kMBlock; }

hipError_t launch_ffn_mfma(const MfmaArgs& m, hipStream_t s) {
  const ExpertList& L = m.L;
  hipError_t e;
  // x rows -> fp16 (and the union's M-block prefix)
  PackArgs px{};
  px.src = m.x;
  px.src_bf16 = m.x_bf16;
  px.K = m.d;
  px.rows = m.x_rows;
  px.gather = m.x_gather;
  px.dst = m.xh;
  px.unit = m.xunit;
  if (!L.single) {
    px.offsets = L.offsets;
    px.n_uniq = L.n_uniq;
    px.mbo = m.mbo;
    px.mblock = kMBlock;
  }
  const unsigned gx = (unsigned)((m.x_rows + 3) / 4) + (L.single ? 0u : 1u);
  e = launch(4, k_pack, dim3(gx), dim3(256), s, px);
  if (e != hipSuccess) return e;

  const unsigned mb = L.single ? (unsigned)((L.single_n + kMBlock - 1) / kMBlock)
                               : (unsigned)m.mb_bound;
  GemmArgs ga{L, m.mbo, m.d, m.f, m.xh, m.xunit, m.a32};
  const unsigned wg = (unsigned)((m.f / 32 + kGWaves - 1) / kGWaves);
  e = launch(5, k_gemm<kGateUp, kMfmaMW>, dim3(wg, mb), dim3(64 * kGWaves), s, ga);
  if (e != hipSuccess) return e;

  PackArgs pa{};
  pa.src = m.a32;
  pa.K = m.f;
  pa.rows = m.slots;
  pa.dst = m.ah;
  pa.unit = m.aunit;
  e = launch(4, k_pack, dim3((unsigned)((m.slots + 3) / 4)), dim3(256), s, pa);
  if (e != hipSuccess) return e;

  GemmArgs gd{L, m.mbo, m.d, m.f, m.ah, m.aunit, m.y};
  const unsigned wd = (unsigned)((m.d / kWaveRows + kGWaves - 1) / kGWaves);
  return launch(6, k_gemm<kDown, kMfmaMW>, dim3(wd, mb), dim3(64 * kGWaves), s, gd);
}

}  // namespace moe

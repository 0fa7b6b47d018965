// Activation rows -> the grouped GEMM's fp16 A operand, and the union's
// M-block map.  Used by k_pack (any batch) and by the one-block small-batch
// routing kernel, which packs the batch's rows after routing it.
//
// A row is scaled by a power of two so that max|v| < 2^14 and rounded to fp16
// (relative 2^-12): x' = fp16(v * 2^(14 - e)) with max|v| < 2^e, and
// unit[r] = 2^(e - 14), so x = x' * unit.  Within every block of 8 columns,
// position p holds column (p >> 1) + 4 (p & 1): the order in which the GEMM's
// dequantisation splits a 32-bit word of 8 codes into fp16 pairs.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {

constexpr int kPackExp = 14;  // packed |x'| < 2^14

__device__ __forceinline__ int slot_of_col(int e) { return 2 * (e & 3) + (e >> 2); }

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

// The thin grouped GEMM feeds the codes to the matrix cores as the fp16
// subnormals (q + o) * 2^-24 (o = corr_off: 8 for int4) and starts each
// 64-column group's partial sum at -o * 2^-24 * (sum of the group's packed
// values), which makes the partial
// 2^-24 * sum of q * x'.  corr_of8 sums a lane's 8 packed values (as stored),
// the 8 lanes of a 64-column group add theirs with a DPP butterfly (quad
// swaps, then the half-row mirror pairs the two quads), and the group's first
// lane writes the correction.  fp32 in a fixed order: its rounding (about
// 2^-24 of 8 |sum x'|) is some 2^-18 of a group's partial.
__device__ __forceinline__ float corr_of8(const float (&v)[8], float up) {
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (float)(_Float16)(v[j] * up);
  return s;
}
__device__ __forceinline__ void store_corr(const PackArgs& p, int r, int c, float s, int lane) {
  s += dpp<kDppXor1>(s);
  s += dpp<kDppXor2>(s);
  s += dpp<kDppHalfMirror>(s);
  if ((lane & 7) == 0) p.corr[(size_t)r * (p.K / 64) + c / 64] = -p.corr_off * 0x1p-24f * s;
}

// Rows of up to kPackRegCols columns are read once into registers (every
// load of the row in flight together), longer ones twice (max, then convert).
constexpr int kPackRegChunks = 12;                   // 8-column chunks per lane
constexpr int kPackRegCols = 64 * 8 * kPackRegChunks;  // 6144

__device__ __forceinline__ void store8(_Float16* drow, int c, const float (&v)[8], float up) {
  typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
  _Float16 h[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) h[slot_of_col(j)] = (_Float16)(v[j] * up);
  f16x8_t hv;
#pragma unroll
  for (int j = 0; j < 8; ++j) hv[j] = h[j];
  *reinterpret_cast<f16x8_t*>(drow + c) = hv;
}

// Integer activations: row r of p as int8, each 64-column group as q = v / s
// rounded to the nearest integer (ties to even), s = max|v| / 127, both in
// fp32 (a group of zeros: s = 0, q = 0); q in column order into dst (bytes),
// s into corr[r][K / 64].  A whole wave takes the row's 512-column chunks
// part, part + nw, ... (one wave: all of them); K is a multiple of 512, so
// in every step all 64 lanes hold a chunk and the 8 lanes of a group take its
// maximum with DPP (quad swaps, then the half-row mirror pairs the two
// quads).  No group spans two chunks, so the waves of a row need no exchange.
__device__ __forceinline__ void pack_row_i8(const PackArgs& p, int r, int lane, int part = 0,
                                            int nw = 1) {
  const size_t base = (p.gather ? (size_t)p.gather[r] : (size_t)r) * p.K;
  int8_t* drow = reinterpret_cast<int8_t*>(p.dst) + (size_t)r * p.K;
  for (int c = (part * 64 + lane) * 8; c < p.K; c += 512 * nw) {
    float v[8];
    load8(p.src, p.src_bf16, base + c, v);
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    m = fmaxf(m, dpp<kDppXor1>(m));
    m = fmaxf(m, dpp<kDppXor2>(m));
    m = fmaxf(m, dpp<kDppHalfMirror>(m));
    const float s = m / 127.0f;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float q = m > 0.0f ? fminf(fmaxf(rintf(v[j] / s), -127.0f), 127.0f) : 0.0f;
      w[j >> 2] |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * (j & 3));
    }
    *reinterpret_cast<uint2*>(drow + c) = make_uint2(w[0], w[1]);
    if ((lane & 7) == 0) p.corr[(size_t)r * (p.K / 64) + c / 64] = s;
  }
  if (part == 0 && lane == 0 && p.unit) p.unit[r] = 1.0f;
}

// Row r of p, by one whole wave (lane = its lane).
__device__ __forceinline__ void pack_row(const PackArgs& p, int r, int lane) {
  const size_t src_row = p.gather ? (size_t)p.gather[r] : (size_t)r;
  const size_t base = src_row * p.K;
  if (p.K <= kPackRegCols) {
    float v[kPackRegChunks][8];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kPackRegChunks; ++i) {
      const int c = (i * 64 + lane) * 8;
      if (c < p.K) {
        load8(p.src, p.src_bf16, base + c, v[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[i][j]));
      }
    }
    m = wave_max(m);
    int e = 0;
    if (m > 0.0f) frexpf(m, &e);  // m < 2^e
    const float up = m > 0.0f ? ldexpf(1.0f, kPackExp - e) : 1.0f;
    _Float16* drow = p.dst + (size_t)r * p.K;
#pragma unroll
    for (int i = 0; i < kPackRegChunks; ++i) {
      const int c = (i * 64 + lane) * 8;
      if (c < p.K) store8(drow, c, v[i], up);
      // K is a multiple of 512: a chunk's 64 lanes are all in or all out
      if (p.corr && i * 512 < p.K) store_corr(p, r, c, corr_of8(v[i], up), lane);
    }
    if (lane == 0) p.unit[r] = m > 0.0f ? ldexpf(1.0f, e - kPackExp) : 1.0f;
    return;
  }
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
    _Float16 h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) h[slot_of_col(j)] = (_Float16)(v[j] * up);
    typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
    f16x8_t hv;
#pragma unroll
    for (int j = 0; j < 8; ++j) hv[j] = h[j];
    *reinterpret_cast<f16x8_t*>(drow + c) = hv;
    if (p.corr) store_corr(p, r, c, corr_of8(v, up), lane);
  }
  if (lane == 0) p.unit[r] = m > 0.0f ? ldexpf(1.0f, e - kPackExp) : 1.0f;
}

// Row r of p by nw waves of one workgroup, this wave being wave `part` of them
// (r < 0: no row; the wave still reaches the barrier).  It takes the
// 512-column chunks part, part + nw, ... and holds up to kSplitRegChunks of
// them in registers (more are read twice: for the maximum, then to convert).
// The row's maximum is combined through s_m, one float per wave of the
// workgroup with the row's nw waves consecutive and this one at s_m[slot],
// after a workgroup barrier that every wave of the workgroup must reach.  A
// maximum does not depend on the order it is taken in, and each 64-column
// group's correction lies inside one chunk, so every value written is the one
// pack_row writes.  Holding a sixth of a 6144-column row per wave keeps the
// register count (and so the workgroups a compute unit holds at once) of the
// kernels that pack rows this way at that of their other work.
constexpr int kSplitRegChunks = 6;
__device__ __forceinline__ void pack_row_split(const PackArgs& p, int r, int part, int nw,
                                               float* s_m, int slot, int lane) {
  const int nch = (p.K + 511) / 512;
  const int mine = r < 0 ? 0 : (nch - part + nw - 1) / nw;  // chunks part + nw j < nch
  const bool regs = mine <= kSplitRegChunks;
  const size_t base = r < 0 ? 0 : (p.gather ? (size_t)p.gather[r] : (size_t)r) * p.K;
  float v[kSplitRegChunks][8];
  float m = 0.0f;
  if (regs) {
#pragma unroll
    for (int j = 0; j < kSplitRegChunks; ++j) {
      const int c = ((part + nw * j) * 64 + lane) * 8;
      if (j < mine && c < p.K) {
        load8(p.src, p.src_bf16, base + c, v[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j][i]));
      }
    }
  } else {
    for (int j = 0; j < mine; ++j) {
      const int c = ((part + nw * j) * 64 + lane) * 8;
      if (c < p.K) {
        float t[8];
        load8(p.src, p.src_bf16, base + c, t);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(t[i]));
      }
    }
  }
  m = wave_max(m);
  if (lane == 0) s_m[slot] = m;
  __syncthreads();
  if (r < 0) return;
  m = s_m[slot - part];
  for (int q = 1; q < nw; ++q) m = fmaxf(m, s_m[slot - part + q]);
  int e = 0;
  if (m > 0.0f) frexpf(m, &e);  // m < 2^e
  const float up = m > 0.0f ? ldexpf(1.0f, kPackExp - e) : 1.0f;
  _Float16* drow = p.dst + (size_t)r * p.K;
  if (regs) {
#pragma unroll
    for (int j = 0; j < kSplitRegChunks; ++j) {
      const int ch = part + nw * j, c = (ch * 64 + lane) * 8;
      if (j < mine) {
        if (c < p.K) store8(drow, c, v[j], up);
        // K is a multiple of 512 where corrections are asked for
        if (p.corr) store_corr(p, r, c, corr_of8(v[j], up), lane);
      }
    }
  } else {
    for (int j = 0; j < mine; ++j) {
      const int c = ((part + nw * j) * 64 + lane) * 8;
      float t[8] = {};
      if (c < p.K) {
        load8(p.src, p.src_bf16, base + c, t);
        store8(drow, c, t, up);
      }
      if (p.corr) store_corr(p, r, c, corr_of8(t, up), lane);
    }
  }
  if (lane == 0 && part == 0) p.unit[r] = m > 0.0f ? ldexpf(1.0f, e - kPackExp) : 1.0f;
}

// M-block map of a union of at most 64 experts (offs[0..U]), by one whole
// wave: experts of more than kThinTokens tokens (none with thin_all) get
// ceil(count / mblock) M-blocks (mbo[u] = M-blocks before u, mbo[U] the total,
// blk_u[j] = the expert of M-block j); the others run as thin tiles
// (thin_tiles_wave).
__device__ __forceinline__ int wave_excl_scan(int c, int lane, int& total) {
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int nb = __shfl_up(incl, o, 64);
    if (lane >= o) incl += nb;
  }
  total = __shfl(incl, 63, 64);
  return incl - c;
}
__device__ __forceinline__ void mblock_map_wave(const int32_t* offs, int U, int mblock,
                                                int32_t* mbo, int32_t* blk_u, int thin_all,
                                                int lane) {
  const int n = lane < U ? offs[lane + 1] - offs[lane] : 0;
  const bool thin = lane < U && (thin_all || n <= kThinTokens);
  const int c = lane < U && !thin ? (n + mblock - 1) / mblock : 0;
  int tot;
  const int run = wave_excl_scan(c, lane, tot);
  if (lane < U) {
    mbo[lane] = run;
    for (int j = 0; j < c; ++j) blk_u[run + j] = lane;
  }
  if (lane == 0) mbo[U] = tot;
}

// The thin tiles of a union of at most 64 experts (offs[0..U], uniq, rows:
// the union's list), by one whole wave: the experts of at most kThinTokens
// tokens (every expert with thin_all), expert by expert, kThinTokens tokens a
// tile, each a record (blob, first list entry, token count, first token) and
// its kTileSlots slot ids; the records from the last tile to tt_n are marked
// empty.
__device__ __forceinline__ void thin_tiles_wave(const int32_t* offs, const int32_t* uniq,
                                                const int32_t* rows, int U,
                                                const uint8_t* const* table, ThinTile* tt,
                                                int32_t* tslot, int tt_n, int thin_all,
                                                int lane) {
  const int n = lane < U ? offs[lane + 1] - offs[lane] : 0;
  const bool thin = lane < U && (thin_all || n <= kThinTokens);
  const int ct = thin ? (n + kThinTokens - 1) / kThinTokens : 0;
  int tot;
  const int run = wave_excl_scan(ct, lane, tot);
  if (ct > 0) {
    const uint8_t* blob = table[uniq[lane]];
    const int off = offs[lane];
    for (int j = 0; j < ct && run + j < tt_n; ++j) {
      ThinTile r{};
      r.blob = blob;
      r.off = off;
      r.cnt = n;
      r.tok0 = j * kThinTokens;
      tt[run + j] = r;
      for (int i = 0; i < kTileSlots; ++i)
        tslot[(size_t)(run + j) * kTileSlots + i] = rows[off + min(j * kThinTokens + i, n - 1)];
    }
  }
  for (int j = tot + lane; j < tt_n; j += 64) tt[j] = ThinTile{};
}

}  // namespace moe

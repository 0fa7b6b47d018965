// Device helpers for the gfx950 kernels: wave64 reductions, the activation
// digit split and the exact int4 x digit dot product of one 16-byte chunk.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_internal.h"

namespace moe {

// DPP lane exchange within rows of 16 lanes.
template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(dpp_i<kCtrl>(__float_as_int(v)));
}

// DPP controls that, applied in this order, form a butterfly over a row of 16
// lanes: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
// After the first two every quad is uniform, so the mirrors pair whole quads
// and then whole half-rows.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
// quad_perm [3,2,1,0] (lane ^ 3) and row_ror:8 (lane ^ 8 inside a row of 16)
constexpr int kDppXor3 = 0x1B, kDppRor8 = 0x128;

// Sum over the 64 lanes, the same value in every lane, in a fixed order:
// butterflies inside each row of 16 lanes (DPP quad permutes and mirrors),
// then the four row sums read out in row order.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// Transposed reduction of 8 per-lane values over the wave: on return, lanes
// 8i .. 8i+7 hold the sum over all 64 lanes of v[i].  Each exchange step halves
// the values a lane carries (a lane keeps the half selected by one lane-index
// bit and receives its partner's copy of that half), then the last three
// steps are DPP butterflies inside groups of 8 lanes.  Fixed order, so
// bit-reproducible.  All 64 lanes must be active.
__device__ __forceinline__ float reduce8(const float (&v)[8], int lane) {
  const bool h5 = lane & 32, h4 = lane & 16, h3 = lane & 8;
  float a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float keep = h5 ? v[i + 4] : v[i], send = h5 ? v[i] : v[i + 4];
    a[i] = keep + __shfl_xor(send, 32, 64);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float keep = h4 ? a[i + 2] : a[i], send = h4 ? a[i] : a[i + 2];
    b[i] = keep + __shfl_xor(send, 16, 64);
  }
  float c = (h3 ? b[1] : b[0]) + __shfl_xor(h3 ? b[0] : b[1], 8, 64);
  c += dpp<kDppXor1>(c);
  c += dpp<kDppXor2>(c);
  c += dpp<kDppHalfMirror>(c);
  return c;
}

template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int hi = dpp_i<kCtrl>((int)(b >> 32)), lo = dpp_i<kCtrl>((int)b);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

__device__ __forceinline__ double readlane_d(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  const int lo = __builtin_amdgcn_readlane((int)b, l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// fp64 sum over the 64 lanes in a fixed order, the same in every lane:
// butterflies inside each row of 16 lanes, then the four row sums in order.
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
  return ((readlane_d(v, 0) + readlane_d(v, 16)) + readlane_d(v, 32)) + readlane_d(v, 48);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}


// Byte position of column cc (0..31) of a chunk inside one 32-byte digit
// plane: a 32-bit word of codes holds columns 8b..8b+7 as nibbles; masking it
// with 0x0F0F0F0F yields the even columns in bytes 0..3 and shifting it right
// by 4 first yields the odd ones.  The plane stores, per 8 columns, the 4 even
// columns' digits in one word and the 4 odd columns' digits in the next.
__device__ __forceinline__ int digit_pos(int cc) {
  const int blk = cc >> 3, odd = cc & 1, byte = (cc & 7) >> 1;
  return (2 * blk + odd) * 4 + byte;
}

template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<kCtrl>(__float_as_int(v)));
}

// Max and integer sum over each row of 16 lanes (every lane of the row gets
// the result).  All 64 lanes must be active.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}

// Float sum over each row of 16 lanes in a fixed order (every lane of the row
// gets it).  All 64 lanes must be active.
__device__ __forceinline__ float row16_fsum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ int row16_sum(int v) {
  v += dpp_i<kDppXor1>(v);
  v += dpp_i<kDppXor2>(v);
  v += dpp_i<kDppHalfMirror>(v);
  v += dpp_i<kDppMirror>(v);
  return v;
}

// Max and integer sum over each half (32 lanes) of the wave.
__device__ __forceinline__ float half_max(float v) {
  return fmaxf(row16_max(v), __shfl_xor(row16_max(v), 16, 64));
}

__device__ __forceinline__ int half_sum(int v) {
  const int r = row16_sum(v);
  return r + __shfl_xor(r, 16, 64);
}

// Digit split of one 32-wide group per half wave: lane l holds column `col`
// of a row of activations, and the 32 lanes of its half hold the 32 columns
// of one group (col & ~31 the same for all of them).  With m the group's
// largest magnitude and E the exponent with m < 2^E <= 2m,
// X = rint(v * 2^(20-E)), so |X| <= 2^20 and the absolute error is at most
// 2^(E-21) <= m * 2^-20; X = D2*2^14 + D1*2^7 + D0 with D0, D1 in [-64, 63]
// and D2 in [-64, 64].  `valid` = false halves still take part in the lane
// exchanges but store nothing.  All 64 lanes must be active.
__device__ __forceinline__ void digitize32(float v, int col, bool valid, int8_t* q_row,
                                           int32_t* sx_row, float* sc_row) {
  const float m = half_max(fabsf(v));
  int E = 0;
  if (m > 0.0f) (void)frexpf(m, &E);
  const int X = m > 0.0f ? (int)rintf(ldexpf(v, kFixBits - E)) : 0;
  const int D0 = ((X + 64) & 127) - 64;
  const int X1 = (X - D0) / 128;
  const int D1 = ((X1 + 64) & 127) - 64;
  const int D2 = (X1 - D1) / 128;
  const int sx = half_sum(X);
  if (!valid) return;
  int8_t* plane = q_row + (size_t)(col >> 5) * kChunkDigitBytes;
  const int pos = digit_pos(col & 31);
  plane[pos] = (int8_t)D0;
  plane[kChunk + pos] = (int8_t)D1;
  plane[2 * kChunk + pos] = (int8_t)D2;
  if ((col & 31) == 0) {
    sx_row[col >> 5] = sx;
    sc_row[col >> 5] = ldexpf(1.0f, E - kFixBits);
  }
}

// Integer activations (int8 per 64-column group) in the same digit form: the
// wave's 64 lanes hold the 64 columns of one group (col & 63 == lane), and
// q = rint(v / s) (ties to even), s = max|v| / 127 in fp32 (a group of
// zeros: s = 0, q = 0).  X = q is stored as D0 in [-64, 63], D1 in [-1, 1],
// D2 = 0 with unit s in both 32-column halves, so the digit dot products give
// exactly sum q_w q, times s.  All 64 lanes must be active.
__device__ __forceinline__ void digitize64_i8(float v, int col, bool valid, int8_t* q_row,
                                              int32_t* sx_row, float* sc_row) {
  const float hm = half_max(fabsf(v));
  const float m = fmaxf(hm, __shfl_xor(hm, 32, 64));
  const float s = m / 127.0f;
  const int X = m > 0.0f ? (int)fminf(fmaxf(rintf(v / s), -127.0f), 127.0f) : 0;
  const int D0 = ((X + 64) & 127) - 64;
  const int D1 = (X - D0) / 128;
  const int sx = half_sum(X);
  if (!valid) return;
  int8_t* plane = q_row + (size_t)(col >> 5) * kChunkDigitBytes;
  const int pos = digit_pos(col & 31);
  plane[pos] = (int8_t)D0;
  plane[kChunk + pos] = (int8_t)D1;
  plane[2 * kChunk + pos] = 0;
  if ((col & 31) == 0) {
    sx_row[col >> 5] = sx;
    sc_row[col >> 5] = s;
  }
}

// Digits of one chunk held in registers: w[p][i] is word i of plane p.
struct ChunkDigits {
  int w[kPlanes][8];
};

__device__ __forceinline__ ChunkDigits load_chunk_digits(const int8_t* plane_base) {
  ChunkDigits cd;
  const int4* p = reinterpret_cast<const int4*>(plane_base);
#pragma unroll
  for (int pl = 0; pl < kPlanes; ++pl) {
    const int4 a = p[2 * pl], b = p[2 * pl + 1];
    cd.w[pl][0] = a.x; cd.w[pl][1] = a.y; cd.w[pl][2] = a.z; cd.w[pl][3] = a.w;
    cd.w[pl][4] = b.x; cd.w[pl][5] = b.y; cd.w[pl][6] = b.z; cd.w[pl][7] = b.w;
  }
  return cd;
}

// Exact sum over a chunk of n'_c * X_c, where n'_c = q_c + 8 is the
// offset-binary form of the int4 weight (bit 3 of every nibble flipped) and
// X_c the activation's fixed-point value: digit plane by digit plane, most
// significant first, each partial sum scaled by 2^7 before the next.  Products
// and sums are exact in int32 (|result| < 2^30).  The caller subtracts
// 8 * sum(X) to get sum q_c X_c.
__device__ __forceinline__ int chunk_dot(const uint4 codes, const ChunkDigits& cd) {
  const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
  int lo[4], hi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v = cw[i] ^ 0x88888888u;
    lo[i] = (int)(v & 0x0F0F0F0Fu);
    hi[i] = (int)((v >> 4) & 0x0F0F0F0Fu);
  }
  int acc = 0;
#pragma unroll
  for (int p = kPlanes - 1; p >= 0; --p) {
    if (p != kPlanes - 1) acc *= 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_amdgcn_sdot4(lo[i], cd.w[p][2 * i], acc, false);
      acc = __builtin_amdgcn_sdot4(hi[i], cd.w[p][2 * i + 1], acc, false);
    }
  }
  return acc;
}

// The same for int2 codes: a chunk's 32 columns are 8 bytes, column 4b + j
// of each 32-bit word in bits 2j..2j+1 of its byte b.  Flipping the top bit
// of every field makes it n'_c = q_c + 2 in [0, 3].  v_perm takes two
// neighbouring bytes from the word and from the word shifted right by 4, so
// that byte i of the result holds columns 2i and 2i + 1 of an 8-column block
// in bits 0-1 and 2-3 (its bits 4-7, from the next byte, are masked off): one
// mask gives the block's even columns and a shift and mask its odd ones, in
// the order the digit planes hold them.  The caller subtracts 2 * sum(X).
__device__ __forceinline__ int chunk_dot2(const uint2 codes, const ChunkDigits& cd) {
  const uint32_t cw[2] = {codes.x, codes.y};
  int ev[4], od[4];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint32_t v = cw[m] ^ 0xAAAAAAAAu, v4 = v >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // bytes [v(b), v4(b), v(b + 1), v4(b + 1)] for b = 2h
      const uint32_t s = __builtin_amdgcn_perm(v4, v, h ? 0x07030602u : 0x05010400u);
      ev[2 * m + h] = (int)(s & 0x03030303u);
      od[2 * m + h] = (int)((s >> 2) & 0x03030303u);
    }
  }
  int acc = 0;
#pragma unroll
  for (int p = kPlanes - 1; p >= 0; --p) {
    if (p != kPlanes - 1) acc *= 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_amdgcn_sdot4(ev[i], cd.w[p][2 * i], acc, false);
      acc = __builtin_amdgcn_sdot4(od[i], cd.w[p][2 * i + 1], acc, false);
    }
  }
  return acc;
}

// The same for int8 codes (32 bytes, column order): v_perm gathers each
// 8-column block's even and odd columns.  The codes are signed, so no offset
// is subtracted.  A plane's sum is exact in int32 (|sum| < 2^19), but the
// chunk's total can reach 2^32, so the three planes' sums are combined in
// fp32: sum = P2 * 2^14 + (P1 * 2^7 + P0), the bracket exact in int32, one
// rounding converting it and one in the fma (relative error < 2^-23).
__device__ __forceinline__ float chunk_dot8(const uint4 c0, const uint4 c1, const ChunkDigits& cd) {
  const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  int ev[4], od[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    ev[b] = (int)__builtin_amdgcn_perm(cw[2 * b + 1], cw[2 * b], 0x06040200u);  // 0 2 4 6
    od[b] = (int)__builtin_amdgcn_perm(cw[2 * b + 1], cw[2 * b], 0x07050301u);  // 1 3 5 7
  }
  static_assert(kPlanes == 3, "three digit planes");
  int P[kPlanes] = {0, 0, 0};
#pragma unroll
  for (int p = 0; p < kPlanes; ++p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      P[p] = __builtin_amdgcn_sdot4(ev[i], cd.w[p][2 * i], P[p], false);
      P[p] = __builtin_amdgcn_sdot4(od[i], cd.w[p][2 * i + 1], P[p], false);
    }
  }
  return fmaf((float)P[2], 16384.0f, (float)(P[1] * 128 + P[0]));
}

__device__ __forceinline__ float f16_to_f32(const _Float16* p) { return (float)*p; }

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

}  // namespace moe

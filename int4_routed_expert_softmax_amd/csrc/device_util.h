// Device helpers for the gfx950 kernels: wave64 reductions, the activation
// digit split and the exact int4 x digit dot product of one 16-byte chunk.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_internal.h"

namespace moe {

// DPP lane exchange within rows of 16 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sum over the 64 lanes, the same value in every lane, in a fixed order:
// butterflies inside each row of 16 lanes (DPP quad permutes and mirrors),
// then the four row sums read out in row order.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum within each 32-lane half of the wave.
__device__ __forceinline__ int half_sum(int v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
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

// One wave turns the 64 values of group g of a row (lane l holds column
// 64g + l) into digit form.  With m the group's largest magnitude and E the
// exponent with m < 2^E <= 2m, X = rint(v * 2^(20-E)) so |X| <= 2^20 and the
// absolute error is at most 2^(E-21) <= m * 2^-20; X = D2*2^14 + D1*2^7 + D0
// with D0, D1 in [-64, 63] and D2 in [-64, 64].
__device__ __forceinline__ void digitize_group(float v, int lane, int g, int8_t* q_row,
                                               int32_t* sx_row, float* sc_row) {
  const float m = wave_max(fabsf(v));
  int E = 0;
  if (m > 0.0f) (void)frexpf(m, &E);
  const int X = m > 0.0f ? (int)rintf(ldexpf(v, kFixBits - E)) : 0;
  const int D0 = ((X + 64) & 127) - 64;
  const int X1 = (X - D0) / 128;
  const int D1 = ((X1 + 64) & 127) - 64;
  const int D2 = (X1 - D1) / 128;
  const int c = 2 * g + (lane >> 5);
  int8_t* plane = q_row + (size_t)c * kChunkDigitBytes;
  const int pos = digit_pos(lane & 31);
  plane[pos] = (int8_t)D0;
  plane[kChunk + pos] = (int8_t)D1;
  plane[2 * kChunk + pos] = (int8_t)D2;
  const int sx = half_sum(X);
  if ((lane & 31) == 0) sx_row[c] = sx;
  if (lane == 0) sc_row[g] = ldexpf(1.0f, E - kFixBits);
}

// Digits of one chunk held in registers: planes[p][w] is word w of plane p.
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

// Exact sum over a chunk of n'_c * X_c, where n'_c = q_c + 8 is the offset
// binary form of the int4 weight (flip bit 3 of every nibble) and X_c the
// activation's fixed-point value; products and sums are exact in int32
// (|result| < 2^30).  The caller subtracts 8 * sum(X) to get sum q_c X_c.
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
  for (int i = 0; i < 4; ++i) {
    acc = __builtin_amdgcn_sdot4(lo[i], cd.w[2][2 * i], acc, false);
    acc = __builtin_amdgcn_sdot4(hi[i], cd.w[2][2 * i + 1], acc, false);
  }
  acc *= 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = __builtin_amdgcn_sdot4(lo[i], cd.w[1][2 * i], acc, false);
    acc = __builtin_amdgcn_sdot4(hi[i], cd.w[1][2 * i + 1], acc, false);
  }
  acc *= 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = __builtin_amdgcn_sdot4(lo[i], cd.w[0][2 * i], acc, false);
    acc = __builtin_amdgcn_sdot4(hi[i], cd.w[0][2 * i + 1], acc, false);
  }
  return acc;
}

__device__ __forceinline__ float f16_to_f32(const _Float16* p) { return (float)*p; }

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

}  // namespace moe

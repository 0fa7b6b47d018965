// Internal declarations of the gfx950 MoE library: workspace layout, kernel
// argument blocks and launchers.  Not part of the public ABI (include/moe.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace moe {

// Weights per fp16 scale along a row (the "gs64" container).
constexpr int kGroup = 64;
// Columns covered by one 16-byte load of 4-bit codes.
constexpr int kChunk = 32;
// Activations enter the int4 dot products as 21-bit fixed point per 64-wide
// group, split into three signed int8 digit planes of base 2^7.  A 32-column
// chunk therefore carries 3 x 32 digit bytes.
constexpr int kPlanes = 3;
constexpr int kChunkDigitBytes = kPlanes * kChunk;
// Exponent offset of the fixed point: a group whose largest magnitude is below
// 2^E is stored as X = rint(v * 2^(kFixBits - E)), |X| <= 2^kFixBits.
constexpr int kFixBits = 20;

// Activations in digit form for `rows` rows of length K.
//   q  [rows][K/32][3][32] int8: digit planes D0, D1, D2 of X = D2*2^14 + D1*2^7 + D0,
//      bytes of each plane in code order (per 8 columns: the 4 even columns,
//      then the 4 odd columns), matching how a 32-bit word of nibbles splits
//      into its low and high nibbles
//   sx [rows][K/32] int32: sum of X over the chunk
//   sc [rows][K/64] f32:   value of one unit of X in the group, 2^(E - 20)
struct Digits {
  int8_t* q;
  int32_t* sx;
  float* sc;
};

struct Layout {
  size_t tickets, z, xn, xq, xsx, xsc, idx, w, uniq, offs, nuniq, rows, aq, asx, asc, y, total;
};

Layout layout(int d, int f, int E, int k, int T);

// Expert list handed to the FFN kernels.  Either a device union (uniq, n_uniq,
// offsets, list of slot ids; x row of a slot = slot / kdiv) read from the
// device, or one expert (`single` blob, single_n rows, slot i = x row i).
struct ExpertList {
  const uint8_t* const* table;
  const uint8_t* single;
  int single_n;
  const int32_t* uniq;
  const int32_t* n_uniq;
  const int32_t* offsets;
  const int32_t* list;
  int kdiv;
};

hipError_t launch_rmsnorm(const float* h, float* xn, int T, int d, float eps, hipStream_t s);
hipError_t launch_logits(const void* x, int x_bf16, int T, int d, int E, const float* Wr,
                         const float* bias, double* z, hipStream_t s);
hipError_t launch_topk(const double* z, int T, int E, int k, int32_t* idx, float* w,
                       hipStream_t s);
hipError_t launch_union(const int32_t* idx, int T, int E, int k, int32_t* uniq, int32_t* n_uniq,
                        int32_t* offsets, int32_t* rows, int32_t* stats, hipStream_t s);
hipError_t launch_digitize(const void* x, int x_bf16, const int32_t* gather, int rows, int K,
                           Digits out, hipStream_t s);
hipError_t launch_gateup(const ExpertList& L, int max_experts, int d, int f, Digits xd, Digits ad,
                         hipStream_t s);
hipError_t launch_down(const ExpertList& L, int max_experts, int d, int f, Digits ad, float* y,
                       hipStream_t s);
hipError_t launch_combine(const float* y, const float* w, const float* resid, float* out, int T,
                          int d, int k, hipStream_t s);

}  // namespace moe

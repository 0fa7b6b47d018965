// Internal declarations of the gfx950 MoE library: workspace layout, kernel
// argument blocks and launchers.  Not part of the public ABI (include/moe.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace moe {

// Weights per fp16 scale along a row (the "gs64" container).
constexpr int kGroup = 64;
// Columns covered by one 16-byte load of 4-bit codes.
constexpr int kChunk = 32;
// Activations enter the int4 dot products as 21-bit fixed point per 32-wide
// group, split into three signed int8 digit planes of base 2^7.  A group is
// one 32-column chunk (one 16-byte load of codes) and carries 3 x 32 digit
// bytes.
constexpr int kPlanes = 3;
constexpr int kChunkDigitBytes = kPlanes * kChunk;
constexpr int kXGroup = 32;
// Exponent offset of the fixed point: a group whose largest magnitude is below
// 2^E is stored as X = rint(v * 2^(kFixBits - E)), |X| <= 2^kFixBits.
constexpr int kFixBits = 20;

// Activations in digit form for `rows` rows of length K.
//   q  [rows][K/32][3][32] int8: digit planes D0, D1, D2 of X = D2*2^14 + D1*2^7 + D0,
//      bytes of each plane in code order (per 8 columns: the 4 even columns,
//      then the 4 odd columns), matching how a 32-bit word of nibbles splits
//      into its low and high nibbles
//   sx [rows][K/32] int32: sum of X over the group
//   sc [rows][K/32] f32:   value of one unit of X in the group, 2^(E - 20)
struct Digits {
  int8_t* q;
  int32_t* sx;
  float* sc;
};

struct Layout {
  size_t tickets, z, xn, xq, xsx, xsc, idx, w, uniq, offs, nuniq, rows, aq, asx, asc, y;
  size_t xh, xunit, xcorr, a32, ah, aunit, aunitg, acorr, mbo, blku, xtab, tt, tslot,
      plan, total;
};

Layout layout(int d, int f, int E, int k, int T);

// MOE_OK for hipSuccess, else MOE_EHIP with the error kept for moe_strerror.
int hip_error_status(hipError_t e);

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
  int per_row;  // blobs carry one scale per row (else one per kGroup weights)
  int bits;     // code width: 4, 8 or 2
  int i8act;    // integer activations: a is digit-split as int8 per 64 columns
  // with hit set: only union positions u with hit[u] == want_hit are computed
  // (the slot cache's hits, resident before the call, or its misses)
  const int32_t* hit;
  int want_hit;
};

// Code width of a layer: dims.code_bits, 0 meaning int4.
inline int code_bits(int b) { return b == 0 ? 4 : b; }

// Scales of one row of K weights in a blob: K / kGroup, or 1 with per-row
// scales.  A blob's scales follow its codes: gate [f][srow(d)], up
// [f][srow(d)], down [d][srow(f)].
__host__ __device__ inline int srow(int K, int per_row) { return per_row ? 1 : K / kGroup; }
// Scale of 32-weight chunk c within its row.
__host__ __device__ inline unsigned scol(unsigned c, int per_row) { return per_row ? 0u : c / 2u; }

// Opt-in kernel timing (moe_timing_arm): launches of an armed kernel record
// caller-provided start/stop events around their execution.
struct TimingSlot {
  hipEvent_t const* start = nullptr;
  hipEvent_t const* stop = nullptr;
  int n = 0, next = 0;
};
extern TimingSlot g_timing[11];

template <typename K, typename... Args>
hipError_t launch(int kernel_id, K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  TimingSlot& t = g_timing[kernel_id];
  if (t.next < t.n) {
    const int i = t.next++;
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t.start[i], t.stop[i], 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  }
  return hipGetLastError();
}

// Experts with at most this many tokens in a batch run on the thin grouped
// GEMM (one 16-row M-tile per block); the others on the M-blocked one.
constexpr int kThinTokens = 16;

// One thin-GEMM tile of a union: kThinTokens tokens of one expert.  The map
// builder writes one record per thin block of the launch (blob == nullptr:
// no tile, the block exits), and the tile's slot ids beside it, so a block
// finds its expert, its tokens and their rows with one dependent load.
struct ThinTile {
  const uint8_t* blob;  // the expert's blob (nullptr: past the last tile)
  int32_t off;          // the expert's first list entry
  int32_t cnt;          // the expert's token count
  int32_t tok0;         // the tile's first token (a multiple of kThinTokens)
  int32_t pad[3];
};
// tslot[j][i]: slot of token tok0 + i of tile j (past the expert's last
// token: its last slot).
constexpr int kTileSlots = 16;

// Rows of activations to pack into the grouped GEMM's fp16 A operand (one
// power of two per row), their per-64-column group sums for the thin GEMM,
// and optionally the union's M-block maps.
struct PackArgs {
  const void* src;
  int src_bf16, K, rows;
  const int32_t* gather;  // source row of row r (nullptr: r)
  _Float16* dst;          // [rows][K]
  float* unit;            // [rows]
  float* corr;            // [rows][K / 64]: -corr_off * 2^-24 * (sum of the group's packed values)
  float corr_off;         // the code width's offset: 8 (int4), 128 (int8), 2 (int2)
  int thin_all;           // map every expert onto thin blocks (int8 and int2 layers,
                          // integer activations)
  int i8;                 // integer activations: rows -> int8 per 64-column group
                          // (dst as bytes, the group scales in corr)
  const int32_t* offsets;
  const int32_t* n_uniq;
  // with mbo set: experts of more than kThinTokens tokens (none with
  // thin_all) get ceil(count / mblock) M-blocks (mbo[u] prefix, blk_u[j] =
  // expert of M-block j); the others run as thin tiles (tt below)
  int32_t* mbo;
  int32_t* blk_u;
  int mblock;
  // with xtab set: the M-blocked experts placed on the 8 XCDs (each expert's
  // M-blocks on one, largest first onto the least loaded): xtab[x * xs + i]
  // = the i-th M-block index of XCD x, xcnt[x] = their number
  int32_t* xtab;
  int32_t* xcnt;
  int xs;
  // with tt set: the thin tiles (tt_n records: the thin blocks of the
  // launch, those past the last tile marked empty) and their slots; the
  // blobs come from table[uniq[u]], the slots from the union's list
  ThinTile* tt;
  int32_t* tslot;  // [tt_n][kTileSlots]
  int tt_n;
  const uint8_t* const* table;
  const int32_t* uniq;
  const int32_t* list;
};

// Arguments of the small-batch router front end (optional RMSNorm, logits and
// digit split in one launch; xd.q == nullptr skips the digit split).
struct RouterArgs {
  const void* x;
  int x_bf16, T, d, E, k, prenorm;
  float eps;
  const float* Wr;
  const float* bias;
  double* z;
  Digits xd;
  PackArgs px;  // px.dst set: workgroups past the logits and digit split pack px.rows rows
  int tsplit;   // logit workgroups per expert, each over its own tokens (set by the launcher)
  int i8;       // the digit split as integer activations (int8 per 64 columns)
};
constexpr int kSmallBatch = 8;
// The small-batch path recomputes routing inside the gate/up kernel with one
// wave for the union, so it needs T * k <= 64 picks.
constexpr int kSmallPicks = 64;
// A small batch (at most kSmallBatch tokens and kSmallPicks picks) takes its
// logits, bias added, from the router front end and its top-k and union from
// one workgroup (the gate/up kernel of the GEMV path, or k_route_small).
// Larger batches have their logits computed as kLogSplit partial sums.
inline bool small_batch(int T, int k) { return T <= kSmallBatch && T * k <= kSmallPicks; }
bool mfma_shape_ok(int d, int f);

// What the down projection of a small batch needs of union expert u, in one
// record: its blob and its slots (a token picks an expert at most once, so
// an expert of a batch of at most kSmallBatch tokens has at most that many).
struct DownPlan {
  const uint8_t* blob;
  int32_t n;
  int32_t slot[kSmallBatch];
  int32_t pad;
};
static_assert(sizeof(DownPlan) == 48, "DownPlan is three 16-byte pieces");

// Routing results of a small batch: the gate/up kernel recomputes top-k and
// the union from the logits at the start of every block (cheaper than a
// separate launch) and block (0, 0) publishes them here, with the down plan.
struct RouteOut {
  const double* z;
  int T, E, k;
  int32_t* idx;
  float* w;
  int32_t *uniq, *n_uniq, *offsets, *rows, *stats;
  DownPlan* plan;  // [kSmallPicks]
};

hipError_t launch_router_front(const RouterArgs& a, hipStream_t s);
// Top-k and union of a small batch from complete logits (ro.z), written to
// ro's outputs; with ro.plan set, also the down plan, whose blob addresses
// come from the expert table (else table may be null).  With map (not null),
// the same block also writes the union's M-block map for the grouped GEMM
// (map->mbo, map->blk_u, in M-blocks of map->mblock tokens).
hipError_t launch_route_small(const RouteOut& ro, const uint8_t* const* table, hipStream_t s,
                              const PackArgs* map = nullptr);
hipError_t launch_rmsnorm(const float* h, float* xn, int T, int d, float eps, hipStream_t s);
// Logits of batches past the small-batch limits: kLogSplit partial sums per
// logit, zp[s][t][e] (no bias); launch_topk(nsplit = kLogSplit, bias) adds
// them.  The small-batch front end writes complete logits (nsplit = 1, bias
// already added).
constexpr int kLogSplit = 8;
hipError_t launch_logits(const void* x, int x_bf16, int T, int d, int E, const float* Wr,
                         double* zp, hipStream_t s);
hipError_t launch_topk(const double* z, int nsplit, const float* bias, int T, int E, int k,
                       int32_t* idx, float* w, hipStream_t s);
hipError_t launch_union(const int32_t* idx, int T, int E, int k, int32_t* uniq, int32_t* n_uniq,
                        int32_t* offsets, int32_t* rows, int32_t* stats, hipStream_t s);
// i8: integer activations (int8 per 64 columns, digitize64_i8)
hipError_t launch_digitize(const void* x, int x_bf16, const int32_t* gather, int rows, int K,
                           Digits out, hipStream_t s, int i8 = 0);
hipError_t launch_gateup(const ExpertList& L, const RouteOut* small_route, int max_experts, int d,
                         int f, Digits xd, Digits ad, int tokens_per_expert_max, int token_groups,
                         hipStream_t s);

hipError_t launch_down(const ExpertList& L, int max_experts, int d, int f, Digits ad, float* y,
                       int tokens_per_expert_max, hipStream_t s);

// Down projection fused with the combine, for small batches (T * k <= 64),
// of int4, int2 or int8 codes (bits).
struct CombineArgs {
  const float* w;      // [T][k] router weights
  const float* resid;  // [T][d] or nullptr
  float* out;          // [T][d]
  int T, k;
};
hipError_t launch_down_combine(const DownPlan* plan, const int32_t* n_uniq, int d, int f,
                               Digits ad, const CombineArgs& cb, int per_row, int bits,
                               hipStream_t s);
hipError_t launch_combine(const float* y, const float* w, const float* resid, float* out, int T,
                          int d, int k, hipStream_t s);

// Grouped-GEMM expert FFN on the MFMA units (multi-token batches).  x rows are
// packed to fp16 with a power of two per row (xh, xunit), gate/up writes
// silu(g) * u per slot (a32), which is packed the same way (ah, aunit), and
// down writes y per slot.  Slots of the union: list entries; x row = slot /
// kdiv.  A single expert: slot i = x row i.
struct MfmaArgs {
  ExpertList L;
  int d, f;
  const void* x;
  int x_bf16;
  int x_rows;                // rows to pack (T tokens, or n rows of a single expert)
  const int32_t* x_gather;   // source row of packed row r (nullptr: r)
  int slots;                 // rows of a32 / ah / y
  int mb_bound;              // union: upper bound on the M-blocked GEMM's M-blocks
  int thin_bound;            // union: upper bound on the number of thin experts
  _Float16* xh;
  float* xunit;
  float* xcorr;              // [x_rows][d / 64]
  float* a32;
  _Float16* ah;
  float* aunit;
  float* aunit_g;            // [slots][f / 64]: a's unit per group (every expert thin)
  float* acorr;              // [slots][f / 64]
  int32_t* mbo;              // [n_experts + 1]
  int32_t* blk_u;            // [mb_bound]
  int32_t* xtab;             // [kXcds][xs] M-blocks per XCD
  int32_t* xcnt;             // [kXcds]
  int xs;
  ThinTile* tt;              // [thin_bound] thin tiles
  int32_t* tslot;            // [thin_bound][kTileSlots]
  float* y;
  int x_packed;              // xh, xunit, xcorr and the M-block maps are already written
  int i8act;                 // integer activations (MOE_INT8_ACT): xh and ah hold int8 rows,
                             // xcorr and acorr their group scales; every expert thin
};
// The x pack (and M-block map) launch_ffn_mfma would run for m.
PackArgs mfma_x_pack_args(const MfmaArgs& m);
// M-block (tokens per GEMM block) for a batch of `rows` activation rows.
int mfma_mblock(int rows);
constexpr int kMinMBlock = 16;
// The mixed launch of a union's grouped GEMM: an upper bound on its M-blocks
// (experts past kThinTokens tokens: fewer than T k / (kThinTokens + 1) of
// them, each with ceil(count / 64) < count / 64 + 1 M-blocks), and the length
// of each XCD's list of M-blocks.  Placing whole experts, each onto the XCD
// least loaded so far, leaves no XCD more than floor(total / 8) plus one
// expert's M-blocks (at most ceil(T / 64): an expert has at most T tokens).
constexpr int kXcds = 8;
inline int mixed_mb_bound(int T, int k, int maxU) {
  const int nthick = T * k / (kThinTokens + 1) < maxU ? T * k / (kThinTokens + 1) : maxU;
  return (T * k + 63) / 64 + nthick;
}
inline int xcd_stride(int T, int k, int maxU) {
  return mixed_mb_bound(T, k, maxU) / kXcds + (T + 63) / 64 + 1;
}
// The grouped GEMM needs d and f to be multiples of 512.
bool mfma_shape_ok(int d, int f);
// Batches from this many tokens on take the grouped GEMM when the shape
// allows it, also within the small-batch limits: its dequantisation work per
// weight does not grow with the tokens an expert serves, the GEMV's does.
constexpr int kMfmaMinTokens = 2;
inline bool gemv_small_path(int T, int k, int d, int f) {
  return small_batch(T, k) && !(T >= kMfmaMinTokens && mfma_shape_ok(d, f));
}
hipError_t launch_ffn_mfma(const MfmaArgs& m, hipStream_t s);
// Streaming read of bytes (a multiple of 16) with `blocks` workgroups of 256
// threads; sink holds blocks * 256 words and is written only in practice never.
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                             hipStream_t s);

}  // namespace moe

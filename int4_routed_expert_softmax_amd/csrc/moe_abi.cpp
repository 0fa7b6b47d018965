// extern "C" entry points of libmoe.so (declared in include/moe.h): argument
// validation, workspace carving and the launch sequence of each call.
// Validation never calls into HIP, so an invalid call touches no device.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>

#include "cache.h"
#include "moe_internal.h"
#include "trace.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {

static size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

// Reserved counters at the start of the workspace (unused: kept zero).
constexpr int kTicketWords = 64;

Layout layout(int d, int f, int E, int k, int T) {
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const size_t Tk = (size_t)T * k;
  const size_t cap = (size_t)(E < (long)Tk ? E : Tk);
  L.tickets = take(kTicketWords * sizeof(uint32_t));
  L.z = take((size_t)T * E * (gemv_small_path(T, k, d, f) ? 1 : kLogSplit) * sizeof(double));
  L.xn = take((size_t)T * d * sizeof(float));
  L.xq = take((size_t)T * (d / kChunk) * kChunkDigitBytes);
  L.xsx = take((size_t)T * (d / kXGroup) * sizeof(int32_t));
  L.xsc = take((size_t)T * (d / kXGroup) * sizeof(float));
  L.idx = take(Tk * sizeof(int32_t));
  L.w = take(Tk * sizeof(float));
  L.uniq = take(cap * sizeof(int32_t));
  L.offs = take((cap + 1) * sizeof(int32_t));
  L.nuniq = take(sizeof(int32_t));
  L.rows = take(Tk * sizeof(int32_t));
  L.aq = take(Tk * (f / kChunk) * kChunkDigitBytes);
  L.asx = take(Tk * (f / kXGroup) * sizeof(int32_t));
  L.asc = take(Tk * (f / kXGroup) * sizeof(float));
  L.y = take(Tk * d * sizeof(float));
  L.xh = take((size_t)T * d * sizeof(uint16_t));
  L.xunit = take((size_t)T * sizeof(float));
  L.xcorr = take((size_t)T * (d / kGroup) * sizeof(float));
  L.a32 = take(Tk * f * sizeof(float));
  L.ah = take(Tk * f * sizeof(uint16_t));
  L.aunit = take(Tk * sizeof(float));
  L.aunitg = take(Tk * (f / kGroup) * sizeof(float));
  L.acorr = take(Tk * (f / kGroup) * sizeof(float));
  L.mbo = take((cap + 1) * sizeof(int32_t));
  L.blku = take((cap + Tk / kMinMBlock + 1) * sizeof(int32_t));
  L.xtab = take(((size_t)kXcds * xcd_stride(T, k, (int)cap) + kXcds) * sizeof(int32_t));
  // thin tiles: at most cap + ceil(T k / kThinTokens) (the launch's thin blocks)
  const size_t ntile = cap + (Tk + kThinTokens - 1) / kThinTokens;
  L.tt = take(ntile * sizeof(ThinTile));
  L.tslot = take(ntile * kTileSlots * sizeof(int32_t));
  L.plan = take(kSmallPicks * sizeof(DownPlan));
  L.total = o;
  return L;
}

TimingSlot g_timing[MOE_KERNEL_COUNT];

}  // namespace moe

using namespace moe;

namespace {

thread_local char g_hip_msg[192];

int dims_status(const moe_dims* dm) {
  if (!dm) return MOE_EINVAL;
  if (dm->d <= 0 || dm->f <= 0 || dm->n_experts <= 0 || dm->top_k <= 0) return MOE_EINVAL;
  if (dm->top_k > dm->n_experts) return MOE_EINVAL;
  if (dm->group_size != kGroup && dm->group_size != 0) return MOE_EUNSUPPORTED;
  if (dm->d % kGroup || dm->f % kGroup || dm->d > 65536 || dm->f > 65536) return MOE_EUNSUPPORTED;
  if (dm->n_experts > 1024 || dm->top_k > 32) return MOE_EUNSUPPORTED;
  const int bits = code_bits(dm->code_bits);
  if (bits != 4 && bits != 8 && bits != 2) return MOE_EUNSUPPORTED;
  if (bits != 4 && !mfma_shape_ok(dm->d, dm->f)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The cached layer's table and copy list follow the layout: [E] table
// pointers, [cap] sources, [cap] destinations, the copy count, [cap] hit flags.
size_t cache_ws_bytes(int E) {
  return align_up(8 * (size_t)E) + 2 * align_up(8 * (size_t)kSmallPicks) + align_up(4) +
         align_up(4 * (size_t)kSmallPicks);
}

// What every entry point requires of ws_bytes: moe_workspace_bytes(dims, T).
size_t ws_need(const Layout& L, int E) { return L.total + cache_ws_bytes(E); }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  snprintf(g_hip_msg, sizeof g_hip_msg, "HIP error: %s", hipGetErrorString(e));
  return MOE_EHIP;
}

}  // namespace

int moe::hip_error_status(hipError_t e) { return hip_status(e); }

namespace {

#define MOE_TRY(call)                       \
  do {                                      \
    const int _st = hip_status(call);       \
    if (_st != MOE_OK) return _st;          \
  } while (0)

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

Digits x_digits(void* ws, const Layout& L) {
  return Digits{at<int8_t>(ws, L.xq), at<int32_t>(ws, L.xsx), at<float>(ws, L.xsc)};
}

Digits a_digits(void* ws, const Layout& L) {
  return Digits{at<int8_t>(ws, L.aq), at<int32_t>(ws, L.asx), at<float>(ws, L.asc)};
}

MfmaArgs mfma_args(void* ws, const Layout& L, int d, int f) {
  MfmaArgs m{};
  m.d = d;
  m.f = f;
  m.xh = at<_Float16>(ws, L.xh);
  m.xunit = at<float>(ws, L.xunit);
  m.xcorr = at<float>(ws, L.xcorr);
  m.a32 = at<float>(ws, L.a32);
  m.ah = at<_Float16>(ws, L.ah);
  m.aunit = at<float>(ws, L.aunit);
  m.aunit_g = at<float>(ws, L.aunitg);
  m.acorr = at<float>(ws, L.acorr);
  m.mbo = at<int32_t>(ws, L.mbo);
  m.blk_u = at<int32_t>(ws, L.blku);
  m.xtab = at<int32_t>(ws, L.xtab);
  m.tt = at<ThinTile>(ws, L.tt);
  m.tslot = at<int32_t>(ws, L.tslot);
  return m;
}

// Row offsets inside the packed activations are 32-bit element indices.
bool rows_fit(size_t rows, const moe_dims* dm) {
  const size_t K = dm->d > dm->f ? dm->d : dm->f;
  return rows * K < (size_t(1) << 31);
}

}  // namespace

MOE_API size_t moe_expert_blob_bytes(const moe_dims* dm) {
  if (dims_status(dm) != MOE_OK) return 0;
  const size_t fd = (size_t)dm->f * dm->d;
  const int pr = dm->group_size == 0;
  return 3 * fd * code_bits(dm->code_bits) / 8 +
         2 * (2 * (size_t)dm->f * srow(dm->d, pr) + (size_t)dm->d * srow(dm->f, pr));
}

MOE_API size_t moe_workspace_bytes(const moe_dims* dm, int32_t T_max) {
  if (dims_status(dm) != MOE_OK || T_max < 1) return 0;
  return ws_need(layout(dm->d, dm->f, dm->n_experts, dm->top_k, T_max), dm->n_experts);
}

MOE_API int moe_workspace_routing(const moe_dims* dm, int32_t T, moe_routing_offsets* out) {
  const int st = dims_status(dm);
  if (st != MOE_OK) return st;
  if (T < 1 || !out) return MOE_EINVAL;
  const Layout L = layout(dm->d, dm->f, dm->n_experts, dm->top_k, T);
  out->topk_idx = L.idx;
  out->topk_w = L.w;
  out->uniq = L.uniq;
  out->n_uniq = L.nuniq;
  out->offsets = L.offs;
  out->rows = L.rows;
  return MOE_OK;
}

MOE_API size_t moe_cache_state_bytes(const moe_dims* dm, int32_t n_slots) {
  if (dims_status(dm) != MOE_OK || n_slots < 1 || n_slots > dm->n_experts) return 0;
  return align_up(cache_state_bytes(dm->n_experts, n_slots));
}

MOE_API const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null/misaligned pointer, inconsistent dims, T < 1)";
    case MOE_EUNSUPPORTED:
      return "unsupported (group_size != 64, d or f not a multiple of 64, k > 32, E > 1024, "
             "bad dtype or flags)";
    case MOE_ENOSPC: return "workspace too small (see moe_workspace_bytes)";
    case MOE_EHIP: return g_hip_msg[0] ? g_hip_msg : "HIP error";
    default: return "unknown status";
  }
}

MOE_API int moe_route(const moe_dims* dm, const void* x, int x_dtype, int32_t T,
                      const float* w_router, const float* bias, int32_t* topk_idx, float* topk_w,
                      void* ws, size_t ws_bytes, void* stream) {
  int st = dims_status(dm);
  if (st != MOE_OK) return st;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (T < 1 || !x || !w_router || !topk_idx || !topk_w || !ws || !aligned(ws, 16)) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(w_router, 16)) return MOE_EINVAL;
  const Layout L = layout(dm->d, dm->f, dm->n_experts, dm->top_k, T);
  if (ws_bytes < ws_need(L, dm->n_experts)) return MOE_ENOSPC;
  hipStream_t s = static_cast<hipStream_t>(stream);
  double* z = at<double>(ws, L.z);
  if (T <= kSmallBatch) {
    RouterArgs ra{};
    ra.x = x;
    ra.x_bf16 = x_dtype == MOE_BF16;
    ra.T = T;
    ra.d = dm->d;
    ra.E = dm->n_experts;
    ra.k = dm->top_k;
    ra.Wr = w_router;
    ra.bias = bias;
    ra.z = z;
    MOE_TRY(launch_router_front(ra, s));
    MOE_TRY(launch_topk(z, 1, nullptr, T, dm->n_experts, dm->top_k, topk_idx, topk_w, s));
  } else {
    MOE_TRY(launch_logits(x, x_dtype == MOE_BF16, T, dm->d, dm->n_experts, w_router, z, s));
    MOE_TRY(launch_topk(z, kLogSplit, bias, T, dm->n_experts, dm->top_k, topk_idx, topk_w, s));
  }
  return MOE_OK;
}

MOE_API int moe_union(const moe_dims* dm, const int32_t* topk_idx, int32_t T, int32_t* uniq,
                      int32_t* n_uniq, int32_t* offsets, int32_t* rows, void* stream) {
  int st = dims_status(dm);
  if (st != MOE_OK) return st;
  if (T < 1 || !topk_idx || !uniq || !n_uniq || !offsets || !rows) return MOE_EINVAL;
  MOE_TRY(launch_union(topk_idx, T, dm->n_experts, dm->top_k, uniq, n_uniq, offsets, rows, nullptr,
                       static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

MOE_API int moe_expert_ffn(const moe_dims* dm, const void* expert_blob, const void* x, int x_dtype,
                           const int32_t* rows, int32_t n, float* y, void* ws, size_t ws_bytes,
                           void* stream) {
  int st = dims_status(dm);
  if (st != MOE_OK) return st;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (n < 1 || !expert_blob || !x || !y || !ws || !aligned(ws, 16)) return MOE_EINVAL;
  if (!aligned(expert_blob, 16) || !aligned(x, 4) || !aligned(y, 4)) return MOE_EINVAL;
  const Layout L = layout(dm->d, dm->f, dm->n_experts, dm->top_k, n);
  if (ws_bytes < ws_need(L, dm->n_experts)) return MOE_ENOSPC;
  if (!rows_fit((size_t)n * dm->top_k, dm)) return MOE_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ExpertList EL{};
  EL.single = static_cast<const uint8_t*>(expert_blob);
  EL.single_n = n;
  EL.kdiv = 1;
  EL.per_row = dm->group_size == 0;
  EL.bits = code_bits(dm->code_bits);
  // int8 and int2 experts take the matrix cores for any n (dims_status has
  // checked the shape)
  if ((n >= kMfmaMinTokens || EL.bits != 4) && mfma_shape_ok(dm->d, dm->f)) {
    MfmaArgs m = mfma_args(ws, L, dm->d, dm->f);
    m.L = EL;
    m.x = x;
    m.x_bf16 = x_dtype == MOE_BF16;
    m.x_rows = n;
    m.x_gather = rows;
    m.slots = n;
    m.y = y;
    MOE_TRY(launch_ffn_mfma(m, s));
    return MOE_OK;
  }
  const Digits xd = x_digits(ws, L), ad = a_digits(ws, L);
  MOE_TRY(launch_digitize(x, x_dtype == MOE_BF16, rows, n, dm->d, xd, s));
  MOE_TRY(launch_gateup(EL, nullptr, 1, dm->d, dm->f, xd, ad, n, 1, s));
  MOE_TRY(launch_down(EL, 1, dm->d, dm->f, ad, y, n, s));
  return MOE_OK;
}

MOE_API int moe_layer_forward(const moe_dims* dm, const void* x, int x_dtype, int32_t T,
                              const float* w_router, const float* bias,
                              const void* const* expert_table, float* out, uint32_t flags,
                              float rms_eps, int32_t* stats, void* ws, size_t ws_bytes,
                              void* stream) {
  int st = dims_status(dm);
  if (st != MOE_OK) return st;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (flags & ~(uint32_t)(MOE_PRENORM_RMS | MOE_RESIDUAL | MOE_BATCH_INVARIANT | MOE_INT8_ACT))
    return MOE_EUNSUPPORTED;
  if ((flags & (MOE_PRENORM_RMS | MOE_RESIDUAL)) && x_dtype != MOE_F32) return MOE_EUNSUPPORTED;
  const bool invariant = (flags & MOE_BATCH_INVARIANT) != 0;
  const bool i8act = (flags & MOE_INT8_ACT) != 0;
  if (invariant && T >= 1 && !small_batch(T, dm->top_k)) return MOE_EUNSUPPORTED;
  if (T < 1 || !x || !w_router || !expert_table || !out || !ws || !aligned(ws, 16)) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(out, 4)) return MOE_EINVAL;
  if ((flags & MOE_PRENORM_RMS) && !(rms_eps >= 0.0f)) return MOE_EINVAL;
  const int d = dm->d, f = dm->f, E = dm->n_experts, k = dm->top_k;
  const Layout L = layout(d, f, E, k, T);
  if (ws_bytes < ws_need(L, dm->n_experts)) return MOE_ENOSPC;
  if (!rows_fit((size_t)T * k, dm)) return MOE_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);

  double* z = at<double>(ws, L.z);
  int32_t* idx = at<int32_t>(ws, L.idx);
  float* w = at<float>(ws, L.w);
  int32_t* uniq = at<int32_t>(ws, L.uniq);
  int32_t* offs = at<int32_t>(ws, L.offs);
  int32_t* nuniq = at<int32_t>(ws, L.nuniq);
  int32_t* rows = at<int32_t>(ws, L.rows);
  float* y = at<float>(ws, L.y);
  const Digits xd = x_digits(ws, L), ad = a_digits(ws, L);
  const float* resid = (flags & MOE_RESIDUAL) ? static_cast<const float*>(x) : nullptr;
  ExpertList EL{};
  EL.table = reinterpret_cast<const uint8_t* const*>(expert_table);
  EL.uniq = uniq;
  EL.n_uniq = nuniq;
  EL.offsets = offs;
  EL.list = rows;
  EL.kdiv = k;
  EL.per_row = dm->group_size == 0;
  EL.bits = code_bits(dm->code_bits);
  const int maxU = E < T * k ? E : T * k;

  EL.i8act = i8act;
  // One token, and batch-invariant batches, on the single-token kernel
  // family, for every code width.  Integer activations take this path as the
  // others do: the digit split then holds one int8 per column (one scale per
  // 64 columns).
  if (invariant || gemv_small_path(T, k, d, f)) {
    // 1: [RMSNorm], logits, digit split; 2: top-k + union (one token: in
    // every gate/up block's prologue; 2+: one k_route_small block) and
    // gate/up; 3: down + combine.  Every step keeps one order of
    // arithmetic per token whatever the batch (the kernels for 1 and for 2+
    // tokens accumulate a token's terms alike), which MOE_BATCH_INVARIANT
    // relies on.
    RouterArgs ra{};
    ra.x = x;
    ra.x_bf16 = x_dtype == MOE_BF16;
    ra.T = T;
    ra.d = d;
    ra.E = E;
    ra.k = k;
    ra.prenorm = (flags & MOE_PRENORM_RMS) != 0;
    ra.eps = rms_eps;
    ra.Wr = w_router;
    ra.bias = bias;
    ra.z = z;
    ra.xd = xd;
    ra.i8 = i8act;
    MOE_TRY(launch_router_front(ra, s));
    DownPlan* plan = at<DownPlan>(ws, L.plan);
    RouteOut ro{z, T, E, k, idx, w, uniq, nuniq, offs, rows, stats, plan};
    if (T == 1) {
      MOE_TRY(launch_gateup(EL, &ro, maxU, d, f, xd, ad, 1, 1, s));
    } else {
      // 2+ tokens: routing once, in one block; then one gate/up block per
      // (row block, expert, token) running the single-token kernel (the
      // two-token one runs out of registers at 12 waves a block), the
      // blocks of one expert's rows back to back on one XCD so its rows
      // come from HBM once
      MOE_TRY(launch_route_small(ro, EL.table, s));
      MOE_TRY(launch_gateup(EL, nullptr, maxU, d, f, xd, ad, 1, T, s));
    }
    CombineArgs cb{w, resid, out, T, k};
    MOE_TRY(launch_down_combine(plan, nuniq, d, f, ad, cb, EL.per_row, EL.bits, s));
    return MOE_OK;
  }

  const void* xr = x;  // what the router and the experts see
  int xr_bf16 = x_dtype == MOE_BF16;
  if (flags & MOE_PRENORM_RMS) {
    float* xn = at<float>(ws, L.xn);
    MOE_TRY(launch_rmsnorm(static_cast<const float*>(x), xn, T, d, rms_eps, s));
    xr = xn;
    xr_bf16 = 0;
  }
  int x_packed = 0;
  // the thin GEMM's blocks per projection: int4, one per thin expert; int8
  // and int2 layers and integer activations, one per 16 tokens of every
  // expert (ceil(count / 16) < count / 16 + 1)
  const int thin_bound = EL.bits == 4 && !i8act
                             ? maxU
                             : maxU + (T * k + kThinTokens - 1) / kThinTokens;
  if (small_batch(T, k)) {
    // a few tokens on the grouped GEMM: logits (+ bias) by the small-batch
    // router front end, top-k and union in one block
    RouterArgs ra{};
    ra.x = xr;
    ra.x_bf16 = xr_bf16;
    ra.T = T;
    ra.d = d;
    ra.E = E;
    ra.k = k;
    ra.Wr = w_router;
    ra.bias = bias;
    ra.z = z;
    RouteOut ro{z, T, E, k, idx, w, uniq, nuniq, offs, rows, stats, nullptr};
    if (mfma_shape_ok(d, f)) {
      // the grouped GEMM's x pack runs in extra workgroups of the router
      // front end and its M-block map in the routing block: two launches
      // fewer than the pack kernel's
      MfmaArgs m = mfma_args(ws, L, d, f);
      m.L = EL;
      m.x = xr;
      m.x_bf16 = xr_bf16;
      m.x_rows = T;
      m.thin_bound = thin_bound;
      m.i8act = i8act;  // int8 rows (the front end's pack workgroups) and every expert thin
      ra.px = mfma_x_pack_args(m);
      MOE_TRY(launch_router_front(ra, s));
      MOE_TRY(launch_route_small(ro, nullptr, s, &ra.px));
      x_packed = 1;
    } else {
      MOE_TRY(launch_router_front(ra, s));
      MOE_TRY(launch_route_small(ro, nullptr, s));
    }
  } else {
    MOE_TRY(launch_logits(xr, xr_bf16, T, d, E, w_router, z, s));
    MOE_TRY(launch_topk(z, kLogSplit, bias, T, E, k, idx, w, s));
    MOE_TRY(launch_union(idx, T, E, k, uniq, nuniq, offs, rows, stats, s));
  }
  if (mfma_shape_ok(d, f)) {
    MfmaArgs m = mfma_args(ws, L, d, f);
    m.L = EL;
    m.x = xr;
    m.x_bf16 = xr_bf16;
    m.x_rows = T;
    m.slots = T * k;
    m.mb_bound = mixed_mb_bound(T, k, maxU);
    m.xs = xcd_stride(T, k, maxU);
    m.xcnt = m.xtab + (size_t)kXcds * m.xs;
    m.thin_bound = thin_bound;
    m.y = y;
    m.x_packed = x_packed;
    m.i8act = i8act;
    MOE_TRY(launch_ffn_mfma(m, s));
  } else {
    MOE_TRY(launch_digitize(xr, xr_bf16, nullptr, T, d, xd, s, i8act));
    MOE_TRY(launch_gateup(EL, nullptr, maxU, d, f, xd, ad, T, 1, s));
    MOE_TRY(launch_down(EL, maxU, d, f, ad, y, T, s));
  }
  MOE_TRY(launch_combine(y, w, resid, out, T, d, k, s));
  return MOE_OK;
}

MOE_API int moe_layer_forward_cached(const moe_dims* dm, const void* x, int x_dtype, int32_t T,
                                     const float* w_router, const float* bias,
                                     const void* const* home_table, void* slots, int32_t n_slots,
                                     void* cache_state, float* out, uint32_t flags, float rms_eps,
                                     int32_t* stats, void* ws, size_t ws_bytes, void* stream) {
  int st = dims_status(dm);
  if (st != MOE_OK) return st;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (flags & ~(uint32_t)(MOE_PRENORM_RMS | MOE_RESIDUAL | MOE_BATCH_INVARIANT | MOE_INT8_ACT))
    return MOE_EUNSUPPORTED;
  if ((flags & (MOE_PRENORM_RMS | MOE_RESIDUAL)) && x_dtype != MOE_F32) return MOE_EUNSUPPORTED;
  if (T < 1 || !x || !w_router || !home_table || !slots || !cache_state || !out || !ws ||
      !aligned(ws, 16))
    return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(out, 4) || !aligned(slots, 256) ||
      !aligned(cache_state, 4))
    return MOE_EINVAL;
  if ((flags & MOE_PRENORM_RMS) && !(rms_eps >= 0.0f)) return MOE_EINVAL;
  const int d = dm->d, f = dm->f, E = dm->n_experts, k = dm->top_k;
  if (!small_batch(T, k)) return MOE_EUNSUPPORTED;
  if (code_bits(dm->code_bits) != 4) return MOE_EUNSUPPORTED;  // the cache serves int4 layers
  const int cap = E < T * k ? E : T * k;
  if (n_slots < cap || n_slots > E) return MOE_EUNSUPPORTED;
  const Layout L = layout(d, f, E, k, T);
  if (ws_bytes < ws_need(L, E)) return MOE_ENOSPC;
  hipStream_t s = static_cast<hipStream_t>(stream);

  double* z = at<double>(ws, L.z);
  int32_t* idx = at<int32_t>(ws, L.idx);
  float* w = at<float>(ws, L.w);
  int32_t* uniq = at<int32_t>(ws, L.uniq);
  int32_t* offs = at<int32_t>(ws, L.offs);
  int32_t* nuniq = at<int32_t>(ws, L.nuniq);
  int32_t* rows = at<int32_t>(ws, L.rows);
  DownPlan* plan = at<DownPlan>(ws, L.plan);
  const Digits xd = x_digits(ws, L), ad = a_digits(ws, L);
  size_t o = L.total;
  const uint8_t** eff = at<const uint8_t*>(ws, o);
  o += align_up(8 * (size_t)E);
  const uint8_t** fill_src = at<const uint8_t*>(ws, o);
  o += align_up(8 * (size_t)kSmallPicks);
  uint8_t** fill_dst = at<uint8_t*>(ws, o);
  o += align_up(8 * (size_t)kSmallPicks);
  int32_t* n_fill = at<int32_t>(ws, o);
  o += align_up(4);
  int32_t* hit = at<int32_t>(ws, o);

  // 1: [RMSNorm], logits, digit split
  RouterArgs ra{};
  ra.x = x;
  ra.x_bf16 = x_dtype == MOE_BF16;
  ra.T = T;
  ra.d = d;
  ra.E = E;
  ra.k = k;
  ra.prenorm = (flags & MOE_PRENORM_RMS) != 0;
  ra.eps = rms_eps;
  ra.Wr = w_router;
  ra.bias = bias;
  ra.z = z;
  ra.xd = xd;
  ra.i8 = (flags & MOE_INT8_ACT) != 0;
  MOE_TRY(launch_router_front(ra, s));
  // 2: top-k, union and the down plan (blobs at home for now)
  const uint8_t* const* home = reinterpret_cast<const uint8_t* const*>(home_table);
  RouteOut ro{z, T, E, k, idx, w, uniq, nuniq, offs, rows, stats, plan};
  MOE_TRY(launch_route_small(ro, home, s));
  // 3: placement (the table and the down plan now point at slots), 4: copies
  CacheArgs ca{};
  ca.state = static_cast<uint8_t*>(cache_state);
  ca.E = E;
  ca.S = n_slots;
  ca.slots = static_cast<uint8_t*>(slots);
  ca.blob_bytes = moe_expert_blob_bytes(dm);
  ca.home = home;
  ca.uniq = uniq;
  ca.n_uniq = nuniq;
  ca.plan = plan;
  ca.eff = eff;
  ca.fill_src = fill_src;
  ca.fill_dst = fill_dst;
  ca.n_fill = n_fill;
  ca.hit = hit;
  MOE_TRY(launch_cache_place(ca, s));
  // 5: the single-token kernels on the slots (one gate/up block per row
  // block, expert and token; each token's arithmetic as in a resident call):
  // the hits' gate/up in one launch with the misses' copies, then the
  // misses' gate/up, then down + combine over the whole union
  ExpertList EL{};
  EL.table = eff;
  EL.uniq = uniq;
  EL.n_uniq = nuniq;
  EL.offsets = offs;
  EL.list = rows;
  EL.kdiv = k;
  EL.per_row = dm->group_size == 0;
  EL.bits = 4;
  EL.i8act = (flags & MOE_INT8_ACT) != 0;
  EL.hit = hit;
  EL.want_hit = 1;
  MOE_TRY(launch_gateup_fill(EL, cap, d, f, xd, ad, T, ca, cap, s));
  EL.want_hit = 0;
  MOE_TRY(launch_gateup(EL, nullptr, cap, d, f, xd, ad, 1, T, s));
  CombineArgs cb{w, (flags & MOE_RESIDUAL) ? static_cast<const float*>(x) : nullptr, out, T, k};
  MOE_TRY(launch_down_combine(plan, nuniq, d, f, ad, cb, EL.per_row, EL.bits, s));
  return MOE_OK;
}

MOE_API int moe_timing_arm(int kernel, void* const* start_events, void* const* stop_events, int n) {
  if (kernel < 0 || kernel >= MOE_KERNEL_COUNT || n < 0) return MOE_EINVAL;
  if (n > 0 && (!start_events || !stop_events)) return MOE_EINVAL;
  TimingSlot& t = g_timing[kernel];
  const int recorded = t.next;
  t.start = reinterpret_cast<hipEvent_t const*>(start_events);
  t.stop = reinterpret_cast<hipEvent_t const*>(stop_events);
  t.n = n;
  t.next = 0;
  return recorded;
}

MOE_API int moe_trace_read(int which, void* dst, size_t bytes) {
  if (which < 0 || which >= MOE_TRACE_COUNT || !dst) return MOE_EINVAL;
  if (!kTrace) return MOE_EUNSUPPORTED;
  if (bytes > sizeof(uint64_t) * kTraceBlocks * kTraceWords) return MOE_EINVAL;
  hipError_t e;
  switch (which) {
    case MOE_TRACE_GATEUP_GEMV: e = trace_read_gemv(0, dst, bytes); break;
    case MOE_TRACE_ROUTE_SMALL: e = trace_read_gemv(1, dst, bytes); break;
    case MOE_TRACE_DOWN_T1: e = trace_read_gemv(2, dst, bytes); break;
    case MOE_TRACE_ROUTER_FRONT: e = trace_read_route(0, dst, bytes); break;
    default: e = trace_read_mfma(which - MOE_TRACE_GATEUP_THIN, dst, bytes); break;
  }
  return hip_status(e);
}

MOE_API int moe_trace_reset(void) {
  if (!kTrace) return MOE_EUNSUPPORTED;
  MOE_TRY(trace_reset_gemv());
  MOE_TRY(trace_reset_mfma());
  MOE_TRY(trace_reset_route());
  return MOE_OK;
}

MOE_API int moe_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks,
                               void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || blocks < 1) return MOE_EINVAL;
  if (!aligned(buf, 16)) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(launch_read_probe(buf, bytes, sink, blocks, s));
  return MOE_OK;
}

// Expert FFN for decode-sized batches: fused int4 dequant GEMVs on gfx950.
//
// Each chosen expert runs its feed-forward computation once per batch over all
// tokens that picked it (colibri 技术解读 (linlog.top), "集群模式与开放问题清单";
// batch union: colibrì README (简体中文), 工作原理 › 绝不为同一次磁盘读取等待两遍).
// The expert is y = Wd (silu(Wg x) * (Wu x)) on signed int4 weights with one
// fp16 scale per 64 inputs.
//
// HBM-bound design.  The lanes of a wave read 64 consecutive 16-byte chunks of
// a weight row (1 KB, one coalesced instruction), so a lane only needs the
// activation digits of its one 32-column chunk in registers and a wave keeps
// many rows' loads in flight.  The fp16 group scale is applied in registers,
// each row is reduced across the wave with DPP and across column slices
// through LDS in a fixed order.  The int4 x activation products are exact
// integer dot products (v_dot4_i32_i8 on the activation's three int8 digit
// planes), about 1.7 VALU operations per weight including the reductions,
// inside the ~2.6 per weight the chip's vector rate allows at full HBM
// bandwidth.
//
// No kernel waits on another workgroup of the same launch: on this chip a
// device-scope release/acquire writes back and invalidates the L2 of the
// XCD, which costs far more than a kernel boundary.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_util.h"
#include "moe_internal.h"
#include "cache.h"
#include "trace.h"
#include "pack.h"
#include "small_route.h"
#include "select.h"

namespace moe {

MOE_TRACE_STORAGE(g_trace_gemv, 3)
hipError_t trace_read_gemv(int slot, void* dst, size_t bytes) {
  return g_trace_gemv_read(slot, dst, bytes);
}
hipError_t trace_reset_gemv() { return g_trace_gemv_reset(); }

constexpr int kStreams = 4;                          // row streams per block
constexpr int kRowsPerStream = 16;
constexpr int kRowsPerBlock = kStreams * kRowsPerStream;  // 64 rows of one expert per block

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

// Digit form of chunk c of activation row `row` (zeros when inactive).
struct ChunkAct {
  ChunkDigits dig;
  int sxo;   // the codes' offset (8 int4, 2 int2, 0 int8) times the sum of X over the chunk
  float sc;  // value of one unit of X
};

template <int BITS = 4>
__device__ __forceinline__ ChunkAct load_act(const Digits& D, int row, int nch, int c, bool act) {
  static_assert(BITS == 4 || BITS == 2 || BITS == 8, "int4, int2 or int8 codes");
  constexpr int kOff = BITS == 4 ? 8 : BITS == 2 ? 2 : 0;
  ChunkAct a;
  if (act) {
    a.dig = load_chunk_digits(D.q + ((size_t)row * nch + c) * kChunkDigitBytes);
    a.sxo = kOff ? kOff * D.sx[(size_t)row * nch + c] : 0;
    a.sc = D.sc[(size_t)row * nch + c];
  } else {
    a.dig = ChunkDigits{};
    a.sxo = 0;
    a.sc = 0.0f;
  }
  return a;
}

// sum over a chunk of q * x: the exact integer sum, times the activation
// group's unit and the weight row's group scale s.
__device__ __forceinline__ float chunk_term(uint4 codes, float s, const ChunkAct& a) {
  return (float)(chunk_dot(codes, a.dig) - a.sxo) * (s * a.sc);
}
// int2 codes (8 bytes a chunk)
__device__ __forceinline__ float chunk_term(uint2 codes, float s, const ChunkAct& a) {
  return (float)(chunk_dot2(codes, a.dig) - a.sxo) * (s * a.sc);
}
// int8 codes (32 bytes a chunk)
struct I8Chunk {
  uint4 lo, hi;
};
__device__ __forceinline__ float chunk_term(const I8Chunk& codes, float s, const ChunkAct& a) {
  return chunk_dot8(codes.lo, codes.hi, a.dig) * (s * a.sc);
}

// Weight bytes are read once per batch and never again soon: non-temporal
// loads keep them from displacing the activations and small tables in cache.
// The pointers are cast to the global address space so the loads are
// global_load (not flat_load).
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const v4u* gv4u_ptr;
typedef __attribute__((address_space(1))) const unsigned short* gu16_ptr;
__device__ __forceinline__ uint4 stream_load16(const uint8_t* p) {
  const v4u v = __builtin_nontemporal_load((gv4u_ptr)(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const v2u* gv2u_ptr;
__device__ __forceinline__ uint2 stream_load8(const uint8_t* p) {
  const v2u v = __builtin_nontemporal_load((gv2u_ptr)(p));
  return make_uint2(v.x, v.y);
}
// A chunk of codes (32 columns): 16 bytes of int4, 8 of int2 or 32 of int8,
// and its load.
template <int BITS>
struct CodeChunk;
template <>
struct CodeChunk<4> {
  using T = uint4;
  static __device__ __forceinline__ T load(const uint8_t* p) { return stream_load16(p); }
};
template <>
struct CodeChunk<2> {
  using T = uint2;
  static __device__ __forceinline__ T load(const uint8_t* p) { return stream_load8(p); }
};
template <>
struct CodeChunk<8> {
  using T = I8Chunk;
  static __device__ __forceinline__ T load(const uint8_t* p) {
    return I8Chunk{stream_load16(p), stream_load16(p + 16)};
  }
};
__device__ __forceinline__ float stream_scale(const _Float16* p) {
  const unsigned short b = __builtin_nontemporal_load((gu16_ptr)(p));
  return (float)__builtin_bit_cast(_Float16, b);
}

// Rows are processed in batches whose loads are all issued before any is
// used, so each lane keeps 2 * kBatch (gate/up) or kBatch (down) code loads
// (16 bytes of int4, 8 of int2) in flight; int8 gate/up takes batches of
// kBatch / 2 rows of 32 bytes (the same registers).  Lanes whose chunk lies past the end of the row read chunk
// 0 of the row instead (always in bounds) and add zero (their activation
// digits and units are zero).
constexpr int kGUBatch = 4;
constexpr int kDnBatch = 4;

// Routing of a small batch in one block: top-k and union (the single-token
// gate/up kernel does the same in its own prologue, with the same per-token
// arithmetic), and the down plan when ro.plan is set (table: the expert
// table, read only then).  With px.mbo set, wave 15 also writes the union's
// M-block maps for the grouped GEMMs.
__global__ __launch_bounds__(1024) void k_route_small(RouteOut ro, const uint8_t* const* table,
                                                      PackArgs px) {
  __shared__ SmallRoute sr;
  // the expert table travels with the logits into LDS, so the blobs of the
  // union (down plan, thin tiles) are known without another memory round
  // trip once it is formed
  __shared__ const uint8_t* s_tab[kMaxE];
  const uint8_t* const* tab = table ? table : px.tt ? px.table : nullptr;
  if (tab)
    for (int e = threadIdx.x; e < ro.E; e += 1024) s_tab[e] = tab[e];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // trace points: 1 per-group sorts, 2 merges, 3 union, 4 published
  BlockTrace tr;
  tr.start();
  small_route(ro, sr, wave, 16, &tr);  // ends with a block barrier
  if (px.mbo && wave == 15) {
    mblock_map_wave(sr.offsets, sr.n, px.mblock, px.mbo, px.blk_u, px.thin_all, lane);
    if (px.tt)
      thin_tiles_wave(sr.offsets, sr.uniq, sr.rows, sr.n, s_tab, px.tt, px.tslot, px.tt_n,
                      px.thin_all, lane);
  }
  publish_small_route(ro, sr, table ? s_tab : nullptr, 1024);
  if constexpr (kTrace) {
    __syncthreads();
    tr.mark(4);
    tr.store(g_trace_gemv, 1, 0, 1);
  }
}

// Rows [r0, r0 + 16) of gate and up for NT tokens: per row, the slice's part
// of g and u, reduced over the wave, is left in s_g / s_u[j][row][slice].
template <int C, int NT, int BITS>
__device__ __forceinline__ void gateup_rows(const uint8_t* gcode, const uint8_t* ucode,
                                            const _Float16* gsc, const _Float16* usc, int d,
                                            int r0, int rl0, int slice, int lane,
                                            const Digits& xd, const int (&xrow)[NT], int nt,
                                            float (*s_g)[kRowsPerBlock][C],
                                            float (*s_u)[kRowsPerBlock][C], int pr) {
  const int nch = d / kChunk, ngx = srow(d, pr);
  const size_t row_bytes = (size_t)d * BITS / 8;
  constexpr unsigned kCB = 4 * BITS;  // code bytes of a chunk
  using Codes = typename CodeChunk<BITS>::T;
  constexpr int kB = BITS == 8 ? kGUBatch / 2 : kGUBatch, kNB = kRowsPerStream / kB;
  // batches whose 2 * kB gate and up terms fill one 8-value reduction
  constexpr int kP = 4 / kB;
  static_assert(2 * kB * kP == 8 && kNB % kP == 0, "whole reductions");
  for (int p = 0; p * 64 * C < nch; ++p) {
    const int c = (p * C + slice) * 64 + lane;
    const bool act = c < nch;
    const int cl = act ? c : 0;
    // software pipeline: the loads of batch i+1 are in flight while batch i
    // is computed
    Codes wg[2][kB], wu[2][kB];
    float sg[2][kB], su[2][kB];
    auto issue = [&](int buf, int rb0) {
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        const size_t r = (size_t)r0 + rb0 + b;
        wg[buf][b] = CodeChunk<BITS>::load(gcode + r * row_bytes + (unsigned)cl * kCB);
        wu[buf][b] = CodeChunk<BITS>::load(ucode + r * row_bytes + (unsigned)cl * kCB);
        sg[buf][b] = stream_scale(gsc + r * ngx + scol((unsigned)cl, pr));
        su[buf][b] = stream_scale(usc + r * ngx + scol((unsigned)cl, pr));
      }
    };
    issue(0, 0);
    ChunkAct xa[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) xa[j] = load_act<BITS>(xd, xrow[j], nch, c, act && j < nt);
    float v[NT][8];
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      const int cur = i & 1;
      if (i + 1 < kNB) issue(cur ^ 1, (i + 1) * kB);
      const int v0 = (i % kP) * 2 * kB;  // this batch's place in the reduction
#pragma unroll
      for (int j = 0; j < NT; ++j) {
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          v[j][v0 + b] = chunk_term(wg[cur][b], sg[cur][b], xa[j]);
          v[j][v0 + kB + b] = chunk_term(wu[cur][b], su[cur][b], xa[j]);
        }
        if (i % kP != kP - 1) continue;
        const float tot = reduce8(v[j], lane);  // lanes 8m..8m+7: value m
        if ((lane & 7) == 0) {
          // value m: batch i - kP + 1 + m / (2 kB), gate then up rows
          const int m = lane >> 3, w = m % (2 * kB);
          const int row = rl0 + (i - kP + 1 + m / (2 * kB)) * kB + (w & (kB - 1));
          float* dst = w < kB ? &s_g[j][row][slice] : &s_u[j][row][slice];
          *dst = p == 0 ? tot : *dst + tot;
        }
      }
    }
  }
}

// Gate/up: block (rb, u) computes rows [64 rb, 64 rb + 64) of gate and up of
// union expert u for all its tokens, forms a = silu(g) * u and stores those
// four 16-wide groups of a in digit form for the down projection.  The block
// has 4 row streams x C column slices of 64 chunks (d = 6144: 192 chunks,
// C = 3, 12 waves).  SMALL: the block first recomputes top-k and the union
// from the logits in ro.z; block (0, 0) publishes them.
// Block coordinates (row block rb < nx, union position u < ny, token group
// grp < G) of flat block index F (x fastest).  With several token groups, the
// groups of one (row block, expert) pair go to one XCD, dispatched back to
// back: blocks go to the 8 XCDs in turn, so F maps to pair 8 (F / 8 / G) +
// F % 8, group (F / 8) % G, and the groups' re-reads of the pair's rows meet
// in that XCD's L2.
__device__ __forceinline__ void gateup_coords(int F, int nx, int ny, int G, int& rb, int& u,
                                              int& grp) {
  if (G > 1 && (nx * ny) % 8 == 0) {
    const int hi = F >> 3, pair = (hi / G) * 8 + (F & 7);
    grp = hi % G;
    rb = pair % nx;
    u = pair / nx;
  } else {
    rb = F % nx;
    u = (F / nx) % ny;
    grp = F / (nx * ny);
  }
}

template <int C, bool SMALL, int NT, int BITS>
__device__ __forceinline__ void gateup_block(const ExpertList& L, const RouteOut& ro, int d, int f,
                                             const Digits& xd, const Digits& ad, int rb, int u,
                                             int grp, int G) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: row bases stay scalar
  const int stream = wave / C, slice = wave % C;
  // trace points: 1-3 the routing prologue's (one token: sorts, merges,
  // union), 4 the first wave's rows streamed, 5 every wave's (block barrier)
  BlockTrace tr;
  tr.start();
  const unsigned tblock = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  __shared__ float s_g[NT][kRowsPerBlock][C], s_u[NT][kRowsPerBlock][C];
  ExpertRef ex;
  const int32_t* list;
  int kdiv;
  if constexpr (SMALL) {
    __shared__ SmallRoute sr;
    const int E = ro.E, k = ro.k;
    // the expert table travels alongside the routing, so the blob address is
    // in LDS once the union is known
    __shared__ const uint8_t* s_tab[kMaxE];
    for (int e = threadIdx.x; e < E; e += 256 * C) s_tab[e] = L.table[e];
    small_route(ro, sr, wave, 4 * C, &tr);
    if (rb == 0 && u == 0) publish_small_route(ro, sr, s_tab, 256 * C);
    if (u >= sr.n) {
      tr.store(g_trace_gemv, 0, tblock, 0);
      return;
    }
    ex.blob = s_tab[sr.uniq[u]];
    ex.beg = sr.offsets[u];
    ex.n = sr.offsets[u + 1] - ex.beg;
    list = sr.rows;
    kdiv = k;
  } else {
    if ((!L.single && u >= *L.n_uniq) || (L.hit && L.hit[u] != L.want_hit)) {
      tr.store(g_trace_gemv, 0, tblock, 0);
      return;
    }
    ex = expert_ref(L, u);
    list = L.single ? nullptr : L.list;
    kdiv = L.kdiv;
  }
  const size_t fdb = (size_t)f * d * BITS / 8;  // code bytes of one matrix
  const uint8_t* gcode = ex.blob;
  const uint8_t* ucode = ex.blob + fdb;
  const _Float16* gsc = reinterpret_cast<const _Float16*>(ex.blob + 3 * fdb);
  const _Float16* usc = gsc + (size_t)f * srow(d, L.per_row);
  const int rl0 = stream * kRowsPerStream;
  const int r0 = rb * kRowsPerBlock + rl0;
  auto slot_at = [&](int i) { return list ? list[ex.beg + i] : i; };

  // grid z splits an expert's tokens: group grp takes tokens grp NT, then
  // every G NT further on
  for (int t0 = grp * NT; t0 < ex.n; t0 += NT * G) {
    const int nt = min(NT, ex.n - t0);
    int xrow[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) xrow[j] = j < nt ? slot_at(t0 + j) / kdiv : 0;
    gateup_rows<C, NT, BITS>(gcode, ucode, gsc, usc, d, r0, rl0, slice, lane, xd, xrow, nt, s_g, s_u,
                       L.per_row);
    if (t0 == grp * NT) tr.mark(4);
    __syncthreads();
    if (t0 == grp * NT) tr.mark(5);
    if (wave < nt) {
      // wave j: token j, the block's 64 rows (four 16-wide groups of a)
      const int j = wave;
      float g = 0.0f, uu = 0.0f;
#pragma unroll
      for (int sl = 0; sl < C; ++sl) {
        g += s_g[j][lane][sl];
        uu += s_u[j][lane][sl];
      }
      const int slot = slot_at(t0 + j);
      const int nca = f / kChunk, nga = f / kXGroup;
      // integer activations: the block's 64 rows are one 64-column group of a
      if (L.i8act)
        digitize64_i8(silu(g) * uu, rb * kRowsPerBlock + lane, true,
                      ad.q + (size_t)slot * nca * kChunkDigitBytes, ad.sx + (size_t)slot * nga,
                      ad.sc + (size_t)slot * nga);
      else
        digitize32(silu(g) * uu, rb * kRowsPerBlock + lane, true,
                   ad.q + (size_t)slot * nca * kChunkDigitBytes, ad.sx + (size_t)slot * nga,
                   ad.sc + (size_t)slot * nga);
    }
    __syncthreads();
  }
  tr.store(g_trace_gemv, 0, tblock, 1);
}

template <int C, bool SMALL, int NT, int BITS = 4>
__global__ __launch_bounds__(256 * C) void k_gateup(ExpertList L, RouteOut ro, int d, int f,
                                                    Digits xd, Digits ad) {
  int rb = blockIdx.x, u = blockIdx.y, grp = blockIdx.z;
  if (gridDim.z > 1)
    gateup_coords(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), gridDim.x,
                  gridDim.y, gridDim.z, rb, u, grp);
  gateup_block<C, SMALL, NT, BITS>(L, ro, d, f, xd, ad, rb, u, grp, gridDim.z);
}

// The slot cache's copies and its hits' gate/up in one launch: the first
// max_fill * kFillParts blocks copy the missed blobs (dispatched first, so
// the slow copies start at once), the others run the single-token gate/up of
// the positions with L.hit[u] == L.want_hit.  kFillParts is a multiple of 8,
// so a gate/up block keeps the XCD of its flat index.
constexpr int kFillParts = 128;
template <int C>
__global__ __launch_bounds__(256 * C) void k_gateup_fill(ExpertList L, int d, int f, Digits xd,
                                                         Digits ad, int nx, int ny, int G,
                                                         int n_fill_blocks, CacheArgs a) {
  const int F = blockIdx.x;
  if (F < n_fill_blocks) {
    fill_part(a.fill_src, a.fill_dst, a.n_fill, a.blob_bytes, F / kFillParts, F % kFillParts,
              kFillParts);
    return;
  }
  int rb, u, grp;
  gateup_coords(F - n_fill_blocks, nx, ny, G, rb, u, grp);
  gateup_block<C, false, 1, 4>(L, RouteOut{}, d, f, xd, ad, rb, u, grp, G);
}

// Rows [r0, r0 + 16) of the down projection for NT tokens into s_y[j][row].
template <int NT>
__device__ __forceinline__ void down_rows(const uint8_t* dcode, const _Float16* dsc, int f, int r0,
                                          int rl0, int lane, const Digits& ad,
                                          const int (&slot)[NT], int nt,
                                          float (*s_y)[kRowsPerBlock], int pr) {
  const int nch = f / kChunk, nga = srow(f, pr);
  constexpr int kB = kDnBatch, kNB = kRowsPerStream / kDnBatch;
  for (int p = 0; p * 64 < nch; ++p) {
    const int c = p * 64 + lane;
    const bool act = c < nch;
    const int cl = act ? c : 0;
    uint4 wd[2][kB];
    float sd[2][kB];
    auto issue = [&](int buf, int rb0) {
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        const size_t r = (size_t)r0 + rb0 + b;
        wd[buf][b] = stream_load16(dcode + r * (f / 2) + (unsigned)cl * 16u);
        sd[buf][b] = stream_scale(dsc + r * nga + scol((unsigned)cl, pr));
      }
    };
    issue(0, 0);
    ChunkAct aa[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) aa[j] = load_act(ad, slot[j], nch, c, act && j < nt);
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      const int cur = i & 1;
      if (i + 1 < kNB) issue(cur ^ 1, (i + 1) * kB);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        float v[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) v[b] = b < kB ? chunk_term(wd[cur][b], sd[cur][b], aa[j]) : 0.0f;
        const float tot = reduce8(v, lane);
        if ((lane & 7) == 0 && (lane >> 3) < kB) {
          const int row = rl0 + i * kB + (lane >> 3);
          s_y[j][row] = p == 0 ? tot : s_y[j][row] + tot;
        }
      }
    }
  }
}

// Down: block (rb, u) computes rows [64 rb, 64 rb + 64) of y = Wd a for every
// token of union expert u (4 waves x 16 rows); y is indexed by slot.
template <int NT>
__global__ __launch_bounds__(256) void k_down(ExpertList L, int d, int f, Digits ad,
                                              float* __restrict__ y) {
  const int u = blockIdx.y;
  if (!L.single && u >= *L.n_uniq) return;
  const ExpertRef ex = expert_ref(L, u);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: row bases stay scalar
  const int rb = blockIdx.x;
  const size_t fd = (size_t)f * d;
  const uint8_t* dcode = ex.blob + fd;
  const _Float16* dsc =
      reinterpret_cast<const _Float16*>(ex.blob + 3 * fd / 2) + 2 * (size_t)f * srow(d, L.per_row);
  const int rl0 = wave * kRowsPerStream;
  const int r0 = rb * kRowsPerBlock + rl0;
  __shared__ float s_y[NT][kRowsPerBlock];
  auto slot_at = [&](int i) { return L.single ? i : L.list[ex.beg + i]; };

  for (int t0 = 0; t0 < ex.n; t0 += NT) {
    const int nt = min(NT, ex.n - t0);
    int slot[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) slot[j] = j < nt ? slot_at(t0 + j) : 0;
    down_rows<NT>(dcode, dsc, f, r0, rl0, lane, ad, slot, nt, s_y, L.per_row);
    __syncthreads();
    for (int i = threadIdx.x; i < nt * kRowsPerBlock; i += 256) {
      const int j = i / kRowsPerBlock, row = i % kRowsPerBlock;
      y[(size_t)slot_at(t0 + j) * d + (size_t)rb * kRowsPerBlock + row] = s_y[j][row];
    }
    __syncthreads();
  }
}

// Down projection and combine for small batches of 2 or more tokens (one
// token: k_down_combine_t1).  Block rb owns output rows
// [8 rb, 8 rb + 8) for every union expert (wave w takes experts w, w + 4,
// ...), so each expert's down matrix is still read exactly once, and the
// block forms out[t][rows] = (x[t][rows]) + sum_j w[t][j] y[t*k+j][rows] in
// ascending j from its own results: no other block is involved.  Everything
// a wave needs of an expert is one DownPlan record, so a weight load waits
// on a single dependent load; the router weights and the residual are
// fetched at the start.
constexpr int kDcRows = 8;
constexpr int kDcWaves = 4;

template <int NT, int BITS = 4>
__global__ __launch_bounds__(64 * kDcWaves) void k_down_combine(const DownPlan* __restrict__ plan,
                                                                 const int32_t* __restrict__ n_uniq,
                                                                 int d, int f, Digits ad,
                                                                 CombineArgs cb, int pr) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r0 = blockIdx.x * kDcRows;
  const int U = *n_uniq;
  const int nch = f / kChunk, nga = srow(f, pr);
  const size_t fdb = (size_t)f * d * BITS / 8, row_bytes = (size_t)f * BITS / 8;
  constexpr unsigned kCB = 4 * BITS;
  using Codes = typename CodeChunk<BITS>::T;
  __shared__ float s_y[kSmallPicks][kDcRows];
  __shared__ float s_w[kSmallPicks];
  // epilogue operands first: thread i < T * 8 owns (token i / 8, row i % 8)
  const int nk = cb.T * cb.k;
  if (threadIdx.x < nk) s_w[threadIdx.x] = cb.w[threadIdx.x];
  const bool owner = threadIdx.x < cb.T * kDcRows;
  const size_t o = (size_t)(threadIdx.x / kDcRows) * d + r0 + threadIdx.x % kDcRows;
  const float res = (owner && cb.resid) ? cb.resid[o] : 0.0f;

  auto dcode = [&](const uint8_t* blob) { return blob + 2 * fdb + (size_t)r0 * row_bytes; };
  auto dscale = [&](const uint8_t* blob) {
    return reinterpret_cast<const _Float16*>(blob + 3 * fdb) + 2 * (size_t)f * srow(d, pr) +
           (size_t)r0 * nga;
  };
  for (int u = wave; u < U; u += kDcWaves) {
    const DownPlan pl = plan[u];
    const uint8_t* dc = dcode(pl.blob);
    const _Float16* ds = dscale(pl.blob);
    for (int p = 0; p * 64 < nch; ++p) {
      const int c = p * 64 + lane;
      const bool act = c < nch;
      const unsigned cl = act ? (unsigned)c : 0u;
      Codes wd[kDcRows];
      float sd[kDcRows];
#pragma unroll
      for (int b = 0; b < kDcRows; ++b) {
        wd[b] = CodeChunk<BITS>::load(dc + (size_t)b * row_bytes + cl * kCB);
        sd[b] = stream_scale(ds + (size_t)b * nga + scol(cl, pr));
      }
      for (int t0 = 0; t0 < pl.n; t0 += NT) {
        const int nt = min(NT, pl.n - t0);
        int slot[NT];
        ChunkAct aa[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          slot[j] = j < nt ? pl.slot[t0 + j] : 0;
          aa[j] = load_act<BITS>(ad, slot[j], nch, c, act && j < nt);
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          float v[8];
#pragma unroll
          for (int b = 0; b < kDcRows; ++b) v[b] = chunk_term(wd[b], sd[b], aa[j]);
          const float tot = reduce8(v, lane);
          if ((lane & 7) == 0 && j < nt) {
            float* dst = &s_y[slot[j]][lane >> 3];
            *dst = p == 0 ? tot : *dst + tot;
          }
        }
      }
    }
  }
  __syncthreads();
  if (owner) {
    const int t = threadIdx.x / kDcRows, b = threadIdx.x % kDcRows;
    float acc = 0.0f;
    for (int j = 0; j < cb.k; ++j) acc += s_w[t * cb.k + j] * s_y[t * cb.k + j][b];
    if (cb.resid) acc = res + acc;
    cb.out[o] = acc;
  }
}

// Down projection and combine for one token (its k picks are k distinct
// union experts).  Block rb owns output rows [R rb, R rb + R); wave w takes
// experts w, w + 8, ... over all R rows, so an expert's activation digits are
// loaded once per R rows and each lane has R weight loads in flight.
constexpr int kD1Waves = 8;

template <int R, int BITS = 4>
__global__ __launch_bounds__(64 * kD1Waves) void k_down_combine_t1(const DownPlan* __restrict__ plan,
                                                                     const int32_t* __restrict__ n_uniq,
                                                                     int d, int f, Digits ad,
                                                                     CombineArgs cb, int pr) {
  static_assert(R % 8 == 0, "rows in groups of 8 (one DPP reduction each)");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r0 = blockIdx.x * R;
  // one token picks k distinct experts: the union has k entries, known
  // without waiting for the published count
  const int U = cb.k;
  (void)n_uniq;
  const int nch = f / kChunk, nga = srow(f, pr);
  const size_t fdb = (size_t)f * d * BITS / 8, row_bytes = (size_t)f * BITS / 8;
  constexpr unsigned kCB = 4 * BITS;
  using Codes = typename CodeChunk<BITS>::T;
  // trace points: 1 the first wave's experts streamed, 2 every wave's
  BlockTrace tr;
  tr.start();
  __shared__ float s_y[kSmallPicks][R];
  __shared__ float s_w[kSmallPicks];
  // epilogue operands first: thread t < R owns output row r0 + t
  if (threadIdx.x < cb.k) s_w[threadIdx.x] = cb.w[threadIdx.x];
  const bool owner = threadIdx.x < R;
  const float res = (owner && cb.resid) ? cb.resid[r0 + threadIdx.x] : 0.0f;

  for (int u = wave; u < U; u += kD1Waves) {
    const DownPlan pl = plan[u];
    const int slot = pl.slot[0];
    const uint8_t* dc = pl.blob + 2 * fdb + (size_t)r0 * row_bytes;
    const _Float16* ds =
        reinterpret_cast<const _Float16*>(pl.blob + 3 * fdb) + 2 * (size_t)f * srow(d, pr) +
        (size_t)r0 * nga;
    for (int p = 0; p * 64 < nch; ++p) {
      const int c = p * 64 + lane;
      const bool act = c < nch;
      const unsigned cl = act ? (unsigned)c : 0u;
      Codes wv[R];
      float sv[R];
#pragma unroll
      for (int b = 0; b < R; ++b) {
        wv[b] = CodeChunk<BITS>::load(dc + (size_t)b * row_bytes + cl * kCB);
        sv[b] = stream_scale(ds + (size_t)b * nga + scol(cl, pr));
      }
      const ChunkAct a = load_act<BITS>(ad, slot, nch, c, act);
#pragma unroll
      for (int g = 0; g < R / 8; ++g) {
        float v[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) v[b] = chunk_term(wv[8 * g + b], sv[8 * g + b], a);
        const float tot = reduce8(v, lane);
        if ((lane & 7) == 0) {
          float* dst = &s_y[slot][8 * g + (lane >> 3)];
          *dst = p == 0 ? tot : *dst + tot;
        }
      }
    }
  }
  tr.mark(1);
  __syncthreads();
  tr.mark(2);
  if (owner) {
    float acc = 0.0f;
    for (int j = 0; j < cb.k; ++j) acc += s_w[j] * s_y[j][threadIdx.x];
    if (cb.resid) acc = res + acc;
    cb.out[r0 + threadIdx.x] = acc;
  }
  tr.store(g_trace_gemv, 2, blockIdx.x, 1);
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

// The same with four columns per thread (16-byte loads and stores), for a
// 16-byte aligned out (and residual); d is a multiple of 64.
__global__ __launch_bounds__(256) void k_combine4(const float* __restrict__ y,
                                                  const float* __restrict__ w, const float* resid,
                                                  float* out, int d, int k) {
  const int t = blockIdx.y;
  const int c4 = blockIdx.x * 256 + threadIdx.x;
  if (4 * c4 >= d) return;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const float4 v = reinterpret_cast<const float4*>(y + ((size_t)t * k + j) * d)[c4];
    acc.x += wj * v.x;
    acc.y += wj * v.y;
    acc.z += wj * v.z;
    acc.w += wj * v.w;
  }
  if (resid) {
    const float4 r = reinterpret_cast<const float4*>(resid + (size_t)t * d)[c4];
    acc = make_float4(r.x + acc.x, r.y + acc.y, r.z + acc.z, r.w + acc.w);
  }
  reinterpret_cast<float4*>(out + (size_t)t * d)[c4] = acc;
}

// Column slices: ceil(chunks per row / 64), at most 3 (wider rows take
// passes): four would make 16-wave blocks, whose 128-register cap the gate/up
// loop does not fit in without spilling.
static int slices(int K) {
  const int c = (K / kChunk + 63) / 64;
  return c < 1 ? 1 : (c > 3 ? 3 : c);
}

template <bool SMALL, int NT, int BITS>
static hipError_t gateup_cb(const ExpertList& L, const RouteOut& ro, int maxU, int d, int f,
                            Digits xd, Digits ad, int groups, hipStream_t s) {
  const dim3 grid(f / kRowsPerBlock, maxU, groups);
  const int c = slices(d);
  if (c == 1)
    return launch(5, k_gateup<1, SMALL, NT, BITS>, grid, dim3(256), s, L, ro, d, f, xd, ad);
  if (c == 2)
    return launch(5, k_gateup<2, SMALL, NT, BITS>, grid, dim3(512), s, L, ro, d, f, xd, ad);
  // two tokens at a time fit a block's registers only up to 2 slices
  if constexpr (NT == 1)
    return launch(5, k_gateup<3, SMALL, NT, BITS>, grid, dim3(768), s, L, ro, d, f, xd, ad);
  return hipErrorInvalidValue;
}

// int4 codes, or int2 and int8 codes one token at a time (the layer's
// single-token path)
template <bool SMALL, int NT>
static hipError_t gateup_c(const ExpertList& L, const RouteOut& ro, int maxU, int d, int f,
                           Digits xd, Digits ad, int groups, hipStream_t s) {
  if (L.bits == 4) return gateup_cb<SMALL, NT, 4>(L, ro, maxU, d, f, xd, ad, groups, s);
  if constexpr (NT == 1) {
    if (L.bits == 2) return gateup_cb<SMALL, 1, 2>(L, ro, maxU, d, f, xd, ad, groups, s);
    if (L.bits == 8) return gateup_cb<SMALL, 1, 8>(L, ro, maxU, d, f, xd, ad, groups, s);
  }
  return hipErrorInvalidValue;
}

// tokens_per_expert_max: 1 selects the single-token kernels (each block takes
// one token at a time), else two at a time where the block's registers allow
// (rows of up to 128 chunks).  token_groups: blocks per (row block, expert),
// each taking every token_groups-th one (or pair) of the expert's tokens.
// A small route (the routing prologue) takes one token and one group.
hipError_t launch_gateup(const ExpertList& L, const RouteOut* ro, int max_experts, int d, int f,
                         Digits xd, Digits ad, int tokens_per_expert_max, int token_groups,
                         hipStream_t s) {
  if (token_groups < 1) return hipErrorInvalidValue;
  if (ro) {
    // the routing prologue serves single tokens only
    if (token_groups != 1 || tokens_per_expert_max > 1) return hipErrorInvalidValue;
    return gateup_c<true, 1>(L, *ro, max_experts, d, f, xd, ad, 1, s);
  }
  if (tokens_per_expert_max > 1 && slices(d) < 3)
    return gateup_c<false, 2>(L, RouteOut{}, max_experts, d, f, xd, ad, token_groups, s);
  return gateup_c<false, 1>(L, RouteOut{}, max_experts, d, f, xd, ad, token_groups, s);
}

hipError_t launch_gateup_fill(const ExpertList& L, int max_experts, int d, int f, Digits xd,
                              Digits ad, int token_groups, const CacheArgs& a, int max_fill,
                              hipStream_t s) {
  if (token_groups < 1 || max_fill < 1 || max_experts < 1 || a.blob_bytes % 16 || !L.hit)
    return hipErrorInvalidValue;
  const int nx = f / kRowsPerBlock, ny = max_experts, G = token_groups;
  const int nfill = max_fill * kFillParts;
  const dim3 grid(nfill + nx * ny * G);
  const int c = slices(d);
  if (c == 1)
    return launch(5, k_gateup_fill<1>, grid, dim3(256), s, L, d, f, xd, ad, nx, ny, G, nfill, a);
  if (c == 2)
    return launch(5, k_gateup_fill<2>, grid, dim3(512), s, L, d, f, xd, ad, nx, ny, G, nfill, a);
  return launch(5, k_gateup_fill<3>, grid, dim3(768), s, L, d, f, xd, ad, nx, ny, G, nfill, a);
}

hipError_t launch_down(const ExpertList& L, int max_experts, int d, int f, Digits ad, float* y,
                       int tokens_per_expert_max, hipStream_t s) {
  if (L.bits != 4) return hipErrorInvalidValue;
  const dim3 grid(d / kRowsPerBlock, max_experts);
  if (tokens_per_expert_max <= 1) return launch(6, k_down<1>, grid, dim3(256), s, L, d, f, ad, y);
  return launch(6, k_down<2>, grid, dim3(256), s, L, d, f, ad, y);
}

hipError_t launch_route_small(const RouteOut& ro, const uint8_t* const* table, hipStream_t s,
                              const PackArgs* map) {
  if (ro.plan && !table) return hipErrorInvalidValue;
  PackArgs px{};
  if (map) {
    // one wave maps a union of at most 64 experts
    if (!map->mbo || !map->blk_u || map->mblock < 1 ||
        ro.T * ro.k > 64)
      return hipErrorInvalidValue;
    px.mbo = map->mbo;
    px.blk_u = map->blk_u;
    px.mblock = map->mblock;
    px.thin_all = map->thin_all;
    px.tt = map->tt;
    px.tslot = map->tslot;
    px.tt_n = map->tt_n;
    px.table = map->table;
    if (px.tt && (!px.tslot || !px.table)) return hipErrorInvalidValue;
  }
  return launch(3, k_route_small, dim3(1), dim3(1024), s, ro, table, px);
}

template <int BITS>
static hipError_t down_combine_b(const DownPlan* plan, const int32_t* n_uniq, int d, int f,
                                 Digits ad, const CombineArgs& cb, int per_row, hipStream_t s) {
  if (cb.T == 1) {
    // int8: 8 rows of 32 bytes a lane hold as many registers as 16 of int4
    if constexpr (BITS == 8) {
      return launch(6, k_down_combine_t1<8, 8>, dim3(d / 8), dim3(64 * kD1Waves), s, plan, n_uniq,
                    d, f, ad, cb, per_row);
    } else {
      if (d % 24 == 0)
        return launch(6, k_down_combine_t1<24, BITS>, dim3(d / 24), dim3(64 * kD1Waves), s, plan,
                      n_uniq, d, f, ad, cb, per_row);
      return launch(6, k_down_combine_t1<16, BITS>, dim3(d / 16), dim3(64 * kD1Waves), s, plan,
                    n_uniq, d, f, ad, cb, per_row);
    }
  }
  return launch(6, k_down_combine<2, BITS>, dim3(d / kDcRows), dim3(64 * kDcWaves), s, plan,
                n_uniq, d, f, ad, cb, per_row);
}

hipError_t launch_down_combine(const DownPlan* plan, const int32_t* n_uniq, int d, int f,
                               Digits ad, const CombineArgs& cb, int per_row, int bits,
                               hipStream_t s) {
  if (bits == 4) return down_combine_b<4>(plan, n_uniq, d, f, ad, cb, per_row, s);
  if (bits == 2) return down_combine_b<2>(plan, n_uniq, d, f, ad, cb, per_row, s);
  if (bits == 8) return down_combine_b<8>(plan, n_uniq, d, f, ad, cb, per_row, s);
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const float* y, const float* w, const float* resid, float* out, int T,
                          int d, int k, hipStream_t s) {
  const bool wide = ((uintptr_t)out % 16 == 0) && ((uintptr_t)resid % 16 == 0) && d % 4 == 0;
  if (wide)
    return launch(7, k_combine4, dim3((d / 4 + 255) / 256, T), dim3(256), s, y, w, resid, out, d, k);
  return launch(7, k_combine, dim3((d + 255) / 256, T), dim3(256), s, y, w, resid, out, d, k);
}

}  // namespace moe

// Expert FFN for multi-token batches (prefill, batched verification): a
// grouped GEMM on the MFMA units.
//
// Each chosen expert runs its feed-forward computation once per batch over all
// of its tokens, so its bytes are read once (colibri 技术解读 (linlog.top),
// "集群模式与开放问题清单"; colibrì README (简体中文), 工作原理 › 绝不为同一次磁盘读取等待两遍).
//
// Arithmetic:
//   x = x' * unit[m]      x' in fp16 (k_pack: a power of two per row, |x'| < 2^14)
//   W[n][k] = fp16(q * s[n][g])    q in [-8, 7] is formed exactly as the fp16
//                         number 1032 + q (one AND/OR per two codes) minus 1032;
//                         the product with the group's fp16 scale is rounded
//                         once (relative error <= 2^-11, exact when q * s fits)
//   out[m][n] = unit[m] * sum_k x'[m][k] W[n][k]    v_mfma_f32_16x16x32_f16, fp32
//                         accumulation straight through the MFMA C operand
// q * s stays a normal fp16 number for 2^-14 <= |s| <= 2^12; smaller scales
// lose relative precision gradually (fp16 subnormals), larger ones overflow.
//
// Work unit: one block (16 waves of 32 weight rows; 4 waves of 32 rows for
// batches of up to 16 rows and for one expert over many tokens) = one expert
// x one M-block of up to 64 (16) of its tokens x 512 (128) weight rows
// (gate/up:
// a wave's rows are half gate rows and the same rows of up, so SwiGLU is
// local to the wave).  K is walked in 128-column
// stages copied global -> LDS without passing through registers, into a ring
// of 3 stages; the A and B fragments come from LDS.  d and f must be multiples
// of 512.
// A 32-bit word of 8 codes splits into fp16 pairs (column j, column j + 4), so
// k_pack stores each block of 8 columns in that order: position p holds column
// (p >> 1) + 4 (p & 1).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <type_traits>

#include "device_util.h"
#include "moe.h"
#include "moe_internal.h"
#include "pack.h"
#include "trace.h"

namespace moe {

MOE_TRACE_STORAGE(g_trace_mfma, 4)
hipError_t trace_read_mfma(int slot, void* dst, size_t bytes) {
  return g_trace_mfma_read(slot, dst, bytes);
}
hipError_t trace_reset_mfma() { return g_trace_mfma_reset(); }

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4* g_u32x4_ptr;

constexpr float kBias = 1032.0f;

__device__ __forceinline__ u32x4 nt_load16(const uint8_t* p) {
  return __builtin_nontemporal_load((g_u32x4_ptr)(p));
}
// 16 bytes through the global address space (no generic-pointer checks)
__device__ __forceinline__ uint4 gload16(const void* p) {
  const u32x4 v = *(g_u32x4_ptr)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 8 codes (column j in bits 4j..4j+3) and their group's scale (both halves)
// -> 8 fp16 weights q * s in slot order (col 0, 4, 1, 5, 2, 6, 3, 7).
__device__ __forceinline__ f16x8 dequant8(uint32_t w, f16x2 s2) {
  const f16x2 off = {(_Float16)kBias, (_Float16)kBias};
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t h = (((w >> (4 * j)) & 0x000F000Fu) ^ 0x00080008u) | 0x64006400u;
    const f16x2 q = __builtin_bit_cast(f16x2, h) - off;  // exact
    const f16x2 ws = q * s2;                             // one rounding
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
// One wave per row (pack.h); with mbo set, the last block instead writes the
// union's M-block prefix (mbo[u] = sum over u' < u of ceil(count(u') /
// mblock), u = 0..U), with tt set the thin tiles, with xtab set the XCD
// placement of the M-blocks.
__global__ __launch_bounds__(256) void k_pack(PackArgs p) {
  if (p.mbo && blockIdx.x == gridDim.x - 1) {
    // thread t maps experts 4t .. 4t + 3: thin ones (at most kThinTokens
    // tokens, or every expert with thin_all) take one thin tile per
    // kThinTokens tokens, the others ceil(count / mblock) M-blocks; two
    // block-wide exclusive scans place them
    __shared__ int s_tot[2][4];
    __shared__ int s_tb[4 * 256 + 1];  // thin tiles before expert u, u = 0..U
    const int U = *p.n_uniq, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int c[4], th[4], sum = 0, sum_t = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = 4 * t + i;
      const int n = u < U ? p.offsets[u + 1] - p.offsets[u] : 0;
      const bool thin = u < U && (p.thin_all || n <= kThinTokens);
      th[i] = thin ? (n + kThinTokens - 1) / kThinTokens : 0;
      c[i] = u < U && !thin ? (n + p.mblock - 1) / p.mblock : 0;
      sum += c[i];
      sum_t += th[i];
    }
    int incl = sum, incl_t = sum_t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int nb = __shfl_up(incl, o, 64), nt = __shfl_up(incl_t, o, 64);
      if (lane >= o) {
        incl += nb;
        incl_t += nt;
      }
    }
    if (lane == 63) {
      s_tot[0][wave] = incl;
      s_tot[1][wave] = incl_t;
    }
    __syncthreads();
    int run = incl - sum, run_t = incl_t - sum_t;
    for (int w = 0; w < wave; ++w) {
      run += s_tot[0][w];
      run_t += s_tot[1][w];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = 4 * t + i;
      if (u < U) {
        p.mbo[u] = run;
        for (int j = 0; j < c[i]; ++j) p.blk_u[run + j] = u;
        s_tb[u] = run_t;
      }
      run += c[i];
      run_t += th[i];
    }
    const int tot_t = s_tot[1][0] + s_tot[1][1] + s_tot[1][2] + s_tot[1][3];
    if (t == 0) {
      p.mbo[U] = s_tot[0][0] + s_tot[0][1] + s_tot[0][2] + s_tot[0][3];
      s_tb[U] = tot_t;
    }
    if (p.tt) {
      // the thin tiles, expert by expert, kThinTokens tokens a tile: one
      // tile a thread, its 16 slot loads issued together (an expert of
      // several hundred tokens has tens of tiles)
      __syncthreads();
      const int nt = min(tot_t, p.tt_n);
      for (int j = t; j < nt; j += (int)blockDim.x) {
        // the tile's expert: s_tb[u] <= j < s_tb[u + 1] (experts without
        // thin tiles have s_tb[u] == s_tb[u + 1])
        int lo = 0, hi = U;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_tb[mid] <= j) lo = mid;
          else hi = mid;
        }
        const int off = p.offsets[lo], n = p.offsets[lo + 1] - off;
        const int tok0 = (j - s_tb[lo]) * kThinTokens;
        int v[kTileSlots];
#pragma unroll
        for (int q = 0; q < kTileSlots; ++q) v[q] = p.list[off + min(tok0 + q, n - 1)];
        ThinTile r{};
        r.blob = p.table[p.uniq[lo]];
        r.off = off;
        r.cnt = n;
        r.tok0 = tok0;
        p.tt[j] = r;
        int4* ds = reinterpret_cast<int4*>(p.tslot + (size_t)j * kTileSlots);
#pragma unroll
        for (int q = 0; q < kTileSlots / 4; ++q)
          ds[q] = make_int4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      }
      for (int j = tot_t + t; j < p.tt_n; j += (int)blockDim.x) p.tt[j] = ThinTile{};
    }
    if (!p.xtab) return;
    // The M-blocked experts onto the 8 XCDs (blocks of a launch go to the
    // XCDs in turn, and an XCD's blocks share its L2): whole experts, in
    // order of decreasing M-block count (then ascending union position),
    // each onto the XCD with the fewest M-blocks so far (ties: the lower
    // XCD), so the blocks of one expert read its weights and its tokens'
    // activation rows through one L2.  No list outgrows xs (see
    // xcd_stride); the guard only keeps a write in bounds.
    __shared__ int s_c[4 * 256], s_beg[4 * 256], s_cmax;  // 4 experts a thread
    if (t == 0) s_cmax = 0;
    __syncthreads();
    int cm = 0;
    run = incl - sum;
    for (int w = 0; w < wave; ++w) run += s_tot[0][w];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = 4 * t + i;
      if (u < U) {
        s_c[u] = c[i];
        s_beg[u] = run;
      }
      run += c[i];
      cm = max(cm, c[i]);
    }
    atomicMax(&s_cmax, cm);
    __syncthreads();
    if (wave != 0) return;
    int load = 0;  // lane x < kXcds: M-blocks placed on XCD x
    for (int cc = s_cmax; cc >= 1; --cc) {
      for (int u0 = 0; u0 < U; u0 += 64) {
        uint64_t pick = __ballot(u0 + lane < U && s_c[u0 + lane] == cc);
        while (pick) {
          const int u = u0 + __builtin_ctzll(pick);
          pick &= pick - 1;
          int mn = lane < kXcds ? load : INT_MAX;
#pragma unroll
          for (int o = 1; o < kXcds; o <<= 1) mn = min(mn, __shfl_xor(mn, o, 64));
          const int x = __builtin_ctzll(__ballot(lane < kXcds && load == mn));
          const int pos = __shfl(load, x, 64);
          for (int i = lane; i < cc; i += 64)
            if (pos + i < p.xs) p.xtab[x * p.xs + pos + i] = s_beg[u] + i;
          if (lane == x) load += cc;
        }
      }
    }
    if (lane < kXcds) p.xcnt[lane] = min(load, p.xs);
    return;
  }
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= p.rows) return;
  if (p.i8) pack_row_i8(p, r, threadIdx.x & 63);
  else pack_row(p, r, threadIdx.x & 63);
}

// ---------------------------------------------------------------- projection
enum { kGateUp = 0, kDown = 1 };

struct GemmArgs {
  ExpertList L;
  const int32_t* mbo;    // union: M-block prefix
  const int32_t* blk_u;  // union: expert of each M-block
  int d, f;
  const _Float16* a;     // packed A rows [rows][K]
  const float* unit;     // [rows]
  float* out;            // gate/up: silu(g) * u [slots][f]; down: y [slots][d]
  const float* corr;     // thin: [rows][K / 64] group corrections of A
  const ThinTile* tt;    // thin union: the record of thin block jy
  const int32_t* tslot;  // thin union: [jy][kTileSlots] the tile's slots
  int thick_blocks;      // mixed launch: M-blocked blocks before the thin ones
  // mixed launch: gx blocks along the weight rows; the M-blocked blocks of
  // XCD x are the entries of xtab[x * xs ..] (xcnt[x] of them)
  int gx;
  const int32_t* xtab;
  const int32_t* xcnt;
  int xs;
  // pa: a travels packed by 64-column groups between the thin GEMMs.  Gate/up
  // then writes a' [slots][f] fp16 in pack order, a_unit and a_corr
  // [slots][f / 64] (corr_off: the code width's offset) instead of out; down
  // reads unit as [rows][K / 64] per-group units.
  int pa;
  _Float16* a_out;
  float* a_unit;
  float* a_corr;
  float corr_off;
  // ia (integer activations, with pa): a is int8 [rows][K] (bytes) with one
  // fp32 scale per 64-column group in corr; gate/up writes a as int8 into
  // a_out and its group scales into a_corr
  int ia;
};

typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

// Global -> LDS copies that bypass registers: lane l's 16 bytes land at
// lds + 16 l, `lds` being wave-uniform (M0); completion is tracked by vmcnt
// only.  They are issued as inline assembly so that the compiler, which
// cannot tell which LDS bytes a copy writes, does not drain every copy in
// flight before each LDS read; the ring protocol below waits for exactly the
// stage it reads.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_u8_t*)p);
}
__device__ __forceinline__ void dma16(const void* src, void* lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_addr(lds)) : "memory", "m0");
}
// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt unconstrained)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70);
}

// LDS: a ring of kRing stages, each covering 128 K-columns (two scale groups),
//   B  [wave][64 rows][64 B]   codes; row r holds its 16-byte piece p at slot
//                              p ^ ((r >> 1) & 3) ^ ((r >> 3) & 1)
//   A  [64 rows][256 B]        packed activations; piece p (8 columns) of row r
//                              at slot p ^ (r & 15)
// followed by per-wave scales, two buffers of [wave rows][8 groups] fp16 (8
// groups = 4 stages), refilled every 4 stages.
constexpr int kSC = 128;
// Block shapes: GW waves (GW x 16 NTW weight rows) x an M-block of MB tokens
// (each wave copies MB / GW activation rows), over a ring of R stages (R - 1
// in flight).  GW = 16, NTW = 2, R = 3, MB = 64: 160 KB, one block per CU,
// four waves per SIMD (prefill; 8 waves of 64 rows in the same LDS were 2%
// slower); GW = 4, NTW = 2, MB = 16, R = 3: 40 KB, several blocks per CU, so a
// batch of a few tokens over a dozen experts keeps enough waves and bytes in
// flight (8 tokens over 13 experts: gate/up 48 us, down 25 us; 2 waves of 64
// rows with 5- and 4-stage rings took 54 and 29 us, 4 waves with them 50 and
// 26 us); GW = 4, NTW = 2, MB = 64, R = 3: 76 KB, one
// expert over many tokens: 128 rows a block, as many blocks as CUs at 512
// tokens, every SIMD busy (2 waves of 64 rows left half of them idle: one
// expert at M = 512 took 84 us instead of 56).
// The scale pieces are double-buffered (4 stages each): a piece is refilled
// R - 1 stages before its first use, which must come after the last use of the
// piece two back, so R <= 5.
template <int GW, int R, int MB, int NTW>
struct RingShape {
  static constexpr int kNt = NTW;                 // 16-row N-tiles per wave
  static constexpr int kWaveRows = 16 * NTW;      // weight rows per wave
  static constexpr int kBWave = kWaveRows * (kSC / 2);
  static constexpr int kScaleWave = 2 * kWaveRows * 16;  // two buffers of [rows][8 groups]
  static constexpr int kRing = R;
  static constexpr int kMBlock = MB;
  static constexpr int kARows = MB / GW;       // activation rows copied per wave
  static constexpr int kACopies = kARows / 4;  // 1 KB copies (4 rows) per wave and stage
  static constexpr int kMT = kMBlock / 16;
  static constexpr int kStageB = GW * kBWave;
  static constexpr int kStage = kStageB + kMBlock * kSC * 2;
  static constexpr int kScaleOff = kRing * kStage;
  static constexpr int kLdsBytes = kScaleOff + GW * kScaleWave;
  static_assert(kLdsBytes <= 160 * 1024, "fits one CU");
  static_assert(R >= 3 && R <= 5, "ring depth");
  static_assert(MB % 16 == 0 && kARows % 4 == 0, "whole M-tiles, whole copies");
  static_assert(NTW == 2 || NTW == 4, "gate/up rows split evenly into gate and up");
};

// Copies a wave has in flight after issuing stages st + 1 .. st + R - 2, with
// st % 4 == PH: NB code copies, NA activation copies, and (NS = 1) a scale
// copy in stages that are multiples of 4.
template <int R, int PH, int NB, int NA, int NS>
constexpr int copies_ahead() {
  int c = 0;
  for (int i = 1; i <= R - 2; ++i) c += NB + NA + (NS && ((PH + i) & 3) == 0 ? 1 : 0);
  return c;
}
// copies per wave and stage: NTW (codes, 16 rows each) + kACopies (activations: wave w copies
// rows kARows w .. kARows (w + 1) - 1), plus 1 (scales) in stages 0, 4, 8, ...
// A wave whose first row lies past the block's last token copies no
// activations (the A rows it would fill only feed output rows that are never
// stored: an MFMA output row depends on its own A row alone); rows past the
// block's tokens in a wave that does copy take the last token's row.

// One block: GW waves, each owning 16 NTW weight rows, times one M-block of up
// to MB tokens of one expert.  Stage st is copied while stage st - 2 is computed;
// every copy of stage st is issued before any of stage st + 1, so "stage st has
// landed" is "at most the copies of stage st + 1 are in flight".
//
// The body takes the block's LDS and its coordinates (jx along the weight rows, jy along
// the M-blocks), so the
// mixed launch below can run it beside thin blocks.
template <int MODE, int GW, int R, int MB, int NTW>
__device__ __forceinline__ void gemm_body(const GemmArgs& g, uint8_t* s_lds, int jx, int jy) {
  using Shape = RingShape<GW, R, MB, NTW>;
  constexpr int kNt = Shape::kNt, kWaveRows = Shape::kWaveRows, kBWave = Shape::kBWave;
  constexpr int kScaleWave = Shape::kScaleWave;
  constexpr int kHalf = kWaveRows / 2;
  constexpr int kARows = Shape::kARows, kACopies = Shape::kACopies;
  constexpr int kRing = Shape::kRing;
  constexpr int kMBlock = Shape::kMBlock, kMT = Shape::kMT, kStageB = Shape::kStageB;
  constexpr int kStage = Shape::kStage, kScaleOff = Shape::kScaleOff;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int d = g.d, f = g.f;
  const int K = MODE == kGateUp ? d : f;
  const int pr = g.L.per_row;
  const int ng = srow(K, pr);  // scales per weight row

  // ---- the block's expert and tokens
  const ExpertList& L = g.L;
  int off, cnt, tok0;
  const uint8_t* blob;
  if (L.single) {
    off = 0;
    cnt = L.single_n;
    tok0 = jy * kMBlock;
    if (tok0 >= cnt) return;
    blob = L.single;
  } else {
    const int j = jy;
    if (j >= g.mbo[*L.n_uniq]) return;
    const int u = g.blk_u[j];
    off = L.offsets[u];
    cnt = L.offsets[u + 1] - off;
    tok0 = (j - g.mbo[u]) * kMBlock;
    blob = L.table[L.uniq[u]];
  }
  const int nmt = (min(kMBlock, cnt - tok0) + 15) >> 4;
  // packed row of the block's token i (past the last token: the last one)
  auto row_of = [&](int i) -> uint32_t {
    const int ti = min(tok0 + i, cnt - 1);
    if (L.single) return (uint32_t)ti;
    const int slot = L.list[off + ti];
    return (uint32_t)(MODE == kGateUp ? slot / L.kdiv : slot);
  };

  // ---- this wave's weight rows (ring rows 0..31 and 32..63); waves past the
  // last row copy the last wave's rows and compute nothing
  const int nwaves = MODE == kGateUp ? f / kHalf : d / kWaveRows;
  const int wv = jx * GW + wave;
  const bool active = wv < nwaves;
  const int wc = min(wv, nwaves - 1);
  const size_t fd = (size_t)f * d;
  const _Float16* sbase = reinterpret_cast<const _Float16*>(blob + 3 * (fd / 2));
  const size_t gate_sc = (size_t)f * srow(d, pr);  // scales of the gate (and of the up) matrix
  const uint8_t *c0, *c1;
  const _Float16 *s0, *s1;
  if (MODE == kGateUp) {
    c0 = blob + (size_t)(kHalf * wc) * (K / 2);
    c1 = c0 + fd / 2;
    s0 = sbase + (size_t)(kHalf * wc) * ng;
    s1 = s0 + gate_sc;
  } else {
    c0 = blob + fd + (size_t)(kWaveRows * wc) * (K / 2);
    c1 = c0 + (size_t)kHalf * (K / 2);
    s0 = sbase + 2 * gate_sc + (size_t)(kWaveRows * wc) * ng;
    s1 = s0 + (size_t)kHalf * ng;
  }
  const int n = lane & 15, kg = lane >> 4;

  // ---- per-lane copy sources
  // codes, copy i: lane l -> ring row 16 i + l / 4, slot l % 4 (piece slot ^ swizzle)
  const uint32_t b_piece = (uint32_t)((lane & 3) ^ ((lane >> 3) & 3) ^ ((lane >> 5) & 1));
  const uint32_t b_off = (uint32_t)(lane >> 2) * (uint32_t)(K / 2) + b_piece * 16u;
  const uint32_t b_half = 16u * (uint32_t)(K / 2);
  // activations, copy i of wave w: lane l -> row 8 w + 4 i + l / 16, slot l % 16
  // (M-tile w / 2)
  uint32_t a_off[kACopies];
#pragma unroll
  for (int i = 0; i < kACopies; ++i) {
    const int r = kARows * wave + 4 * i + (lane >> 4);
    a_off[i] = row_of(r) * (uint32_t)K + (uint32_t)((lane & 15) ^ (r & 15)) * 8u;
  }
  // scales: lane l < kWaveRows -> ring row l, 8 groups (the other lanes copy
  // nothing)
  const int sr_lane = lane % kWaveRows;
  const _Float16* s_lane = (sr_lane < kHalf ? s0 : s1) + (size_t)(sr_lane % kHalf) * ng;
  uint8_t* s_scales = s_lds + kScaleOff + wave * kScaleWave;
  if (pr && lane < kWaveRows) {
    // one scale per row: put in every group of both buffers, once (this
    // wave's own LDS; the first stage's wait covers the writes)
    const uint32_t h = *reinterpret_cast<const uint16_t*>(s_lane);
    const uint32_t hh = h | (h << 16);
    const uint4 v = make_uint4(hh, hh, hh, hh);
    *reinterpret_cast<uint4*>(s_scales + lane * 16) = v;
    *reinterpret_cast<uint4*>(s_scales + kWaveRows * 16 + lane * 16) = v;
  }

  const int nst = K / kSC;
  // a wave copies its activation rows only when the first is one of the
  // block's tokens (wave-uniform)
  const bool a_copy = kARows * wave < min(kMBlock, cnt - tok0);
  auto issue = [&](int st) {
    uint8_t* base = s_lds + (st % kRing) * kStage;
    const uint32_t so = (uint32_t)st * (kSC / 2);
#pragma unroll
    for (int i = 0; i < kNt; ++i)
      dma16((i < kNt / 2 ? c0 : c1) + (i % (kNt / 2)) * b_half + so + b_off,
            base + wave * kBWave + i * 1024);
    if (a_copy) {
#pragma unroll
      for (int i = 0; i < kACopies; ++i)
        dma16(g.a + a_off[i] + st * kSC, base + kStageB + (kARows * wave + 4 * i) * (kSC * 2));
    }
    if ((st & 3) == 0 && !pr && lane < kWaveRows)
      dma16(s_lane + 2 * st, s_scales + ((st >> 2) & 1) * (kWaveRows * 16));
  };

  f32x4 acc[kMT][kNt];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNt; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // scale group 2 st + gg of a landed stage.  Lane (n, kg) takes, for MFMA
  // step j, columns 16 kg + 8 j .. + 8 of the group: dword 2 kg + j of the
  // row's 32 code bytes and 8-column block 2 kg + j of the activations.
  auto group = [&](int st, int gg) {
    const uint8_t* base = s_lds + (st % kRing) * kStage;
    const int gi = 2 * st + gg;
    const uint8_t* sc = s_scales + ((gi >> 3) & 1) * (kWaveRows * 16) + (gi & 7) * 2;
    f16x8 b0[kNt], b1[kNt];
#pragma unroll
    for (int nt = 0; nt < kNt; ++nt) {
      const int r = 16 * nt + n;
      const int slot = (2 * gg + (kg >> 1)) ^ ((r >> 1) & 3) ^ ((r >> 3) & 1);
      const uint2 w = *reinterpret_cast<const uint2*>(base + wave * kBWave + r * (kSC / 2) +
                                                      slot * 16 + 8 * (kg & 1));
      const uint32_t h = *reinterpret_cast<const uint16_t*>(sc + r * 16);
      const f16x2 s2 = __builtin_bit_cast(f16x2, h | (h << 16));
      b0[nt] = dequant8(w.x, s2);
      b1[nt] = dequant8(w.y, s2);
    }
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      if (mt < nmt) {
        const uint8_t* ar = base + kStageB + (16 * mt + n) * (kSC * 2);
        const int p0 = 8 * gg + 2 * kg;
        const f16x8 a0 = *reinterpret_cast<const f16x8*>(ar + (p0 ^ n) * 16);
        const f16x8 a1 = *reinterpret_cast<const f16x8*>(ar + ((p0 + 1) ^ n) * 16);
#pragma unroll
        for (int nt = 0; nt < kNt; ++nt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0[nt], acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1[nt], acc[mt][nt], 0, 0, 0);
        }
      }
    }
  };

#pragma unroll
  for (int i = 0; i < kRing - 1; ++i) issue(i);
  // one step: wait for stage st, barrier, refill the slot of stage st - 1,
  // compute stage st.  Unrolled by the 4-stage scale period so that every
  // wait count is a constant.
  auto step = [&](int st, auto phase) {
    constexpr int PH = decltype(phase)::value;
    if (st + kRing - 2 < nst) {
      // stage st has landed once at most the copies of stages st + 1 ..
      // st + R - 2 are in flight
      // (per-row scales: no scale copies)
      if (a_copy && !pr) wait_vm_lgkm0<copies_ahead<kRing, PH, kNt, kACopies, 1>()>();
      else if (a_copy) wait_vm_lgkm0<copies_ahead<kRing, PH, kNt, kACopies, 0>()>();
      else if (!pr) wait_vm_lgkm0<copies_ahead<kRing, PH, kNt, 0, 1>()>();
      else wait_vm_lgkm0<copies_ahead<kRing, PH, kNt, 0, 0>()>();
    } else {
      wait_vm_lgkm0<0>();
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // every wave is past stage st - 1: its ring slot takes stage st + R - 1
    if (st + kRing - 1 < nst) issue(st + kRing - 1);
    if (active) {
      group(st, 0);
      group(st, 1);
    }
  };
  for (int st0 = 0; st0 < nst; st0 += 4) {  // nst is a multiple of 4
    step(st0, std::integral_constant<int, 0>());
    step(st0 + 1, std::integral_constant<int, 1>());
    step(st0 + 2, std::integral_constant<int, 2>());
    step(st0 + 3, std::integral_constant<int, 3>());
  }
  if (!active) return;

  // epilogue: lane (n, kg) holds, per tile, tokens 4 kg + i of the M-tile for
  // weight row 16 nt + n
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    if (mt >= nmt) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ti = tok0 + 16 * mt + 4 * kg + i;
      if (ti >= cnt) continue;
      const int slot = L.single ? ti : L.list[off + ti];
      if (MODE == kGateUp) {
        const int xr = L.single ? ti : slot / L.kdiv;
        const float us = g.unit[xr];
        float* orow = g.out + (size_t)slot * f + kHalf * wv;
#pragma unroll
        for (int h = 0; h < kNt / 2; ++h) {
          const float gv = acc[mt][h][i] * us, uv = acc[mt][h + kNt / 2][i] * us;
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

template <int MODE, int GW, int R, int MB, int NTW>
__global__ __launch_bounds__(64 * GW) void k_gemm(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[RingShape<GW, R, MB, NTW>::kLdsBytes];
  gemm_body<MODE, GW, R, MB, NTW>(g, s_lds, blockIdx.x, blockIdx.y);
}

// ---------------------------------------------------------------- thin GEMM
// One block = one 16-row M-tile of one expert (int4 layers: the experts of at
// most kThinTokens tokens, most of a prefill chunk's union and every expert of
// a small batch; int8 and int2 layers: every M-tile of every expert) x GW
// waves of 32 weight rows.  The weights' per-64-column scales multiply the
// fp32 partial sum of each group instead of every weight: the codes enter the
// MFMA as the exact fp16 subnormals (q + o) * 2^-24, o = 8 (int4), 128
// (int8) or 2 (int2) (a few bit operations per two codes), each group's
// partial starts from the group's correction -o * 2^-24 * sum(x') (written by
// k_pack), so it ends as 2^-24 * sum(x' q), and partial times scale is added
// to the accumulator.  That is about half the VALU work of scaling every
// weight before the MFMA, the weights stay exact (only x' is rounded), and the
// scale's size is not limited by fp16.  Every code width feeds the MFMA the
// same 8 columns per lane and step in the same order (column j with column
// j + 4), so the activations are packed alike for all of them.
// A stage (128 columns: two scale groups) holds, for every wave, its 32 rows
// of codes, and for the block the M-tile's activation rows (copied by waves
// 0..3) and group corrections (wave 0); the ring has R stages, R - 1 in
// flight.  Each wave copies its rows' scales 16 bytes (8 groups, 4 stages) at
// a time into two buffers of its own.
constexpr int kThinWaveRows = 32;
constexpr int kSwWindows = 4;  // scales in registers: 32-group windows, K <= 8192

template <int GW, int R, int BITS, bool PA = false, bool SW = false, bool IA = false>
struct ThinShape {
  static constexpr int kRowStage = 16 * BITS;                 // code bytes of a row per stage
  static constexpr int kPieces = kRowStage / 16;              // its 16-byte pieces
  static constexpr int kRowsPerCopy = 64 / kPieces;           // rows one 1 KB copy covers
  static constexpr int kCopies = kThinWaveRows / kRowsPerCopy;  // code copies per wave and stage
  static constexpr int kBWave = kThinWaveRows * kRowStage;
  static constexpr int kStageB = GW * kBWave;
  // 16 activation rows of 128 columns: fp16 (256 B a row), or int8 (IA)
  static constexpr int kStageA = kThinTokens * kSC * (IA ? 1 : 2);
  // [2 groups][16 tokens] f32 corrections (IA: the activations' group
  // scales), then (per-group A units) the same of units
  static constexpr int kStageC = (PA && !IA ? 64 : 32) * 4;
  static constexpr int kStage = kStageB + kStageA + kStageC;
  static constexpr int kScalePiece = kThinWaveRows * 16;      // [32 rows][8 groups] fp16
  static constexpr int kScaleOff = R * kStage;
  // scales in registers (SW): no scale buffers
  static constexpr int kLdsBytes = kScaleOff + (SW ? 0 : GW * 2 * kScalePiece);
  // the per-group pack of a's reductions ([2][GW][16 tokens] f32) use a ring
  // slot no wave reads after the last stage
  static_assert(2 * GW * kThinTokens * 4 <= kStage, "reduction area fits a stage");
  static_assert(BITS == 4 || BITS == 8 || BITS == 2, "code width");
  static_assert(kLdsBytes <= 160 * 1024, "fits one CU");
  // a scale piece is copied R - 1 stages before its first use, which must
  // come after the last use of the piece two back
  static_assert(R >= 3 && (SW || R <= 5), "ring depth");
  static_assert(GW >= 4, "waves 0..3 copy the 16 activation rows");
  static_assert(!IA || PA, "integer activations: a travels as int8 by groups");
  static_assert(kThinTokens == 16, "one M-tile");
};

// Slot of 16-byte piece p of row r of a wave's stage (a permutation of the
// row's pieces that spreads neighbouring rows over the LDS banks).
template <int BITS>
__device__ __forceinline__ int thin_slot(int p, int r) {
  if constexpr (BITS == 4) return p ^ ((r >> 1) & 3) ^ ((r >> 3) & 1);
  else if constexpr (BITS == 8) return p ^ (r & 7);
  else return p ^ ((r >> 2) & 1);
}

// 8 int4 codes (column j in bits 4j..4j+3) -> the fp16 subnormals (q + 8) *
// 2^-24 in slot order (col 0, 4, 1, 5, 2, 6, 3, 7): q + 8 is the code with
// its sign bit flipped.
__device__ __forceinline__ f16x8 raw8(uint32_t w) {
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t h = ((w >> (4 * j)) & 0x000F000Fu) ^ 0x00080008u;
    const f16x2 q = __builtin_bit_cast(f16x2, h);
    r[2 * j] = q[0];
    r[2 * j + 1] = q[1];
  }
  return r;
}
// 8 int8 codes (columns 0..3 in lo, 4..7 in hi) -> (q + 128) * 2^-24, same
// slot order: byte i of lo and byte i of hi into the low bytes of the two
// halves (v_perm), sign bits flipped.
__device__ __forceinline__ f16x8 raw8_i8(uint32_t lo, uint32_t hi) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t sel = (uint32_t)i | (0x0Cu << 8) | ((uint32_t)(4 + i) << 16) | (0x0Cu << 24);
    const uint32_t h = __builtin_amdgcn_perm(hi, lo, sel) ^ 0x00800080u;
    const f16x2 q = __builtin_bit_cast(f16x2, h);
    r[2 * i] = q[0];
    r[2 * i + 1] = q[1];
  }
  return r;
}
// 8 int2 codes (bytes 2j and 2j + 1 of w: columns 0..3 and 4..7) -> (q + 2) *
// 2^-24, same slot order.
__device__ __forceinline__ f16x8 raw8_i2(uint32_t w, int j) {
  const uint32_t sel = (uint32_t)(2 * j) | (0x0Cu << 8) | ((uint32_t)(2 * j + 1) << 16) | (0x0Cu << 24);
  const uint32_t x = __builtin_amdgcn_perm(w, w, sel);
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h = ((x >> (2 * i)) & 0x00030003u) ^ 0x00020002u;
    const f16x2 q = __builtin_bit_cast(f16x2, h);
    r[2 * i] = q[0];
    r[2 * i + 1] = q[1];
  }
  return r;
}

// 4-byte global -> LDS copy: lane l's word lands at lds + 4 l.
__device__ __forceinline__ void dma4(const void* src, void* lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(lds_addr(lds)) : "memory", "m0");
}

// SW (scales in registers; group scales, K <= 8192): a 16-byte scale piece
// per row every 4 stages would take each 128-byte line of a row's scales 8
// times, 4 stages apart, and under a whole chip's streaming the L2 drops the
// line between the takes (prefill: about 9 fetches per scale line).  Instead
// all of a wave's scales are loaded into registers before the first stage,
// each line at once: lane (n, kg) holds groups 32 w + 8 kg .. + 8 of rows n
// and 16 + n for every window w of 32 groups, and a stage's two scales of a
// row come from lane n + 16 ((st % 16) / 4) with a permute (those of 4
// stages at once).  (Loaded any later, their first use would make the
// compiler wait for every copy in flight, the ring's included.)
// PA (per-group A): the batch's experts all run the thin GEMM and a travels
// from gate/up to down packed by 64-column groups: gate/up forms each
// token's group of a (its 4-wave quad's 64 columns), scales it by a power of
// two so that the group's max|a| < 2^14, rounds it to fp16 and writes it with
// the unit and the group correction; down takes the unit per group (beside
// the corrections, one dword copy per stage) into the group's scale.
// Scales in registers: the scales of groups 2 st .. 2 st + 7 (stages st ..
// st + 3, st a multiple of 4) of rows n (sd[i][0]) and 16 + n (sd[i][1]):
// dword i of window st / 16 in lane src = n + 16 ((st % 16) / 4).
__device__ __forceinline__ void sw_scales(int w, int src, uint4 a0, uint4 a1, uint4 b0, uint4 b1,
                                          uint4 c0, uint4 c1, uint4 e0, uint4 e1,
                                          uint32_t (&sd)[4][2]) {
  const uint4 r0 = w == 0 ? a0 : w == 1 ? b0 : w == 2 ? c0 : e0;
  const uint4 r1 = w == 0 ? a1 : w == 1 ? b1 : w == 2 ? c1 : e1;
  sd[0][0] = (uint32_t)__shfl((int)r0.x, src, 64);
  sd[1][0] = (uint32_t)__shfl((int)r0.y, src, 64);
  sd[2][0] = (uint32_t)__shfl((int)r0.z, src, 64);
  sd[3][0] = (uint32_t)__shfl((int)r0.w, src, 64);
  sd[0][1] = (uint32_t)__shfl((int)r1.x, src, 64);
  sd[1][1] = (uint32_t)__shfl((int)r1.y, src, 64);
  sd[2][1] = (uint32_t)__shfl((int)r1.z, src, 64);
  sd[3][1] = (uint32_t)__shfl((int)r1.w, src, 64);
}

// Integer activations: a lane's 16 weights of a group (columns 16 kg ..
// 16 kg + 15) as 16 signed bytes in column order, the B operand of
// v_mfma_i32_16x16x64_i8 (lane (n, kg): K bytes 16 kg .. 16 kg + 15 of row or
// column n, for A and B alike).  A byte field b of width w in two's
// complement becomes its int8 value as ((b ^ 2^(w-1)) + 0x80 - 2^(w-1)) ^
// 0x80 per byte: the sum stays below 0x100, so no byte carries into the next.
typedef int i32x4 __attribute__((ext_vector_type(4)));
// 8 int4 codes (column j in bits 4j..4j+3) -> columns 0..3 and 4..7
__device__ __forceinline__ void i4x8_to_i8(uint32_t w, int& c03, int& c47) {
  const uint32_t lo = (((w & 0x0F0F0F0Fu) ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;  // 0 2 4 6
  const uint32_t hi = ((((w >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;  // 1 3 5 7
  c03 = (int)__builtin_amdgcn_perm(hi, lo, 0x05010400u);
  c47 = (int)__builtin_amdgcn_perm(hi, lo, 0x07030602u);
}
// 4 int2 codes (byte t: column j in bits 2j..2j+1) -> 4 bytes
__device__ __forceinline__ int i2x4_to_i8(uint32_t t) {
  const uint32_t x = (t | (t << 6) | (t << 12) | (t << 18)) & 0x03030303u;
  return (int)(((x ^ 0x02020202u) + 0x7E7E7E7Eu) ^ 0x80808080u);
}

// Trace points (tr): 1 the tile known and its first copies issued, 2 the
// first stage landed, 3 the last stage computed.
template <int MODE, int GW, int R, int BITS, bool PA = false, bool SW = false, bool IA = false,
          typename Marks = NoMarks>
__device__ __forceinline__ void thin_body(const GemmArgs& g, uint8_t* s_lds, int jx, int jy,
                                          Marks& tr) {
  using Shape = ThinShape<GW, R, BITS, PA, SW, IA>;
  // IA (integer activations): A is int8 [rows][K] with one fp32 scale per
  // 64-column group in corr; each group is one v_mfma_i32_16x16x64_i8 per
  // 16 weight rows (exact), times the weight scale and the A scale in fp32.
  constexpr bool kUnitsA = PA && MODE == kDown && !IA;
  static_assert(!PA || GW % 4 == 0, "a group of a spans 4 waves");
  constexpr int kBWave = Shape::kBWave, kStageB = Shape::kStageB, kRowStage = Shape::kRowStage;
  constexpr int kPieces = Shape::kPieces, kRowsPerCopy = Shape::kRowsPerCopy;
  constexpr int kCopies = Shape::kCopies;
  constexpr int kStageA = Shape::kStageA, kStage = Shape::kStage, kScalePiece = Shape::kScalePiece;
  constexpr int kHalf = kThinWaveRows / 2;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int d = g.d, f = g.f;
  const int K = MODE == kGateUp ? d : f;
  const int pr = g.L.per_row;
  const int ng = srow(K, pr);  // scales per weight row
  const int ngc = K / kGroup;  // correction groups per activation row
  const size_t row_bytes = (size_t)K * BITS / 8;

  // ---- the block's expert and M-tile (tokens tok0 .. tok0 + 15)
  const ExpertList& L = g.L;
  int off, cnt, tok0;
  const uint8_t* blob;
  if (L.single) {
    off = 0;
    cnt = L.single_n;
    tok0 = jy * kThinTokens;
    if (tok0 >= cnt) return;
    blob = L.single;
  } else {
    // the tile's record: expert, tokens (one dependent load)
    const ThinTile tile = g.tt[jy];
    if (!tile.blob) return;
    off = tile.off;
    cnt = tile.cnt;
    tok0 = tile.tok0;
    blob = tile.blob;
  }
  (void)off;
  const int mcnt = min(kThinTokens, cnt - tok0);
  const int32_t* tsl = L.single ? nullptr : g.tslot + (size_t)jy * kTileSlots;
  // slot of the tile's token i (past the last token: the last one)
  auto slot_of = [&](int i) -> int { return L.single ? min(tok0 + i, cnt - 1) : tsl[i]; };
  // packed activation row of a slot
  auto row_of_slot = [&](int slot) -> uint32_t {
    return (uint32_t)(MODE == kGateUp && !L.single ? slot / L.kdiv : slot);
  };
  // the epilogue's slots and units of this lane's tokens 4 kg + i (lane
  // (n, kg), n = lane & 15).  4-wave blocks request the slots now, with the
  // activation rows' slots (one wait covers both), and the units (which
  // depend on the slots) at the start of the last stage, whose wait for every
  // copy covers them too: a load of the units here would be waited for
  // before the first copies.  16-wave blocks (one a CU, long main loops) load
  // both at the end and keep the registers.
  // This lane's slots: its activation row's, its correction row's and (4-wave
  // blocks) the epilogue's, read in one branch so that a union's loads of
  // them go out together and one wait covers them.
  const int tl = threadIdx.x & 63, tkg = tl >> 4;
  // the activation row this lane copies: 16 lanes (fp16) or 8 lanes (int8)
  // a row, waves 0..3 (fp16) or 0..1 (int8)
  const int a_row = IA ? 8 * (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1) + (tl >> 3)
                       : 4 * (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 3) + tkg;
  constexpr bool kEpiEarly = GW <= 4;
  int eslot[4], sl_a, sl_c;
  float eunit[4];
  if (L.single) {
    sl_a = min(tok0 + a_row, cnt - 1);
    sl_c = min(tok0 + (tl & 15), cnt - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) eslot[i] = min(tok0 + 4 * tkg + i, cnt - 1);
  } else {
    sl_a = tsl[a_row];
    sl_c = tsl[tl & 15];
    if constexpr (kEpiEarly) {
#pragma unroll
      for (int i = 0; i < 4; ++i) eslot[i] = tsl[4 * tkg + i];
    }
  }
  auto epi_slots = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) eslot[i] = slot_of(4 * tkg + i);
  };
  auto epi_units = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (IA) eunit[i] = 1.0f;  // the A scales were applied per group
      else if (MODE == kGateUp) eunit[i] = g.unit[L.single ? eslot[i] : eslot[i] / L.kdiv];
      else eunit[i] = kUnitsA ? 1.0f : g.unit[eslot[i]];
    }
  };

  // ---- this wave's 32 weight rows (gate/up: 16 gate rows and the same 16 up
  // rows); waves past the last row copy the last wave's rows, compute nothing
  const int nwaves = MODE == kGateUp ? f / kHalf : d / kThinWaveRows;
  const int wv = jx * GW + wave;
  const bool active = wv < nwaves;
  const int wc = min(wv, nwaves - 1);
  const size_t mat_codes = (size_t)f * d * BITS / 8;
  const _Float16* sbase = reinterpret_cast<const _Float16*>(blob + 3 * mat_codes);
  const size_t gate_sc = (size_t)f * srow(d, pr);
  const uint8_t *c0, *c1;
  const _Float16 *s0, *s1;
  if (MODE == kGateUp) {
    c0 = blob + (size_t)(kHalf * wc) * row_bytes;
    c1 = c0 + mat_codes;
    s0 = sbase + (size_t)(kHalf * wc) * ng;
    s1 = s0 + gate_sc;
  } else {
    c0 = blob + 2 * mat_codes + (size_t)(kThinWaveRows * wc) * row_bytes;
    c1 = c0 + (size_t)kHalf * row_bytes;
    s0 = sbase + 2 * gate_sc + (size_t)(kThinWaveRows * wc) * ng;
    s1 = s0 + (size_t)kHalf * ng;
  }
  const int n = lane & 15, kg = lane >> 4;

  // ---- per-lane copy sources.  Codes, copy i: lane l -> wave row
  // r = kRowsPerCopy i + l / kPieces, LDS slot l % kPieces (holding piece
  // slot ^ swizzle); rows 0..15 come from c0, 16..31 from c1.
  const uint8_t* b_src[kCopies];
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int r = kRowsPerCopy * i + lane / kPieces;
    const int piece = thin_slot<BITS>(lane % kPieces, r);
    b_src[i] = (r < kHalf ? c0 : c1) + (size_t)(r % kHalf) * row_bytes + piece * 16;
  }
  const bool a_copy = IA ? wave < 2 && 8 * wave < mcnt : wave < 4 && 4 * wave < mcnt;  // wave-uniform
  // fp16: 16-byte piece (lane & 15) ^ row of a 256-byte row stage; int8:
  // piece (lane & 7) ^ (row & 7) of a 128-byte one (elements of the row)
  const uint32_t a_off =
      IA ? row_of_slot(sl_a) * (uint32_t)K + (uint32_t)((lane & 7) ^ (a_row & 7)) * 16u
         : row_of_slot(sl_a) * (uint32_t)K + (uint32_t)((lane & 15) ^ (a_row & 15)) * 8u;
  // corrections: lane l -> token l & 15, group 2 st + ((l >> 4) & 1); with
  // per-group A units, lanes 32..63 copy the units the same way
  const size_t cu_row = (size_t)row_of_slot(sl_c) * ngc + ((lane >> 4) & 1);
  const float* cu_lane = (kUnitsA && lane >= 32 ? g.unit : g.corr) + cu_row;
  // scales: lane l < 32 -> row l of the wave, 16 bytes (8 groups) every 4 stages
  const int sr_lane = lane % kThinWaveRows;
  const _Float16* s_lane = (sr_lane < kHalf ? s0 : s1) + (size_t)(sr_lane % kHalf) * ng;
  uint8_t* s_scales = s_lds + Shape::kScaleOff + wave * (2 * kScalePiece);
  if (!SW && pr && lane < kThinWaveRows) {
    // one scale per row: put in every group of both buffers, once (this
    // wave's own LDS; the first stage's wait covers the writes)
    const uint32_t h = *reinterpret_cast<const uint16_t*>(s_lane);
    const uint32_t hh = h | (h << 16);
    const uint4 v = make_uint4(hh, hh, hh, hh);
    *reinterpret_cast<uint4*>(s_scales + lane * 16) = v;
    *reinterpret_cast<uint4*>(s_scales + kScalePiece + lane * 16) = v;
  }
  // SW: windows 0..3 of rows n (x0) and 16 + n (x1), 8 groups each
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
  uint4 a0 = z4, a1 = z4, b0 = z4, b1 = z4, c0w = z4, c1w = z4, e0 = z4, e1 = z4;
  if constexpr (SW) {
    static_assert(kSwWindows == 4, "four named windows");
    const _Float16* srw0 = s0 + (size_t)n * ng;
    const _Float16* srw1 = s1 + (size_t)n * ng;
    const int g0 = 8 * kg;  // ng is a multiple of 8: a lane's 8 are all in or out
    if (g0 < ng) a0 = gload16(srw0 + g0), a1 = gload16(srw1 + g0);
    if (g0 + 32 < ng) b0 = gload16(srw0 + g0 + 32), b1 = gload16(srw1 + g0 + 32);
    if (g0 + 64 < ng) c0w = gload16(srw0 + g0 + 64), c1w = gload16(srw1 + g0 + 64);
    if (g0 + 96 < ng) e0 = gload16(srw0 + g0 + 96), e1 = gload16(srw1 + g0 + 96);
  }

  const int nst = K / kSC;
  auto issue = [&](int st) __attribute__((always_inline)) {
    uint8_t* base = s_lds + (st % R) * kStage;
    const uint32_t so = (uint32_t)st * kRowStage;
#pragma unroll
    for (int i = 0; i < kCopies; ++i) dma16(b_src[i] + so, base + wave * kBWave + i * 1024);
    if (a_copy) {
      if constexpr (IA)
        dma16(reinterpret_cast<const int8_t*>(g.a) + a_off + st * kSC,
              base + kStageB + 8 * wave * kSC);
      else
        dma16(g.a + a_off + st * kSC, base + kStageB + 4 * wave * (kSC * 2));
    }
    // the correction copy fills 32 x 4 bytes (64 x 4 with the units); without
    // units lanes 32..63 stay out of it
    if (wave == 0 && (kUnitsA || lane < 32)) dma4(cu_lane + 2 * st, base + kStageB + kStageA);
    if (!SW && (st & 3) == 0 && !pr && lane < kThinWaveRows)
      dma16(s_lane + 2 * st, s_scales + ((st >> 2) & 1) * kScalePiece);
  };

  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // group 2 st + gg of a landed stage: lane (n, kg) takes, for MFMA step j,
  // columns 16 kg + 8 j .. + 8 of the group
  auto group = [&](int st, int gg, const uint32_t (&sd)[2]) __attribute__((always_inline)) {
    const uint8_t* base = s_lds + (st % R) * kStage;
    const int gi = 2 * st + gg;
    const uint8_t* sc = s_scales + ((gi >> 3) & 1) * kScalePiece + (gi & 7) * 2;
    if constexpr (IA) {
      // A: token n's 16 bytes of the group (piece 4 gg + kg, swizzled by the
      // row), its scales for tokens 4 kg .. 4 kg + 3
      const uint8_t* ar = base + kStageB + n * kSC;
      const i32x4 av = *reinterpret_cast<const i32x4*>(ar + (((4 * gg + kg) ^ (n & 7)) * 16));
      const f32x4 s4 =
          *reinterpret_cast<const f32x4*>(base + kStageB + kStageA + (16 * gg + 4 * kg) * 4);
      const i32x4 z4 = {0, 0, 0, 0};
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int r = 16 * nt + n;
        const uint8_t* row = base + wave * kBWave + r * kRowStage;
        i32x4 bv;
        if constexpr (BITS == 4) {
          const uint2 w = *reinterpret_cast<const uint2*>(
              row + thin_slot<4>(2 * gg + (kg >> 1), r) * 16 + 8 * (kg & 1));
          int b0, b1, b2, b3;
          i4x8_to_i8(w.x, b0, b1);
          i4x8_to_i8(w.y, b2, b3);
          bv = i32x4{b0, b1, b2, b3};
        } else if constexpr (BITS == 8) {
          bv = *reinterpret_cast<const i32x4*>(row + thin_slot<8>(4 * gg + kg, r) * 16);
        } else {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(row + thin_slot<2>(gg, r) * 16 + 4 * kg);
#pragma unroll
          for (int m = 0; m < 4; ++m) bv[m] = i2x4_to_i8((w >> (8 * m)) & 0xFFu);
        }
        const i32x4 pi = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, z4, 0, 0, 0);
        float sv;
        if constexpr (SW)
          sv = (float)__builtin_bit_cast(_Float16, (uint16_t)(sd[nt] >> (16 * gg)));
        else
          sv = (float)*reinterpret_cast<const _Float16*>(sc + r * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][i] = fmaf((float)pi[i], sv * s4[i], acc[nt][i]);
      }
      return;
    }
    const uint8_t* ar = base + kStageB + n * (kSC * 2);
    const int p0 = 8 * gg + 2 * kg;
    const f16x8 a0 = *reinterpret_cast<const f16x8*>(ar + (p0 ^ n) * 16);
    const f16x8 a1 = *reinterpret_cast<const f16x8*>(ar + ((p0 + 1) ^ n) * 16);
    const f32x4 c4 =
        *reinterpret_cast<const f32x4*>(base + kStageB + kStageA + (16 * gg + 4 * kg) * 4);
    f32x4 u4 = {1.f, 1.f, 1.f, 1.f};
    if constexpr (kUnitsA)
      u4 = *reinterpret_cast<const f32x4*>(base + kStageB + kStageA + 128 + (16 * gg + 4 * kg) * 4);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int r = 16 * nt + n;
      const uint8_t* row = base + wave * kBWave + r * kRowStage;
      f16x8 b0, b1;
      if constexpr (BITS == 4) {
        const uint2 w = *reinterpret_cast<const uint2*>(
            row + thin_slot<4>(2 * gg + (kg >> 1), r) * 16 + 8 * (kg & 1));
        b0 = raw8(w.x);
        b1 = raw8(w.y);
      } else if constexpr (BITS == 8) {
        const uint4 w = *reinterpret_cast<const uint4*>(row + thin_slot<8>(4 * gg + kg, r) * 16);
        b0 = raw8_i8(w.x, w.y);
        b1 = raw8_i8(w.z, w.w);
      } else {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(row + thin_slot<2>(gg, r) * 16 + 4 * kg);
        b0 = raw8_i2(w, 0);
        b1 = raw8_i2(w, 1);
      }
      f32x4 pg = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0, c4, 0, 0, 0);
      pg = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1, pg, 0, 0, 0);
      float sv;
      if constexpr (SW)
        sv = (float)__builtin_bit_cast(_Float16, (uint16_t)(sd[nt] >> (16 * gg)));
      else
        sv = (float)*reinterpret_cast<const _Float16*>(sc + r * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[nt][i] = fmaf(kUnitsA ? sv * u4[i] : sv, pg[i], acc[nt][i]);
    }
  };

  // copies a wave issues per stage besides its scale pieces: kCopies of
  // codes, 1 of activations (waves 0..3 with tokens), 1 of corrections (wave 0)
  const int extra = (a_copy ? 1 : 0) + (wave == 0 ? 1 : 0);
#pragma unroll
  for (int i = 0; i < R - 1; ++i)
    if (i < nst) issue(i);
  tr.mark(1);
  auto step = [&](int st, auto phase, const uint32_t (&sd)[2]) __attribute__((always_inline)) {
    constexpr int PH = decltype(phase)::value;  // stage % 4
    if (kEpiEarly && st == nst - 1) epi_units();
    if (st + R - 2 < nst) {
      // stage st has landed once at most the copies of stages st + 1 ..
      // st + R - 2 are in flight
      if (SW || pr) {
        if (extra == 0) wait_vm_lgkm0<copies_ahead<R, PH, kCopies, 0, 0>()>();
        else if (extra == 1) wait_vm_lgkm0<copies_ahead<R, PH, kCopies + 1, 0, 0>()>();
        else wait_vm_lgkm0<copies_ahead<R, PH, kCopies + 2, 0, 0>()>();
      } else {
        if (extra == 0) wait_vm_lgkm0<copies_ahead<R, PH, kCopies, 0, 1>()>();
        else if (extra == 1) wait_vm_lgkm0<copies_ahead<R, PH, kCopies + 1, 0, 1>()>();
        else wait_vm_lgkm0<copies_ahead<R, PH, kCopies + 2, 0, 1>()>();
      }
    } else {
      wait_vm_lgkm0<0>();
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st == 0) tr.mark(2);
    // every wave is past stage st - 1: its ring slot takes stage st + R - 1
    if (st + R - 1 < nst) issue(st + R - 1);
    if (active) {
      group(st, 0, sd);
      group(st, 1, sd);
    }
  };
  for (int st0 = 0; st0 < nst; st0 += 4) {  // nst is a multiple of 4
    // SW: a stage's scales of rows n and 16 + n (both lanes' permutes run in
    // every wave, active or not)
    uint32_t sd[4][2] = {};
    if constexpr (SW) {
      const int src = n + 16 * ((st0 & 15) >> 2), w = st0 >> 4;
      sw_scales(w, src, a0, a1, b0, b1, c0w, c1w, e0, e1, sd);
    }
    step(st0, std::integral_constant<int, 0>(), sd[0]);
    step(st0 + 1, std::integral_constant<int, 1>(), sd[1]);
    step(st0 + 2, std::integral_constant<int, 2>(), sd[2]);
    step(st0 + 3, std::integral_constant<int, 3>(), sd[3]);
  }
  tr.mark(3);

  if constexpr (!kEpiEarly) {
    epi_slots();
    epi_units();
  }

  if constexpr (PA && MODE == kGateUp) {
    // lane (n, kg): a at column c = 16 wv + n for tile tokens 4 kg + i (rows
    // past the tile repeat the last token and are not stored).  The group's
    // max|a| and the sum of its packed values are taken over the row of 16
    // lanes (DPP), then over the quad's 4 waves through LDS, in a fixed order;
    // every wave of the block reaches both barriers (a quad's waves are all
    // active or all past the last row: f / 16 is a multiple of 32).
    const int c = kHalf * wv + n;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float us = IA ? 1.0f : eunit[i] * 0x1p24f;
      v[i] = silu(acc[0][i] * us) * (acc[1][i] * us);
    }
    // ring slot nst % R: its last stage (nst - R) was computed by every wave
    // before the barrier of stage nst - 1, and no copy is issued after that
    float* red_m = reinterpret_cast<float*>(s_lds + (nst % R) * kStage);
    float* red_s = red_m + GW * kThinTokens;
    const int q0 = wave & ~3;
    float mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[i] = row16_max(fabsf(v[i]));
    // lane n < 4 of each row posts token 4 kg + n
    if (n < 4) red_m[wave * kThinTokens + 4 * kg + n] = n == 0 ? mx[0] : n == 1 ? mx[1] : n == 2 ? mx[2] : mx[3];
    __syncthreads();
    if constexpr (IA) {
      // a's group of 64 columns as int8: q = a / s to the nearest (ties to
      // even), s = max|a| / 127 in fp32, into a_out (bytes, column order) and
      // s into a_corr
      if (!active) return;
      const int grp = c / kGroup, ngroups = f / kGroup;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * kg + i >= mcnt) continue;
        const int t = 4 * kg + i;
        const float gmi =
            fmaxf(fmaxf(red_m[q0 * kThinTokens + t], red_m[(q0 + 1) * kThinTokens + t]),
                  fmaxf(red_m[(q0 + 2) * kThinTokens + t], red_m[(q0 + 3) * kThinTokens + t]));
        const float sa = gmi / 127.0f;
        const float q = gmi > 0.0f ? fminf(fmaxf(rintf(v[i] / sa), -127.0f), 127.0f) : 0.0f;
        const int slot = eslot[i];
        reinterpret_cast<int8_t*>(g.a_out)[(size_t)slot * f + c] = (int8_t)(int)q;
        if (wave == q0 && n == i) g.a_corr[(size_t)slot * ngroups + grp] = sa;
      }
      return;
    }
    float gm[4], up[4], hs[4];
    int ex[4];
    _Float16 h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * kg + i;
      gm[i] = fmaxf(fmaxf(red_m[q0 * kThinTokens + t], red_m[(q0 + 1) * kThinTokens + t]),
                    fmaxf(red_m[(q0 + 2) * kThinTokens + t], red_m[(q0 + 3) * kThinTokens + t]));
      ex[i] = 0;
      if (gm[i] > 0.0f) frexpf(gm[i], &ex[i]);  // gm < 2^ex
      up[i] = gm[i] > 0.0f ? ldexpf(1.0f, kPackExp - ex[i]) : 1.0f;
      h[i] = (_Float16)(v[i] * up[i]);
      hs[i] = row16_fsum((float)h[i]);
    }
    if (n < 4) red_s[wave * kThinTokens + 4 * kg + n] = n == 0 ? hs[0] : n == 1 ? hs[1] : n == 2 ? hs[2] : hs[3];
    __syncthreads();
    if (!active) return;
    const int grp = c / kGroup, ngroups = f / kGroup;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (4 * kg + i >= mcnt) continue;
      const int slot = eslot[i];
      g.a_out[(size_t)slot * f + (c & ~7) + slot_of_col(c & 7)] = h[i];
      if (wave == q0 && n == i) {
        const int t = 4 * kg + i;
        const float sum = (red_s[q0 * kThinTokens + t] + red_s[(q0 + 1) * kThinTokens + t]) +
                          (red_s[(q0 + 2) * kThinTokens + t] + red_s[(q0 + 3) * kThinTokens + t]);
        g.a_corr[(size_t)slot * ngroups + grp] = -g.corr_off * 0x1p-24f * sum;
        g.a_unit[(size_t)slot * ngroups + grp] = gm[i] > 0.0f ? ldexpf(1.0f, ex[i] - kPackExp) : 1.0f;
      }
    }
    return;
  }
  if (!active) return;

  // epilogue: lane (n, kg) holds tile tokens 4 kg + i for weight rows 16 nt + n;
  // the partials were in units of 2^-24
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (4 * kg + i >= mcnt) continue;
    const int slot = eslot[i];
    if (MODE == kGateUp) {
      const float us = IA ? 1.0f : eunit[i] * 0x1p24f;
      const float gv = acc[0][i] * us, uv = acc[1][i] * us;
      g.out[(size_t)slot * f + kHalf * wv + n] = silu(gv) * uv;
    } else {
      const float us = IA ? 1.0f : eunit[i] * 0x1p24f;
      float* orow = g.out + (size_t)slot * d + kThinWaveRows * wv;
      orow[n] = acc[0][i] * us;
      orow[16 + n] = acc[1][i] * us;
    }
  }
}

template <int MODE, int GW, int R, int BITS, bool PA, bool SW, bool IA = false>
__global__ __launch_bounds__(64 * GW) void k_gemm_thin(GemmArgs g) {
  __shared__ __attribute__((aligned(16)))
  uint8_t s_lds[ThinShape<GW, R, BITS, PA, SW, IA>::kLdsBytes];
  BlockTrace tr;
  tr.start();
  thin_body<MODE, GW, R, BITS, PA, SW, IA>(g, s_lds, blockIdx.x, blockIdx.y, tr);
  tr.store(g_trace_mfma, MODE, blockIdx.x + gridDim.x * blockIdx.y, 1);
}

// One launch for a batch's whole union: the first g.thick_blocks blocks run
// the M-blocked GEMM (16 waves, 64-token M-blocks: the hot experts, whose
// matrix-core and dequantisation work is the longest, dispatched first), the
// others the thin GEMM (16 waves) over the experts of at most kThinTokens
// tokens, so the streaming of the many small experts overlaps the compute of
// the few large ones.  Both cover 512 weight rows a block.  Block F runs on
// XCD F % 8 (blocks are dispatched to the XCDs in turn): the M-blocked
// blocks of XCD x take the M-blocks of its list, each over all gx row
// blocks, so an expert's blocks share one L2 (its weights across its
// M-blocks, its activation rows across the row blocks).
constexpr int kMixedThinRing = 3;
template <int MODE, bool SW>
__global__ __launch_bounds__(1024) void k_gemm_mixed(GemmArgs g) {
  constexpr int kA = RingShape<16, 3, 64, 2>::kLdsBytes;
  constexpr int kB = ThinShape<16, kMixedThinRing, 4, false, SW>::kLdsBytes;
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kA > kB ? kA : kB];
  // trace: start and end of every workgroup, tag 1 M-blocked, 2 thin, 3 an
  // empty M-block slot
  BlockTrace tr;
  tr.start();
  NoMarks none;
  const int F = blockIdx.x;
  int tag = 2;
  if (F < g.thick_blocks) {
    const int x = F % kXcds, q = F / kXcds, i = q / g.gx;
    if (i >= g.xcnt[x]) {
      tag = 3;
    } else {
      gemm_body<MODE, 16, 3, 64, 2>(g, s_lds, q % g.gx, g.xtab[x * g.xs + i]);
      tag = 1;
    }
  } else {
    const int Ft = F - g.thick_blocks;
    thin_body<MODE, 16, kMixedThinRing, 4, false, SW>(g, s_lds, Ft % g.gx, Ft / g.gx, none);
  }
  tr.store(g_trace_mfma, 2 + MODE, F, tag);
}

// ---------------------------------------------------------------- launchers

// Block shape of the M-blocked GEMM (experts of more than kThinTokens tokens):
// one expert over 128 rows or more (the compute-bound case) takes 4-wave
// blocks of 128 rows with 64-token M-blocks, four times as many blocks as the
// 16-wave shape; everything else 16-wave blocks (32 rows a wave) with 64-token
// M-blocks.
struct GemmShape {
  int gw, mblock, ntw;
};
static GemmShape gemm_shape(int rows, bool single) {
  if (single && rows >= 128) return {4, 64, 2};
  return {16, 64, 2};
}
int mfma_mblock(int) { return 64; }

bool mfma_shape_ok(int d, int f) { return d % 512 == 0 && f % 512 == 0; }

// Thin GEMM on its own (batches of at most kThinTokens rows, one expert of
// that many): 4 waves of 32 rows, a ring of 4 stages, several blocks a CU, so
// a dozen experts still give hundreds of blocks.
constexpr int kThinGW = 4;
constexpr int kThinRing = 4;
// Down (K = f, a few stages) keeps 3: with 4 stages (54 KB of LDS) many CUs
// took only two of its blocks, and at 624 blocks over 256 CUs a second round
// of blocks started 16 us late (verify8 down 27.5 -> 25.6 us with 3).
constexpr int kThinRingDown = 3;

// The offset that makes a code of this width non-negative (its value plus
// the offset is the field with the sign bit flipped).
static float corr_offset(int bits) { return bits == 8 ? 128.0f : bits == 2 ? 2.0f : 8.0f; }

PackArgs mfma_x_pack_args(const MfmaArgs& m) {
  const ExpertList& L = m.L;
  PackArgs px{};
  px.src = m.x;
  px.src_bf16 = m.x_bf16;
  px.K = m.d;
  px.rows = m.x_rows;
  px.gather = m.x_gather;
  px.dst = m.xh;
  px.unit = m.xunit;
  px.corr = m.xcorr;
  px.corr_off = corr_offset(L.bits);
  px.thin_all = L.bits != 4 || m.i8act;
  px.i8 = m.i8act;
  if (!L.single) {
    px.offsets = L.offsets;
    px.n_uniq = L.n_uniq;
    px.mbo = m.mbo;
    px.blk_u = m.blk_u;
    px.mblock = mfma_mblock(m.x_rows);
    px.xtab = m.xtab;
    px.xcnt = m.xcnt;
    px.xs = m.xs;
    px.tt = m.tt;
    px.tslot = m.tslot;
    px.tt_n = m.thin_bound;
    px.table = L.table;
    px.uniq = L.uniq;
    px.list = L.list;
  }
  return px;
}

// A projection.  int4: batches of at most kThinTokens rows (every expert
// thin) and a single expert of that many run the thin GEMM alone; a single
// larger expert the M-blocked GEMM; larger batches the mixed launch
// (M-blocked blocks for the experts past kThinTokens tokens, then thin blocks
// for the others).  int8 and int2: the thin GEMM over every M-tile of 16
// tokens of every expert.
// Scales in registers (SW) with one scale per 64 weights (a row's scales then
// fill whole 8-group lane slices: K is a multiple of 512) and K <= 8192.
static bool scales_in_regs(const GemmArgs& ga, int K) {
  return K % 512 == 0 && K <= 32 * 64 * kSwWindows && !ga.L.per_row;
}

// big: a batch of more than kThinTokens rows (prefill of int8 and int2
// layers).  Only there does the whole chip stream at once, so that the L2
// drops scale lines between the takes of a per-stage piece: with a few
// experts the pieces hit, and the register windows only cost (decode of an
// int8 layer: gate/up 41.7 -> 45.8 us with them).
template <int MODE, int BITS, int R>
static hipError_t thin_launch(int kid, unsigned gx, unsigned gy, bool big, hipStream_t s,
                              const GemmArgs& ga) {
  const dim3 grid(gx, gy), block(64 * kThinGW);
  const bool sw = big && scales_in_regs(ga, MODE == kGateUp ? ga.d : ga.f);
  if (ga.ia) {
    if (!ga.pa) return hipErrorInvalidValue;
    if (sw) return launch(kid, k_gemm_thin<MODE, kThinGW, R, BITS, true, true, true>, grid, block, s, ga);
    return launch(kid, k_gemm_thin<MODE, kThinGW, R, BITS, true, false, true>, grid, block, s, ga);
  }
  if (ga.pa) {
    if (sw) return launch(kid, k_gemm_thin<MODE, kThinGW, R, BITS, true, true>, grid, block, s, ga);
    return launch(kid, k_gemm_thin<MODE, kThinGW, R, BITS, true, false>, grid, block, s, ga);
  }
  if (sw) return launch(kid, k_gemm_thin<MODE, kThinGW, R, BITS, false, true>, grid, block, s, ga);
  return launch(kid, k_gemm_thin<MODE, kThinGW, R, BITS, false, false>, grid, block, s, ga);
}

// Every expert of the call runs the thin GEMM: int8 and int2 layers, integer
// activations, and int4 batches (or a single expert) of at most kThinTokens
// rows.
static bool all_thin(const MfmaArgs& m) {
  const int rows = m.L.single ? m.L.single_n : m.x_rows;
  return m.L.bits != 4 || m.i8act || rows <= kThinTokens;
}

template <int MODE>
static hipError_t project(const MfmaArgs& m, GemmArgs ga, hipStream_t s) {
  const ExpertList& L = m.L;
  const int rows = L.single ? L.single_n : m.x_rows;
  const int kid = MODE == kGateUp ? MOE_KERNEL_GATEUP : MOE_KERNEL_DOWN;
  const int kid_thin = MODE == kGateUp ? MOE_KERNEL_GATEUP_THIN : MOE_KERNEL_DOWN_THIN;
  const int N = MODE == kGateUp ? m.f : m.d;  // weight rows (gate/up: gate rows; up alike)
  const int wrows = MODE == kGateUp ? 16 : 32;  // of N a wave covers
  const int nw = N / wrows;
  const unsigned gx = (unsigned)((nw + kThinGW - 1) / kThinGW);
  const unsigned gy = L.single ? (unsigned)((L.single_n + kThinTokens - 1) / kThinTokens)
                               : (unsigned)m.thin_bound;
  const bool big = rows > kThinTokens;
  if (L.bits == 8) return thin_launch<MODE, 8, 3>(kid_thin, gx, gy, big, s, ga);
  if (L.bits == 2) return thin_launch<MODE, 2, 4>(kid_thin, gx, gy, big, s, ga);
  if (rows <= kThinTokens || ga.ia)
    return thin_launch<MODE, 4, MODE == kDown ? kThinRingDown : kThinRing>(kid_thin, gx, gy, big,
                                                                          s, ga);
  if (L.single) {
    const GemmShape sh = gemm_shape(rows, true);
    const unsigned mb = (unsigned)((L.single_n + sh.mblock - 1) / sh.mblock);
    const unsigned gxs = (unsigned)((nw + sh.gw - 1) / sh.gw);
    if (sh.gw == 4) return launch(kid, k_gemm<MODE, 4, 3, 64, 2>, dim3(gxs, mb), dim3(256), s, ga);
    return launch(kid, k_gemm<MODE, 16, 3, 64, 2>, dim3(gxs, mb), dim3(1024), s, ga);
  }
  ga.gx = (nw + 15) / 16;
  ga.xtab = m.xtab;
  ga.xcnt = m.xcnt;
  ga.xs = m.xs;
  ga.thick_blocks = kXcds * ga.gx * m.xs;
  const dim3 grid((unsigned)(ga.thick_blocks + ga.gx * m.thin_bound));
  if (scales_in_regs(ga, MODE == kGateUp ? m.d : m.f))
    return launch(kid, k_gemm_mixed<MODE, true>, grid, dim3(1024), s, ga);
  return launch(kid, k_gemm_mixed<MODE, false>, grid, dim3(1024), s, ga);
}

hipError_t launch_ffn_mfma(const MfmaArgs& m, hipStream_t s) {
  const ExpertList& L = m.L;
  hipError_t e;
  if (!m.x_packed) {
    // x rows -> fp16 with their group corrections (and the union's M-block maps)
    const PackArgs px = mfma_x_pack_args(m);
    const unsigned gx = (unsigned)((m.x_rows + 3) / 4) + (L.single ? 0u : 1u);
    e = launch(MOE_KERNEL_DIGITIZE, k_pack, dim3(gx), dim3(256), s, px);
    if (e != hipSuccess) return e;
  }
  GemmArgs ga{L, m.mbo, m.blk_u, m.d, m.f, m.xh, m.xunit, m.a32, m.xcorr, m.tt, m.tslot, 0};
  const bool pa_groups = all_thin(m);
  if (pa_groups) {
    // gate/up writes a packed by groups; no pack launch between the GEMMs
    ga.pa = 1;
    ga.a_out = m.ah;
    ga.a_unit = m.aunit_g;
    ga.a_corr = m.acorr;
    ga.corr_off = corr_offset(L.bits);
    ga.ia = m.i8act;
  }
  e = project<kGateUp>(m, ga, s);
  if (e != hipSuccess) return e;
  if (pa_groups) {
    GemmArgs gd{L, m.mbo, m.blk_u, m.d, m.f, m.ah, m.aunit_g, m.y, m.acorr, m.tt, m.tslot, 0};
    gd.pa = 1;
    gd.ia = m.i8act;
    return project<kDown>(m, gd, s);
  }

  PackArgs pa{};
  pa.src = m.a32;
  pa.K = m.f;
  pa.rows = m.slots;
  pa.dst = m.ah;
  pa.unit = m.aunit;
  pa.corr = m.acorr;
  pa.corr_off = corr_offset(L.bits);
  e = launch(MOE_KERNEL_DIGITIZE, k_pack, dim3((unsigned)((m.slots + 3) / 4)), dim3(256), s, pa);
  if (e != hipSuccess) return e;

  GemmArgs gd{L, m.mbo, m.blk_u, m.d, m.f, m.ah, m.aunit, m.y, m.acorr, m.tt, m.tslot, 0};
  return project<kDown>(m, gd, s);
}

}  // namespace moe

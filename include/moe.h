/*
 * moe.h — C ABI of the MI355X (gfx950) int4 routed-expert MoE layer library.
 *
 * One sparse MoE layer forward pass over group-scaled int4 routed experts:
 * each token's router picks k of E experts; the picks of a batch are merged
 * into a union of distinct experts so each expert's bytes are read once; each
 * chosen expert runs a SwiGLU FFN on its int4 weights; the outputs are summed
 * with the router weights.
 *
 * Sources for the method (pages on the colibrì engine):
 *  - the per-token path through a MoE layer is route -> union -> place ->
 *    overlap -> learn, with repeated picks of one expert in a batch merged into
 *    a single read: colibri 技术解读 (linlog.top), "引擎结构：一个 C 文件，五步
 *    token 路径"; colibrì README (简体中文), 工作原理 › 绝不为同一次磁盘读取等待两遍;
 *  - 8 of 256 routed experts per token and layer, about 19 MB each at int4:
 *    colibri 技术解读, "MoE 的稀疏性"; README 核心概念;
 *  - the three matrices of an expert stored next to each other and fetched in
 *    one read: README 工作原理 › 绝不为同一次磁盘读取等待两遍;
 *  - group-scaled int4 ("gs64") as the weight container: README 开始使用 › 获取模型;
 *  - where an expert's bytes live decides only speed, never the result:
 *    README 工作原理 › 每个 token 的处理路径.
 * The pages do not fix the gate function, the FFN form or the bit layout.  The
 * readings this library implements (and its CPU oracle checks) are:
 *  - gate: softmax over all E logits, the k largest logits chosen (ties to the
 *    lower expert id), their softmax weights renormalised to sum to 1; logits
 *    are accumulated in fp64 so the choice does not depend on summation order;
 *  - expert: y = Wd (silu(Wg x) * (Wu x)), silu(v) = v / (1 + exp(-v));
 *  - weights: signed two's-complement int4, element 2i of a row in the low
 *    nibble of byte i, one IEEE binary16 scale per 64 consecutive weights along
 *    the input (contiguous) dimension, w = q * s.
 *
 * Expert blob (canonical layout, 64-byte aligned sections for d, f % 64 == 0):
 *   gate codes [f][d/2] | up codes [f][d/2] | down codes [d][f/2]
 *   | gate scales [f][d/64] | up scales [f][d/64] | down scales [d][f/64]
 * Size: moe_expert_blob_bytes(); 20,054,016 bytes at d = 6144, f = 2048.
 * Per-row variant (dims.group_size = 0; the per-row scaling the nxmr blog
 * names, «纯C语言»): the same codes, then one scale per row,
 *   | gate scales [f] | up scales [f] | down scales [d]
 * so w[r][c] = q[r][c] * s[r]; 18,894,848 bytes at d = 6144, f = 2048.  Every
 * entry point takes both layouts and computes the same way on them.
 * Code widths (dims.code_bits; the nxmr blog, «纯C语言», names hand-written
 * int8 and packed int2 kernels beside packed int4): a row of `cols` weights
 * takes cols * bits / 8 bytes of codes, int8 one two's-complement byte per
 * weight, int2 four two's-complement 2-bit fields per byte (weight 4i + j in
 * bits 2j..2j+1 of byte i); the scale tensors follow all the codes as above.
 * 38,928,384 (int8) and 10,616,832 (int2) bytes per gs64 expert at d = 6144,
 * f = 2048.  d and f must be multiples of 512 for both.  int8 layers run
 * every call on the matrix cores in 16-token tiles, where a token's result
 * does not depend on the other tokens of its call.  int2 layers take the
 * single-token kernel family for one token (and for MOE_BATCH_INVARIANT
 * batches) in moe_layer_forward, as int4 layers do, and the matrix cores for
 * other batches and in moe_expert_ffn.  moe_layer_forward_cached takes int4
 * layers only.
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers (or host memory mapped into the device
 *    address space, e.g. from hipHostMalloc) unless said otherwise.  `dims`
 *    points at host memory.  The caller owns every buffer; the library
 *    allocates and frees nothing and keeps no state between calls (apart
 *    from the opt-in kernel timing below).
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued on it; nothing is synchronised, nothing is copied to the host.
 *    Calls enqueue only kernels (no memset/memcpy), so they may be captured in
 *    a HIP graph.
 *  - `ws` is a caller-provided device workspace of at least
 *    moe_workspace_bytes(dims, T) bytes, 16-byte aligned (hipMalloc and
 *    torch's allocator return 256-byte aligned blocks; a misaligned ws is
 *    MOE_EINVAL).  Its contents need not be
 *    initialised: every call writes each word of it before reading it.  Calls
 *    that share a workspace must not overlap in time.
 *  - All arguments are validated before anything is enqueued; on error the
 *    call returns a negative code and enqueues nothing.  Device-side faults
 *    surface at the caller's next synchronisation.  There is no CPU fallback.
 *  - Scale range.  Calls on 2 or more tokens (rows) with d and f multiples of
 *    512, without MOE_BATCH_INVARIANT, run the matrix-core path, which forms
 *    each weight q * s as one IEEE binary16 number.  That is exact-to-rounding
 *    for 2^-14 <= |s| <= 2^12 (2^-12 relative); smaller scales lose relative
 *    precision gradually (binary16 subnormals) and |s| > 8188 overflows
 *    (8 * |s| > 65504).  Every other path (one token, other shapes,
 *    MOE_BATCH_INVARIANT, the cached layer) applies s in fp32 and takes any
 *    finite scale; experts with scales outside the range belong there.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_dims {
  int32_t d;          /* hidden size; multiple of 64, 64..65536 */
  int32_t f;          /* expert FFN width; multiple of 64, 64..65536 */
  int32_t n_experts;  /* E; 1..1024 */
  int32_t top_k;      /* k; 1..min(E, 32) */
  int32_t group_size; /* weights per fp16 scale: 64, or 0 for one scale per row */
  int32_t code_bits;  /* code width: 4 (or 0) int4, 8 int8, 2 int2; 8 and 2 need d
                         and f multiples of 512 (see "Code widths" below) */
} moe_dims;

/* Activation dtypes (x_dtype). */
enum { MOE_F32 = 0, MOE_BF16 = 1 };

/* moe_layer_forward flags. */
enum {
  MOE_PRENORM_RMS = 1u,    /* route and run experts on RMSNorm(x), unit gain (x must be f32) */
  MOE_RESIDUAL = 2u,       /* out = x + MoE(...) (x must be f32).  The residual is the
                              layer input itself (h_{l+1} = h_l + MoE(RMSNorm(h_l))): no
                              separate residual pointer is taken, so a residual other than
                              x cannot be expressed; callers with one add it themselves */
  MOE_BATCH_INVARIANT = 4u, /* each token's result as if it were alone in the call (see below) */
  MOE_INT8_ACT = 8u         /* integer activations: int8 per 64-column group (see below) */
};

/* Return codes. */
enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* null or inconsistent argument, T < 1 */
  MOE_EUNSUPPORTED = -2, /* group_size not 64 or 0, d/f not multiples of 64, k > 32, E > 1024,
                            code_bits not 0, 2, 4 or 8 (8 and 2: d or f not a multiple
                            of 512), bad dtype/flags,
                            MOE_BATCH_INVARIANT with T > 8 or T * k > 64 */
  MOE_ENOSPC = -3,       /* ws_bytes smaller than moe_workspace_bytes() */
  MOE_EHIP = -4          /* a kernel launch failed; moe_strerror() names the HIP error */
};

/* Bytes of one expert blob (canonical layout above); 0 for invalid dims. */
size_t moe_expert_blob_bytes(const moe_dims* dims);

/* Workspace bytes any entry point needs for up to T_max tokens (or rows);
 * 0 for invalid dims or T_max < 1. */
size_t moe_workspace_bytes(const moe_dims* dims, int32_t T_max);

/* Static text for a return code (MOE_EHIP: includes the last HIP error seen
 * by this thread). */
const char* moe_strerror(int code);

/*
 * Where a call leaves its routing in the workspace: byte offsets from ws of
 * the routing results of the last moe_layer_forward or
 * moe_layer_forward_cached call for T tokens on that workspace (the layout
 * depends on the call's T, not on the T_max the workspace was sized for):
 *   topk_idx  int32 [T][k]   chosen ids in slot order (as moe_route)
 *   topk_w    f32   [T][k]   renormalised router weights (as moe_route)
 *   uniq      int32 [min(E, T*k)]      distinct ids ascending, then -1 (as moe_union)
 *   n_uniq    int32 [1]                U
 *   offsets   int32 [min(E, T*k) + 1]  per-expert slot ranges (as moe_union)
 *   rows      int32 [T*k]              slot ids grouped by expert, ascending t
 * These are the lists the call's expert kernels walked, so a caller can check
 * or reuse them (they are valid once the call's work on its stream has
 * completed and until the next call on the workspace).  Returns MOE_OK, or
 * MOE_EINVAL / MOE_EUNSUPPORTED for invalid dims, T < 1 or a NULL `out`.
 * Source: route, then union, per token and layer — colibri 技术解读,
 * "引擎结构：一个 C 文件，五步 token 路径"; README 工作原理 › 绝不为同一次磁盘读取等待两遍.
 */
typedef struct moe_routing_offsets {
  size_t topk_idx, topk_w, uniq, n_uniq, offsets, rows;
} moe_routing_offsets;
int moe_workspace_routing(const moe_dims* dims, int32_t T, moe_routing_offsets* out);

/*
 * moe_route — router logits, top-k and renormalised weights.
 *   x          [T][d] activations, f32 or bf16 (x_dtype), row-major
 *   w_router   [E][d] f32 router matrix, row-major
 *   bias       [E] f32 added to the logits before selection and softmax, or NULL
 *   topk_idx   [T][k] int32 out: chosen expert ids, slot j in descending logit
 *              order, equal logits ordered by ascending id
 *   topk_w     [T][k] f32 out: softmax(z)[id] / sum over the token's k ids
 * Logits z[t][e] = sum_i x[t][i] * w_router[e][i] + bias[e] are accumulated
 * in fp64 (each fp32 product is exact in fp64).
 * Source: the router picks 8 of 256 routed experts per token and layer —
 * colibri 技术解读, "MoE 的稀疏性" and "引擎结构：一个 C 文件，五步 token 路径".
 */
int moe_route(const moe_dims* dims, const void* x, int x_dtype, int32_t T, const float* w_router,
              const float* bias, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
              void* stream);

/*
 * moe_union — batch union of the routed experts.
 *   topk_idx   [T][k] int32 expert ids, each in [0, E), distinct within a token
 *   uniq       [min(E, T*k)] int32 out: the U distinct ids ascending, then -1
 *   n_uniq     [1] int32 out: U (stays on the device)
 *   offsets    [min(E, T*k) + 1] int32 out: expert uniq[u] owns
 *              rows[offsets[u] .. offsets[u+1]); entries after U equal
 *              offsets[U] (= T*k when every id is valid)
 *   rows       [T*k] int32 out: slot ids t*k + j grouped by expert in uniq
 *              order, ascending t within an expert
 * Each distinct expert appears once, so a consumer that walks uniq reads each
 * expert's bytes once per batch.
 * Source: repeated picks of one expert across the positions of a batch are
 * merged into one read ("batch union") — colibrì README (简体中文), 工作原理 ›
 * 绝不为同一次磁盘读取等待两遍; colibri 技术解读, "引擎结构：一个 C 文件，五步 token 路径".
 * Ids outside [0, E) are skipped: they are listed under no expert, offsets
 * after U then equal the number of valid ids, and the tail of rows beyond
 * offsets[U] is left unwritten.
 */
int moe_union(const moe_dims* dims, const int32_t* topk_idx, int32_t T, int32_t* uniq,
              int32_t* n_uniq, int32_t* offsets, int32_t* rows, void* stream);

/*
 * moe_expert_ffn — one expert's SwiGLU FFN on n activation rows.
 *   expert_blob  the expert's canonical blob (device or host-mapped memory)
 *   x            [*][d] activations (f32 or bf16)
 *   rows         [n] int32 indices into x (each a valid row of x), or NULL
 *                for rows 0..n-1
 *   y            [n][d] f32 out: y[i] = Wd (silu(Wg x[rows[i]]) * (Wu x[rows[i]]))
 * The result does not depend on where the blob's bytes live.
 * Source: the chosen experts run their feed-forward computation — colibri
 * 技术解读, "集群模式与开放问题清单"; blob of three adjacent matrices — README
 * 工作原理 › 绝不为同一次磁盘读取等待两遍.
 */
int moe_expert_ffn(const moe_dims* dims, const void* expert_blob, const void* x, int x_dtype,
                   const int32_t* rows, int32_t n, float* y, void* ws, size_t ws_bytes,
                   void* stream);

/*
 * moe_layer_forward — the whole layer for T tokens.
 *   x             [T][d] f32 or bf16 layer input
 *   w_router      [E][d] f32; bias [E] f32 or NULL
 *   expert_table  device array of E pointers to expert blobs (each device or
 *                 host-mapped memory); entries of experts no token picks are
 *                 never dereferenced
 *   out           [T][d] f32 out: out[t] = sum_j w[t][j] * y_{idx[t][j]}(x'[t])
 *                 (+ x[t] with MOE_RESIDUAL), summed in ascending slot j, where
 *                 x' = RMSNorm(x) with MOE_PRENORM_RMS, else x.  out may alias x.
 *   flags         MOE_PRENORM_RMS | MOE_RESIDUAL (both need x_dtype MOE_F32)
 *                 | MOE_BATCH_INVARIANT (any dtype; T <= 8 and T * k <= 64):
 *                 token t's out[t] and its counts in stats are bit-identical
 *                 to those of a call with x[t] alone (T = 1, same flags,
 *                 table and weights), so a batched verify of drafted tokens
 *                 computes exactly the function that produced them one at a
 *                 time.  The batch runs the single-token kernel family with
 *                 every token's arithmetic in the single-token order; each
 *                 distinct expert is still streamed once per call.  Without
 *                 the flag, batches of 2 or more tokens may take the matrix-
 *                 core path, whose rounding differs from the single-token
 *                 path within the output tolerance.
 *                 Source: drafts and their batched verification must compute
 *                 the same function, pinned to one kernel family — README
 *                 工作原理 › 诚实的推测解码; 技术解读, "精度与语义：速度可以牺牲，语义不能".
 *                 | MOE_INT8_ACT: the experts take integer activations, as
 *                 the pages' hand-written integer dot-product kernels do (int4
 *                 weights times integer activations, no BLAS — 技术解读,
 *                 "int4 量化与手写内核"; the nxmr blog's int8 kernels, «纯C语言»).
 *                 Each 64-column group of an expert's input row (x', and
 *                 a = silu(g) * u) is held as int8 q = v / s rounded to the
 *                 nearest integer (ties to even), s = max|v| / 127, both in
 *                 fp32 (a group of zeros: s = 0); each group's dot product
 *                 with the weight codes is exact in int32 on the int8 matrix
 *                 cores, then times the weight scale and s in fp32.  Routing
 *                 is unchanged.  The result is this quantised function: within
 *                 2e-3 * max|ref| of an fp64 evaluation of it, and about
 *                 1e-2 * max|ref| from the unquantised layer (the int8
 *                 rounding of the activations).  int4 and int2 layers run one
 *                 token (and, with MOE_BATCH_INVARIANT, batches of up to 8;
 *                 int4 also every batch when d or f is not a multiple of 512)
 *                 on the single-token kernel family with these int8 values in
 *                 its digit form, other batches on the int8 matrix cores; int8
 *                 layers run every batch on the matrix cores, in 16-token
 *                 tiles, so there a token's result never depends on its
 *                 batch.  MOE_BATCH_INVARIANT keeps its meaning, and
 *                 moe_layer_forward_cached takes the flag too.
 *   rms_eps       RMSNorm epsilon (used with MOE_PRENORM_RMS)
 *   stats         device [1 + E] int32 out, or NULL: stats[0] = U, stats[1+e]
 *                 = number of tokens that picked expert e
 * Routing is as moe_route, the union as moe_union; each distinct expert's
 * bytes are streamed once for the whole batch.  Results are bit-reproducible
 * run to run (no floating-point atomics).
 * Source: route -> union -> place -> overlap -> learn per token and layer —
 * colibri 技术解读, "引擎结构：一个 C 文件，五步 token 路径"; the residual stream kept
 * on the device across layers — README 工作原理 › 绝不为同一次磁盘读取等待两遍.
 */
int moe_layer_forward(const moe_dims* dims, const void* x, int x_dtype, int32_t T,
                      const float* w_router, const float* bias, const void* const* expert_table,
                      float* out, uint32_t flags, float rms_eps, int32_t* stats, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * HBM slot cache in front of the experts' home memory.
 *
 * moe_cache_state_bytes — bytes of the cache state for n_slots slots; 0 for
 * invalid dims or n_slots outside [1, E].  The state lives in caller device
 * memory, zero-filled once before its first use (every slot empty), and is
 * then owned by the calls that take it.  Layout (32-bit words):
 *   header: clock (calls so far), hits, misses (union experts found in a
 *           slot / copied into one, over all calls), last_hits, last_misses,
 *           3 reserved
 *   slot_of[E]   slot + 1 holding expert e, 0 if none
 *   expert_of[S] expert + 1 held by slot s, 0 if empty
 *   stamp[S]     clock value of slot s's last use
 */
size_t moe_cache_state_bytes(const moe_dims* dims, int32_t n_slots);

/*
 * moe_layer_forward_cached — the layer for a small batch (T <= 8, T * k <= 64)
 * whose experts live in home memory (pinned host memory mapped into the device
 * address space, or any device-readable memory) behind an HBM cache of
 * n_slots expert slots.
 *   home_table  device array of E pointers to the experts' blobs in their home
 *               memory (16-byte aligned); only missed experts are read there
 *   slots       device memory of n_slots * moe_expert_blob_bytes() bytes,
 *               256-byte aligned, owned by the cache
 *   n_slots     min(E, T * k) <= n_slots <= E
 *   cache_state device buffer of moe_cache_state_bytes(dims, n_slots)
 *   other arguments as moe_layer_forward (every flag accepted).
 * Per call, on the device: the router and the union; placement in one
 * workgroup (experts of the union found in a slot keep it and count as hits;
 * each other one, in ascending id, takes the least recently used slot not
 * used by this call, ties to the lower slot, and evicts its expert); the
 * missed blobs are copied from home into their slots by the first workgroups
 * of a launch whose other workgroups run the gate/up of the hits, so the
 * hits compute while the misses are in flight; the misses' gate/up follows
 * once their copies have landed, then down + combine over the whole union,
 * every expert read from its slot.  The batch runs the single-token
 * kernel family, so out (and stats) are bit-identical to moe_layer_forward
 * with MOE_BATCH_INVARIANT added (for one token: with the same flags) and the blobs
 * resident, for any cache contents: where an expert's bytes come from
 * decides only the speed.  Calls sharing one
 * cache state must be ordered (one stream); the clock wraps after 2^32 calls.
 * Errors as moe_layer_forward; MOE_EUNSUPPORTED also for T or n_slots out of
 * range.
 * Source: an expert is fetched once per batch from wherever it lives and
 * resident experts are served from the faster tier, the placement following
 * each token's routing — README 工作原理 › 绝不为同一次磁盘读取等待两遍 (place,
 * overlap); colibri 技术解读, "引擎结构：一个 C 文件，五步 token 路径"
 * (route → union → place → overlap → learn).
 */
int moe_layer_forward_cached(const moe_dims* dims, const void* x, int x_dtype, int32_t T,
                             const float* w_router, const float* bias,
                             const void* const* home_table, void* slots, int32_t n_slots,
                             void* cache_state, float* out, uint32_t flags, float rms_eps,
                             int32_t* stats, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_forward_noalloc — moe_layer_forward for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The arguments and results are those of
 * moe_layer_forward without ws / ws_bytes: the workspace is instead a fixed
 * array of MOE_NOALLOC_SCRATCH_BYTES in the library's own device memory,
 * one per GPU, held from the first call on that GPU until the process ends.
 * The call allocates and frees nothing (no hipMalloc, no allocating library
 * routine); its first call on a device looks up that device's copy of the
 * array, with the device current.  The caller still owns x, the router, the
 * expert table, out and stats.
 *   - A call needs moe_workspace_bytes(dims, T) <= MOE_NOALLOC_SCRATCH_BYTES
 *     (GLM-5.2-shaped layers, d = 6144, f = 2048, 256 experts, top-8: up to
 *     T = 64 tokens and a little more: 79 with the current workspace layout);
 *     larger calls return MOE_ENOSPC and enqueue nothing.
 *   - Every call on a GPU shares that GPU's array, which keeps the last
 *     call's contents (no part of it needs to start at zero: every call
 *     writes each word before it reads it).  Calls that overlap in time on
 *     one GPU (other streams, other threads) race on it and must not be made.
 *   - moe_workspace_routing applies to the array as to a workspace, but the
 *     array is not addressable by the caller.
 * Errors as moe_layer_forward, plus MOE_ENOSPC for a call past the limit and
 * MOE_EHIP when the array's address cannot be looked up.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_layer_forward_noalloc(const moe_dims* dims, const void* x, int x_dtype, int32_t T,
                              const float* w_router, const float* bias,
                              const void* const* expert_table, float* out, uint32_t flags,
                              float rms_eps, int32_t* stats, void* stream);

/*
 * Kernel timing — instrumentation, not part of the layer's computation.
 * Kernels of the library, by name:                                          */
enum {
  MOE_KERNEL_RMSNORM = 0,
  MOE_KERNEL_LOGITS = 1,
  MOE_KERNEL_TOPK = 2,
  MOE_KERNEL_UNION = 3,
  MOE_KERNEL_DIGITIZE = 4,
  MOE_KERNEL_GATEUP = 5, /* gate/up projections + SwiGLU (the largest byte stream) */
  MOE_KERNEL_DOWN = 6,   /* down projection */
  MOE_KERNEL_COMBINE = 7,
  MOE_KERNEL_READ_PROBE = 8, /* moe_hbm_read_probe */
  MOE_KERNEL_GATEUP_THIN = 9, /* gate/up of experts with at most 16 tokens (batches of 2+) */
  MOE_KERNEL_DOWN_THIN = 10,  /* down of those experts */
  MOE_KERNEL_COUNT = 11
};
/*
 * moe_timing_arm — the next n launches of `kernel` record start_events[i]
 * when launch i starts executing and stop_events[i] when it ends (hipEvent_t
 * handles created by the caller, recorded on the launch's stream through
 * hipExtLaunchKernelGGL).  The handle arrays are host memory that must stay
 * valid until the n launches have been enqueued or the kernel is re-armed;
 * n = 0 disarms.  Returns how many launches the previous arming recorded, or
 * MOE_EINVAL for a bad kernel id, negative n, or n > 0 with NULL arrays.
 * Process-wide state: not for concurrent use from several threads.
 */
int moe_timing_arm(int kernel, void* const* start_events, void* const* stop_events, int n);

/*
 * Phase trace — instrumentation, not part of the layer's computation.  Only
 * lib/libmoe_trace.so (the same sources built with MOE_PHASE_TRACE, same
 * entry points) records; in libmoe.so both calls return MOE_EUNSUPPORTED and
 * the kernels carry no trace code.  Every workgroup of a traced kernel writes
 * a record of 8 uint64 words, record b for workgroup index b (flattened over
 * the grid, modulo 32768), after it finishes:
 *   [0] start, [1..5] the kernel's trace points (0: not reached), [6] end:
 *       readings of the device's 100 MHz clock (one counter for the whole
 *       chip, so records of one launch share a time line);
 *   [7] (compute unit id << 8) | tag.
 * Traced kernels (`which`), their points and tags:
 *   MOE_TRACE_GATEUP_GEMV   single-token gate/up family: 1-3 routing prologue
 *                           (per-group sorts, merges, union; one token only),
 *                           4 the first wave's rows streamed, 5 every wave's;
 *                           tag 1, or 0 for a block without an expert;
 *   MOE_TRACE_ROUTE_SMALL   k_route_small: 1 sorts, 2 merges, 3 union,
 *                           4 maps and routing published;
 *   MOE_TRACE_DOWN_T1       one-token down + combine: 1 the first wave's
 *                           experts streamed, 2 every wave's;
 *   MOE_TRACE_ROUTER_FRONT  small-batch router front end: tag 1 logits,
 *                           2 x pack, 3 digit split;
 *   MOE_TRACE_GATEUP_THIN, MOE_TRACE_DOWN_THIN  thin grouped GEMM alone:
 *                           1 tile known and first copies issued (0: no
 *                           tile), 2 first stage landed, 3 last stage done;
 *   MOE_TRACE_GATEUP_MIXED, MOE_TRACE_DOWN_MIXED  mixed launch: start and end
 *                           only; tag 1 M-blocked, 2 thin, 3 empty M-block slot.
 * moe_trace_read copies the first `bytes` bytes (at most 32768 records) of a
 * kernel's records into host memory `dst`, synchronously; moe_trace_reset
 * zeroes every record.  Records stay until a later launch of the kernel
 * overwrites them.  Neither call may run while traced kernels are in flight.
 */
enum {
  MOE_TRACE_GATEUP_GEMV = 0,
  MOE_TRACE_ROUTE_SMALL = 1,
  MOE_TRACE_DOWN_T1 = 2,
  MOE_TRACE_ROUTER_FRONT = 3,
  MOE_TRACE_GATEUP_THIN = 4,
  MOE_TRACE_DOWN_THIN = 5,
  MOE_TRACE_GATEUP_MIXED = 6,
  MOE_TRACE_DOWN_MIXED = 7,
  MOE_TRACE_COUNT = 8
};
int moe_trace_read(int which, void* dst, size_t bytes);
int moe_trace_reset(void);

/*
 * moe_hbm_read_probe — measurement helper, not part of the layer: one kernel
 * that streams `bytes` bytes of device memory at `buf` (16-byte aligned,
 * bytes a multiple of 16) through non-temporal 16-byte loads, eight in
 * flight per lane, over `blocks` workgroups of 256 threads.  Timed over a
 * buffer far larger than the 256 MB Infinity Cache, it gives the read
 * bandwidth a plain kernel reaches on the device, the ceiling against which
 * the expert kernels' achieved GB/s is also read (besides the published peak).
 * `sink` is device memory of blocks * 256 uint32 words; the kernel writes a
 * word only when its XOR of the data equals a fixed key (so the loads
 * cannot be elided), which callers must not rely on either way.  Enqueued on
 * `stream`; never synchronises.  MOE_EINVAL for null pointers, a misaligned
 * buffer, bytes == 0 or not a multiple of 16, or blocks < 1; MOE_EHIP when
 * the launch fails.
 */
int moe_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */

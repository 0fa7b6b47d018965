/*
 * CPU oracle of the int4 routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  The product
 * (the HIP library and its Python binding) never links, loads or calls it, and
 * it shares no code, header or table with the product.
 *
 * It is deliberately plain: each step is its definition written out, in fp64,
 * with sequential sums (OpenMP only splits independent output rows across
 * threads; each row is still summed in order).
 *
 * What it computes (the pages describe the path of each token through a MoE
 * layer as route -> union -> place -> overlap -> learn; colibri 技术解读
 * (linlog.top), "引擎结构：一个 C 文件，五步 token 路径"; colibrì README
 * (简体中文), 工作原理 › 每个 token 的处理路径).  Place, overlap and learn only
 * decide where bytes come from and how fast, never the result, so the layer's
 * value is:
 *
 *   z[t,e] = sum_i x[t,i] * Wr[e,i] + b[e]                        (router)
 *   S_t    = the k experts of largest z[t,.], ties to the lower id (top-k)
 *   w[t,j] = softmax(z[t,.])[S_tj] / sum_j' softmax(z[t,.])[S_tj'] (renormalised)
 *   U      = distinct experts of all S_t, each read once           (batch union)
 *   y_e(x) = Wd_e (silu(Wg_e x) * (Wu_e x))                        (SwiGLU FFN)
 *   out[t] = sum_j w[t,j] * y_{S_tj}(x[t])                         (recombine)
 *
 * The pages name top-8-of-256 routing and the batch union (colibri 技术解读,
 * "MoE 的稀疏性" and the five-step path; README 工作原理 › 绝不为同一次磁盘读取
 * 等待两遍) but not the gate function, the FFN form or the weight layout; the
 * readings taken here (softmax over all experts, top-k on the logits,
 * renormalisation, SwiGLU, signed two's-complement int4 with one fp16 scale per
 * 64 consecutive input weights, element 2i in the low nibble) are listed with
 * their reasons in the design notes.
 *
 * Expert blob (the three matrices stored next to each other so one read fetches
 * an expert: README 工作原理 › 绝不为同一次磁盘读取等待两遍):
 *   gate codes [f][d/2] | up codes [f][d/2] | down codes [d][f/2]
 *   | gate scales [f][d/64] | up scales [f][d/64] | down scales [d][f/64]
 * codes are bytes holding two 4-bit weights, scales are IEEE binary16.  The
 * functions that read a blob take gs, the scale group: 64 for the layout
 * above (gs64, README 开始使用 › 获取模型), or 0 for one scale per row (the
 * per-row scaling of the nxmr blog, «纯C语言»): gate scales [f], up scales
 * [f], down scales [d], each weight w[r][c] = q[r][c] * s[r].
 * They also take bits, the code width: 4 (the layout above), or the 8-bit
 * and 2-bit codes the nxmr blog's hand-written kernels name next to packed
 * int4 («纯C语言»): a row of `cols` weights then takes cols * bits / 8 bytes,
 * int8 one two's-complement byte per weight, int2 four per byte (weight 4i + j
 * in bits 2j..2j+1 of byte i, lowest first; two's complement, -2..1), and the
 * scale tensors follow all the codes as above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define REF_PRENORM 1u
#define REF_RESIDUAL 2u
#define REF_I8ACT 8u

/* ---- encodings ------------------------------------------------------------ */

/* Weight number c of a row of 4-bit codes: byte c/2, low nibble when c is
 * even, high nibble when odd; the nibble is a two's-complement int4. */
int ref_nibble(const uint8_t* row_codes, int64_t c) {
  int b = row_codes[c / 2];
  int n = (c % 2 == 0) ? (b & 0xF) : (b >> 4);
  return n >= 8 ? n - 16 : n;
}

/* Weight number c of a row of `bits`-wide codes (8, 4 or 2): the byte holding
 * it, the field (lowest first) and two's complement of that width. */
int ref_code(const uint8_t* row_codes, int64_t c, int bits) {
  if (bits == 4) return ref_nibble(row_codes, c);
  if (bits == 8) {
    int b = row_codes[c];
    return b >= 128 ? b - 256 : b;
  }
  int b = row_codes[c / 4];
  int v = (b >> (2 * (c % 4))) & 3;
  return v >= 2 ? v - 4 : v;
}

/* IEEE 754 binary16 -> double, from the format's definition. */
double ref_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1F;
  int man = h & 0x3FF;
  double v;
  if (ex == 0)
    v = ldexp((double)man, -24); /* subnormal: m/1024 * 2^-14 */
  else if (ex == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp(1.0 + man / 1024.0, ex - 15);
  return sign ? -v : v;
}

/* bfloat16 -> double: the upper half of an IEEE binary32. */
double ref_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ---- expert blob ----------------------------------------------------------- */

/* Scales of one row of `cols` weights: cols / gs (gs = 64), or 1 (gs = 0). */
static int64_t row_scales(int cols, int gs) { return gs ? cols / gs : 1; }

/* Bytes of the codes of one f x d matrix. */
static int64_t mat_code_bytes(int d, int f, int bits) { return (int64_t)f * d * bits / 8; }

int64_t ref_blob_bytes(int d, int f, int gs, int bits) {
  return 3 * mat_code_bytes(d, f, bits) +
         2LL * (2LL * f * row_scales(d, gs) + (int64_t)d * row_scales(f, gs));
}

/* which: 0 gate [f x d], 1 up [f x d], 2 down [d x f]. */
static void mat_view(const uint8_t* blob, int d, int f, int gs, int bits, int which,
                     const uint8_t** codes, const uint16_t** scales, int* rows, int* cols) {
  *codes = blob + which * mat_code_bytes(d, f, bits);
  *scales = (const uint16_t*)(blob + 3 * mat_code_bytes(d, f, bits)) + which * (f * row_scales(d, gs));
  *rows = which == 2 ? d : f;
  *cols = which == 2 ? f : d;
}

/* Row r of a matrix, dequantised: w[c] = q[r,c] * s[r, c/gs] (gs64) or
 * q[r,c] * s[r] (per row), exact in fp64. */
static void dequant_row(const uint8_t* codes, const uint16_t* scales, int cols, int gs, int bits,
                        int r, double* w) {
  const uint8_t* rc = codes + (int64_t)r * cols * bits / 8;
  const uint16_t* rs = scales + (int64_t)r * row_scales(cols, gs);
  for (int c = 0; c < cols; ++c)
    w[c] = (double)ref_code(rc, c, bits) * ref_f16(rs[gs ? c / gs : 0]);
}

/* Dense dequantised matrix (rows x cols doubles), for tests on small shapes. */
void ref_dequant(const uint8_t* blob, int d, int f, int gs, int bits, int which, double* W) {
  const uint8_t* codes;
  const uint16_t* scales;
  int rows, cols;
  mat_view(blob, d, f, gs, bits, which, &codes, &scales, &rows, &cols);
  for (int r = 0; r < rows; ++r) dequant_row(codes, scales, cols, gs, bits, r, W + (int64_t)r * cols);
}

double ref_silu(double v) { return v / (1.0 + exp(-v)); }

/* SwiGLU expert FFN on n input rows x[n][d] -> y[n][d], reading the blob once:
 *   g = Wg x, u = Wu x, a = silu(g) * u, y = Wd a.
 * The pages only say the chosen experts run their feed-forward computation
 * (colibri 技术解读, "集群模式与开放问题清单"); SwiGLU is the reading taken. */
void ref_expert_ffn(int d, int f, int gs, int bits, const uint8_t* blob, const double* x, int n,
                    double* y) {
  const uint8_t *gc, *uc, *dc;
  const uint16_t *gsc, *usc, *dsc;
  int rows, cols;
  mat_view(blob, d, f, gs, bits, 0, &gc, &gsc, &rows, &cols);
  mat_view(blob, d, f, gs, bits, 1, &uc, &usc, &rows, &cols);
  mat_view(blob, d, f, gs, bits, 2, &dc, &dsc, &rows, &cols);
  double* a = (double*)malloc(sizeof(double) * (size_t)n * f);
#pragma omp parallel
  {
    double* wg = (double*)malloc(sizeof(double) * d);
    double* wu = (double*)malloc(sizeof(double) * d);
#pragma omp for schedule(static)
    for (int r = 0; r < f; ++r) {
      dequant_row(gc, gsc, d, gs, bits, r, wg);
      dequant_row(uc, usc, d, gs, bits, r, wu);
      for (int t = 0; t < n; ++t) {
        const double* xt = x + (int64_t)t * d;
        double g = 0.0, u = 0.0;
        for (int c = 0; c < d; ++c) {
          g += wg[c] * xt[c];
          u += wu[c] * xt[c];
        }
        a[(int64_t)t * f + r] = ref_silu(g) * u;
      }
    }
    free(wg);
    free(wu);
    double* wd = (double*)malloc(sizeof(double) * f);
#pragma omp for schedule(static)
    for (int c = 0; c < d; ++c) {
      dequant_row(dc, dsc, f, gs, bits, c, wd);
      for (int t = 0; t < n; ++t) {
        const double* at = a + (int64_t)t * f;
        double acc = 0.0;
        for (int r = 0; r < f; ++r) acc += wd[r] * at[r];
        y[(int64_t)t * d + c] = acc;
      }
    }
    free(wd);
  }
  free(a);
}

/* ---- integer activations ------------------------------------------------- */

/* The pages run the experts through hand-written integer dot-product kernels:
 * int4 weights times integer activations, no BLAS (colibri 技术解读
 * (linlog.top), "int4 量化与手写内核"; the nxmr blog's int8 kernels, «纯C语言»),
 * without fixing how the activations are quantised.  Reading taken: each
 * 64-column group of an activation row (the weights' scale group) is held as
 * int8 q with one scale s = max|v| / 127, q = v / s rounded to the nearest
 * integer (ties to even); a group of zeros has s = 0 and q = 0.  Both the
 * scale and the rounding are taken in fp32 (the kernel's precision, so that
 * both sides make the same integer decision on the same fp32 input).  cols is
 * a multiple of 64; q[cols], s[cols / 64]. */
void ref_quant_i8(const float* v, int cols, int8_t* q, float* s) {
  for (int g = 0; g < cols / 64; ++g) {
    const float* vg = v + (int64_t)g * 64;
    float m = 0.0f;
    for (int j = 0; j < 64; ++j)
      if (fabsf(vg[j]) > m) m = fabsf(vg[j]);
    const float sc = m / 127.0f;
    s[g] = sc;
    for (int j = 0; j < 64; ++j) {
      float r = m > 0.0f ? rintf(vg[j] / sc) : 0.0f;
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      q[(int64_t)g * 64 + j] = (int8_t)r;
    }
  }
}

/* One row of a matrix times int8 activation rows: for each 64-column group g,
 * the exact integer sum of code * q over the group, times the weight scale of
 * the group (or of the row) and the activation scale s[g], summed over the
 * groups in order in fp64. */
static double row_dot_i8(const uint8_t* codes, const uint16_t* scales, int cols, int gs, int bits,
                         int r, const int8_t* q, const float* s) {
  const uint8_t* rc = codes + (int64_t)r * cols * bits / 8;
  const uint16_t* rs = scales + (int64_t)r * row_scales(cols, gs);
  double acc = 0.0;
  for (int g = 0; g < cols / 64; ++g) {
    int64_t dot = 0;
    for (int j = 64 * g; j < 64 * g + 64; ++j) dot += (int64_t)ref_code(rc, j, bits) * q[j];
    acc += ref_f16(rs[gs ? (64 * g) / gs : 0]) * (double)s[g] * (double)dot;
  }
  return acc;
}

/* The SwiGLU expert FFN with integer activations: x rows are quantised as
 * above, g and u are integer dot products per group, a = silu(g) * u is
 * rounded to fp32 (the precision the kernel holds it in) and quantised the
 * same way, and y = Wd a is again integer dot products per group.  x[n][d]
 * fp32 -> y[n][d] fp64; d and f multiples of 64. */
void ref_expert_ffn_i8act(int d, int f, int gs, int bits, const uint8_t* blob, const float* x,
                          int n, double* y) {
  const uint8_t *gc, *uc, *dc;
  const uint16_t *gsc, *usc, *dsc;
  int rows, cols;
  mat_view(blob, d, f, gs, bits, 0, &gc, &gsc, &rows, &cols);
  mat_view(blob, d, f, gs, bits, 1, &uc, &usc, &rows, &cols);
  mat_view(blob, d, f, gs, bits, 2, &dc, &dsc, &rows, &cols);
  int8_t* xq = (int8_t*)malloc((size_t)n * d);
  float* xs = (float*)malloc(sizeof(float) * (size_t)n * (d / 64));
  for (int t = 0; t < n; ++t)
    ref_quant_i8(x + (int64_t)t * d, d, xq + (int64_t)t * d, xs + (int64_t)t * (d / 64));
  float* a = (float*)malloc(sizeof(float) * (size_t)n * f);
#pragma omp parallel for schedule(static)
  for (int r = 0; r < f; ++r)
    for (int t = 0; t < n; ++t) {
      const double g = row_dot_i8(gc, gsc, d, gs, bits, r, xq + (int64_t)t * d, xs + (int64_t)t * (d / 64));
      const double u = row_dot_i8(uc, usc, d, gs, bits, r, xq + (int64_t)t * d, xs + (int64_t)t * (d / 64));
      a[(int64_t)t * f + r] = (float)(ref_silu(g) * u);
    }
  int8_t* aq = (int8_t*)malloc((size_t)n * f);
  float* as = (float*)malloc(sizeof(float) * (size_t)n * (f / 64));
  for (int t = 0; t < n; ++t)
    ref_quant_i8(a + (int64_t)t * f, f, aq + (int64_t)t * f, as + (int64_t)t * (f / 64));
#pragma omp parallel for schedule(static)
  for (int c = 0; c < d; ++c)
    for (int t = 0; t < n; ++t)
      y[(int64_t)t * d + c] =
          row_dot_i8(dc, dsc, f, gs, bits, c, aq + (int64_t)t * f, as + (int64_t)t * (f / 64));
  free(xq);
  free(xs);
  free(a);
  free(aq);
  free(as);
}

/* ---- router ---------------------------------------------------------------- */

typedef struct {
  double z;
  int e;
} zpair;

/* Order: larger logit first; equal logits -> lower expert id first. */
static int zpair_cmp(const void* pa, const void* pb) {
  const zpair* a = (const zpair*)pa;
  const zpair* b = (const zpair*)pb;
  if (a->z > b->z) return -1;
  if (a->z < b->z) return 1;
  return (a->e > b->e) - (a->e < b->e);
}

static double x_at(const void* x, int x_is_bf16, int64_t i) {
  return x_is_bf16 ? ref_bf16(((const uint16_t*)x)[i]) : (double)((const float*)x)[i];
}

/* Router logits, top-k and renormalised weights for T tokens.
 * z[t][e] (optional output) is the fp64 logit; idx[t][j] the j-th largest
 * (slot order); w[t][j] the renormalised softmax weight.  The router picking
 * 8 of 256 experts per token and layer is on the pages (colibri 技术解读,
 * "MoE 的稀疏性"); the softmax/top-k/renormalise gate is the reading taken. */
void ref_route(int d, int E, int k, const void* x, int x_is_bf16, int T, const float* Wr,
               const float* bias, int32_t* idx, double* w, double* z_out) {
  double* z = (double*)malloc(sizeof(double) * (size_t)T * E);
#pragma omp parallel for collapse(2) schedule(static)
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i)
        acc += x_at(x, x_is_bf16, (int64_t)t * d + i) * (double)Wr[(int64_t)e * d + i];
      z[(int64_t)t * E + e] = acc + (bias ? (double)bias[e] : 0.0);
    }
  zpair* pr = (zpair*)malloc(sizeof(zpair) * E);
  double* p = (double*)malloc(sizeof(double) * E);
  for (int t = 0; t < T; ++t) {
    const double* zt = z + (int64_t)t * E;
    for (int e = 0; e < E; ++e) {
      pr[e].z = zt[e];
      pr[e].e = e;
    }
    qsort(pr, E, sizeof(zpair), zpair_cmp);
    /* softmax over all E experts */
    double m = pr[0].z, den = 0.0;
    for (int e = 0; e < E; ++e) {
      p[e] = exp(zt[e] - m);
      den += p[e];
    }
    for (int e = 0; e < E; ++e) p[e] /= den;
    double sel = 0.0;
    for (int j = 0; j < k; ++j) sel += p[pr[j].e];
    for (int j = 0; j < k; ++j) {
      idx[(int64_t)t * k + j] = pr[j].e;
      w[(int64_t)t * k + j] = p[pr[j].e] / sel;
    }
  }
  if (z_out) memcpy(z_out, z, sizeof(double) * (size_t)T * E);
  free(p);
  free(pr);
  free(z);
}

/* ---- batch union ----------------------------------------------------------- */

/* Distinct experts of a batch, each listed once, ascending id; for each, the
 * slots (t*k + j) that chose it, ascending t.  Returns U.  (Repeated picks of
 * one expert in a batch become a single read: README 工作原理 › 绝不为同一次
 * 磁盘读取等待两遍.)  uniq and offsets need min(E, T*k) and that + 1 entries. */
int ref_union(int E, int k, int T, const int32_t* idx, int32_t* uniq, int32_t* offsets,
              int32_t* rows) {
  char* seen = (char*)calloc(E, 1);
  for (int64_t i = 0; i < (int64_t)T * k; ++i) seen[idx[i]] = 1;
  int U = 0, pos = 0;
  for (int e = 0; e < E; ++e) {
    if (!seen[e]) continue;
    uniq[U] = e;
    offsets[U] = pos;
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (idx[(int64_t)t * k + j] == e) rows[pos++] = t * k + j;
    ++U;
  }
  offsets[U] = pos;
  free(seen);
  return U;
}

/* ---- RMSNorm (unit gain) --------------------------------------------------- */

/* xn = h / sqrt(mean(h^2) + eps), mean and root in fp64, rounded to fp32. */
void ref_rmsnorm(int d, const float* h, double eps, float* xn) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += (double)h[i] * (double)h[i];
  double r = 1.0 / sqrt(ss / d + eps);
  for (int i = 0; i < d; ++i) xn[i] = (float)((double)h[i] * r);
}

/* ---- whole layer ----------------------------------------------------------- */

/* One MoE layer over T tokens.  table[e] points at expert e's blob (any
 * memory; entries of experts no token selects may be NULL).  flags:
 *   REF_PRENORM  route and run experts on RMSNorm(x) (x fp32)
 *   REF_RESIDUAL out = x + MoE(...) (x fp32)
 *   REF_I8ACT    the experts take integer activations (ref_expert_ffn_i8act)
 * Outputs: out[T][d] (fp64), idx/w [T][k], uniq/offsets/rows as ref_union,
 * reads[E] += 1 for every time an expert's blob is read.  Returns U, or -1 if
 * a selected expert has no blob. */
int ref_layer_forward(int d, int f, int gs, int bits, int E, int k, const void* x, int x_is_bf16, int T,
                      const float* Wr, const float* bias, const uint8_t* const* table,
                      uint32_t flags, double eps, double* out, int32_t* idx, double* w,
                      int32_t* uniq, int32_t* offsets, int32_t* rows, int32_t* reads) {
  const void* xin = x;
  int xin_bf16 = x_is_bf16;
  float* xn = NULL;
  if (flags & REF_PRENORM) {
    xn = (float*)malloc(sizeof(float) * (size_t)T * d);
    for (int t = 0; t < T; ++t) ref_rmsnorm(d, (const float*)x + (int64_t)t * d, eps, xn + (int64_t)t * d);
    xin = xn;
    xin_bf16 = 0;
  }
  ref_route(d, E, k, xin, xin_bf16, T, Wr, bias, idx, w, NULL);
  int U = ref_union(E, k, T, idx, uniq, offsets, rows);
  for (int u = 0; u < U; ++u)
    if (!table[uniq[u]]) {
      free(xn);
      return -1;
    }

  double* yslot = (double*)malloc(sizeof(double) * (size_t)T * k * d);
  for (int u = 0; u < U; ++u) {
    int e = uniq[u];
    int n = offsets[u + 1] - offsets[u];
    double* xs = (double*)malloc(sizeof(double) * (size_t)n * d);
    double* ys = (double*)malloc(sizeof(double) * (size_t)n * d);
    for (int i = 0; i < n; ++i) {
      int t = rows[offsets[u] + i] / k;
      for (int c = 0; c < d; ++c) xs[(int64_t)i * d + c] = x_at(xin, xin_bf16, (int64_t)t * d + c);
    }
    if (flags & REF_I8ACT) {
      /* the rows are fp32 values (fp32 or bf16 input, or the fp32 RMSNorm) */
      float* xf = (float*)malloc(sizeof(float) * (size_t)n * d);
      for (int64_t i = 0; i < (int64_t)n * d; ++i) xf[i] = (float)xs[i];
      ref_expert_ffn_i8act(d, f, gs, bits, table[e], xf, n, ys); /* the one read of expert e */
      free(xf);
    } else {
      ref_expert_ffn(d, f, gs, bits, table[e], xs, n, ys); /* the one read of expert e */
    }
    reads[e] += 1;
    for (int i = 0; i < n; ++i)
      memcpy(yslot + (int64_t)rows[offsets[u] + i] * d, ys + (int64_t)i * d, sizeof(double) * d);
    free(xs);
    free(ys);
  }
  for (int t = 0; t < T; ++t)
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) acc += w[(int64_t)t * k + j] * yslot[((int64_t)t * k + j) * d + c];
      if (flags & REF_RESIDUAL) acc += (double)((const float*)x)[(int64_t)t * d + c];
      out[(int64_t)t * d + c] = acc;
    }
  free(yslot);
  free(xn);
  return U;
}

/*
 * Sanitizer run of the CPU oracle (TEST INFRASTRUCTURE).
 *
 * Built together with moe_ref.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitized.py), it calls every
 * oracle function on small layers whose shapes reach the edges of the
 * oracle's loops: one token, k = 1, k = E, per-row and gs64 scales, bf16
 * input, RMSNorm + residual, experts no token picks left out of the table.
 * Any out-of-bounds access, use of freed memory or undefined operation stops
 * the run with the sanitizer's report.  Beyond that it checks a few facts
 * that hold for any input: router weights sum to 1 per token, the union's
 * offsets run from 0 to T*k, every selected expert is read exactly once and
 * no other, outputs are finite.
 *
 * Inputs are a fixed xorshift pattern (no part of the layer's arithmetic).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ref_nibble(const uint8_t* row_codes, int64_t c);
double ref_f16(uint16_t h);
double ref_bf16(uint16_t b);
int ref_code(const uint8_t* row_codes, int64_t c, int bits);
int64_t ref_blob_bytes(int d, int f, int gs, int bits);
void ref_dequant(const uint8_t* blob, int d, int f, int gs, int bits, int which, double* W);
double ref_silu(double v);
void ref_quant_i8(const float* v, int cols, int8_t* q, float* s);
void ref_expert_ffn(int d, int f, int gs, int bits, const uint8_t* blob, const double* x, int n,
                    double* y);
void ref_route(int d, int E, int k, const void* x, int x_is_bf16, int T, const float* Wr,
               const float* bias, int32_t* idx, double* w, double* z_out);
int ref_union(int E, int k, int T, const int32_t* idx, int32_t* uniq, int32_t* offsets,
              int32_t* rows);
void ref_rmsnorm(int d, const float* h, double eps, float* xn);
int ref_layer_forward(int d, int f, int gs, int bits, int E, int k, const void* x, int x_is_bf16, int T,
                      const float* Wr, const float* bias, const uint8_t* const* table,
                      uint32_t flags, double eps, double* out, int32_t* idx, double* w,
                      int32_t* uniq, int32_t* offsets, int32_t* rows, int32_t* reads);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
  g_state ^= g_state << 13;
  g_state ^= g_state >> 7;
  g_state ^= g_state << 17;
  return g_state;
}
static double next_unit(void) { return (double)(next_u64() >> 11) / 9007199254740992.0; }

static int failures = 0;
#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");             \
      ++failures;                        \
    }                                    \
  } while (0)

/* One expert blob in exactly its own allocation (so ASan sees its end):
 * random codes, scales = fp16 bit patterns of values in [0.004, 0.03). */
static uint8_t* make_blob(int d, int f, int gs, int bits) {
  const int64_t n = ref_blob_bytes(d, f, gs, bits);
  uint8_t* b = (uint8_t*)malloc((size_t)n);
  const int64_t codes = 3LL * f * d * bits / 8;
  for (int64_t i = 0; i < codes; ++i) b[i] = (uint8_t)next_u64();
  uint16_t* s = (uint16_t*)(b + codes);
  for (int64_t i = 0; i < (n - codes) / 2; ++i)
    s[i] = (uint16_t)(0x1C00u + (next_u64() % 0x0C00u)); /* 2^-8 .. 2^-5 */
  return b;
}

static void run_layer(const char* name, int d, int f, int gs, int bits, int E, int k, int T,
                      int bf16, uint32_t flags, int sparse_table) {
  float* xf = (float*)malloc(sizeof(float) * (size_t)T * d);
  uint16_t* xb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)T * d);
  for (int64_t i = 0; i < (int64_t)T * d; ++i) {
    xf[i] = (float)(2.0 * next_unit() - 1.0);
    uint32_t u;
    memcpy(&u, &xf[i], 4);
    xb[i] = (uint16_t)(u >> 16);
  }
  float* Wr = (float*)malloc(sizeof(float) * (size_t)E * d);
  for (int64_t i = 0; i < (int64_t)E * d; ++i) Wr[i] = (float)(0.04 * next_unit() - 0.02);
  float* bias = (float*)malloc(sizeof(float) * E);
  for (int e = 0; e < E; ++e) bias[e] = (float)(-0.1 * log(e + 1.0));
  const void* x = bf16 ? (const void*)xb : (const void*)xf;

  /* the experts the router picks, found first so the table can leave the
   * others out */
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)T * k);
  double* w = (double*)malloc(sizeof(double) * (size_t)T * k);
  double* z = (double*)malloc(sizeof(double) * (size_t)T * E);
  float* xn = NULL;
  const void* xr = x;
  int xr_bf16 = bf16;
  if (flags & 1u) {
    xn = (float*)malloc(sizeof(float) * (size_t)T * d);
    for (int t = 0; t < T; ++t) ref_rmsnorm(d, xf + (int64_t)t * d, 1e-6, xn + (int64_t)t * d);
    xr = xn;
    xr_bf16 = 0;
  }
  ref_route(d, E, k, xr, xr_bf16, T, Wr, bias, idx, w, z);
  const uint8_t** table = (const uint8_t**)calloc(E, sizeof(*table));
  uint8_t** owned = (uint8_t**)calloc(E, sizeof(*owned));
  for (int e = 0; e < E; ++e) {
    int picked = 0;
    for (int64_t i = 0; i < (int64_t)T * k; ++i) picked |= idx[i] == e;
    if (picked || !sparse_table) table[e] = owned[e] = make_blob(d, f, gs, bits);
  }
  const int cap = E < T * k ? E : T * k;
  double* out = (double*)malloc(sizeof(double) * (size_t)T * d);
  int32_t* uniq = (int32_t*)malloc(sizeof(int32_t) * cap);
  int32_t* offs = (int32_t*)malloc(sizeof(int32_t) * (cap + 1));
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)T * k);
  int32_t* reads = (int32_t*)calloc(E, sizeof(int32_t));
  const int U = ref_layer_forward(d, f, gs, bits, E, k, bf16 && !(flags & 3u) ? (const void*)xb
                                                                       : (const void*)xf,
                                  bf16 && !(flags & 3u), T, Wr, bias, table, flags, 1e-6, out,
                                  idx, w, uniq, offs, rows, reads);
  CHECK(U >= 1 && U <= cap, "%s: U = %d", name, U);
  CHECK(offs[0] == 0 && offs[U] == T * k, "%s: offsets run %d..%d", name, offs[0], offs[U]);
  for (int t = 0; t < T; ++t) {
    double s = 0.0;
    for (int j = 0; j < k; ++j) s += w[(int64_t)t * k + j];
    CHECK(fabs(s - 1.0) < 1e-12, "%s: token %d weights sum to %.17g", name, t, s);
  }
  for (int e = 0; e < E; ++e) {
    int in_union = 0;
    for (int u = 0; u < U; ++u) in_union |= uniq[u] == e;
    CHECK(reads[e] == in_union, "%s: expert %d read %d times", name, e, reads[e]);
  }
  for (int64_t i = 0; i < (int64_t)T * d; ++i) CHECK(isfinite(out[i]), "%s: out[%lld]", name, (long long)i);

  /* union on its own, and the expert FFN on its own */
  int32_t* uq2 = (int32_t*)malloc(sizeof(int32_t) * cap);
  int32_t* of2 = (int32_t*)malloc(sizeof(int32_t) * (cap + 1));
  int32_t* rw2 = (int32_t*)malloc(sizeof(int32_t) * (size_t)T * k);
  CHECK(ref_union(E, k, T, idx, uq2, of2, rw2) == U, "%s: union size", name);
  double* xd = (double*)malloc(sizeof(double) * (size_t)T * d);
  for (int64_t i = 0; i < (int64_t)T * d; ++i) xd[i] = xf[i];
  double* y = (double*)malloc(sizeof(double) * (size_t)T * d);
  ref_expert_ffn(d, f, gs, bits, table[uniq[0]], xd, T, y);
  for (int which = 0; which < 3; ++which) {
    const int rws = which == 2 ? d : f, cls = which == 2 ? f : d;
    double* W = (double*)malloc(sizeof(double) * (size_t)rws * cls);
    ref_dequant(table[uniq[0]], d, f, gs, bits, which, W);
    free(W);
  }

  for (int e = 0; e < E; ++e) free(owned[e]);
  free(owned);
  free((void*)table);
  free(xf), free(xb), free(Wr), free(bias), free(idx), free(w), free(z), free(xn), free(out);
  free(uniq), free(offs), free(rows), free(reads), free(uq2), free(of2), free(rw2), free(xd), free(y);
  printf("sanitized oracle: %s ok (U = %d)\n", name, U);
}

int main(void) {
  /* encodings over their whole domains */
  for (int b = 0; b < 256; ++b) {
    const uint8_t byte = (uint8_t)b;
    CHECK(ref_nibble(&byte, 0) >= -8 && ref_nibble(&byte, 1) <= 7, "nibble %d", b);
  }
  for (int h = 0; h < 65536; ++h) {
    (void)ref_f16((uint16_t)h);
    (void)ref_bf16((uint16_t)h);
  }
  CHECK(ref_silu(-800.0) == 0.0 || ref_silu(-800.0) > -1e-300, "silu limit");
  for (int b = 0; b < 256; ++b) {
    const uint8_t byte = (uint8_t)b;
    CHECK(ref_code(&byte, 0, 8) == (int8_t)byte, "int8 code %d", b);
    for (int j = 0; j < 4; ++j) CHECK(ref_code(&byte, j, 2) >= -2 && ref_code(&byte, j, 2) <= 1, "int2");
  }
  run_layer("tiny gs64", 128, 64, 64, 4, 16, 2, 4, 0, 0u, 0);
  run_layer("one token", 64, 64, 64, 4, 8, 1, 1, 0, 0u, 1);
  run_layer("k = E", 64, 128, 64, 4, 8, 8, 3, 0, 0u, 0);
  run_layer("per-row scales", 192, 64, 0, 4, 12, 3, 5, 0, 0u, 1);
  run_layer("bf16 input", 128, 64, 64, 4, 10, 4, 6, 1, 0u, 1);
  run_layer("rmsnorm + residual", 128, 128, 64, 4, 16, 2, 3, 0, 3u, 1);
  run_layer("wide union", 64, 64, 64, 4, 96, 32, 3, 0, 0u, 1);
  run_layer("int8 codes", 128, 64, 64, 8, 12, 3, 5, 0, 0u, 1);
  run_layer("int2 codes, per-row", 192, 64, 0, 2, 12, 3, 5, 0, 3u, 1);
  run_layer("integer activations", 128, 64, 64, 4, 12, 3, 5, 0, 8u, 1);
  run_layer("integer activations, int8 codes, bf16", 128, 64, 64, 8, 10, 4, 6, 1, 8u, 1);
  run_layer("integer activations, int2, per-row, rmsnorm + residual", 192, 64, 0, 2, 12, 3, 5, 0, 11u, 1);
  {
    float v[128] = {0};
    int8_t q[128];
    float sc[2];
    v[70] = -1e-38f;
    v[100] = 3e38f;
    ref_quant_i8(v, 128, q, sc);
    CHECK(sc[0] == 0.0f && q[0] == 0 && q[63] == 0, "quant: zero group");
    CHECK(q[100] == 127 && q[70] == 0, "quant: extreme group");
  }
  if (failures) {
    fprintf(stderr, "sanitized oracle: %d failures\n", failures);
    return 1;
  }
  printf("sanitized oracle: all ok\n");
  return 0;
}

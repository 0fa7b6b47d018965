/*
 * Seeded synthetic inputs for the int4 routed-expert MoE layer.
 *
 * This file is harness code shared by the tests, the benchmark and the CPU
 * oracle's callers.  It holds none of the layer's arithmetic (no routing, no
 * dequantisation, no matmul): it only produces random bytes, normals and
 * fp16/bf16 encodings of random values.
 *
 * Randomness is counter based, so any element of any tensor of any layer can
 * be regenerated on its own (the oracle regenerates single experts of a
 * 48-layer stack without holding all of it):
 *
 *   key    = mix(mix(mix(seed) ^ layer) ^ (tensor << 32 | expert))
 *   draw_i = SplitMix64 output number i of the generator whose state starts
 *            at key, i.e. fin(key + (i + 1) * 0x9E3779B97F4A7C15)
 *
 * SplitMix64 is the generator of Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators" (OOPSLA 2014); fin() is its output mixing
 * function.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_fin(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t expert) {
  uint64_t k = sm64_fin(seed + SM64_GAMMA);
  k = sm64_fin(k ^ (uint64_t)layer);
  k = sm64_fin(k ^ (((uint64_t)tensor << 32) | (uint64_t)expert));
  return k;
}

uint64_t synth_draw(uint64_t key, uint64_t i) { return sm64_fin(key + (i + 1) * SM64_GAMMA); }

/* Uniform double in (0, 1] from the top 53 bits. */
static inline double u01_open0(uint64_t r) { return (double)((r >> 11) + 1) * 0x1.0p-53; }
/* Uniform double in [0, 1) from the top 53 bits. */
static inline double u01(uint64_t r) { return (double)(r >> 11) * 0x1.0p-53; }

/* Normal draws by the Box-Muller transform (Box and Muller, 1958): element i
 * uses draws 2i and 2i+1.  out[i] = (float)(mean + std * z_i). */
void synth_normal_f32(uint64_t key, int64_t n, double mean, double std, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double u1 = u01_open0(synth_draw(key, 2 * (uint64_t)i));
    double u2 = u01(synth_draw(key, 2 * (uint64_t)i + 1));
    double z = sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
    out[i] = (float)(mean + std * z);
  }
}

/* Random bytes: byte i is byte (i % 8) of draw i / 8 (little end first).
 * Each byte therefore carries two independent uniform 4-bit fields. */
void synth_bytes(uint64_t key, int64_t nbytes, uint8_t* out) {
  int64_t nw = nbytes / 8;
#pragma omp parallel for schedule(static)
  for (int64_t w = 0; w < nw; ++w) {
    uint64_t r = synth_draw(key, (uint64_t)w);
    memcpy(out + 8 * w, &r, 8);
  }
  for (int64_t i = 8 * nw; i < nbytes; ++i)
    out[i] = (uint8_t)(synth_draw(key, (uint64_t)(i / 8)) >> (8 * (i % 8)));
}

/* IEEE binary16 encoding of a double, round to nearest even. */
uint16_t synth_f64_to_f16(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00; /* rounds to infinity */
  if (a >= 0x1.0p-14) {
    int e;
    frexp(a, &e);              /* a = m * 2^e, m in [0.5, 1) */
    int E = e - 1;             /* a = 1.xxx * 2^E */
    double mant = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (mant >= 2048.0) { mant = 1024.0; E += 1; }
    if (E > 15) return sign | 0x7C00;
    return (uint16_t)(sign | ((E + 15) << 10) | ((int)mant - 1024));
  }
  double mant = nearbyint(ldexp(a, 24)); /* subnormal steps of 2^-24 */
  return (uint16_t)(sign | (int)mant);   /* mant == 1024 is the smallest normal */
}

/* n fp16 values uniform on [lo, hi): u has 24 random bits, v = lo + (hi-lo)*u
 * in double, then rounded to binary16. */
void synth_uniform_f16(uint64_t key, int64_t n, double lo, double hi, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double u = (double)(synth_draw(key, (uint64_t)i) >> 40) * 0x1.0p-24;
    out[i] = synth_f64_to_f16(lo + (hi - lo) * u);
  }
}

/* bfloat16 encoding of fp32 values, round to nearest even. */
void synth_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, &in[i], 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
      out[i] = (uint16_t)((u >> 16) | 0x40);
      continue;
    }
    u += 0x7FFFu + ((u >> 16) & 1u);
    out[i] = (uint16_t)(u >> 16);
  }
}

/* Tensor ids (the "tensor" field of the key). */
enum { T_X = 1, T_XNOISE = 2, T_WR = 3, T_NIB = 4, T_SCALE = 5, T_H0 = 6 };

/* One expert's bytes: nib_bytes random bytes (every nibble uniform on its 16
 * codes) followed by n_scales fp16 values uniform on [s_lo, s_hi). */
void synth_expert_blob(uint64_t seed, uint32_t layer, uint32_t expert, int64_t nib_bytes,
                       int64_t n_scales, double s_lo, double s_hi, uint8_t* out) {
  synth_bytes(synth_key(seed, layer, T_NIB, expert), nib_bytes, out);
  synth_uniform_f16(synth_key(seed, layer, T_SCALE, expert), n_scales, s_lo, s_hi,
                    (uint16_t*)(out + nib_bytes));
}

/* All experts [e0, e0+ne) of one layer into out (ne * blob_bytes). */
void synth_layer_blobs(uint64_t seed, uint32_t layer, uint32_t e0, uint32_t ne, int64_t nib_bytes,
                       int64_t n_scales, double s_lo, double s_hi, uint8_t* out) {
  int64_t blob = nib_bytes + 2 * n_scales;
  for (uint32_t e = 0; e < ne; ++e)
    synth_expert_blob(seed, layer, e0 + e, nib_bytes, n_scales, s_lo, s_hi, out + (int64_t)e * blob);
}

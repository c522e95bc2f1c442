/*
 * synth.c -- seeded synthetic inputs for the MSA decode path.
 *
 * Both the CPU oracle and the HIP library are fed from here; this file holds
 * none of the method's arithmetic (no scoring, pooling, selection or
 * attention), only random numbers and the encoders that turn them into the
 * stored formats.
 *
 * Random numbers are counter based: element i of stream (seed, stream) is a
 * pure function of (seed, stream, i), so any slice can be produced on its own
 * and in parallel.  Mixer: the splitmix64 finaliser (Steele, Lea, Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014).  Normals:
 * Box-Muller in binary32 on two 24-bit uniforms cut from one 64-bit draw,
 * pair k giving elements 2k (cos) and 2k+1 (sin).
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + 0x9E3779B97F4A7C15ULL) ^ (stream * 0xD1B54A32D192ED03ULL + 1));
}

static inline uint64_t draw(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

/* uniform 64-bit words: out[i] = word i of the stream */
void synth_u64(uint64_t key, uint64_t first, uint64_t n, uint64_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = draw(key, first + i);
}

static inline void normal_pair(uint64_t key, uint64_t k, float* c, float* s) {
  uint64_t a = draw(key, k);
  float u1 = (float)((a >> 40) + 1) * 0x1.0p-24f;          /* (0, 1] */
  float u2 = (float)((a >> 8) & 0xFFFFFFu) * 0x1.0p-24f;   /* [0, 1) */
  float r = sqrtf(-2.0f * logf(u1));
  float sn, cs;
  sincosf(6.28318530717958647692f * u2, &sn, &cs);
  *c = r * cs;
  *s = r * sn;
}

void synth_normal_f32(uint64_t key, uint64_t first, uint64_t n, float* out) {
  uint64_t i = 0;
  while (i < n) {
    uint64_t e = first + i;
    float c, s;
    normal_pair(key, e >> 1, &c, &s);
    if ((e & 1) == 0) {
      out[i++] = (float)c;
      if (i < n) out[i++] = (float)s;
    } else {
      out[i++] = (float)s;
    }
  }
}

/* fp32 -> OCP e4m3fn, round to nearest even, saturating to +-448 (the
 * largest finite e4m3 value); NaN maps to 0x7F. */
static inline uint8_t enc_e4m3(float xf) {
  uint32_t u;
  memcpy(&u, &xf, 4);
  uint8_t s = (uint8_t)((u >> 24) & 0x80u);
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7F;
  if (a >= 0x43E00000u) return s | 0x7E; /* |x| >= 448 */
  if (a < 0x3C800000u) {                  /* |x| < 2^-6: quantum 2^-9 */
    float f;
    memcpy(&f, &a, 4);
    float q = f * 512.0f; /* exact: scaling by a power of two */
    uint32_t i = (uint32_t)q;
    float frac = q - (float)i;
    if (frac > 0.5f || (frac == 0.5f && (i & 1u))) ++i;
    return s | (uint8_t)i; /* i == 8 is code 8 = 2^-6 */
  }
  uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20; /* keep 3 mantissa bits, RNE */
  int e = (int)(r >> 3) - 127 + 7;
  return s | (uint8_t)((e << 3) | (int)(r & 7u));
}

void synth_encode_e4m3(const float* x, uint64_t n, uint8_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = enc_e4m3(x[i]);
}

/* fp32 -> bfloat16, round to nearest even. */
void synth_encode_bf16(const float* x, uint64_t n, uint16_t* out) {
  for (uint64_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, &x[i], 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
      out[i] = (uint16_t)((u >> 16) | 0x40);
      continue;
    }
    u += 0x7FFFu + ((u >> 16) & 1u);
    out[i] = (uint16_t)(u >> 16);
  }
}

/* normals straight to e4m3 */
void synth_normal_e4m3(uint64_t key, uint64_t first, uint64_t n, uint8_t* out) {
  float buf[1024];
  uint64_t done = 0;
  while (done < n) {
    uint64_t m = n - done < 1024 ? n - done : 1024;
    synth_normal_f32(key, first + done, m, buf);
    synth_encode_e4m3(buf, m, out + done);
    done += m;
  }
}

/* nearest E2M1 code of a magnitude, ties to the even code:
 * magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 -> midpoints .25 .75 1.25 1.75 2.5 3.5 5 */
static inline uint8_t enc_e2m1_mag(double a) {
  if (a <= 0.25) return 0;
  if (a < 0.75) return 1;
  if (a <= 1.25) return 2;
  if (a < 1.75) return 3;
  if (a <= 2.5) return 4;
  if (a < 3.5) return 5;
  if (a <= 5.0) return 6;
  return 7;
}

static inline double dec_e4m3_local(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  double v = e == 0 ? (double)m * 0x1.0p-9 : (double)(8 + m) * (double)(1u << e) * 0x1.0p-10;
  return (c & 0x80) ? -v : v;
}

/* NVFP4 quantiser for `rows` rows of `dim` values: per 16-element group the
 * scale is e4m3(amax / (6 * g)); each value becomes the nearest E2M1 of
 * x / (scale * g), clamped to +-6.  g is the per-tensor scale (the dequant
 * multiplier).  data[rows][dim/2] (even element in the low nibble),
 * scales[rows][dim/16]. */
void synth_nvfp4_rows(const float* x, uint64_t rows, int dim, float g,
                      uint8_t* data, uint8_t* scales) {
  for (uint64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * (uint64_t)dim;
    uint8_t* dr = data + r * (uint64_t)(dim / 2);
    uint8_t* sr = scales + r * (uint64_t)(dim / 16);
    memset(dr, 0, (size_t)(dim / 2));
    for (int grp = 0; grp < dim / 16; ++grp) {
      double amax = 0.0;
      for (int i = 0; i < 16; ++i) {
        double a = fabs((double)xr[grp * 16 + i]);
        if (a > amax) amax = a;
      }
      uint8_t sc = enc_e4m3((float)(amax / (6.0 * (double)g)));
      sr[grp] = sc;
      double sv = dec_e4m3_local(sc) * (double)g;
      for (int i = 0; i < 16; ++i) {
        int el = grp * 16 + i;
        double v = sv > 0.0 ? (double)xr[el] / sv : 0.0;
        uint8_t code = enc_e2m1_mag(fabs(v));
        if (v < 0.0 && code) code |= 8;
        dr[el / 2] |= (uint8_t)((el & 1) ? (code << 4) : code);
      }
    }
  }
}

/* ---- whole cache blocks, generated and encoded in one pass -------------- */

/* K/V pool blocks [p0, p0+np) in e4m3: out[np][2][G][BS*D].  Element values
 * follow the logical order [p][kv][g][t][d] of the stream; plane kv = 1 (V)
 * is stored transposed, [d][t]. */
void synth_kv_fp8(uint64_t key, uint64_t p0, uint64_t np, int G, int BS, int D, uint8_t* out) {
  const uint64_t per = (uint64_t)BS * (uint64_t)D;
  float* buf = (float*)__builtin_alloca(sizeof(float) * per);
  for (uint64_t p = 0; p < np; ++p) {
    for (int kv = 0; kv < 2; ++kv) {
      for (int g = 0; g < G; ++g) {
        uint64_t plane = ((p0 + p) * 2 + (uint64_t)kv) * (uint64_t)G + (uint64_t)g;
        uint8_t* o = out + ((p * 2 + (uint64_t)kv) * (uint64_t)G + (uint64_t)g) * per;
        synth_normal_f32(key, plane * per, per, buf);
        if (kv == 0) {
          for (uint64_t i = 0; i < per; ++i) o[i] = enc_e4m3(buf[i]);
        } else {
          for (int t = 0; t < BS; ++t)
            for (int d = 0; d < D; ++d) o[(uint64_t)d * BS + t] = enc_e4m3(buf[(uint64_t)t * D + d]);
        }
      }
    }
  }
}

/* K/V pool blocks in NVFP4: data[np][2][G][BS*D/2], scales[np][2][G][BS*D/16].
 * Both K and V are quantised per token in groups of 16 along d; K is stored
 * [t][d/2] + [t][d/16], V transposed as [d][t/2] (even t in the low nibble)
 * + [d/16][t]. */
void synth_kv_nvfp4(uint64_t key, uint64_t p0, uint64_t np, int G, int BS, int D, float gs,
                    uint8_t* data, uint8_t* scales) {
  const uint64_t per = (uint64_t)BS * (uint64_t)D;
  float* buf = (float*)__builtin_alloca(sizeof(float) * per);
  uint8_t* td = (uint8_t*)__builtin_alloca(per / 2);
  uint8_t* ts = (uint8_t*)__builtin_alloca(per / 16);
  for (uint64_t p = 0; p < np; ++p) {
    for (int kv = 0; kv < 2; ++kv) {
      for (int g = 0; g < G; ++g) {
        uint64_t plane = ((p0 + p) * 2 + (uint64_t)kv) * (uint64_t)G + (uint64_t)g;
        uint64_t lp = (p * 2 + (uint64_t)kv) * (uint64_t)G + (uint64_t)g;
        uint8_t* od = data + lp * (per / 2);
        uint8_t* os = scales + lp * (per / 16);
        synth_normal_f32(key, plane * per, per, buf);
        if (kv == 0) {
          synth_nvfp4_rows(buf, (uint64_t)BS, D, gs, od, os);
        } else {
          synth_nvfp4_rows(buf, (uint64_t)BS, D, gs, td, ts);
          memset(od, 0, per / 2);
          for (int t = 0; t < BS; ++t) {
            for (int d = 0; d < D; ++d) {
              uint8_t b = td[(uint64_t)t * (D / 2) + d / 2];
              uint8_t c = (d & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
              od[(uint64_t)d * (BS / 2) + t / 2] |= (uint8_t)((t & 1) ? (c << 4) : c);
            }
            for (int gi = 0; gi < D / 16; ++gi)
              os[(uint64_t)gi * BS + t] = ts[(uint64_t)t * (D / 16) + gi];
          }
        }
      }
    }
  }
}

/* index-key pool blocks [p0, p0+np), rows [t][d]: dtype 2 = e4m3 (data
 * [np][BS][Di]), 3 = NVFP4 (data [np][BS][Di/2], scales [np][BS][Di/16]). */
void synth_ik(uint64_t key, uint64_t p0, uint64_t np, int BS, int Di, int dtype, float gs,
              uint8_t* data, uint8_t* scales) {
  const uint64_t per = (uint64_t)BS * (uint64_t)Di;
  float* buf = (float*)__builtin_alloca(sizeof(float) * per);
  for (uint64_t p = 0; p < np; ++p) {
    synth_normal_f32(key, (p0 + p) * per, per, buf);
    if (dtype == 2)
      synth_encode_e4m3(buf, per, data + p * per);
    else
      synth_nvfp4_rows(buf, (uint64_t)BS, Di, gs, data + p * (per / 2), scales + p * (per / 16));
  }
}

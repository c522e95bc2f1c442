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
 * Box-Muller on two 53-bit uniforms, pair k giving elements 2k (cos) and
 * 2k+1 (sin).
 */
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

static inline void normal_pair(uint64_t key, uint64_t k, double* c, double* s) {
  uint64_t a = draw(key, 2 * k), b = draw(key, 2 * k + 1);
  double u1 = (double)((a >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
  double u2 = (double)(b >> 11) * 0x1.0p-53;       /* [0, 1) */
  double r = sqrt(-2.0 * log(u1));
  double ang = 6.283185307179586476925 * u2;
  *c = r * cos(ang);
  *s = r * sin(ang);
}

void synth_normal_f32(uint64_t key, uint64_t first, uint64_t n, float* out) {
  uint64_t i = 0;
  while (i < n) {
    uint64_t e = first + i;
    double c, s;
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
  double x = (double)xf;
  if (isnan(x)) return 0x7F;
  uint8_t s = signbit(x) ? 0x80 : 0;
  double a = fabs(x);
  if (a >= 448.0) return s | 0x7E;
  if (a < 0x1.0p-6) { /* subnormal range, quantum 2^-9; 8 quanta = 2^-6 = code 8 */
    double q = nearbyint(a * 512.0);
    return s | (uint8_t)q;
  }
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int E = e - 1;
  double q = nearbyint(ldexp(a, -(E - 3))); /* 8..16 */
  if (q >= 16.0) {
    q = 8.0;
    E += 1;
  }
  int be = E + 7;
  if (be > 15 || (be == 15 && q > 14.0)) return s | 0x7E;
  return s | (uint8_t)(be << 3) | (uint8_t)((int)q - 8);
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

/* nearest E2M1 code of a magnitude in [0, 6], ties to the even code */
static inline uint8_t enc_e2m1_mag(double a) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  if (a >= 6.0) return 7;
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    double dc = fabs(a - mag[c]), db = fabs(a - mag[best]);
    if (dc < db || (dc == db && (c & 1) == 0)) best = c;
  }
  return (uint8_t)best;
}

static inline double dec_e4m3_local(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  double v = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
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

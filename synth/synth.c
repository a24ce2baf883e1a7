/*
 * Seeded synthetic inputs for the quantized MoE expert FFN.
 *
 * This module produces the workload both sides consume: Gaussian expert and
 * router weights, Gaussian activations and router logits, and the 4-bit
 * super-block encoding of the expert weights. It holds no step of the MoE
 * computation itself (no dequantization, no GEMV, no routing): the GPU library
 * and the CPU oracle each decode the encoded blocks with their own code.
 *
 * Random numbers: Philox4x32-10, the counter-based generator of Salmon,
 * Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
 * (SC 2011), keyed per stream; each 32-bit output becomes a uniform that is
 * mapped to a normal by the inverse normal CDF. Element i of a stream uses
 * counter block i/4, so any slice of any stream can be regenerated
 * independently.
 *
 * Encoding. The pages name the Q4_K super-block but print no bit layout, so
 * this canonical block is our reading of it: 144 bytes per 256 weights, made
 * of fp16 d, fp16 dmin, sixteen 6-bit fields packed LSB-first from byte 4
 * (eight sub-block scales sc_0..sc_7, then eight sub-block mins m_0..m_7) and
 * 128 bytes of 4-bit codes: sub-block j (32 weights) sits in bytes
 * 16+16j..31+16j, element 2i of the sub-block in the low nibble of byte i and
 * element 2i+1 in the high nibble. A weight decodes as d*sc_j*q - dmin*m_j.
 * The quantizer is plain round-to-nearest per sub-block (no search).
 *
 * MXFP4 encoding (the pages' FP4 expert weights with 32-value E8M0 scale
 * blocks): 17 bytes per 32 weights, one E8M0 scale byte e (2^(e-127)) then
 * 16 bytes of FP4 E2M1 codes, element 2i in the low nibble of byte 1+i. The
 * quantizer takes the shared exponent floor(log2(max|x|)) - 2 (2 is the
 * largest E2M1 exponent), kept to e in [2, 252] (so every nonzero weight is a
 * normal bf16 and fp32 number), and rounds x / 2^(e-127) to the nearest E2M1
 * value, ties to the even code, saturating at +-6. An all-zero block gets
 * e = 127 and zero codes.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <omp.h>

#define QK 256
#define QBLOCK_BYTES 144
#define MXK 32
#define MXBLOCK_BYTES 17

/* ---------------- Philox4x32-10 ---------------- */
static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
  const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  uint32_t n0 = hi1 ^ c[1] ^ k[0];
  uint32_t n1 = lo1;
  uint32_t n2 = hi0 ^ c[3] ^ k[1];
  uint32_t n3 = lo0;
  c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
  uint32_t k[2] = {key_in[0], key_in[1]};
  for (int r = 0; r < 10; ++r) {
    if (r) { k[0] += 0x9E3779B9u; k[1] += 0xBB67AE85u; }
    philox_round(c, k);
  }
  out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/* splitmix64 finaliser, used only to derive stream keys from small ids */
static inline uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t synth_key(int64_t a, int64_t b, int64_t c, int64_t d, int64_t e) {
  uint64_t h = mix64(0x5EED5EED00000000ull ^ (uint64_t)a);
  h = mix64(h ^ (uint64_t)b);
  h = mix64(h ^ (uint64_t)c);
  h = mix64(h ^ (uint64_t)d);
  h = mix64(h ^ (uint64_t)e);
  return h;
}

/* Standard normal quantile by P. J. Acklam's rational approximation of the
 * inverse normal CDF (relative error below 1.2e-9): a rational function of
 * (p - 1/2) in the central region, of sqrt(-2 log p) in the tails. */
static inline double normal_quantile(double p) {
  static const double a[6] = {-3.969683028665376e+01, 2.209460984245205e+02, -2.759285104469687e+02,
                              1.383577518672690e+02, -3.066479806614716e+01, 2.506628277459239e+00};
  static const double b[5] = {-5.447609879822406e+01, 1.615858368580409e+02, -1.556989798598866e+02,
                              6.680131188771972e+01, -1.328068155288572e+01};
  static const double c[6] = {-7.784894002430293e-03, -3.223964580411365e-01, -2.400758277161838e+00,
                              -2.549732539343734e+00, 4.374664141464968e+00, 2.938163982698783e+00};
  static const double d[4] = {7.784695709041462e-03, 3.224671290700398e-01, 2.445134137142996e+00,
                              3.754408661907416e+00};
  const double plow = 0.02425;
  if (p < plow) {
    double q = sqrt(-2.0 * log(p));
    return (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
           ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1.0);
  }
  if (p > 1.0 - plow) {
    double q = sqrt(-2.0 * log(1.0 - p));
    return -(((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
           ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1.0);
  }
  double q = p - 0.5, r = q * q;
  return (((((a[0] * r + a[1]) * r + a[2]) * r + a[3]) * r + a[4]) * r + a[5]) * q /
         (((((b[0] * r + b[1]) * r + b[2]) * r + b[3]) * r + b[4]) * r + 1.0);
}

/* four standard normals from counter block `blk` of stream `key` */
static inline void normals4(uint64_t key, uint64_t blk, float z[4]) {
  uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), 0x4E4F524Du, 0x414C5321u};
  uint32_t k[2] = {(uint32_t)key, (uint32_t)(key >> 32)};
  uint32_t r[4];
  synth_philox4x32_10(ctr, k, r);
  for (int j = 0; j < 4; ++j) {
    /* uniform strictly inside (0,1) on a 2^-32 grid offset by half a step */
    double u = ((double)r[j] + 0.5) * (1.0 / 4294967296.0);
    z[j] = (float)normal_quantile(u);
  }
}

/* out[i] = scale * N_i for i in [start, start+n) of stream key */
void synth_normal_f32(uint64_t key, uint64_t start, uint64_t n, float scale, float* out) {
  uint64_t i = 0;
  while (i < n) {
    uint64_t g = start + i;
    float z[4];
    normals4(key, g >> 2, z);
    for (uint64_t j = g & 3; j < 4 && i < n; ++j, ++i) out[i] = scale * z[j];
  }
}

/* ---------------- fp16 / bf16 rounding (input encoding only) ---------------- */
/* round-to-nearest-even double -> IEEE binary16 bits; finite inputs */
uint16_t synth_f64_to_f16(double v) {
  uint16_t sign = 0;
  if (v < 0 || (v == 0 && signbit(v))) { sign = 0x8000; v = -v; }
  if (v == 0) return sign;
  if (v >= 65520.0) return sign | 0x7C00;          /* rounds to infinity */
  int e;
  (void)frexp(v, &e);                              /* v = f * 2^e, f in [0.5,1) */
  int E = e - 1;                                   /* v in [2^E, 2^(E+1)) */
  if (E < -14) {                                   /* subnormal range: units of 2^-24 */
    double q = rint(ldexp(v, 24));
    return sign | (uint16_t)q;                     /* q == 1024 is the smallest normal */
  }
  double sig = rint(ldexp(v, 10 - E));             /* in [1024, 2048] */
  if (sig >= 2048.0) { sig = 1024.0; E += 1; }
  if (E + 15 >= 31) return sign | 0x7C00;
  return sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)sig - 1024);
}

static double f16_value(uint16_t h) {
  int ex = (h >> 10) & 31, mant = h & 1023;
  double v = ex ? ldexp(1024 + mant, ex - 25) : ldexp(mant, -24);
  return (h & 0x8000) ? -v : v;
}

void synth_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t b;
    memcpy(&b, &in[i], 4);
    uint32_t r = b + 0x7FFFu + ((b >> 16) & 1u);
    out[i] = (uint16_t)(r >> 16);
  }
}

/* ---------------- round-to-nearest 4-bit super-block quantizer ---------------- */
static inline int clampi(double v, int lo, int hi) {
  if (v < lo) return lo;
  if (v > hi) return hi;
  return (int)v;
}

/* encode one super-block of 256 weights into 144 bytes */
void synth_quantize_block(const float* x, uint8_t* blk) {
  double mn[8], s[8], smax = 0, mnmax = 0;
  for (int j = 0; j < 8; ++j) {
    double lo = 0.0, hi = -INFINITY;
    for (int i = 0; i < 32; ++i) {
      double v = x[32 * j + i];
      if (v < lo) lo = v;
      if (v > hi) hi = v;
    }
    mn[j] = lo;
    s[j] = (hi - lo) / 15.0;
    if (s[j] > smax) smax = s[j];
    if (-lo > mnmax) mnmax = -lo;
  }
  uint16_t dh = synth_f64_to_f16(smax / 63.0);
  uint16_t mh = synth_f64_to_f16(mnmax / 63.0);
  double d = f16_value(dh), dmin = f16_value(mh);
  int sc[8], m[8];
  for (int j = 0; j < 8; ++j) {
    sc[j] = d > 0 ? clampi(rint(s[j] / d), 0, 63) : 0;
    m[j] = dmin > 0 ? clampi(rint(-mn[j] / dmin), 0, 63) : 0;
  }
  memset(blk, 0, QBLOCK_BYTES);
  blk[0] = (uint8_t)dh; blk[1] = (uint8_t)(dh >> 8);
  blk[2] = (uint8_t)mh; blk[3] = (uint8_t)(mh >> 8);
  /* 16 six-bit fields, LSB-first, starting at byte 4 */
  for (int f = 0; f < 16; ++f) {
    int v = f < 8 ? sc[f] : m[f - 8];
    for (int b = 0; b < 6; ++b) {
      int bit = 6 * f + b;
      if ((v >> b) & 1) blk[4 + bit / 8] |= (uint8_t)(1u << (bit % 8));
    }
  }
  for (int j = 0; j < 8; ++j) {
    double step = d * sc[j];
    double off = dmin * m[j];
    for (int i = 0; i < 32; ++i) {
      int q = step > 0 ? clampi(rint((x[32 * j + i] + off) / step), 0, 15) : 0;
      uint8_t* p = &blk[16 + 16 * j + i / 2];
      *p |= (uint8_t)((i & 1) ? (q << 4) : q);
    }
  }
}

/* ---------------- round-to-nearest MXFP4 block quantizer ---------------- */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* encode one block of 32 weights into 17 bytes */
void synth_quantize_mx_block(const float* x, uint8_t* blk) {
  double amax = 0.0;
  for (int i = 0; i < MXK; ++i) {
    const double a = fabs((double)x[i]);
    if (a > amax) amax = a;
  }
  int e = 127;
  if (amax > 0.0) {
    e = (int)floor(log2(amax)) - 2 + 127;
    if (e < 2) e = 2;
    if (e > 252) e = 252;
  }
  const double scale = ldexp(1.0, e - 127);
  memset(blk, 0, MXBLOCK_BYTES);
  blk[0] = (uint8_t)e;
  for (int i = 0; i < MXK; ++i) {
    const double v = (double)x[i] / scale;
    const double a = fabs(v);
    int best = 0;
    for (int c = 1; c < 8; ++c) {
      const double dc = fabs(a - E2M1_MAG[c]), db = fabs(a - E2M1_MAG[best]);
      if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    const int code = best | ((v < 0.0 && best != 0) ? 8 : 0);
    blk[1 + i / 2] |= (uint8_t)((i & 1) ? (code << 4) : code);
  }
}

/* rows x cols float weights (cols % 32 == 0) -> rows x cols/32 MXFP4 blocks */
void synth_quantize_mx_rows(const float* w, int64_t rows, int64_t cols, uint8_t* out) {
  int64_t nb = cols / MXK;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b)
      synth_quantize_mx_block(w + r * cols + b * MXK, out + (r * nb + b) * MXBLOCK_BYTES);
}

/* Many matrices, as synth_q4k_matrices, encoded as MXFP4 blocks (the same
 * N(0, sigma) elements: element index r*cols + c of each stream). */
void synth_mx_matrices(const uint64_t* keys, int64_t nmat, int64_t rows, int64_t cols, float sigma,
                       uint8_t* out, int nthreads) {
  int64_t nb = cols / MXK;
  int64_t per = rows * nb * MXBLOCK_BYTES;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
  {
    float buf[MXK];
#pragma omp for schedule(static)
    for (int64_t t = 0; t < nmat * rows; ++t) {
      int64_t mi = t / rows, r = t % rows;
      for (int64_t b = 0; b < nb; ++b) {
        synth_normal_f32(keys[mi], (uint64_t)(r * cols + b * MXK), MXK, sigma, buf);
        synth_quantize_mx_block(buf, out + mi * per + (r * nb + b) * MXBLOCK_BYTES);
      }
    }
  }
}

/* rows x cols float weights (cols % 256 == 0) -> rows x cols/256 blocks */
void synth_quantize_rows(const float* w, int64_t rows, int64_t cols, uint8_t* out) {
  int64_t nb = cols / QK;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b)
      synth_quantize_block(w + r * cols + b * QK, out + (r * nb + b) * QBLOCK_BYTES);
}

/* Generate a rows x cols matrix N(0, sigma) from stream `key` (row-major
 * element index) and encode it; parallel over rows. */
void synth_q4k_matrix(uint64_t key, int64_t rows, int64_t cols, float sigma, uint8_t* out, int nthreads) {
  int64_t nb = cols / QK;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
  {
    float buf[QK];
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      for (int64_t b = 0; b < nb; ++b) {
        synth_normal_f32(key, (uint64_t)(r * cols + b * QK), QK, sigma, buf);
        synth_quantize_block(buf, out + (r * nb + b) * QBLOCK_BYTES);
      }
    }
  }
}

/* Many matrices at once: keys[n], all rows x cols, outputs contiguous
 * (matrix t at out + t*rows*(cols/256)*144). Parallel over (matrix, row). */
void synth_q4k_matrices(const uint64_t* keys, int64_t nmat, int64_t rows, int64_t cols, float sigma,
                        uint8_t* out, int nthreads) {
  int64_t nb = cols / QK;
  int64_t per = rows * nb * QBLOCK_BYTES;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
  {
    float buf[QK];
#pragma omp for schedule(static)
    for (int64_t t = 0; t < nmat * rows; ++t) {
      int64_t mi = t / rows, r = t % rows;
      for (int64_t b = 0; b < nb; ++b) {
        synth_normal_f32(keys[mi], (uint64_t)(r * cols + b * QK), QK, sigma, buf);
        synth_quantize_block(buf, out + mi * per + (r * nb + b) * QBLOCK_BYTES);
      }
    }
  }
}

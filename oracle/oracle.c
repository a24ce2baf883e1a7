/*
 * CPU oracle for the quantized MoE expert FFN -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library. The GPU path shares no code with it and never calls it.
 *
 * Everything is computed slowly and plainly in fp64, one definition at a time:
 *
 *  - fp16 / bf16 decoding and bf16 round-to-nearest-even;
 *  - dequantization of a 144-byte 4-bit super-block. The pages
 *    (sparkinfer README, opening paragraph and kernel table: Q4_K_M GGUF
 *    experts kept quantized and dequantized on read) name the format but print
 *    no bit layout; the canonical block read here is: fp16 d, fp16 dmin,
 *    sixteen 6-bit fields LSB-first from byte 4 (sub-block scales sc_0..sc_7
 *    then sub-block mins m_0..m_7), then 128 bytes of 4-bit codes with
 *    sub-block j in bytes 16+16j..31+16j and element 2i of a sub-block in the
 *    low nibble of byte i. Weight = d*sc_j*q - dmin*m_j, exact in fp64;
 *  - dequantization of a 17-byte MXFP4 block (the pages' FP4 expert
 *    weights with bf16 activations and inline dequant: sparkinfer CuTe-DSL
 *    README, "moe" paragraph; the 32-value E8M0 scale blocks: the same README,
 *    compressed-collective table and the paragraph after it). The canonical
 *    block read here: one E8M0 scale byte e (2^(e-127); 255 is NaN), then 16
 *    bytes of FP4 E2M1 codes, element 2i in the low nibble of byte 1+i. An
 *    E2M1 code is sign (bit 3), 2-bit exponent (bits 2-1, bias 1) and one
 *    mantissa bit (bit 0); exponent 0 is subnormal (0 or 1/2). Weight =
 *    E2M1(q) * 2^(e-127), exact in fp64;
 *  - the quantized GEMV y = Deq(W) x with fp64 accumulation, over either
 *    format (fmt 0: 4-bit super-blocks, fmt 1: MXFP4 blocks);
 *  - the router: logits = W_r x, exact top-k by a full stable sort on
 *    (logit descending, expert id ascending), and the softmax restricted to
 *    the selected experts (softmax over all experts then renormalised over
 *    the top-k, which is the same number);
 *  - the expert FFN y_e = D_e (act(G_e x, U_e x)) and the routing-weighted
 *    sum over the selected experts (the pages' fused MoE expert FFN: sparkinfer
 *    README kernel table; sparkinfer CuTe-DSL README, "moe" paragraph, for the
 *    gated form with top-k ids and weights as inputs). The same paragraph
 *    names SiLU, ReLU2 and SwiGLU-OAI activations without formulas; read
 *    here as act(g, u) = SiLU(g) u (the default), max(g, 0)^2 u (squared ReLU
 *    in place of SiLU), and the clamped SwiGLU variant published with that
 *    name: g' = min(g, 7), u' = min(max(u, -7), 7),
 *    act = g' / (1 + exp(-1.702 g')) * (u' + 1);
 *  - the residual add and RMSNorm between stacked layers (weight 1, eps given
 *    by the caller), rounded to bf16;
 *  - a recipe emulation of the expert FFN: the same FFN with the roundings of
 *    a GPU arithmetic recipe (fp32 accumulation; weights as exact codes with
 *    an fp32 sub-block affine, or rounded to bf16 / fp16 / bf16 hi + lo; the
 *    intermediate h stored as fp32 / bf16 / fp16 / bf16 hi + lo; activations
 *    as given or converted to fp16 toward zero), which predicts a recipe's
 *    error before its kernel exists. It is not the reference: every parity
 *    check compares against the fp64 functions above.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define QK 256
#define QBLOCK_BYTES 144
#define MXK 32
#define MXBLOCK_BYTES 17

/* ---------------------------------------------------------------- numbers */
double oracle_f16(uint16_t h) {
  int sign = h >> 15, ex = (h >> 10) & 31, mant = h & 1023;
  double v;
  if (ex == 0) v = ldexp((double)mant, -24);                 /* zero / subnormal */
  else if (ex == 31) v = mant ? NAN : INFINITY;
  else v = ldexp((double)(1024 + mant), ex - 25);            /* (1 + m/1024) 2^(ex-15) */
  return sign ? -v : v;
}

double oracle_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* nearest bf16 to a finite double, ties to even mantissa */
uint16_t oracle_round_bf16(double v) {
  if (v == 0) return signbit(v) ? 0x8000 : 0;
  uint16_t sign = v < 0 ? 0x8000 : 0;
  double a = fabs(v);
  int e;
  frexp(a, &e);
  int E = e - 1;                                  /* a in [2^E, 2^(E+1)) */
  if (E < -126) E = -126;                         /* subnormal spacing 2^-133 */
  double q = a / ldexp(1.0, E - 7);               /* units of the bf16 spacing */
  double r = floor(q);
  double frac = q - r;
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  double rv = r * ldexp(1.0, E - 7);
  /* rebuild bits from the rounded value */
  float f = (float)rv;                            /* exact: rv has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)(u >> 16);
}

/* ---------------------------------------------------------------- dequant */
static int field6(const uint8_t* blk, int f) {
  int v = 0;
  for (int b = 0; b < 6; ++b) {
    int bit = 6 * f + b;
    v |= ((blk[4 + bit / 8] >> (bit % 8)) & 1) << b;
  }
  return v;
}

/* the fields of one super-block: d, dmin, sub-block scales and mins, codes */
static void q4k_fields(const uint8_t* blk, double* d, double* dmin, int* sc, int* m, int* q) {
  *d = oracle_f16((uint16_t)(blk[0] | (blk[1] << 8)));
  *dmin = oracle_f16((uint16_t)(blk[2] | (blk[3] << 8)));
  for (int j = 0; j < 8; ++j) {
    sc[j] = field6(blk, j);
    m[j] = field6(blk, 8 + j);
    for (int i = 0; i < 32; ++i) {
      uint8_t byte = blk[16 + 16 * j + i / 2];
      q[32 * j + i] = (i & 1) ? (byte >> 4) : (byte & 15);
    }
  }
}

/* one super-block -> 256 weights */
void oracle_dequant_block(const uint8_t* blk, double* w) {
  double d, dmin;
  int sc[8], m[8], q[QK];
  q4k_fields(blk, &d, &dmin, sc, m, q);
  for (int i = 0; i < QK; ++i) w[i] = d * sc[i / 32] * q[i] - dmin * m[i / 32];
}

/* FP4 E2M1 code (low 4 bits) -> value */
double oracle_fp4(int32_t code) {
  const int sign = (code >> 3) & 1, ex = (code >> 1) & 3, man = code & 1;
  const double mag = ex == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, ex - 1);
  return sign ? -mag : mag;
}

/* E8M0 scale code -> 2^(e-127); 255 is NaN */
double oracle_e8m0(int32_t e) { return e == 255 ? NAN : ldexp(1.0, (e & 255) - 127); }

/* one MXFP4 block -> 32 weights */
void oracle_dequant_mx_block(const uint8_t* blk, double* w) {
  const double scale = oracle_e8m0(blk[0]);
  for (int i = 0; i < MXK; ++i) {
    const uint8_t byte = blk[1 + i / 2];
    w[i] = oracle_fp4((i & 1) ? (byte >> 4) : (byte & 15)) * scale;
  }
}

void oracle_dequant_matrix(const uint8_t* blocks, int64_t rows, int64_t cols, double* w) {
  int64_t nb = cols / QK;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b)
      oracle_dequant_block(blocks + (r * nb + b) * QBLOCK_BYTES, w + r * cols + b * QK);
}

void oracle_dequant_mx_matrix(const uint8_t* blocks, int64_t rows, int64_t cols, double* w) {
  int64_t nb = cols / MXK;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b)
      oracle_dequant_mx_block(blocks + (r * nb + b) * MXBLOCK_BYTES, w + r * cols + b * MXK);
}

/* y[r] = sum_c Deq(W)[r][c] * x[c], fp64; blocks [rows][cols/K][bytes] of
 * format fmt (0: 4-bit super-blocks of 256, 1: MXFP4 blocks of 32) */
void oracle_qgemv_fmt(const uint8_t* blocks, int64_t rows, int64_t cols, const double* x, double* y, int32_t fmt) {
  const int K = fmt == 1 ? MXK : QK;
  const int bytes = fmt == 1 ? MXBLOCK_BYTES : QBLOCK_BYTES;
  int64_t nb = cols / K;
  double w[QK];
  for (int64_t r = 0; r < rows; ++r) {
    double acc = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* blk = blocks + (r * nb + b) * bytes;
      if (fmt == 1) oracle_dequant_mx_block(blk, w);
      else oracle_dequant_block(blk, w);
      for (int i = 0; i < K; ++i) acc += w[i] * x[b * K + i];
    }
    y[r] = acc;
  }
}

void oracle_qgemv(const uint8_t* blocks, int64_t rows, int64_t cols, const double* x, double* y) {
  oracle_qgemv_fmt(blocks, rows, cols, x, y, 0);
}

/* ---------------------------------------------------------------- router */
void oracle_router_logits(const float* wr, int64_t E, int64_t H, const uint16_t* x_bf16, double* logits) {
  for (int64_t e = 0; e < E; ++e) {
    double acc = 0.0;
    for (int64_t i = 0; i < H; ++i) acc += (double)wr[e * H + i] * oracle_bf16(x_bf16[i]);
    logits[e] = acc;
  }
}

typedef struct { double l; int32_t id; } scored;

static int by_logit_desc_id_asc(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->l > y->l) return -1;
  if (x->l < y->l) return 1;
  return x->id < y->id ? -1 : (x->id > y->id);
}

/* the k largest logits, descending; equal logits -> lower id first */
void oracle_topk(const double* logits, int64_t E, int64_t k, int32_t* ids) {
  scored* s = (scored*)malloc(sizeof(scored) * (size_t)E);
  for (int64_t e = 0; e < E; ++e) { s[e].l = logits[e]; s[e].id = (int32_t)e; }
  qsort(s, (size_t)E, sizeof(scored), by_logit_desc_id_asc);
  for (int64_t i = 0; i < k; ++i) ids[i] = s[i].id;
  free(s);
}

/* softmax over the selected logits (= full softmax renormalised over top-k) */
void oracle_route_weights(const double* logits, const int32_t* ids, int64_t k, double* w) {
  double mx = -INFINITY;
  for (int64_t s = 0; s < k; ++s) if (logits[ids[s]] > mx) mx = logits[ids[s]];
  double den = 0.0;
  for (int64_t s = 0; s < k; ++s) den += exp(logits[ids[s]] - mx);
  for (int64_t s = 0; s < k; ++s) w[s] = exp(logits[ids[s]] - mx) / den;
}

/* ---------------------------------------------------------------- FFN */
double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* Gate activation h = act(g, u): 0 SiLU, 1 squared ReLU, 2 clamped SwiGLU
 * (readings in the header comment). */
double oracle_act(double g, double u, int32_t act) {
  if (act == 1) {
    const double r = g > 0.0 ? g : 0.0;
    return r * r * u;
  }
  if (act == 2) {
    const double gc = g < 7.0 ? g : 7.0;
    const double uc = u < -7.0 ? -7.0 : (u > 7.0 ? 7.0 : u);
    return gc / (1.0 + exp(-1.702 * gc)) * (uc + 1.0);
  }
  return oracle_silu(g) * u;
}

/* y = D act(G x, U x); G, U: [I x H] blocks, D: [H x I] blocks of format fmt */
void oracle_expert_ffn_fmt(const uint8_t* gate, const uint8_t* up, const uint8_t* down,
                           int64_t H, int64_t I, const double* x, double* y, double* h_out, int32_t act,
                           int32_t fmt) {
  double* g = (double*)malloc(sizeof(double) * (size_t)I);
  double* u = (double*)malloc(sizeof(double) * (size_t)I);
  oracle_qgemv_fmt(gate, I, H, x, g, fmt);
  oracle_qgemv_fmt(up, I, H, x, u, fmt);
  for (int64_t i = 0; i < I; ++i) g[i] = oracle_act(g[i], u[i], act);
  if (h_out) memcpy(h_out, g, sizeof(double) * (size_t)I);
  oracle_qgemv_fmt(down, H, I, g, y, fmt);
  free(g);
  free(u);
}

void oracle_expert_ffn_act(const uint8_t* gate, const uint8_t* up, const uint8_t* down,
                           int64_t H, int64_t I, const double* x, double* y, double* h_out, int32_t act) {
  oracle_expert_ffn_fmt(gate, up, down, H, I, x, y, h_out, act, 0);
}

void oracle_expert_ffn(const uint8_t* gate, const uint8_t* up, const uint8_t* down,
                       int64_t H, int64_t I, const double* x, double* y, double* h_out) {
  oracle_expert_ffn_act(gate, up, down, H, I, x, y, h_out, 0);
}

/* One token through one MoE layer given its selected experts' blocks.
 * gate/up/down: arrays of k pointers (expert of slot s); w: k routing weights. */
void oracle_moe_token_fmt(const uint8_t* const* gate, const uint8_t* const* up, const uint8_t* const* down,
                          const double* w, int64_t k, int64_t H, int64_t I, const uint16_t* x_bf16,
                          double* y, int32_t act, int32_t fmt) {
  double* x = (double*)malloc(sizeof(double) * (size_t)H);
  double* ys = (double*)malloc(sizeof(double) * (size_t)H);
  for (int64_t i = 0; i < H; ++i) { x[i] = oracle_bf16(x_bf16[i]); y[i] = 0.0; }
  for (int64_t s = 0; s < k; ++s) {
    oracle_expert_ffn_fmt(gate[s], up[s], down[s], H, I, x, ys, NULL, act, fmt);
    for (int64_t i = 0; i < H; ++i) y[i] += w[s] * ys[i];
  }
  free(x);
  free(ys);
}

void oracle_moe_token_act(const uint8_t* const* gate, const uint8_t* const* up, const uint8_t* const* down,
                          const double* w, int64_t k, int64_t H, int64_t I, const uint16_t* x_bf16,
                          double* y, int32_t act) {
  oracle_moe_token_fmt(gate, up, down, w, k, H, I, x_bf16, y, act, 0);
}

void oracle_moe_token(const uint8_t* const* gate, const uint8_t* const* up, const uint8_t* const* down,
                      const double* w, int64_t k, int64_t H, int64_t I, const uint16_t* x_bf16,
                      double* y) {
  oracle_moe_token_act(gate, up, down, w, k, H, I, x_bf16, y, 0);
}

/* ---------------------------------------------------------------- stack */
/* r = v / sqrt(mean(v^2) + eps), v = x + y; returned in fp64 and as bf16 */
void oracle_resid_rmsnorm(const uint16_t* x_bf16, const double* y, int64_t n, double eps,
                          double* r, uint16_t* r_bf16) {
  double ss = 0.0;
  double* v = (double*)malloc(sizeof(double) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) { v[i] = oracle_bf16(x_bf16[i]) + y[i]; ss += v[i] * v[i]; }
  double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) {
    double ri = v[i] * inv;
    if (r) r[i] = ri;
    if (r_bf16) r_bf16[i] = oracle_round_bf16(ri);
  }
  free(v);
}

/* ---------------------------------------------------------------- recipe emulation
 * The expert FFN and the routing-weighted sum again, with the roundings of a
 * GPU arithmetic recipe, so that a recipe's error can be predicted before its
 * kernel is written. Every sum is an fp32 sum in the order of the formula
 * (the GPU's order differs; the size of the error is what is predicted), and
 * every product-add is one fused fp32 operation, as on the GPU.
 *   wmode  0: exact codes with an fp32 sub-block affine: for 4-bit
 *             super-blocks, per 32-weight sub-block P = sum q*x and
 *             S = sum x, then acc += a*P - b*S (a = d*sc, b = dmin*m, both
 *             exact in fp32); MXFP4 weights are exact in fp32 and enter as
 *             they are;
 *          1: each weight rounded to bf16 (nearest even);
 *          2: each weight rounded to fp16 (nearest even);
 *          3: each weight as bf16 hi + lo (hi = bf16(w), lo = bf16(w - hi)).
 *   hmode  0: h stored in fp32; 1: bf16; 2: fp16 (nearest even, overflow to
 *          infinity); 3: bf16 hi + lo; 4: FP8 E4M3 hi + lo with one
 *          power-of-two scale per 32 consecutive values and plane (below).
 *   xmode  0: the bf16 activations as they are; 1: converted to fp16 toward
 *          zero (saturating at 65504), as a round-toward-zero conversion does;
 *          2: FP8 E4M3 hi + lo with per-32 scales (below).
 * FP8 hi + lo (the operand form of a block-scaled FP8 x FP4 matrix product
 * with two passes over the activations): per block of 32 values v, the hi
 * plane's scale is the smallest power of two s with max|v| / s <= 448 (the
 * largest E4M3 value, so nothing saturates), hi = E4M3(v / s) * s; the lo
 * plane does the same for the residual r = v - hi; the operand is hi + lo.
 */
/* nearest value (ties to even), or toward zero, with p significant bits and
 * smallest normal exponent emin (below it the spacing stays 2^(emin-p+1)) */
static double round_sig(double v, int p, int emin, int toward_zero) {
  if (v == 0.0 || !isfinite(v)) return v;
  double a = fabs(v);
  int e;
  frexp(a, &e);
  int E = e - 1;                                  /* a in [2^E, 2^(E+1)) */
  if (E < emin) E = emin;
  double unit = ldexp(1.0, E - (p - 1));
  double qv = a / unit;
  double r = floor(qv);
  if (!toward_zero) {
    double frac = qv - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  }
  double out = r * unit;
  return v < 0 ? -out : out;
}

double oracle_emul_bf16(double v) { return round_sig(v, 8, -126, 0); }

double oracle_emul_fp16(double v) {
  double r = round_sig(v, 11, -14, 0);
  return fabs(r) > 65504.0 ? copysign(INFINITY, v) : r;
}

/* FP8 E4M3 (4 significant bits, smallest normal 2^-6, largest 448),
 * nearest even; values beyond 448 saturate */
double oracle_emul_e4m3(double v) {
  double r = round_sig(v, 4, -6, 0);
  return fabs(r) > 448.0 ? copysign(448.0, v) : r;
}

/* v[0..n) in place as FP8 hi + lo operands, blocks of 32 (n a multiple of 32) */
static double pow2_scale(double amax) {
  if (!(amax > 0.0)) return 1.0;
  double s = ldexp(1.0, (int)ceil(log2(amax / 448.0)));
  while (amax / s > 448.0) s *= 2.0;                   /* guard the log2 rounding */
  while (s > 0.0 && amax / (s / 2.0) <= 448.0) s /= 2.0;
  return s;
}
void oracle_emul_fp8_hilo(float* v, int64_t n) {
  for (int64_t b = 0; b < n; b += 32) {
    double amax = 0.0, rmax = 0.0, hi[32], r[32];
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)v[b + i]));
    const double sh = pow2_scale(amax);
    for (int i = 0; i < 32; ++i) {
      hi[i] = oracle_emul_e4m3((double)v[b + i] / sh) * sh;
      r[i] = (double)v[b + i] - hi[i];
      rmax = fmax(rmax, fabs(r[i]));
    }
    const double sl = pow2_scale(rmax);
    for (int i = 0; i < 32; ++i) v[b + i] = (float)(hi[i] + oracle_emul_e4m3(r[i] / sl) * sl);
  }
}

double oracle_emul_fp16_rtz(double v) {
  double r = round_sig(v, 11, -14, 1);
  return fabs(r) > 65504.0 ? copysign(65504.0, v) : r;
}

/* y = Deq(W) x under weight mode wmode, fp32 accumulation; x already in the
 * form the recipe feeds (fp32 values) */
static void emul_qgemv(const uint8_t* blocks, int64_t rows, int64_t cols, const float* x, float* y, int32_t fmt,
                       int32_t wmode) {
  const int K = fmt == 1 ? MXK : QK;
  const int bytes = fmt == 1 ? MXBLOCK_BYTES : QBLOCK_BYTES;
  const int64_t nb = cols / K;
  double w[QK], d, dmin;
  int sc[8], m[8], q[QK];
  for (int64_t r = 0; r < rows; ++r) {
    float acc = 0.0f;
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* blk = blocks + (r * nb + b) * bytes;
      const float* xb = x + b * K;
      if (wmode == 0 && fmt == 0) {
        q4k_fields(blk, &d, &dmin, sc, m, q);
        for (int j = 0; j < 8; ++j) {
          float P = 0.0f, S = 0.0f;
          for (int i = 0; i < 32; ++i) {
            P = fmaf((float)q[32 * j + i], xb[32 * j + i], P);
            S += xb[32 * j + i];
          }
          const float a = (float)(d * sc[j]), bb = (float)(dmin * m[j]);
          acc = fmaf(a, P, acc);
          acc = fmaf(-bb, S, acc);
        }
        continue;
      }
      if (fmt == 1) oracle_dequant_mx_block(blk, w);
      else oracle_dequant_block(blk, w);
      for (int i = 0; i < K; ++i) {
        if (wmode == 0) {
          acc = fmaf((float)w[i], xb[i], acc);                  /* MXFP4: exact in fp32 */
        } else if (wmode == 1) {
          acc = fmaf((float)oracle_emul_bf16(w[i]), xb[i], acc);
        } else if (wmode == 2) {
          acc = fmaf((float)oracle_emul_fp16(w[i]), xb[i], acc);
        } else {
          const double hi = oracle_emul_bf16(w[i]);
          const double lo = oracle_emul_bf16(w[i] - hi);
          acc = fmaf((float)hi, xb[i], acc);
          acc = fmaf((float)lo, xb[i], acc);
        }
      }
    }
    y[r] = acc;
  }
}

/* stored form of one h value under hmode (hi + lo is exact in fp32) */
static float emul_store_h(float h, int32_t hmode) {
  if (hmode == 1) return (float)oracle_emul_bf16(h);
  if (hmode == 2) return (float)oracle_emul_fp16(h);
  if (hmode == 3) {
    const double hi = oracle_emul_bf16(h);
    return (float)(hi + oracle_emul_bf16((double)h - hi));
  }
  return h;
}

/* One token through its k selected experts under the recipe; y (fp64 out)
 * holds the fp32 result. w: the k routing weights (used as fp32). */
void oracle_emul_moe_token(const uint8_t* const* gate, const uint8_t* const* up, const uint8_t* const* down,
                           const double* w, int64_t k, int64_t H, int64_t I, const uint16_t* x_bf16, double* y,
                           int32_t act, int32_t fmt, int32_t wmode, int32_t hmode, int32_t xmode) {
  float* x = (float*)malloc(sizeof(float) * (size_t)H);
  float* g = (float*)malloc(sizeof(float) * (size_t)I);
  float* u = (float*)malloc(sizeof(float) * (size_t)I);
  float* ye = (float*)malloc(sizeof(float) * (size_t)H);
  float* acc = (float*)malloc(sizeof(float) * (size_t)H);
  for (int64_t i = 0; i < H; ++i) {
    const double xv = oracle_bf16(x_bf16[i]);
    x[i] = (float)(xmode == 1 ? oracle_emul_fp16_rtz(xv) : xv);
    acc[i] = 0.0f;
  }
  if (xmode == 2) oracle_emul_fp8_hilo(x, H);
  for (int64_t s = 0; s < k; ++s) {
    emul_qgemv(gate[s], I, H, x, g, fmt, wmode);
    emul_qgemv(up[s], I, H, x, u, fmt, wmode);
    for (int64_t i = 0; i < I; ++i) g[i] = emul_store_h((float)oracle_act(g[i], u[i], act), hmode);
    if (hmode == 4) oracle_emul_fp8_hilo(g, I);
    emul_qgemv(down[s], H, I, g, ye, fmt, wmode);
    for (int64_t i = 0; i < H; ++i) acc[i] = fmaf((float)w[s], ye[i], acc[i]);
  }
  for (int64_t i = 0; i < H; ++i) y[i] = acc[i];
  free(x);
  free(g);
  free(u);
  free(ye);
  free(acc);
}

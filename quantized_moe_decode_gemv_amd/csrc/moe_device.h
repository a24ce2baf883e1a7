// Device helpers shared by the per-token and expert-major GEMV kernels:
// vector loads, dot products of 4-bit codes against bf16 / fp16 operands,
// super-block header decoding and DPP lane sums (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace qmoe {

typedef unsigned int u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr int BLOCK = 256;

__device__ __forceinline__ u32x4 load_nt(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ float dot2_bf16(u32 a, u32 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_f16(u32 a, u32 b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c, false);
}

__device__ __forceinline__ float half_bits_to_float(u32 bits) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)bits);
}

__device__ __forceinline__ float bf16_bits_to_float(u32 bits) { return __builtin_bit_cast(float, bits << 16); }

// Reinterpret a 32-bit value as fp32. Takes the value (not a vector element
// lvalue) so the cast always sees the intended component.
__device__ __forceinline__ float as_f32(u32 v) { return __builtin_bit_cast(float, v); }

// Nearest-even bf16 of a finite fp32.
__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
  u32 b = __builtin_bit_cast(u32, f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// Cross-lane move by a DPP pattern (all lanes of the wave active).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float read_lane(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Sum over groups of W adjacent lanes (W a power of two <= 64); every lane of
// a group ends with the same value, the group's sum. Within a row of 16
// lanes: quad swaps (lane ^ 1, lane ^ 2), then the half-row and row mirrors,
// each pairing a lane with one holding the other half's partial sum (a + b
// and b + a are the same float, so all lanes agree); the four row sums are
// then combined through scalar reads of lanes 0, 16, 32, 48. DPP moves stay
// in the VALU instead of the LDS crossbar. Must be called with the whole
// wave active.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if (W >= 2) v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
  if (W >= 4) v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  if (W >= 8) v += dpp_mov<0x141>(v);   // row_half_mirror
  if (W >= 16) v += dpp_mov<0x140>(v);  // row_mirror
  if (W >= 32) {
    const float r0 = read_lane(v, 0), r1 = read_lane(v, 16), r2 = read_lane(v, 32), r3 = read_lane(v, 48);
    if (W == 32) v = (threadIdx.x & (WAVE - 1)) < 32 ? r0 + r1 : r2 + r3;
    else v = (r0 + r1) + (r2 + r3);
  }
  return v;
}

// Sub-block affine of sub-block jj (0..7) of a super-block header:
// weight = a*q - b. Header dword 0 holds d and dmin (fp16); dwords 1..3 hold
// the 6-bit scales at bit 6*jj and the 6-bit mins at bit 48 + 6*jj of their
// 96 bits, read here with one 64-bit shift each.
struct Affine { float a, b; };
__device__ __forceinline__ Affine header_affine(const u32x4& h, int jj) {
  const float d = half_bits_to_float(h.x & 0xFFFFu);
  const float dmin = half_bits_to_float(h.x >> 16);
  const unsigned long long lo = (unsigned long long)h.y | ((unsigned long long)h.z << 32);
  const unsigned long long hi = (unsigned long long)h.z | ((unsigned long long)h.w << 32);
  const u32 sc = (u32)(lo >> (6 * jj)) & 63u;
  const u32 m = (u32)(hi >> (16 + 6 * jj)) & 63u;
  return {d * (float)sc, dmin * (float)m};   // both products exact in fp32
}

// The 8 codes of code dword v (nibble i = element 8d + i of the sub-block)
// as four 16-bit pairs with high byte K: P[c] = (K<<8 | q_c, K<<8 | q_{c+4}).
// With K = 0x43 each half is the bf16 value 128 + q, with K = 0x64 the fp16
// value 1024 + q, both exact. One byte permute per pair.
__device__ __forceinline__ void code_pairs(u32 v, u32 K4, u32* P) {
  const u32 lo = v & 0x0F0F0F0Fu;          // bytes: q0 q2 q4 q6
  const u32 hi = (v >> 4) & 0x0F0F0F0Fu;   // bytes: q1 q3 q5 q7
  P[0] = __builtin_amdgcn_perm(K4, lo, 0x04020400u);   // (q0, q4)
  P[1] = __builtin_amdgcn_perm(K4, hi, 0x04020400u);   // (q1, q5)
  P[2] = __builtin_amdgcn_perm(K4, lo, 0x04030401u);   // (q2, q6)
  P[3] = __builtin_amdgcn_perm(K4, hi, 0x04030401u);   // (q3, q7)
}

// sum_i (128 + q_i) * x_i over one 32-code sub-block, two codes per dot2.
// X[4d+c] holds the bf16 pair (x[8d+c], x[8d+c+4]) (see load_x_pairs).
__device__ __forceinline__ float dot_codes_bf16(const u32x4& c, const u32* X) {
  const u32 w[4] = {c.x, c.y, c.z, c.w};
  float a = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    u32 P[4];
    code_pairs(w[d], 0x43434343u, P);
#pragma unroll
    for (int q = 0; q < 4; ++q) a = dot2_bf16(P[q], X[4 * d + q], a);
  }
  return a;
}

// The 32 bf16 activations of one sub-block: four 16-byte loads.
__device__ __forceinline__ void load_x_raw(const uint16_t* xs, u32x4* r) {
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = load16(xs + 8 * q);   // elements 8q .. 8q+7
}

// The loaded activations in the pair order of dot_codes_bf16: X[4d+c] =
// (x[8d+c], x[8d+c+4]), c = 0..3. Returns sum(x), taken with
// v_dot2_f32_bf16 against (1, 1).
__device__ __forceinline__ float x_pairs(const u32x4* r, u32* X) {
  const u32 ONES = 0x3F803F80u;           // bf16 (1, 1)
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    X[4 * q + 0] = __builtin_amdgcn_perm(r[q].z, r[q].x, 0x05040100u);   // (8q, 8q+4)
    X[4 * q + 1] = __builtin_amdgcn_perm(r[q].z, r[q].x, 0x07060302u);   // (8q+1, 8q+5)
    X[4 * q + 2] = __builtin_amdgcn_perm(r[q].w, r[q].y, 0x05040100u);   // (8q+2, 8q+6)
    X[4 * q + 3] = __builtin_amdgcn_perm(r[q].w, r[q].y, 0x07060302u);   // (8q+3, 8q+7)
    s = dot2_bf16(r[q].x, ONES, s); s = dot2_bf16(r[q].y, ONES, s);
    s = dot2_bf16(r[q].z, ONES, s); s = dot2_bf16(r[q].w, ONES, s);
  }
  return s;
}

__device__ __forceinline__ float load_x_pairs(const uint16_t* xs, u32* X) {
  u32x4 r[4];
  load_x_raw(xs, r);
  return x_pairs(r, X);
}

// Gate activation h = act(g, u): 0 SiLU(g) * u, 1 max(g, 0)^2 * u, 2 the
// clamped SwiGLU g' * sigmoid(1.702 g') * (u' + 1), g' = min(g, 7),
// u' = clamp(u, -7, 7). act is uniform over the launch.
__device__ __forceinline__ float gate_act(float g, float u, int act) {
  if (act == 1) {
    const float r = fmaxf(g, 0.f);
    return r * r * u;
  }
  if (act == 2) {
    const float gc = fminf(g, 7.0f), uc = fminf(fmaxf(u, -7.0f), 7.0f);
    return gc / (1.0f + expf(-1.702f * gc)) * (uc + 1.0f);
  }
  return g / (1.0f + expf(-g)) * u;
}

// Exact conversion of 4-bit codes: a byte 0x0q read as an FP8 E4M3 number is
// q * 2^-9 (a subnormal m 2^-9 for q = m < 8, (8 + m) 2^-9 for q = 8 + m), so
// gfx950's scaled FP8 conversion with scale 2^9 yields q exactly (checked on
// the device for all 16 codes). One instruction turns two codes (one 16-bit
// word of masked nibbles) into two fp32 or bf16 values.
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <bool HIGH_WORD>
__device__ __forceinline__ f32x2 codes2_f32(u32 nibble_bytes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(nibble_bytes, 512.0f, HIGH_WORD);
}

// sum_i q_i * h_i over one 32-code sub-block with fp32 h (h[i] = element i
// of the sub-block): the codes are converted exactly, products and sums are
// fused fp32 operations; two accumulators halve the dependent chain.
__device__ __forceinline__ float dot_codes_f32(const u32x4& c, const float* h) {
  const u32 w[4] = {c.x, c.y, c.z, c.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const u32 lo = w[d] & 0x0F0F0F0Fu, hi = (w[d] >> 4) & 0x0F0F0F0Fu;   // elements 8d + (0,2,4,6) / (1,3,5,7)
    const f32x2 q02 = codes2_f32<false>(lo), q46 = codes2_f32<true>(lo);
    const f32x2 q13 = codes2_f32<false>(hi), q57 = codes2_f32<true>(hi);
    const float* hd = h + 8 * d;
    a0 = fmaf(q02.x, hd[0], a0); a0 = fmaf(q02.y, hd[2], a0); a0 = fmaf(q46.x, hd[4], a0); a0 = fmaf(q46.y, hd[6], a0);
    a1 = fmaf(q13.x, hd[1], a1); a1 = fmaf(q13.y, hd[3], a1); a1 = fmaf(q57.x, hd[5], a1); a1 = fmaf(q57.y, hd[7], a1);
  }
  return a0 + a1;
}

// ---------------------------------------------------------------- MXFP4
// gfx950 converts one byte of FP4 E2M1 codes (low nibble first) to a bf16
// (or fp32) pair, times a power of two taken from the exponent of an fp32
// operand; with 1.0 the pair holds the exact E2M1 values.
__device__ __forceinline__ void fp4_pairs_bf16(u32 v, u32* P) {
  P[0] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 0));
  P[1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 1));
  P[2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 2));
  P[3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 3));
}

// sum_i E2M1(q_i) * x_i over one 32-code block; X[i] holds the bf16 pair
// (x[2i], x[2i+1]) (the natural order of bf16 words). Products are exact in
// fp32 (2 + 8 significant bits).
__device__ __forceinline__ float dot_fp4_bf16(const u32x4& c, const u32* X) {
  const u32 w[4] = {c.x, c.y, c.z, c.w};
  float a = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    u32 P[4];
    fp4_pairs_bf16(w[d], P);
#pragma unroll
    for (int q = 0; q < 4; ++q) a = dot2_bf16(P[q], X[4 * d + q], a);
  }
  return a;
}

// sum_i E2M1(q_i) * h_i over one 32-code block with fp32 h: each byte of
// codes becomes two exact fp32 values (v_cvt_scalef32_pk_f32_fp4, low nibble
// first, scale 1), then fused fp32 products and sums.
__device__ __forceinline__ float dot_fp4_f32(const u32x4& c, const float* h) {
  const u32 w[4] = {c.x, c.y, c.z, c.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f32x2 v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 0),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 1),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 2),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 3)};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      a0 = fmaf(v[b].x, h[8 * d + 2 * b], a0);
      a1 = fmaf(v[b].y, h[8 * d + 2 * b + 1], a1);
    }
  }
  return a0 + a1;
}

// E8M0 scale code e in [1, 254] -> 2^(e-127) as fp32 (exact; the packer
// rejects 0 and 255).
__device__ __forceinline__ float e8m0_scale(u32 e) { return __builtin_bit_cast(float, e << 23); }

}  // namespace qmoe

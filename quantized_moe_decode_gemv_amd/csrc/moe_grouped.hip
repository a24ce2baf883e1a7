// gfx950 kernels of the batched path: grouped expert GEMMs on the MFMA
// units for token batches routed to the same expert.
//
// The pages' batched prefill dequantizes 4-bit weights into the GEMM operand
// and shares one weight read across a chunk of tokens (SP⚡RKINFER README,
// Qwen3.8-27B prefill notes; sparkinfer-k3 release log, batched prompt
// ingestion); this is our CDNA4 form of it. Tokens are grouped by expert on
// the device (dispatch lists); a workgroup takes a (expert, 64-pair tile,
// feature block) and runs v_mfma_f32_16x16x32_f16 with
//   A = activations in fp16 (bf16 inputs are exact in fp16 above 2^-14),
//   B = q * sc, the 4-bit code times its 6-bit sub-block scale (<= 945,
//       exact in fp16), built with the exact fp16 identity 0x6400|q = 1024+q,
// accumulated over one 256-weight super-block, then scaled by the block's d.
// The min term sum_j dmin*m_j*sum_{i in j} x_i is one more MFMA per
// super-block with A = the sub-block sums split into fp16 hi + lo parts and
// B = m_j, scaled by dmin. Activations are staged in LDS with each group of 8
// stored in the order the code nibbles are unpacked (0,4,1,5,2,6,3,7), two
// super-blocks in flight (LDS double buffer, next weights in registers).
// h = SiLU(gate) * up is kept in fp16 between the two GEMMs; the down GEMM
// writes one fp32 row per (token, slot) pair and the routing-weighted combine
// sums them in slot order (deterministic).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace qmoe {
namespace grouped {

typedef unsigned int u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int BLOCK = 256;
constexpr int MT = 64;       // pairs per tile
constexpr int XS = 256 + 8;  // LDS row stride (halfs) of a staged 256-wide K slice

__device__ __forceinline__ float bf16_to_f32(u32 bits) { return __builtin_bit_cast(float, bits << 16); }
__device__ __forceinline__ float half_bits(u32 b) { return (float)__builtin_bit_cast(_Float16, (unsigned short)b); }

__device__ __forceinline__ u32 field6(const u32x4& h, int p) {
  const int idx = p >> 5, sh = p & 31;
  const u32 lo = idx == 0 ? h.y : (idx == 1 ? h.z : h.w);
  const u32 hi = idx == 0 ? h.z : (idx == 1 ? h.w : 0u);
  return __builtin_amdgcn_alignbit(hi, lo, sh) & 63u;
}

// tile -> (expert, first pair in the expert's group); -1 if past the last tile
__device__ __forceinline__ int find_tile(const int32_t* __restrict__ tile_off, int E, int tile, int* m0) {
  if (tile >= tile_off[E]) return -1;
  int lo = 0, hi = E;            // tile_off[lo] <= tile < tile_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= tile) lo = mid; else hi = mid;
  }
  *m0 = (tile - tile_off[lo]) * MT;
  return lo;
}

// B fragment of one sub-block for this lane: its 8 codes (4 bytes) times the
// sub-block scale, as fp16, in nibble-unpack order (0,4,1,5,2,6,3,7).
// 0x6400|q is 1024+q exactly; subtracting 1024 and multiplying by sc <= 63
// stay exact (q*sc <= 945).
__device__ __forceinline__ half8 codes_times_scale(u32 c4, u32 sc) {
  const u32 M = 0x000F000Fu, B = 0x64006400u;
  const half2 bias = {(_Float16)1024.0f, (_Float16)1024.0f};
  const half2 s2 = {(_Float16)(float)sc, (_Float16)(float)sc};
  half8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32 p = ((c4 >> (4 * i)) & M) | B;
    const half2 v = (__builtin_bit_cast(half2, p) - bias) * s2;
    r[2 * i] = v[0];
    r[2 * i + 1] = v[1];
  }
  return r;
}

// Activation slice staging: thread -> (row i = tid/4, 64 columns).
// Loaded values are held in registers between the load and the LDS write so
// the next slice's loads overlap the current slice's MFMAs.
struct StageRegs {
  u32x4 v[8];
};

template <bool SRC_BF16>
__device__ __forceinline__ void stage_load(const void* __restrict__ src, const int* __restrict__ row_index, int rows,
                                           int ld, int k0, StageRegs& r) {
  const int tid = threadIdx.x;
  const int i = tid >> 2, q = tid & 3;
  const bool ok = i < rows;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    r.v[c] = u32x4{0u, 0u, 0u, 0u};
    if (ok) {
      const size_t off = (size_t)row_index[i] * ld + k0 + 64 * q + 8 * c;
      r.v[c] = SRC_BF16 ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + off)
                        : *reinterpret_cast<const u32x4*>(static_cast<const _Float16*>(src) + off);
    }
  }
}

// Write the staged slice as fp16 in nibble order and the per-row sub-block
// sums (fp16 hi + lo) of sub-blocks 2q, 2q+1.
template <bool SRC_BF16>
__device__ __forceinline__ void stage_store(const StageRegs& r, _Float16* xs, _Float16* shi, _Float16* slo) {
  const int tid = threadIdx.x;
  const int i = tid >> 2, q = tid & 3;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const u32 w[4] = {r.v[c].x, r.v[c].y, r.v[c].z, r.v[c].w};
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (SRC_BF16) { f[2 * e] = bf16_to_f32(w[e] & 0xFFFFu); f[2 * e + 1] = bf16_to_f32(w[e] >> 16); }
      else { f[2 * e] = half_bits(w[e] & 0xFFFFu); f[2 * e + 1] = half_bits(w[e] >> 16); }
    }
    half8 hv;
    // nibble order: 0,4,1,5,2,6,3,7
    hv[0] = (_Float16)f[0]; hv[1] = (_Float16)f[4]; hv[2] = (_Float16)f[1]; hv[3] = (_Float16)f[5];
    hv[4] = (_Float16)f[2]; hv[5] = (_Float16)f[6]; hv[6] = (_Float16)f[3]; hv[7] = (_Float16)f[7];
    *reinterpret_cast<half8*>(xs + i * XS + 64 * q + 8 * c) = hv;
    const float part = ((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]));
    if (c < 4) s0 += part; else s1 += part;
  }
  const _Float16 h0 = (_Float16)s0, h1 = (_Float16)s1;
  shi[i * 8 + 2 * q] = h0;
  slo[i * 8 + 2 * q] = (_Float16)(s0 - (float)h0);
  shi[i * 8 + 2 * q + 1] = h1;
  slo[i * 8 + 2 * q + 1] = (_Float16)(s1 - (float)h1);
}

struct SliceSmem {
  _Float16 x[MT * XS];
  _Float16 shi[MT * 8];
  _Float16 slo[MT * 8];
};

// Weights of one lane's row for one super-block: the lane's 4 code bytes of
// each of the 8 sub-blocks and the 16-byte header.
struct WRegs {
  u32 c4[8];
  u32x4 hd;
};

__device__ __forceinline__ void load_w(const uint8_t* __restrict__ row, int codes_bytes, int b, int kg, WRegs& w) {
#pragma unroll
  for (int s = 0; s < 8; ++s) w.c4[s] = *reinterpret_cast<const u32*>(row + (size_t)b * QCODES + 16 * s + 4 * kg);
  w.hd = *reinterpret_cast<const u32x4*>(row + codes_bytes + (size_t)b * QHDR);
}

// NM weight matrices (row pointers per lane) x the staged slice: accumulate
// one super-block into tot[m][r] (lane: rows 16r + 4*(l/16) + i, column l%16).
template <int NM>
__device__ __forceinline__ void slice_mfma(const SliceSmem& sm, const WRegs* w, f32x4 (*tot)[4]) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int j = lane & 15, kg = lane >> 4;
  f32x4 acc[NM][4];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[m][r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    half8 bf[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) bf[m] = codes_times_scale(w[m].c4[s], field6(w[m].hd, 6 * s));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const half8 af = *reinterpret_cast<const half8*>(sm.x + (16 * r + j) * XS + 32 * s + 8 * kg);
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[m][r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[m], acc[m][r], 0, 0, 0);
    }
  }
  // min term: A' = [sum_hi(8) | sum_lo(8) | 0], B' = [m(8) | m(8) | 0]
  half8 am[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (kg < 2) am[r] = *reinterpret_cast<const half8*>((kg == 0 ? sm.shi : sm.slo) + (16 * r + j) * 8);
    else am[r] = half8{0, 0, 0, 0, 0, 0, 0, 0};
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    half8 bm;
#pragma unroll
    for (int s = 0; s < 8; ++s) bm[s] = kg < 2 ? (_Float16)(float)field6(w[m].hd, 48 + 6 * s) : (_Float16)0.f;
    const float d = half_bits(w[m].hd.x & 0xFFFFu), dmin = half_bits(w[m].hd.x >> 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 mt = __builtin_amdgcn_mfma_f32_16x16x32_f16(am[r], bm, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[m][r][i] += d * acc[m][r][i] - dmin * mt[i];
    }
  }
}

// Pipelined K loop over super-blocks for NM weight matrices.
template <bool SRC_BF16, int NM>
__device__ __forceinline__ void tile_gemm(const uint8_t* const* rows, const int* codes_bytes, int K,
                                          const void* __restrict__ src, const int* __restrict__ row_index, int rows_n,
                                          int ld, SliceSmem* sm, f32x4 (*tot)[4]) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int kg = lane >> 4;
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) tot[m][r] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nb = K / QK;
  StageRegs st;
  WRegs w[NM], wn[NM];
  stage_load<SRC_BF16>(src, row_index, rows_n, ld, 0, st);
#pragma unroll
  for (int m = 0; m < NM; ++m) load_w(rows[m], codes_bytes[m], 0, kg, w[m]);
  stage_store<SRC_BF16>(st, sm[0].x, sm[0].shi, sm[0].slo);
  for (int b = 0; b < nb; ++b) {
    __syncthreads();                                   // slice b is in sm[b & 1]
    const bool more = b + 1 < nb;
    if (more) {
      stage_load<SRC_BF16>(src, row_index, rows_n, ld, (b + 1) * QK, st);
#pragma unroll
      for (int m = 0; m < NM; ++m) load_w(rows[m], codes_bytes[m], b + 1, kg, wn[m]);
    }
    slice_mfma<NM>(sm[b & 1], w, tot);
    if (more) {
      stage_store<SRC_BF16>(st, sm[(b + 1) & 1].x, sm[(b + 1) & 1].shi, sm[(b + 1) & 1].slo);
#pragma unroll
      for (int m = 0; m < NM; ++m) w[m] = wn[m];
    }
  }
}

// ------------------------------------------------------------------ gate/up + SiLU
// Work item: blockIdx.x = tile * nnb + nb (nb fastest, so workgroups reading
// the same weights cycle through the same XCD). Features [64nb, 64nb+64),
// 16 per wave; each wave computes gate and up of its features.
__global__ __launch_bounds__(BLOCK, 2) void gateup_grouped_kernel(
    const uint8_t* __restrict__ gu, size_t gu_expert_bytes, int rp_bytes, int H, int I, int E, int k,
    const uint16_t* __restrict__ x, const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs,
    const int32_t* __restrict__ tile_off, _Float16* __restrict__ h16) {
  __shared__ SliceSmem sm[2];
  __shared__ int rowtok[MT];
  const int nnb = I / 64;
  const int nb = blockIdx.x % nnb, tile = blockIdx.x / nnb;
  int m0 = 0;
  const int e = find_tile(tile_off, E, tile, &m0);
  if (e < 0) return;
  const int n_e = offsets[e + 1] - offsets[e];
  const int rows = min(MT, n_e - m0);
  const int tid = threadIdx.x, wid = tid / WAVE, lane = tid & (WAVE - 1);
  if (tid < MT) rowtok[tid] = tid < rows ? pairs[offsets[e] + m0 + tid] / k : 0;
  __syncthreads();
  const int j = lane & 15, kg = lane >> 4;
  const int f0 = 64 * nb + 16 * wid;       // first feature of this wave
  // row-pair record: gate codes at 0, up codes at H/2, gate headers at H, up headers at H + H/16
  const uint8_t* rec = gu + (size_t)e * gu_expert_bytes + (size_t)(f0 + j) * rp_bytes;
  const uint8_t* rowp[2] = {rec, rec + H / 2};
  const int cb[2] = {H, H / 2 + H / 16};
  f32x4 tot[2][4];
  tile_gemm<true, 2>(rowp, cb, H, x, rowtok, rows, H, sm, tot);
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * r + 4 * kg + i;
      if (row < rows) {
        const float g = tot[0][r][i];
        h16[(size_t)(offsets[e] + m0 + row) * I + f0 + j] = (_Float16)(g / (1.0f + expf(-g)) * tot[1][r][i]);
      }
    }
}

// ------------------------------------------------------------------ down
// Work item: blockIdx.x = tile * nnb + nb; features [128nb, 128nb+128), 32
// per wave (two 16-column MFMA blocks sharing each A fragment). Output rows
// go to their pair index (t*k + s).
__global__ __launch_bounds__(BLOCK, 2) void down_grouped_kernel(
    const uint8_t* __restrict__ dn, size_t dn_expert_bytes, int drow_bytes, int H, int I, int E,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs, const int32_t* __restrict__ tile_off,
    const _Float16* __restrict__ h16, float* __restrict__ ypair) {
  __shared__ SliceSmem sm[2];
  __shared__ int rowpos[MT];
  __shared__ int rowpair[MT];
  const int nnb = H / 128;
  const int nb = blockIdx.x % nnb, tile = blockIdx.x / nnb;
  int m0 = 0;
  const int e = find_tile(tile_off, E, tile, &m0);
  if (e < 0) return;
  const int n_e = offsets[e + 1] - offsets[e];
  const int rows = min(MT, n_e - m0);
  const int tid = threadIdx.x, wid = tid / WAVE, lane = tid & (WAVE - 1);
  if (tid < MT) {
    rowpos[tid] = tid < rows ? offsets[e] + m0 + tid : 0;     // row of h16 (sorted order)
    rowpair[tid] = tid < rows ? pairs[offsets[e] + m0 + tid] : 0;
  }
  __syncthreads();
  const int j = lane & 15, kg = lane >> 4;
  const int f0 = 128 * nb + 32 * wid;
  const uint8_t* base = dn + (size_t)e * dn_expert_bytes;
  const uint8_t* rowp[2] = {base + (size_t)(f0 + j) * drow_bytes, base + (size_t)(f0 + 16 + j) * drow_bytes};
  const int cb[2] = {I / 2, I / 2};
  f32x4 tot[2][4];
  tile_gemm<false, 2>(rowp, cb, I, h16, rowpos, rows, I, sm, tot);
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * r + 4 * kg + i;
        if (row < rows) ypair[(size_t)rowpair[row] * H + f0 + 16 * m + j] = tot[m][r][i];
      }
}

// ------------------------------------------------------------------ combine
// out[t][n] = sum_s w[t][s] * ypair[t*k + s][n], slot order.
__global__ __launch_bounds__(BLOCK) void combine_kernel(const float* __restrict__ ypair, const float* __restrict__ w,
                                                        float* __restrict__ out, int H, int k, int T) {
  const int idx = blockIdx.x * BLOCK + threadIdx.x;     // one float4 of one token
  const int per = H / 4;
  if (idx >= T * per) return;
  const int t = idx / per, c = idx % per;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < k; ++s) {
    const float ws = w[(size_t)t * k + s];
    const float4 v = *reinterpret_cast<const float4*>(ypair + ((size_t)t * k + s) * H + 4 * c);
    acc.x = fmaf(ws, v.x, acc.x); acc.y = fmaf(ws, v.y, acc.y);
    acc.z = fmaf(ws, v.z, acc.z); acc.w = fmaf(ws, v.w, acc.w);
  }
  *reinterpret_cast<float4*>(out + (size_t)t * H + 4 * c) = acc;
}

}  // namespace grouped

int grouped_max_tiles(const Layout& d, int T) { return (T * d.k + grouped::MT - 1) / grouped::MT + d.E; }

hipError_t launch_grouped_ffn(const Layout& d, const uint8_t* layer, const uint16_t* x, const float* w,
                              const int32_t* offsets, const int32_t* pairs, const int32_t* tile_off, _Float16* h16,
                              float* ypair, float* out, int T, hipStream_t s) {
  using namespace grouped;
  const int tiles = grouped_max_tiles(d, T);
  hipLaunchKernelGGL(gateup_grouped_kernel, dim3(tiles * (d.I / 64)), dim3(BLOCK), 0, s, layer + d.gu_off,
                     d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.E, d.k, x, offsets, pairs, tile_off, h16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(down_grouped_kernel, dim3(tiles * (d.H / 128)), dim3(BLOCK), 0, s, layer + d.dn_off,
                     d.dn_expert_bytes, (int)d.drow_bytes, d.H, d.I, d.E, offsets, pairs, tile_off, h16, ypair);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n4 = T * (d.H / 4);
  hipLaunchKernelGGL(combine_kernel, dim3((n4 + BLOCK - 1) / BLOCK), dim3(BLOCK), 0, s, ypair, w, out, d.H, d.k, T);
  return hipGetLastError();
}

}  // namespace qmoe

// gfx950 kernels of the batched path: grouped expert GEMMs on the MFMA
// units for token batches routed to the same expert.
//
// The pages' batched prefill dequantizes 4-bit weights into the GEMM operand
// and shares one weight read across a chunk of tokens (sparkinfer README,
// Qwen3.8-27B prefill notes; sparkinfer-k3 release log, batched prompt
// ingestion); this is our CDNA4 form of it. Tokens are grouped by expert on
// the device (dispatch lists), each workgroup takes a (expert, 64-pair tile,
// feature block) and runs v_mfma_f32_16x16x32_f16 with
//   A = activations in fp16 (bf16 inputs are exact in fp16 above 2^-14),
//   B = q * sc, the 4-bit code times its 6-bit sub-block scale (<= 945,
//       exact in fp16),
// accumulated over one 256-weight super-block, then scaled by the block's d.
// The min term sum_j dmin*m_j*sum_{i in j} x_i is one more MFMA per
// super-block with A = the sub-block sums split into fp16 hi + lo parts and
// B = m_j, scaled by dmin. h = SiLU(gate) * up is kept in fp16 between the
// two GEMMs; the down GEMM writes one fp32 row per (token, slot) pair and the
// routing-weighted combine sums them in slot order (deterministic).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace qmoe {
namespace grouped {

typedef unsigned int u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int BLOCK = 256;
constexpr int MT = 64;       // pairs per tile
constexpr int XS = 256 + 8;  // LDS row stride (halfs) of a staged 256-wide K slice (padding against bank conflicts)

__device__ __forceinline__ float as_f32(u32 v) { return __builtin_bit_cast(float, v); }
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

// B fragment of one 32-weight sub-block for this lane: 8 codes (its k-group)
// times the sub-block scale, as fp16 (exact: at most 15 * 63).
__device__ __forceinline__ half8 codes_times_scale(u32 c4, u32 sc) {
  half8 b;
  const _Float16 s = (_Float16)(float)sc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32 byte = (c4 >> (8 * i)) & 0xFFu;
    b[2 * i] = (_Float16)(float)(byte & 15u) * s;
    b[2 * i + 1] = (_Float16)(float)(byte >> 4) * s;
  }
  return b;
}

// Stage a [MT x 256] activation slice (columns k0..k0+255) into LDS as fp16,
// plus per-row sub-block sums split as fp16 hi + lo. Rows past `rows` are 0.
// src_bf16: true for bf16 rows (x), false for fp16 rows (h).
template <bool SRC_BF16>
__device__ __forceinline__ void stage_rows(const void* __restrict__ src, const int* __restrict__ row_index, int rows,
                                           int ld, int k0, _Float16* xs, _Float16* shi, _Float16* slo) {
  const int tid = threadIdx.x;
  const int i = tid >> 2, q = tid & 3;      // row, quarter of the 256 columns
  const bool ok = i < rows;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {             // 8 x 8 elements
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) {
      const size_t off = (size_t)row_index[i] * ld + k0 + 64 * q + 8 * c;
      v = SRC_BF16 ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + off)
                   : *reinterpret_cast<const u32x4*>(static_cast<const _Float16*>(src) + off);
    }
    half8 hv;
    float part = 0.f;
    const u32 w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a, b;
      if (SRC_BF16) { a = bf16_to_f32(w[e] & 0xFFFFu); b = bf16_to_f32(w[e] >> 16); }
      else { a = half_bits(w[e] & 0xFFFFu); b = half_bits(w[e] >> 16); }
      hv[2 * e] = (_Float16)a;
      hv[2 * e + 1] = (_Float16)b;
      part += a + b;
    }
    *reinterpret_cast<half8*>(xs + i * XS + 64 * q + 8 * c) = hv;
    if (c < 4) s0 += part; else s1 += part;
  }
  // sub-blocks 2q and 2q+1 of this super-block
  const _Float16 h0 = (_Float16)s0, h1 = (_Float16)s1;
  shi[i * 8 + 2 * q] = h0;
  slo[i * 8 + 2 * q] = (_Float16)(s0 - (float)h0);
  shi[i * 8 + 2 * q + 1] = h1;
  slo[i * 8 + 2 * q + 1] = (_Float16)(s1 - (float)h1);
}

// One weight matrix, 16 output features (one per lane column), all MT rows:
// acc over the K range [0, K) in super-blocks, result in tot[4] (lane holds
// rows 16r + 4*(l/16) + i, column l%16).
struct GemmSmem {
  _Float16 x[MT * XS];
  _Float16 shi[MT * 8];
  _Float16 slo[MT * 8];
};

template <bool SRC_BF16>
__device__ __forceinline__ void tile_gemm(const uint8_t* __restrict__ wrow_base, size_t wrow_stride, int codes_bytes,
                                          int K, const void* __restrict__ src, const int* __restrict__ row_index,
                                          int rows, int ld, GemmSmem& sm, f32x4 tot[4]) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int j = lane & 15, kg = lane >> 4;
  const uint8_t* row = wrow_base + (size_t)j * wrow_stride;   // this lane's weight row
#pragma unroll
  for (int r = 0; r < 4; ++r) tot[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < K / QK; ++b) {
    __syncthreads();
    stage_rows<SRC_BF16>(src, row_index, rows, ld, b * QK, sm.x, sm.shi, sm.slo);
    // weights of this lane's row for super-block b: its 4 code bytes of each sub-block + header
    u32 c4[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) c4[s] = *reinterpret_cast<const u32*>(row + (size_t)b * QCODES + 16 * s + 4 * kg);
    const u32x4 hd = *reinterpret_cast<const u32x4*>(row + codes_bytes + (size_t)b * QHDR);
    __syncthreads();
    f32x4 acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const half8 bf = codes_times_scale(c4[s], field6(hd, 6 * s));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const half8 af = *reinterpret_cast<const half8*>(sm.x + (16 * r + j) * XS + 32 * s + 8 * kg);
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc[r], 0, 0, 0);
      }
    }
    // min term: A' = [sum_hi(8) | sum_lo(8) | 0], B' = [m(8) | m(8) | 0]
    half8 bm;
#pragma unroll
    for (int s = 0; s < 8; ++s) bm[s] = kg < 2 ? (_Float16)(float)field6(hd, 48 + 6 * s) : (_Float16)0.f;
    const float d = half_bits(hd.x & 0xFFFFu), dmin = half_bits(hd.x >> 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      half8 am;
      const _Float16* src8 = kg == 0 ? sm.shi : sm.slo;
#pragma unroll
      for (int s = 0; s < 8; ++s) am[s] = kg < 2 ? src8[(16 * r + j) * 8 + s] : (_Float16)0.f;
      const f32x4 mt = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, bm, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[r][i] += d * acc[r][i] - dmin * mt[i];
    }
  }
}

// ------------------------------------------------------------------ gate/up + SiLU
// Work item: blockIdx.x = tile * nnb + nb (nb fastest, so workgroups reading
// the same weights cycle through the same XCD). Features [32nb, 32nb+32):
// waves 0,1 compute gate for 16 features each, waves 2,3 up.
__global__ __launch_bounds__(BLOCK) void gateup_grouped_kernel(
    const uint8_t* __restrict__ gu, size_t gu_expert_bytes, int rp_bytes, int H, int I, int E, int k,
    const uint16_t* __restrict__ x, const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs,
    const int32_t* __restrict__ tile_off, _Float16* __restrict__ h16) {
  __shared__ GemmSmem sm;
  __shared__ int rowtok[MT];
  __shared__ float gtile[MT][33];
  const int nnb = I / 32;
  const int nb = blockIdx.x % nnb, tile = blockIdx.x / nnb;
  int m0 = 0;
  const int e = find_tile(tile_off, E, tile, &m0);
  if (e < 0) return;
  const int n_e = offsets[e + 1] - offsets[e];
  const int rows = min(MT, n_e - m0);
  const int tid = threadIdx.x, wid = tid / WAVE, lane = tid & (WAVE - 1);
  if (tid < MT) rowtok[tid] = tid < rows ? pairs[offsets[e] + m0 + tid] / k : 0;
  __syncthreads();
  const int mat = wid >> 1, cb = wid & 1;
  const int f0 = 32 * nb + 16 * cb;       // first feature of this wave
  const uint8_t* wbase = gu + (size_t)e * gu_expert_bytes + (size_t)f0 * rp_bytes + (size_t)mat * (H / 2);
  // within a row-pair record: gate codes at 0, up codes at H/2, gate headers at H, up headers at H + H/16
  // tile_gemm reads codes at row + 128b and headers at row + codes_bytes + 16b
  const int codes_bytes = H - mat * (H / 2) + mat * (H / 16);
  f32x4 tot[4];
  tile_gemm<true>(wbase, rp_bytes, codes_bytes, H, x, rowtok, rows, H, sm, tot);
  const int j = lane & 15, kg = lane >> 4;
  // gate tile to LDS, then the up waves combine
  if (mat == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) gtile[16 * r + 4 * kg + i][16 * cb + j] = tot[r][i];
  }
  __syncthreads();
  if (mat == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * r + 4 * kg + i;
        if (row < rows) {
          const float g = gtile[row][16 * cb + j];
          const float hval = g / (1.0f + expf(-g)) * tot[r][i];
          h16[(size_t)(offsets[e] + m0 + row) * I + f0 + j] = (_Float16)hval;
        }
      }
  }
}

// ------------------------------------------------------------------ down
// Work item: blockIdx.x = tile * nnb + nb; features [64nb, 64nb+64), 16 per
// wave. Output rows go to their pair index (t*k + s).
__global__ __launch_bounds__(BLOCK) void down_grouped_kernel(
    const uint8_t* __restrict__ dn, size_t dn_expert_bytes, int drow_bytes, int H, int I, int E,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs, const int32_t* __restrict__ tile_off,
    const _Float16* __restrict__ h16, float* __restrict__ ypair) {
  __shared__ GemmSmem sm;
  __shared__ int rowpos[MT];
  __shared__ int rowpair[MT];
  const int nnb = H / 64;
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
  const int f0 = 64 * nb + 16 * wid;
  const uint8_t* wbase = dn + (size_t)e * dn_expert_bytes + (size_t)f0 * drow_bytes;
  f32x4 tot[4];
  tile_gemm<false>(wbase, drow_bytes, I / 2, I, h16, rowpos, rows, I, sm, tot);
  const int j = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * r + 4 * kg + i;
      if (row < rows) ypair[(size_t)rowpair[row] * H + f0 + j] = tot[r][i];
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
  hipLaunchKernelGGL(gateup_grouped_kernel, dim3(tiles * (d.I / 32)), dim3(BLOCK), 0, s, layer + d.gu_off,
                     d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.E, d.k, x, offsets, pairs, tile_off, h16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(down_grouped_kernel, dim3(tiles * (d.H / 64)), dim3(BLOCK), 0, s, layer + d.dn_off,
                     d.dn_expert_bytes, (int)d.drow_bytes, d.H, d.I, d.E, offsets, pairs, tile_off, h16, ypair);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n4 = T * (d.H / 4);
  hipLaunchKernelGGL(combine_kernel, dim3((n4 + BLOCK - 1) / BLOCK), dim3(BLOCK), 0, s, ypair, w, out, d.H, d.k, T);
  return hipGetLastError();
}

}  // namespace qmoe

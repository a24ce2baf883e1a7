// gfx950 kernels of the batched path: grouped expert GEMMs on the MFMA
// units for token batches routed to the same expert.
//
// The pages' batched prefill dequantizes the 4-bit super-blocks into the GEMM
// operand and shares one weight read across a chunk of tokens (SP⚡RKINFER
// README, Qwen3.8-27B prefill notes; sparkinfer-k3 release log, batched
// prompt ingestion); this is our CDNA4 form of it. Tokens are grouped by
// expert on the device (dispatch lists); a workgroup takes (expert, tile of
// MT = 32*WR routed pairs, block of output features) and runs
// v_mfma_f32_32x32x16_f16 with
//   A = activations in fp16 (bf16 inputs are exact in fp16 above 2^-14),
//   B = the dequantized weight d*sc*q - dmin*m rounded once to fp16: the
//       code q comes out exact as fp16(0x6400|q) - 1024, then one packed fp16
//       fma with (d*sc, -dmin*m) per sub-block (relative rounding 2^-11),
// accumulated in fp32 over the whole K. Lane (n = l%32, kg = l/32) of a
// weight row owns the 16-byte code chunks at 32j + 16kg (j = 0..3) of every
// super-block, i.e. sub-blocks 2j + kg, so four consecutive MFMAs cover 64
// consecutive K; activations are staged in LDS half a super-block (128 K) at
// a time, double buffered, with each group of 8 stored in the order the code
// nibbles are unpacked (0,2,4,6,1,3,5,7). h = SiLU(gate) * up is written in
// fp16 in that same order, so the down GEMM stages it by plain copies; the
// down GEMM writes one fp32 row per (token, slot) pair and the
// routing-weighted combine sums them in slot order (deterministic).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moe_device.h"

namespace qmoe {
namespace grouped {

typedef unsigned int u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int KH = 128;            // K per stage (half a super-block)
constexpr int XS = KH + 8;         // LDS row stride (halfs): 272 B = 16 mod 128, conflict-free 16-byte reads
constexpr int NN = 2;              // 32-feature column blocks per wave
constexpr int FB = 4 * NN * 32 / 2;   // gate/up: output features (h) per workgroup = 128
constexpr int FD = 4 * NN * 32;       // down: output features per workgroup = 256

__device__ __forceinline__ u32 field6(const u32x4& h, int p) {
  const int idx = p >> 5, sh = p & 31;
  const u32 lo = idx == 0 ? h.y : (idx == 1 ? h.z : h.w);
  const u32 hi = idx == 0 ? h.z : (idx == 1 ? h.w : 0u);
  return __builtin_amdgcn_alignbit(hi, lo, sh) & 63u;
}

__device__ __forceinline__ float half_bits(u32 b) { return (float)__builtin_bit_cast(_Float16, (unsigned short)b); }

// tile -> (expert, first pair in the expert's group); -1 if past the last tile
__device__ __forceinline__ int find_tile(const int32_t* __restrict__ tile_off, int E, int tile, int mt, int* m0) {
  if (tile >= tile_off[E]) return -1;
  int lo = 0, hi = E;            // tile_off[lo] <= tile < tile_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= tile) lo = mid; else hi = mid;
  }
  *m0 = (tile - tile_off[lo]) * mt;
  return lo;
}

// Work unit of a workgroup: units are dealt so that each XCD (workgroup i
// runs on XCD i % 8) gets a contiguous run of (feature block, tile) units,
// tiles fastest: consecutive tiles of one expert's feature block share the
// XCD's L2.
__device__ __forceinline__ void unit_of_block(int ntiles, int* tile, int* fb) {
  const int per = gridDim.x >> 3;
  const int u = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  *tile = u % ntiles;
  *fb = u / ntiles;
}

// Work unit of a multi-row 16-pair-tile workgroup: tiles are dealt to the
// XCDs round-robin (tile t to XCD t % 8, so empty tiles spread evenly) and
// the bpt row blocks of one tile follow each other on that XCD, so the
// tile's activations (or h) are fetched into one L2 and re-read from there.
// The grid is 8 * bpt * ceil(ntiles / 8); units past the last tile return.
__device__ __forceinline__ bool tile_unit(int ntiles, int bpt, int* tile, int* rb) {
  const int su = (int)(blockIdx.x >> 3);
  *tile = (su / bpt) * 8 + (int)(blockIdx.x & 7);
  *rb = su % bpt;
  return *tile < ntiles;
}
__host__ __forceinline__ unsigned tile_unit_grid(int ntiles, int bpt) {
  return 8u * (unsigned)bpt * (unsigned)((ntiles + 7) / 8);
}

// Per-sub-block dequantization constants (a, -b) as fp16 pairs:
// weight = a*q - b with a = d*sc, b = dmin*m (products exact in fp32, then
// rounded to fp16). The 6-bit fields sit at bit 6*sb (scales) and 48 + 6*sb
// (mins) of header dwords 1..3, read with one 64-bit shift each.
struct SubScale { half2 a2, nb2; };
__device__ __forceinline__ SubScale sub_scale(const u32x4& h, int sb) {
  const float d = half_bits(h.x & 0xFFFFu), dmin = half_bits(h.x >> 16);
  const unsigned long long lo = (unsigned long long)h.y | ((unsigned long long)h.z << 32);
  const unsigned long long hi = (unsigned long long)h.z | ((unsigned long long)h.w << 32);
  const u32 sc = (u32)(lo >> (6 * sb)) & 63u;
  const u32 m = (u32)(hi >> (16 + 6 * sb)) & 63u;
  const _Float16 a = (_Float16)(d * (float)sc);
  const _Float16 nb = (_Float16)(-(dmin * (float)m));
  return {half2{a, a}, half2{nb, nb}};
}

// The 8 weights of one code dword in unpack order (0,2,4,6,1,3,5,7): the low
// and high nibbles of the 4 bytes are split into bytes, and each pair of
// bytes becomes two fp16 values 0x64qq = 1024 + q with one byte permute
// against a register of 0x64 bytes; 1024 is then removed exactly and one
// packed fma applies the sub-block's (a, -b).
__device__ __forceinline__ half8 dequant8(u32 v, const SubScale& s) {
  const u32 K64 = 0x64646464u;
  const u32 lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;   // bytes: e0 e2 e4 e6 / e1 e3 e5 e7
  const u32 p[4] = {__builtin_amdgcn_perm(K64, lo, 0x04010400u), __builtin_amdgcn_perm(K64, lo, 0x04030402u),
                    __builtin_amdgcn_perm(K64, hi, 0x04010400u), __builtin_amdgcn_perm(K64, hi, 0x04030402u)};
  const half2 bias = {(_Float16)1024.0f, (_Float16)1024.0f};
  half8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2 q = __builtin_bit_cast(half2, p[i]) - bias;   // exact
    const half2 w = __builtin_elementwise_fma(q, s.a2, s.nb2);
    r[2 * i] = w[0];
    r[2 * i + 1] = w[1];
  }
  return r;
}

// Position of element e (0..7) of an 8-group in unpack order.
__device__ __forceinline__ int nib_pos(int e) { return (e >> 1) + 4 * (e & 1); }

// Staging of one 128-wide K half of the A tile (MT rows): thread -> chunks of
// 8 values (16 bytes), chunk c = tid + 256*q: row c/16, columns 8*(c%16).
template <int MT>
struct StageRegs { u32x4 v[MT / 16]; };

template <int MT, bool SRC_BF16>
__device__ __forceinline__ void stage_load(const void* __restrict__ src, const int* __restrict__ row_index, int rows,
                                           int ld, int k0, StageRegs<MT>& r) {
#pragma unroll
  for (int q = 0; q < MT / 16; ++q) {
    const int c = (int)threadIdx.x + BLOCK * q;
    const int row = c >> 4, c8 = c & 15;
    r.v[q] = u32x4{0u, 0u, 0u, 0u};
    if (row < rows) {
      const size_t off = (size_t)row_index[row] * ld + k0 + 8 * c8;
      r.v[q] = SRC_BF16 ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + off)
                        : *reinterpret_cast<const u32x4*>(static_cast<const _Float16*>(src) + off);
    }
  }
}

// bf16 sources are converted to fp16 (exact for normal values; the
// round-toward-zero conversion only matters below 2^-14 or above 65504) and
// permuted into unpack order; fp16 sources (h) are already in that order.
template <int MT, bool SRC_BF16>
__device__ __forceinline__ void stage_store(const StageRegs<MT>& r, _Float16* a) {
#pragma unroll
  for (int q = 0; q < MT / 16; ++q) {
    const int c = (int)threadIdx.x + BLOCK * q;
    const int row = c >> 4, c8 = c & 15;
    u32x4 o = r.v[q];
    if (SRC_BF16) {
      const u32 w0 = r.v[q].x, w1 = r.v[q].y, w2 = r.v[q].z, w3 = r.v[q].w;   // (e0,e1) (e2,e3) (e4,e5) (e6,e7)
      auto lo = [](u32 w) { return __builtin_bit_cast(float, w << 16); };
      auto hi = [](u32 w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); };
      o.x = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_pkrtz(lo(w0), lo(w1)));   // (e0, e2)
      o.y = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_pkrtz(lo(w2), lo(w3)));   // (e4, e6)
      o.z = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_pkrtz(hi(w0), hi(w1)));   // (e1, e3)
      o.w = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_pkrtz(hi(w2), hi(w3)));   // (e5, e7)
    }
    *reinterpret_cast<u32x4*>(a + row * XS + 8 * c8) = o;
  }
}

// One lane's weights for one super-block: the four 16-byte code chunks at
// 32j + 16kg (j = 0..3) of its row, i.e. sub-blocks 2j + kg. The four loads
// of a row's 128-byte line leave together, so the line is fetched from HBM
// once; ordinary (cached) loads, since each instruction covers 32 bytes of
// 32 different rows.
struct SbCodes { u32x4 c[4]; };

__device__ __forceinline__ void load_sb(const uint8_t* __restrict__ row, int b, int kg, SbCodes& w) {
  const uint8_t* p = row + (size_t)b * QCODES + 16 * kg;
#pragma unroll
  for (int j = 0; j < 4; ++j) w.c[j] = *reinterpret_cast<const u32x4*>(p + 32 * j);
}

// Grouped GEMM core: MT x (NN*32) outputs per wave over K, NN weight rows
// per lane (rowp[n] = start of the lane's row in column block n, header
// offset hdr_off[n] from that start). The weights of super-block b + 1 are
// requested when super-block b starts; activations are staged half a
// super-block at a time through a double-buffered LDS tile, the next half
// requested before the current one is multiplied.
template <int WR, bool SRC_BF16>
__device__ __forceinline__ void tile_gemm(const uint8_t* const* rowp, const int* hdr_off, int K, const void* __restrict__ src,
                                          const int* __restrict__ row_index, int rows, int ld, _Float16 (*a)[32 * WR * XS],
                                          f32x16 (*acc)[NN]) {
  constexpr int MT = 32 * WR;
  const int lane = threadIdx.x & (WAVE - 1);
  const int i = lane & 31, kg = lane >> 5;
#pragma unroll
  for (int r = 0; r < WR; ++r)
#pragma unroll
    for (int n = 0; n < NN; ++n)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[r][n][q] = 0.f;
  const int nb = K / QK;
  SbCodes w[NN], wn[NN];
  u32x4 hd[NN], hdn[NN];
  StageRegs<MT> st;
#pragma unroll
  for (int n = 0; n < NN; ++n) {
    load_sb(rowp[n], 0, kg, w[n]);
    hd[n] = *reinterpret_cast<const u32x4*>(rowp[n] + hdr_off[n]);
  }
  stage_load<MT, SRC_BF16>(src, row_index, rows, ld, 0, st);
  stage_store<MT, SRC_BF16>(st, a[0]);
  for (int b = 0; b < nb; ++b) {
    if (b + 1 < nb) {
#pragma unroll
      for (int n = 0; n < NN; ++n) {
        load_sb(rowp[n], b + 1, kg, wn[n]);
        hdn[n] = *reinterpret_cast<const u32x4*>(rowp[n] + hdr_off[n] + (size_t)(b + 1) * QHDR);
      }
    }
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const int s = 2 * b + hs;
      __syncthreads();                                 // half s is in a[s & 1]
      const bool more = s + 1 < 2 * nb;
      if (more) stage_load<MT, SRC_BF16>(src, row_index, rows, ld, (s + 1) * KH, st);
      const _Float16* as = a[s & 1];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * hs + jj;
        const int sb = 2 * j + kg;                     // sub-block of this lane's chunk
        SubScale sc[NN];
#pragma unroll
        for (int n = 0; n < NN; ++n) sc[n] = sub_scale(hd[n], sb);
#pragma unroll
        for (int wq = 0; wq < 4; ++wq) {
          half8 bf[NN];
#pragma unroll
          for (int n = 0; n < NN; ++n) {
            const u32x4& c = w[n].c[j];
            const u32 dw = wq == 0 ? c.x : (wq == 1 ? c.y : (wq == 2 ? c.z : c.w));
            bf[n] = dequant8(dw, sc[n]);
          }
          const int col = 64 * jj + 32 * kg + 8 * wq;
#pragma unroll
          for (int r = 0; r < WR; ++r) {
            const half8 af = *reinterpret_cast<const half8*>(as + (32 * r + i) * XS + col);
#pragma unroll
            for (int n = 0; n < NN; ++n) acc[r][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[n], acc[r][n], 0, 0, 0);
          }
        }
      }
      if (more) stage_store<MT, SRC_BF16>(st, a[(s + 1) & 1]);
    }
#pragma unroll
    for (int n = 0; n < NN; ++n) { w[n] = wn[n]; hd[n] = hdn[n]; }
  }
}

template <int WR>
struct Smem {
  _Float16 a[2][32 * WR * XS];
  int rowidx[32 * WR];
};

// ------------------------------------------------------------------ gate/up + SiLU
// Workgroup: one tile (MT pairs of one expert) x 128 features of h; wave w
// computes gate (column block 0) and up (column block 1) of features
// [f0, f0 + 32), f0 = 128*fb + 32*w, and writes h in fp16 at the pairs'
// sorted positions, in unpack order within each group of 8.
template <int WR>
__global__ __launch_bounds__(BLOCK, 2) void gateup_grouped_kernel(
    const uint8_t* __restrict__ gu, size_t gu_expert_bytes, int rp_bytes, int H, int I, int E, int k, int ntiles,
    const uint16_t* __restrict__ x, const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs,
    const int32_t* __restrict__ tile_off, _Float16* __restrict__ h16, int act) {
  constexpr int MT = 32 * WR;
  __shared__ Smem<WR> sm;
  int tile, fb;
  unit_of_block(ntiles, &tile, &fb);
  if (fb >= I / FB) return;
  int m0 = 0;
  const int e = find_tile(tile_off, E, tile, MT, &m0);
  if (e < 0) return;
  const int n_e = offsets[e + 1] - offsets[e];
  const int rows = min(MT, n_e - m0);
  const int tid = threadIdx.x, wid = tid / WAVE, lane = tid & (WAVE - 1);
  if (tid < MT) sm.rowidx[tid] = tid < rows ? pairs[offsets[e] + m0 + tid] / k : 0;
  __syncthreads();
  const int f0 = FB * fb + 32 * wid;
  // row-pair record: gate codes at 0, up codes at H/2, gate headers at H, up headers at H + H/16
  const uint8_t* rec = gu + (size_t)e * gu_expert_bytes + (size_t)(f0 + (lane & 31)) * rp_bytes;
  const uint8_t* rowp[NN] = {rec, rec + H / 2};
  const int hdr[NN] = {H, H / 2 + H / 16};
  f32x16 acc[WR][NN];
  tile_gemm<WR, true>(rowp, hdr, H, x, sm.rowidx, rows, H, sm.a, acc);
  const int kg = lane >> 5;
  const int col = f0 + 8 * ((lane & 31) >> 3) + nib_pos(lane & 7);
  const size_t pos0 = (size_t)offsets[e] + m0;
#pragma unroll
  for (int r = 0; r < WR; ++r)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = 32 * r + 8 * (q >> 2) + 4 * kg + (q & 3);
      if (row < rows) {
        const float g = acc[r][0][q], u = acc[r][1][q];
        h16[(pos0 + row) * I + col] = (_Float16)gate_act(g, u, act);
      }
    }
}

// ------------------------------------------------------------------ down
// Workgroup: one tile x 256 output features; wave w computes features
// [f0, f0 + 64), f0 = 256*fb + 64*w (two column blocks), rows to ypair at
// the pair index t*k + s.
template <int WR>
__global__ __launch_bounds__(BLOCK, 2) void down_grouped_kernel(
    const uint8_t* __restrict__ dn, size_t dn_expert_bytes, int drow_bytes, int H, int I, int E, int ntiles,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs, const int32_t* __restrict__ tile_off,
    const _Float16* __restrict__ h16, float* __restrict__ ypair) {
  constexpr int MT = 32 * WR;
  __shared__ Smem<WR> sm;
  __shared__ int rowpair[MT];
  int tile, fb;
  unit_of_block(ntiles, &tile, &fb);
  if (fb >= H / FD) return;
  int m0 = 0;
  const int e = find_tile(tile_off, E, tile, MT, &m0);
  if (e < 0) return;
  const int n_e = offsets[e + 1] - offsets[e];
  const int rows = min(MT, n_e - m0);
  const int tid = threadIdx.x, wid = tid / WAVE, lane = tid & (WAVE - 1);
  if (tid < MT) {
    sm.rowidx[tid] = tid < rows ? offsets[e] + m0 + tid : 0;     // row of h16 (sorted order)
    rowpair[tid] = tid < rows ? pairs[offsets[e] + m0 + tid] : 0;
  }
  __syncthreads();
  const int f0 = FD * fb + 64 * wid;
  const uint8_t* base = dn + (size_t)e * dn_expert_bytes;
  const uint8_t* rowp[NN] = {base + (size_t)(f0 + (lane & 31)) * drow_bytes,
                             base + (size_t)(f0 + 32 + (lane & 31)) * drow_bytes};
  const int hdr[NN] = {I / 2, I / 2};
  f32x16 acc[WR][NN];
  tile_gemm<WR, false>(rowp, hdr, I, h16, sm.rowidx, rows, I, sm.a, acc);
  const int kg = lane >> 5;
#pragma unroll
  for (int r = 0; r < WR; ++r)
#pragma unroll
    for (int n = 0; n < NN; ++n)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = 32 * r + 8 * (q >> 2) + 4 * kg + (q & 3);
        if (row < rows) ypair[(size_t)rowpair[row] * H + f0 + 32 * n + (lane & 31)] = acc[r][n][q];
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

template <int WR>
static hipError_t launch_wr(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* offsets,
                            const int32_t* pairs, const int32_t* tile_off, _Float16* h16, float* ypair, int T,
                            hipStream_t s) {
  const int tiles = grouped_max_tiles(d, T);
  const int gu_units = tiles * (d.I / FB), dn_units = tiles * (d.H / FD);
  // grids padded to a multiple of 8 (the unit dealing assumes it); extra blocks exit
  hipLaunchKernelGGL((gateup_grouped_kernel<WR>), dim3((gu_units + 7) / 8 * 8), dim3(BLOCK), 0, s, layer + d.gu_off,
                     d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.E, d.k, tiles, x, offsets, pairs, tile_off, h16,
                     d.act);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((down_grouped_kernel<WR>), dim3((dn_units + 7) / 8 * 8), dim3(BLOCK), 0, s, layer + d.dn_off,
                     d.dn_expert_bytes, (int)d.drow_bytes, d.H, d.I, d.E, tiles, offsets, pairs, tile_off, h16, ypair);
  return hipGetLastError();
}


// ------------------------------------------------------------------ 16-pair tiles, all weights in flight
// For batches whose experts carry few pairs (a tile of 32 or 96 rows would be
// mostly padding and its K loop would wait on one super-block at a time),
// v_mfma_f32_16x16x32_f16 on tiles of at most 16 pairs (lane layouts checked
// on the box: A[l%16][8(l/16)+e], B[8(l/16)+e][l%16], D[4(l/16)+r][l%16]).
// Lane (row r = l%16, kg = l/16) of a weight row owns the 16-byte code chunk
// of sub-block 4m + kg for each group m of 128 K, so one group is four MFMAs
// (one per code dword), B dequantized with dequant8 and A the matching eight
// activations in unpack order. Every wave requests all of its weights at once
// and takes its activations straight from L2 into registers: no LDS staging,
// no barrier inside the K loop. Work list: one record {expert, first pair,
// pairs} per tile, written by the dispatch.
struct TileRec { int e, pos0, n, pad; };

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Eight bf16 activations (16 bytes) as fp16 in unpack order (0,2,4,6,1,3,5,7).
__device__ __forceinline__ half8 bf16x8_to_unpack(const u32x4& v) {
  auto lo = [](u32 w) { return __builtin_bit_cast(float, w << 16); };
  auto hi = [](u32 w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); };
  u32x4 o;
  o.x = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_pkrtz(lo(v.x), lo(v.y)));   // (e0, e2)
  o.y = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_pkrtz(lo(v.z), lo(v.w)));   // (e4, e6)
  o.z = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_pkrtz(hi(v.x), hi(v.y)));   // (e1, e3)
  o.w = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_pkrtz(hi(v.z), hi(v.w)));   // (e5, e7)
  return __builtin_bit_cast(half8, o);
}

__device__ __forceinline__ u32 dword_of(const u32x4& c, int i) {
  return i == 0 ? c.x : (i == 1 ? c.y : (i == 2 ? c.z : c.w));
}

// MXFP4 on the 16-pair tiles: the block's E8M0 scale goes into the FP4
// conversion, which yields the exact weights as bf16 (scale codes 2..252 keep
// every value a normal bf16), so v_mfma_f32_16x16x32_bf16 runs on exact
// operands in natural K order: A is the bf16 activations as loaded, B the
// eight weights of one code dword.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 fp4x8_bf16(u32 v, float scale) {
  u32x4 o;
  o.x = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0));
  o.y = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1));
  o.z = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2));
  o.w = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3));
  return __builtin_bit_cast(bf16x8, o);
}

// Gate/up: workgroup = one tile x 16 row pairs (intermediate rows f0 .. f0+15),
// the tile's pairs 16 at a time (a tile holds 16 pairs, or for MXFP4 at
// large batches 64 or 128, which then reuse the weights in registers);
// wave w takes K range [w*H/4, (w+1)*H/4), G = H/512 groups of 128 K. The
// four partial products are added in wave order through LDS, then SiLU(gate)
// * up goes to h16 at the pairs' sorted positions, in unpack order within
// each group of 8 (as the 32/96-pair tiles write it).
// MXFP4 (FMT): h is written as bf16 hi and lo parts, h = hi + lo to about
// 2^-17, natural order, the lo plane hlo elements after the hi plane.
template <int G, int FMT, bool MULTI>
__global__ __launch_bounds__(BLOCK) void gateup_g16_kernel(
    const uint8_t* __restrict__ gu, size_t gu_expert_bytes, int rp_bytes, int H, int I, int k,
    const uint16_t* __restrict__ x, const int32_t* __restrict__ pairs, const TileRec* __restrict__ tiles,
    _Float16* __restrict__ h16, int act, size_t hlo) {
  constexpr bool MX = FMT == FMT_MXFP4;
  // super-blocks per wave (a group is half of one); MXFP4: one scale byte per group
  constexpr int NH = MX ? G : (G + 1) / 2;
  using Hdr = std::conditional_t<MX, u32, u32x4>;
  __shared__ float red[4][2][4][WAVE];
  const int bpt = I / 16;
  const TileRec tr = tiles[blockIdx.x / bpt];
  if (tr.n == 0) return;                        // past the last tile (workgroup-uniform)
  const int f0 = (int)(blockIdx.x % bpt) * 16;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int r = lane & 15, kg = lane >> 4;
  const int sb0 = w * 4 * G;                    // first sub-block of the wave's K range
  // token of tile row t = l%16 first: loads complete in order, so the
  // activation loads, which wait on it, must not queue behind the weights.
  // Rows past the tile's pairs repeat its last row (their outputs are not
  // stored), so every load is unconditional.
  const int pair = pairs[tr.pos0 + min(lane & 15, tr.n - 1)];
  __builtin_amdgcn_sched_barrier(0);
  // weights: row f0 + r; gate codes at 0, up codes at H/2, gate headers at H, up headers at H + H/16
  const uint8_t* rec = gu + (size_t)tr.e * gu_expert_bytes + (size_t)(f0 + r) * rp_bytes;
  u32x4 cg[G], cu[G];
  Hdr hg[NH], hu[NH];
#pragma unroll
  for (int m = 0; m < G; ++m) {
    const int sbi = sb0 + 4 * m + kg;
    cg[m] = *reinterpret_cast<const u32x4*>(rec + 16 * sbi);
    cu[m] = *reinterpret_cast<const u32x4*>(rec + H / 2 + 16 * sbi);
  }
#pragma unroll
  for (int b = 0; b < NH; ++b) {
    if constexpr (MX) {
      const int sbi = sb0 + 4 * b + kg;          // the scale of this lane's block of group b
      hg[b] = rec[H + sbi];
      hu[b] = rec[H + H / MXK + sbi];
    } else {
      const int sup = (sb0 + 8 * b) >> 3;
      hg[b] = *reinterpret_cast<const u32x4*>(rec + H + QHDR * sup);
      hu[b] = *reinterpret_cast<const u32x4*>(rec + H + H / 16 + QHDR * sup);
    }
  }
  // the tile's pairs 16 at a time (tiles of more than 16 pairs, MULTI, reuse
  // the weights held in registers; a 16-pair tile is one pass, compiled as such)
  for (int b0 = 0; b0 < (MULTI ? tr.n : 1); b0 += 16) {
    const int nb = min(16, tr.n - b0);
    if constexpr (MULTI) {
      // the codes stay the live state across blocks (32 registers), not
      // their bf16 conversions (128): convert again per block
#pragma unroll
      for (int m = 0; m < G; ++m) asm volatile("" : "+v"(cg[m]), "+v"(cu[m]));
    }
    const int tok = (b0 == 0 ? pair : pairs[tr.pos0 + b0 + min(lane & 15, nb - 1)]) / k;
    u32x4 xr[G][4];
#pragma unroll
    for (int m = 0; m < G; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xr[m][i] = *reinterpret_cast<const u32x4*>(x + (size_t)tok * H + 32 * (sb0 + 4 * m + kg) + 8 * i);
    __builtin_amdgcn_sched_barrier(0);            // every load is in flight before the first use
    f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    if constexpr (MX) {
#pragma unroll
      for (int m = 0; m < G; ++m) {
        const float sg = e8m0_scale(hg[m]), su = e8m0_scale(hu[m]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, xr[m][i]);
          accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp4x8_bf16(dword_of(cg[m], i), sg), accg, 0, 0, 0);
          accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp4x8_bf16(dword_of(cu[m], i), su), accu, 0, 0, 0);
        }
      }
    } else {
      half8 A[G][4];
#pragma unroll
      for (int m = 0; m < G; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) A[m][i] = bf16x8_to_unpack(xr[m][i]);
#pragma unroll
      for (int m = 0; m < G; ++m) {
        const int sb = (sb0 + 4 * m + kg) & 7;    // sub-block within its super-block
        const SubScale sg = sub_scale(hg[m >> 1], sb), su = sub_scale(hu[m >> 1], sb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accg = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[m][i], dequant8(dword_of(cg[m], i), sg), accg, 0, 0, 0);
          accu = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[m][i], dequant8(dword_of(cu[m], i), su), accu, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      red[w][0][q][lane] = accg[q];
      red[w][1][q][lane] = accu[q];
    }
    __syncthreads();
    // thread -> (tile row tt, intermediate row f0 + rr); D[tt][rr] sits in lane rr + 16*(tt/4), register tt%4
    const int tt = tid >> 4, rr = tid & 15;
    if (tt < nb) {
      const int ln = rr + 16 * (tt >> 2), q = tt & 3;
      const float g = ((red[0][0][q][ln] + red[1][0][q][ln]) + red[2][0][q][ln]) + red[3][0][q][ln];
      const float u = ((red[0][1][q][ln] + red[1][1][q][ln]) + red[2][1][q][ln]) + red[3][1][q][ln];
      const int f = f0 + rr;
      const float hv = gate_act(g, u, act);
      if constexpr (MX) {
        uint16_t* hb = reinterpret_cast<uint16_t*>(h16) + (size_t)(tr.pos0 + b0 + tt) * I + f;
        const uint16_t hi = float_to_bf16_rne(hv);
        hb[0] = hi;
        hb[hlo] = float_to_bf16_rne(hv - bf16_bits_to_float(hi));
      } else {
        h16[(size_t)(tr.pos0 + b0 + tt) * I + (f & ~7) + nib_pos(f & 7)] = (_Float16)hv;
      }
    }
    if constexpr (MULTI)
      if (b0 + 16 < tr.n) __syncthreads();      // red is rewritten by the next block
  }
}

// Down: workgroup = one tile x 64 output rows, wave w rows n0 .. n0+15 over the
// whole K = I (GD = I/128 groups); h16 holds the tile's rows in unpack order,
// so A is a plain load. Rows go to ypair at the pair index t*k + s.
// MXFP4 (FMT): h as its bf16 hi and lo planes, two bf16 MFMAs per slice.
template <int GD, int FMT, bool MULTI>
__global__ __launch_bounds__(BLOCK) void down_g16_kernel(
    const uint8_t* __restrict__ dn, size_t dn_expert_bytes, int drow_bytes, int H, int I,
    const int32_t* __restrict__ pairs, const TileRec* __restrict__ tiles, const _Float16* __restrict__ h16,
    float* __restrict__ ypair, size_t hlo) {
  constexpr bool MX = FMT == FMT_MXFP4;
  constexpr int NH = MX ? GD : (GD + 1) / 2;
  using Hdr = std::conditional_t<MX, u32, u32x4>;
  const int bpt = H / 64;
  const TileRec tr = tiles[blockIdx.x / bpt];
  if (tr.n == 0) return;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int n0 = (int)(blockIdx.x % bpt) * 64 + 16 * w;
  const int r = lane & 15, kg = lane >> 4;
  const uint8_t* row = dn + (size_t)tr.e * dn_expert_bytes + (size_t)(n0 + r) * drow_bytes;
  u32x4 cd[GD];
  Hdr hd[NH];
#pragma unroll
  for (int m = 0; m < GD; ++m) cd[m] = *reinterpret_cast<const u32x4*>(row + 16 * (4 * m + kg));
#pragma unroll
  for (int b = 0; b < NH; ++b) {
    if constexpr (MX) hd[b] = row[I / 2 + 4 * b + kg];
    else hd[b] = *reinterpret_cast<const u32x4*>(row + I / 2 + QHDR * b);
  }
  // the tile's pairs 16 at a time, the weights held in registers
  for (int b0 = 0; b0 < (MULTI ? tr.n : 1); b0 += 16) {
    const int nb = min(16, tr.n - b0);
    // h of tile row t = l%16; rows past the tile's pairs repeat its last row
    // (their outputs are not stored), so the loads are unconditional
    const _Float16* hp = h16 + (size_t)(tr.pos0 + b0 + min(lane & 15, nb - 1)) * I;
    half8 A[MX ? 1 : GD][4];
    if constexpr (!MX) {
#pragma unroll
      for (int m = 0; m < GD; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) A[m][i] = *reinterpret_cast<const half8*>(hp + 32 * (4 * m + kg) + 8 * i);
    }
    // output pair indices of this lane's four accumulator rows (tile rows 4*kg .. 4*kg+3)
    int pr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pr[q] = 4 * kg + q < nb ? pairs[tr.pos0 + b0 + 4 * kg + q] : -1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (MX) {
      const uint16_t* hb = reinterpret_cast<const uint16_t*>(hp);
#pragma unroll
      for (int m = 0; m < GD; ++m) {
        const float sc = e8m0_scale(hd[m]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint16_t* a = hb + 32 * (4 * m + kg) + 8 * i;
          const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(a), alo = *reinterpret_cast<const bf16x8*>(a + hlo);
          const bf16x8 b = fp4x8_bf16(dword_of(cd[m], i), sc);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, acc, 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < GD; ++m) {
        const SubScale sc = sub_scale(hd[m >> 1], (4 * m + kg) & 7);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[m][i], dequant8(dword_of(cd[m], i), sc), acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (pr[q] >= 0) ypair[(size_t)pr[q] * H + n0 + r] = acc[q];
  }
}

// Multi-row gate/up (both encodings: super-block 16-pair tiles above 6
// pairs per expert, MXFP4 tiles of more than 16 pairs up to 6 pairs per
// expert, and wherever I is not a multiple of 64): workgroup = one tile x
// 16*NW row pairs (f0 .. f0 + 16 NW), wave w the K range [w H/4, (w+1) H/4)
// for all NW row blocks; the tile's pairs 16 at a time, each activation slice
// loaded once and used for the NW blocks' gate and up MFMAs, so the
// activations are read I/(16 NW) times per tile instead of I/16. The four
// partial products are added in wave order through LDS, as in the 16-pair
// kernel; h goes to the bf16 hi and lo planes.
template <int G, int NW, int FMT>
__global__ __launch_bounds__(BLOCK) void gateup_g16m_kernel(
    const uint8_t* __restrict__ gu, size_t gu_expert_bytes, int rp_bytes, int H, int I, int k,
    const uint16_t* __restrict__ x, const int32_t* __restrict__ pairs, const TileRec* __restrict__ tiles,
    _Float16* __restrict__ h16, int act, size_t hlo, int ntiles) {
  constexpr bool MX = FMT == FMT_MXFP4;
  constexpr int NH = MX ? G : (G + 1) / 2;     // scale bytes, or super-block headers, per row
  using Hdr = std::conditional_t<MX, u32, u32x4>;
  __shared__ float red[4][2][NW][4][WAVE];
  const int bpt = I / (16 * NW);
  int ti, rb;
  if (!tile_unit(ntiles, bpt, &ti, &rb)) return;
  const TileRec tr = tiles[ti];
  if (tr.n == 0) return;
  const int f0 = rb * 16 * NW;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int r = lane & 15, kg = lane >> 4;
  const int sb0 = w * 4 * G;                    // first 32-block of the wave's K range
  u32x4 cg[NW][G], cu[NW][G];
  Hdr sg[NW][NH], su[NW][NH];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const uint8_t* rec = gu + (size_t)tr.e * gu_expert_bytes + (size_t)(f0 + 16 * j + r) * rp_bytes;
#pragma unroll
    for (int m = 0; m < G; ++m) {
      const int sbi = sb0 + 4 * m + kg;
      cg[j][m] = *reinterpret_cast<const u32x4*>(rec + 16 * sbi);
      cu[j][m] = *reinterpret_cast<const u32x4*>(rec + H / 2 + 16 * sbi);
    }
#pragma unroll
    for (int b = 0; b < NH; ++b) {
      if constexpr (MX) {
        sg[j][b] = rec[H + sb0 + 4 * b + kg];
        su[j][b] = rec[H + H / MXK + sb0 + 4 * b + kg];
      } else {
        const int sup = (sb0 + 8 * b) >> 3;
        sg[j][b] = *reinterpret_cast<const u32x4*>(rec + H + QHDR * sup);
        su[j][b] = *reinterpret_cast<const u32x4*>(rec + H + H / 16 + QHDR * sup);
      }
    }
  }
  for (int b0 = 0; b0 < tr.n; b0 += 16) {
    const int nb = min(16, tr.n - b0);
    // the codes stay the live state across blocks, converted again per block
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
      for (int m = 0; m < G; ++m) asm volatile("" : "+v"(cg[j][m]), "+v"(cu[j][m]));
    const int tok = pairs[tr.pos0 + b0 + min(lane & 15, nb - 1)] / k;
    u32x4 xr[G][4];
#pragma unroll
    for (int m = 0; m < G; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xr[m][i] = *reinterpret_cast<const u32x4*>(x + (size_t)tok * H + 32 * (sb0 + 4 * m + kg) + 8 * i);
    f32x4 accg[NW], accu[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) accg[j] = accu[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < G; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (MX) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, xr[m][i]);
#pragma unroll
          for (int j = 0; j < NW; ++j) {
            accg[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, fp4x8_bf16(dword_of(cg[j][m], i), e8m0_scale(sg[j][m])), accg[j], 0, 0, 0);
            accu[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, fp4x8_bf16(dword_of(cu[j][m], i), e8m0_scale(su[j][m])), accu[j], 0, 0, 0);
          }
        } else {
          const half8 a = bf16x8_to_unpack(xr[m][i]);
          const int sb = (sb0 + 4 * m + kg) & 7;
#pragma unroll
          for (int j = 0; j < NW; ++j) {
            accg[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                a, dequant8(dword_of(cg[j][m], i), sub_scale(sg[j][m >> 1], sb)), accg[j], 0, 0, 0);
            accu[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                a, dequant8(dword_of(cu[j][m], i), sub_scale(su[j][m >> 1], sb)), accu[j], 0, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        red[w][0][j][q][lane] = accg[j][q];
        red[w][1][j][q][lane] = accu[j][q];
      }
    __syncthreads();
    // thread -> (tile row tt, row rr of each block); D[tt][rr] sits in lane rr + 16*(tt/4), register tt%4
    const int tt = tid >> 4, rr = tid & 15;
    if (tt < nb) {
      const int ln = rr + 16 * (tt >> 2), q = tt & 3;
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const float g = ((red[0][0][j][q][ln] + red[1][0][j][q][ln]) + red[2][0][j][q][ln]) + red[3][0][j][q][ln];
        const float u = ((red[0][1][j][q][ln] + red[1][1][j][q][ln]) + red[2][1][j][q][ln]) + red[3][1][j][q][ln];
        const float hv = gate_act(g, u, act);
        const int f = f0 + 16 * j + rr;
        if constexpr (MX) {
          uint16_t* hb = reinterpret_cast<uint16_t*>(h16) + (size_t)(tr.pos0 + b0 + tt) * I + f;
          const uint16_t hi = float_to_bf16_rne(hv);
          hb[0] = hi;
          hb[hlo] = float_to_bf16_rne(hv - bf16_bits_to_float(hi));
        } else {
          h16[(size_t)(tr.pos0 + b0 + tt) * I + (f & ~7) + nib_pos(f & 7)] = (_Float16)hv;
        }
      }
    }
    if (b0 + 16 < tr.n) __syncthreads();        // red is rewritten by the next block
  }
}


// MXFP4 gate/up on tiles of more than 16 pairs between 6 and 12 pairs per
// expert, rows split over the waves: workgroup = one tile x 64 row pairs, wave w rows f0 + 16w .. + 15 (gate and
// up) over the whole K = H with its codes held in registers; each 16-pair
// block of activations is staged in LDS once for the four waves (rows padded
// by 16 bytes), so a tile's activations are read I/64 times and no partial
// sums cross waves.
template <int GK>   // GK = H/128 groups of 128 K
__global__ __launch_bounds__(BLOCK, 2) void gateup_g16r_kernel(
    const uint8_t* __restrict__ gu, size_t gu_expert_bytes, int rp_bytes, int H, int I, int k,
    const uint16_t* __restrict__ x, const int32_t* __restrict__ pairs, const TileRec* __restrict__ tiles,
    _Float16* __restrict__ h16, int act, size_t hlo, int ntiles) {
  constexpr int HK = 128 * GK, LS = HK + 8, CPR = HK / 8;
  __shared__ __align__(16) uint16_t xs[16][LS];
  __shared__ int tok_s[16];
  const int bpt = I / 64;
  int ti, rb;
  if (!tile_unit(ntiles, bpt, &ti, &rb)) return;
  const TileRec tr = tiles[ti];
  if (tr.n == 0) return;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int f0 = rb * 64 + 16 * w;
  const int r = lane & 15, kg = lane >> 4;
  const uint8_t* rec = gu + (size_t)tr.e * gu_expert_bytes + (size_t)(f0 + r) * rp_bytes;
  u32x4 cg[GK], cu[GK];
  u32 sg[GK], su[GK];
#pragma unroll
  for (int m = 0; m < GK; ++m) {
    const int sbi = 4 * m + kg;
    cg[m] = *reinterpret_cast<const u32x4*>(rec + 16 * sbi);
    cu[m] = *reinterpret_cast<const u32x4*>(rec + H / 2 + 16 * sbi);
    sg[m] = rec[H + sbi];
    su[m] = rec[H + H / MXK + sbi];
  }
  for (int b0 = 0; b0 < tr.n; b0 += 16) {
    const int nb = min(16, tr.n - b0);
#pragma unroll
    for (int m = 0; m < GK; ++m) asm volatile("" : "+v"(cg[m]), "+v"(cu[m]));
    if (tid < 16) tok_s[tid] = pairs[tr.pos0 + b0 + min(tid, nb - 1)] / k;
    __syncthreads();
    {
      u32x4 st[16 * CPR / BLOCK];
#pragma unroll
      for (int q = 0; q < 16 * CPR / BLOCK; ++q) {
        const int c = tid + BLOCK * q, row = c / CPR, c8 = c % CPR;
        st[q] = *reinterpret_cast<const u32x4*>(x + (size_t)tok_s[row] * H + 8 * c8);
      }
#pragma unroll
      for (int q = 0; q < 16 * CPR / BLOCK; ++q) {
        const int c = tid + BLOCK * q, row = c / CPR, c8 = c % CPR;
        *reinterpret_cast<u32x4*>(&xs[row][8 * c8]) = st[q];
      }
    }
    __syncthreads();
    f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < GK; ++m) {
      const float scg = e8m0_scale(sg[m]), scu = e8m0_scale(su[m]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&xs[lane & 15][32 * (4 * m + kg) + 8 * i]);
        accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp4x8_bf16(dword_of(cg[m], i), scg), accg, 0, 0, 0);
        accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp4x8_bf16(dword_of(cu[m], i), scu), accu, 0, 0, 0);
      }
    }
    // D[tt][rr]: tile row tt = 4 kg + q, row rr = lane % 16
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tt = 4 * kg + q;
      if (tt < nb) {
        const float hv = gate_act(accg[q], accu[q], act);
        uint16_t* hb = reinterpret_cast<uint16_t*>(h16) + (size_t)(tr.pos0 + b0 + tt) * I + f0 + r;
        const uint16_t hi = float_to_bf16_rne(hv);
        hb[0] = hi;
        hb[hlo] = float_to_bf16_rne(hv - bf16_bits_to_float(hi));
      }
    }
    if (b0 + 16 < tr.n) __syncthreads();          // xs and tok_s are rewritten by the next block
  }
}


// MXFP4 down on tiles of more than 16 pairs: workgroup = one tile x
// 4*NW*16 output rows, wave w the NW blocks of 16 rows from
// n0 = (256*NW/4)*fb + 16*NW*w over the whole K = I; the tile's pairs 16 at a
// time, each slice of h (hi and lo planes) loaded once and used for all NW
// row blocks, so h is read H/(64 NW) times per tile instead of H/16.
// MXFP4 gate/up above 12 pairs per expert (tiles of up to 128 pairs), K
// outermost: workgroup = one
// tile x 64 row pairs (wave w: rows f0 + 16w .. + 15, gate and up). K runs
// in chunks of 128: the tile's activations for the chunk are staged in LDS
// (rows padded by 16 bytes) while the next chunk is loaded into registers,
// and each wave converts its 32-wide code slices once per chunk and feeds
// every 16-pair block of the tile from that one conversion, with one
// accumulator pair per block. The K order of the sums is the same as in the
// row-split kernel (ascending 32-blocks).
constexpr int KCH = 128, KCM = KCH / 128;
template <int NBR, int MT>   // NBR = 16-pair blocks this tile fills (the MFMAs run unconditionally)
__device__ __forceinline__ void g16k_body(const uint8_t* __restrict__ rec, int H, int I, const uint16_t* __restrict__ x,
                                          const TileRec& tr, _Float16* __restrict__ h16, int act, size_t hlo,
                                          int f0, uint16_t (*xs)[KCH + 8], const int* tok_s) {
  constexpr int CPR = KCH / 8, NST = 16 * NBR * CPR / BLOCK;
  static_assert(NST * BLOCK == 16 * NBR * CPR || NBR < 2, "staging split");
  constexpr int NSTX = NST > 0 ? NST : 1;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int r = lane & 15, kg = lane >> 4;
  // staging unit c = tid + BLOCK q: row c / CPR, 16-byte column c % CPR.
  // The row guards below always hold (the units cover exactly 16 NBR rows);
  // they stay because without them the compiler schedules the staging so
  // that the kernel needs 174 registers instead of 163, two waves per SIMD
  // instead of three.
  u32x4 st[NSTX];
  auto load_x = [&](int c0) {
#pragma unroll
    for (int q = 0; q < NSTX; ++q) {
      const int c = tid + BLOCK * q, row = c / CPR;
      if (row < 16 * NBR)
        st[q] = *reinterpret_cast<const u32x4*>(x + (size_t)tok_s[row] * H + c0 + 8 * (c % CPR));
    }
  };
  u32x4 cg[KCM], cu[KCM];
  u32 sg[KCM], su[KCM];
  auto load_codes = [&](int c0) {
#pragma unroll
    for (int m = 0; m < KCM; ++m) {
      const int sbi = c0 / MXK + 4 * m + kg;
      cg[m] = *reinterpret_cast<const u32x4*>(rec + 16 * sbi);
      cu[m] = *reinterpret_cast<const u32x4*>(rec + H / 2 + 16 * sbi);
      sg[m] = rec[H + sbi];
      su[m] = rec[H + H / MXK + sbi];
    }
  };
  f32x4 accg[NBR], accu[NBR];
#pragma unroll
  for (int b = 0; b < NBR; ++b) accg[b] = accu[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  load_x(0);
  load_codes(0);
  for (int c0 = 0; c0 < H; c0 += KCH) {
    if (c0) __syncthreads();                        // the previous chunk's reads of xs are done
#pragma unroll
    for (int q = 0; q < NSTX; ++q) {
      const int c = tid + BLOCK * q, row = c / CPR;
      if (row < 16 * NBR) *reinterpret_cast<u32x4*>(&xs[row][8 * (c % CPR)]) = st[q];
    }
    __syncthreads();
    u32x4 ncg[KCM], ncu[KCM];
    u32 nsg[KCM], nsu[KCM];
#pragma unroll
    for (int m = 0; m < KCM; ++m) { ncg[m] = cg[m]; ncu[m] = cu[m]; nsg[m] = sg[m]; nsu[m] = su[m]; }
    if (c0 + KCH < H) {
      load_x(c0 + KCH);
      load_codes(c0 + KCH);
    }
#pragma unroll
    for (int m = 0; m < KCM; ++m) {
      const float scg = e8m0_scale(nsg[m]), scu = e8m0_scale(nsu[m]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 bg = fp4x8_bf16(dword_of(ncg[m], i), scg);
        const bf16x8 bu = fp4x8_bf16(dword_of(ncu[m], i), scu);
#pragma unroll
        for (int b = 0; b < NBR; ++b) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&xs[16 * b + r][128 * m + 32 * kg + 8 * i]);
          accg[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bg, accg[b], 0, 0, 0);
          accu[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bu, accu[b], 0, 0, 0);
        }
      }
    }
  }
  // D[tt][rr] of block b: pair 16 b + tt, tt = 4 kg + q; row rr = lane % 16
#pragma unroll
  for (int b = 0; b < NBR; ++b) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = 16 * b + 4 * kg + q;
      const float hv = gate_act(accg[b][q], accu[b][q], act);
      if (p < tr.n) {
        uint16_t* hb = reinterpret_cast<uint16_t*>(h16) + (size_t)(tr.pos0 + p) * I + f0 + r;
        const uint16_t hi = float_to_bf16_rne(hv);
        hb[0] = hi;
        hb[hlo] = float_to_bf16_rne(hv - bf16_bits_to_float(hi));
      }
    }
  }
}

template <int NB>   // up to 16 NB pairs per tile
__global__ __launch_bounds__(BLOCK, 2) void gateup_g16k_kernel(
    const uint8_t* __restrict__ gu, size_t gu_expert_bytes, int rp_bytes, int H, int I, int k,
    const uint16_t* __restrict__ x, const int32_t* __restrict__ pairs, const TileRec* __restrict__ tiles,
    _Float16* __restrict__ h16, int act, size_t hlo, int ntiles) {
  constexpr int MT = 16 * NB;
  __shared__ __align__(16) uint16_t xs[MT][KCH + 8];
  __shared__ int tok_s[MT];
  const int bpt = I / 64;
  int ti, rb;
  if (!tile_unit(ntiles, bpt, &ti, &rb)) return;
  const TileRec tr = tiles[ti];
  if (tr.n == 0) return;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int f0 = rb * 64 + 16 * w;
  const uint8_t* rec = gu + (size_t)tr.e * gu_expert_bytes + (size_t)(f0 + (tid & 15)) * rp_bytes;
  if (tid < MT) tok_s[tid] = pairs[tr.pos0 + min(tid, tr.n - 1)] / k;
  __syncthreads();
  const int nblk = (tr.n + 15) >> 4;               // uniform over the workgroup
  if (NB >= 8 && nblk > 4) g16k_body<8, MT>(rec, H, I, x, tr, h16, act, hlo, f0, xs, tok_s);
  else if (nblk > 2) g16k_body<4, MT>(rec, H, I, x, tr, h16, act, hlo, f0, xs, tok_s);
  else if (nblk > 1) g16k_body<2, MT>(rec, H, I, x, tr, h16, act, hlo, f0, xs, tok_s);
  else g16k_body<1, MT>(rec, H, I, x, tr, h16, act, hlo, f0, xs, tok_s);
}

template <int GD, int NW, int FMT>
__global__ __launch_bounds__(BLOCK) void down_g16m_kernel(
    const uint8_t* __restrict__ dn, size_t dn_expert_bytes, int drow_bytes, int H, int I,
    const int32_t* __restrict__ pairs, const TileRec* __restrict__ tiles, const _Float16* __restrict__ h16,
    float* __restrict__ ypair, size_t hlo, int ntiles) {
  constexpr bool MX = FMT == FMT_MXFP4;
  constexpr int NH = MX ? GD : (GD + 1) / 2;
  using Hdr = std::conditional_t<MX, u32, u32x4>;
  // a block's 16 rows of h (MXFP4: hi and lo planes) staged in LDS once for
  // the four waves; rows padded by 16 bytes against bank conflicts
  constexpr int PL = MX ? 2 : 1, IK = 128 * GD, LS = IK + 8, CPR = IK / 8;
  __shared__ __align__(16) uint16_t hs[PL][16][LS];
  const int bpt = H / (64 * NW);
  int ti, rb;
  if (!tile_unit(ntiles, bpt, &ti, &rb)) return;
  const TileRec tr = tiles[ti];
  if (tr.n == 0) return;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int n0 = rb * 64 * NW + 16 * NW * w;
  const int r = lane & 15, kg = lane >> 4;
  const uint8_t* base = dn + (size_t)tr.e * dn_expert_bytes;
  u32x4 cd[NW][GD];
  Hdr sc[NW][NH];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const uint8_t* row = base + (size_t)(n0 + 16 * j + r) * drow_bytes;
#pragma unroll
    for (int m = 0; m < GD; ++m) cd[j][m] = *reinterpret_cast<const u32x4*>(row + 16 * (4 * m + kg));
#pragma unroll
    for (int b = 0; b < NH; ++b) {
      if constexpr (MX) sc[j][b] = row[I / 2 + 4 * b + kg];
      else sc[j][b] = *reinterpret_cast<const u32x4*>(row + I / 2 + QHDR * b);
    }
  }
  for (int b0 = 0; b0 < tr.n; b0 += 16) {
    const int nb = min(16, tr.n - b0);
    // the codes stay the live state across blocks, converted again per block
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
      for (int m = 0; m < GD; ++m) asm volatile("" : "+v"(cd[j][m]));
    {
      // thread -> one (plane, row) and every TPR-th 16-byte column of it:
      // one address per thread, the rest immediate offsets
      constexpr int TPR = BLOCK / (PL * 16), NQ = CPR / TPR;
      static_assert(CPR % TPR == 0, "h staging split");
      const int prw = tid / TPR, pl = prw / 16, row = prw % 16, col0 = tid % TPR;
      const uint16_t* src = reinterpret_cast<const uint16_t*>(h16) + (pl ? hlo : 0) +
                            (size_t)(tr.pos0 + b0 + min(row, nb - 1)) * I + 8 * col0;
      u32x4 st[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) st[q] = *reinterpret_cast<const u32x4*>(src + 8 * TPR * q);
#pragma unroll
      for (int q = 0; q < NQ; ++q) *reinterpret_cast<u32x4*>(&hs[pl][row][8 * col0 + 8 * TPR * q]) = st[q];
      __syncthreads();
    }
    int pr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pr[q] = 4 * kg + q < nb ? pairs[tr.pos0 + b0 + 4 * kg + q] : -1;
    f32x4 acc[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < GD; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t* a = &hs[0][lane & 15][32 * (4 * m + kg) + 8 * i];
        if constexpr (MX) {
          const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(a);
          const bf16x8 alo = *reinterpret_cast<const bf16x8*>(a + 16 * LS);   // the lo plane
#pragma unroll
          for (int j = 0; j < NW; ++j) {
            const bf16x8 b = fp4x8_bf16(dword_of(cd[j][m], i), e8m0_scale(sc[j][m]));
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, acc[j], 0, 0, 0);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, acc[j], 0, 0, 0);
          }
        } else {
          // h16 holds fp16 h in unpack order
          const half8 ah = *reinterpret_cast<const half8*>(a);
          const int sb = (4 * m + kg) & 7;
#pragma unroll
          for (int j = 0; j < NW; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, dequant8(dword_of(cd[j][m], i), sub_scale(sc[j][m >> 1], sb)),
                                                           acc[j], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (pr[q] >= 0) ypair[(size_t)pr[q] * H + n0 + 16 * j + r] = acc[j][q];
    if (b0 + 16 < tr.n) __syncthreads();          // hs is rewritten by the next block
  }
}

// rows: the multi-row kernels (2 / 4 blocks of 16 rows per wave), which read
// a tile's activations and h fewer times but run fewer workgroups: always
// for tiles of more than 16 pairs, and for 16-pair tiles above 6 pairs per
// expert (super-block weights, Qwen3-30B-A3B shape, same box: at 64 tokens
// 109 / 112 us without / with, at 128 and 192 tokens 123 / 119 and 146 / 133).
template <int G, int GD, int FMT, bool MULTI>
static hipError_t launch_g16_f(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* pairs,
                               const TileRec* tiles, int ntiles, _Float16* h16, float* ypair, size_t hlo,
                               int rows, hipStream_t s) {
  constexpr int NWG = 2;                         // row blocks per wave of the multi-row gate/up
  if (FMT == FMT_MXFP4 && MULTI && rows == 3 && d.I % 64 == 0)
    hipLaunchKernelGGL((gateup_g16k_kernel<8>), dim3(tile_unit_grid(ntiles, d.I / 64)), dim3(BLOCK), 0, s,
                       layer + d.gu_off, d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.k, x, pairs, tiles, h16,
                       d.act, hlo, ntiles);
  else if (FMT == FMT_MXFP4 && MULTI && rows >= 2 && d.I % 64 == 0)
    hipLaunchKernelGGL((gateup_g16r_kernel<4 * G>), dim3(tile_unit_grid(ntiles, d.I / 64)), dim3(BLOCK), 0, s,
                       layer + d.gu_off, d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.k, x, pairs, tiles, h16,
                       d.act, hlo, ntiles);
  else if (MULTI || rows)
    hipLaunchKernelGGL((gateup_g16m_kernel<G, NWG, FMT>), dim3(tile_unit_grid(ntiles, d.I / (16 * NWG))), dim3(BLOCK),
                       0, s, layer + d.gu_off, d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.k, x, pairs, tiles, h16,
                       d.act, hlo, ntiles);
  else
    hipLaunchKernelGGL((gateup_g16_kernel<G, FMT, MULTI>), dim3(ntiles * (d.I / 16)), dim3(BLOCK), 0, s,
                       layer + d.gu_off, d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.k, x, pairs, tiles, h16,
                       d.act, hlo);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int NW = 4;                          // row blocks per wave of the multi-row down
  if (MULTI || rows) {
    if (d.H % (64 * NW) == 0) {
      hipLaunchKernelGGL((down_g16m_kernel<GD, NW, FMT>), dim3(tile_unit_grid(ntiles, d.H / (64 * NW))), dim3(BLOCK),
                         0, s, layer + d.dn_off, d.dn_expert_bytes, (int)d.drow_bytes, d.H, d.I, pairs, tiles, h16,
                         ypair, hlo, ntiles);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((down_g16_kernel<GD, FMT, MULTI>), dim3(ntiles * (d.H / 64)), dim3(BLOCK), 0, s,
                     layer + d.dn_off, d.dn_expert_bytes, (int)d.drow_bytes, d.H, d.I, pairs, tiles, h16, ypair, hlo);
  return hipGetLastError();
}

// hlo: elements from the hi plane of h to its lo plane (MXFP4 only)
template <int G, int GD>
static hipError_t launch_g16(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* pairs,
                             const TileRec* tiles, int ntiles, _Float16* h16, float* ypair, size_t hlo, bool multi,
                             int rows, hipStream_t s) {
  if (d.fmt != FMT_MXFP4)
    return launch_g16_f<G, GD, FMT_Q4K, false>(d, layer, x, pairs, tiles, ntiles, h16, ypair, hlo, rows, s);
  if (multi) return launch_g16_f<G, GD, FMT_MXFP4, true>(d, layer, x, pairs, tiles, ntiles, h16, ypair, hlo, rows, s);
  return launch_g16_f<G, GD, FMT_MXFP4, false>(d, layer, x, pairs, tiles, ntiles, h16, ypair, hlo, rows, s);
}

template <int G>
static hipError_t launch_g16_i(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* pairs,
                               const TileRec* tiles, int ntiles, _Float16* h16, float* ypair, size_t hlo,
                               bool multi, int rows, hipStream_t s) {
  switch (d.I) {
    case 256: return launch_g16<G, 2>(d, layer, x, pairs, tiles, ntiles, h16, ypair, hlo, multi, rows, s);
    case 512: return launch_g16<G, 4>(d, layer, x, pairs, tiles, ntiles, h16, ypair, hlo, multi, rows, s);
    case 768: return launch_g16<G, 6>(d, layer, x, pairs, tiles, ntiles, h16, ypair, hlo, multi, rows, s);
    case 1024: return launch_g16<G, 8>(d, layer, x, pairs, tiles, ntiles, h16, ypair, hlo, multi, rows, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace grouped

int grouped_mt(const Layout& d, int T) { return (long long)T * d.k >= 64LL * d.E ? 96 : 32; }

int grouped_max_tiles(const Layout& d, int T) {
  const int mt = grouped_mt(d, T);
  return (T * d.k + mt - 1) / mt + d.E;
}

hipError_t launch_grouped_ffn(const Layout& d, const uint8_t* layer, const uint16_t* x, const float* w,
                              const int32_t* offsets, const int32_t* pairs, const int32_t* tile_off, _Float16* h16,
                              float* ypair, float* out, int T, hipStream_t s) {
  using namespace grouped;
  if (d.I % FB || d.H % FD) return hipErrorInvalidValue;
  const hipError_t e = grouped_mt(d, T) == 96 ? launch_wr<3>(d, layer, x, offsets, pairs, tile_off, h16, ypair, T, s)
                                               : launch_wr<1>(d, layer, x, offsets, pairs, tile_off, h16, ypair, T, s);
  if (e != hipSuccess) return e;
  return launch_combine(d, ypair, w, out, T, s);
}

hipError_t launch_combine(const Layout& d, const float* ypair, const float* w, float* out, int T, hipStream_t s) {
  using namespace grouped;
  if (T <= 0) return hipSuccess;
  const int n4 = T * (d.H / 4);
  hipLaunchKernelGGL(combine_kernel, dim3((n4 + BLOCK - 1) / BLOCK), dim3(BLOCK), 0, s, ypair, w, out, d.H, d.k, T);
  return hipGetLastError();
}

bool g16_supported(const Layout& d) {
  return (d.H == 512 || d.H == 1024 || d.H == 2048) && d.I <= 1024;
}

// Pairs per tile: 16; MXFP4 (whose only MFMA path this is) takes 64 above
// one pair per expert and 128 above 16, walked by the multi-block kernels
// (measured on the Qwen3-30B-A3B-shaped layer: at 41 / 96 / 128 tokens
// 108 / 122 / 126 us against 123 / 151 / 166 us on 16-pair tiles).
int g16_mt(const Layout& d, int T) {
  if (d.fmt != FMT_MXFP4) return 16;
  const long long P = (long long)T * d.k;
  return P <= d.E ? 16 : (P <= 16LL * d.E ? 64 : 128);
}

int g16_max_tiles(const Layout& d, int T) {
  const int P = T * d.k, mt = g16_mt(d, T);
  return (P + mt - 1) / mt + (P < d.E ? P : d.E);
}

hipError_t launch_g16_ffn(const Layout& d, const uint8_t* layer, const uint16_t* x, const float* w,
                          const int32_t* pairs, const void* tiles, _Float16* h16, float* ypair, float* out, int T,
                          hipStream_t s) {
  using namespace grouped;
  if (!g16_supported(d)) return hipErrorInvalidValue;
  if (T <= 0) return hipSuccess;
  const TileRec* tr = static_cast<const TileRec*>(tiles);
  const int nt = g16_max_tiles(d, T);
  // MXFP4: h's bf16 lo plane follows the hi plane (scratch holds 4 bytes per value)
  const size_t hlo = (size_t)T * d.k * d.I;
  const bool multi = g16_mt(d, T) > 16;
  // 0: one row block per wave; 1: multi-row kernels; 2: above 6 pairs per
  // expert, where the MXFP4 gate/up splits rows over the waves (fewer
  // workgroups per tile: a loss below that, measured at 32-64 tokens); 3:
  // above 12 pairs per expert, where it runs K outermost and reuses each
  // converted code slice for all of a tile's blocks (tiles of one block,
  // common below that, gain nothing and pay a barrier pair per 128 K)
  const long long P = (long long)T * d.k;
  const int rows = P > 12LL * d.E ? 3 : (P > 6LL * d.E ? 2 : (multi ? 1 : 0));
  hipError_t e;
  switch (d.H) {
    case 512: e = launch_g16_i<1>(d, layer, x, pairs, tr, nt, h16, ypair, hlo, multi, rows, s); break;
    case 1024: e = launch_g16_i<2>(d, layer, x, pairs, tr, nt, h16, ypair, hlo, multi, rows, s); break;
    default: e = launch_g16_i<4>(d, layer, x, pairs, tr, nt, h16, ypair, hlo, multi, rows, s); break;
  }
  if (e != hipSuccess) return e;
  return launch_combine(d, ypair, w, out, T, s);
}

}  // namespace qmoe

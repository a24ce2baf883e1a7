// gfx950 kernels of the batched path: grouped expert GEMMs on the MFMA
// units for token batches routed to the same expert.
//
// The pages' batched prefill dequantizes the 4-bit super-blocks into the GEMM
// operand and shares one weight read across a chunk of tokens (SP⚡RKINFER
// README, Qwen3.8-27B prefill notes; sparkinfer-k3 release log, batched
// prompt ingestion); this is our CDNA4 form of it. Tokens are grouped by
// expert on the device (dispatch lists); a tile holds 16, 64 or 128 routed
// pairs of one expert and is walked 16 pairs at a time on
// v_mfma_f32_16x16x32_bf16 (lane layouts checked on the box:
// A[l%16][8(l/16)+e], B[8(l/16)+e][l%16], D[4(l/16)+r][l%16]).
//
// Every MFMA operand is exact, so the only roundings are fp32 accumulation
// and the storage of h:
//  - activations: the bf16 inputs as they are;
//  - MXFP4 weights: each code converted together with its block's E8M0 scale
//    to the exact weight as a bf16 (scale codes 2..252 keep it normal);
//  - 4-bit super-block weights: each code converted to the exact bf16 value q;
//    one MFMA covers one 32-weight sub-block, P = A·q, the MFMA against ones
//    gives S = A·1, and the sub-block affine (a = d*sc, b = dmin*m, weight =
//    a q - b) is applied in fp32: acc += a P - b S;
//  - h = act(gate, up) is stored as two bf16 planes, hi = bf16(h) and lo =
//    bf16(h - hi), so h = hi + lo to about 2^-17 relative with bf16's (fp32's)
//    exponent range; the down GEMM runs its MFMAs on both planes.
// Down writes one fp32 row per (token, slot) pair and the routing-weighted
// combine sums them in slot order (deterministic).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moe_device.h"

namespace qmoe {
namespace grouped {

typedef unsigned int u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Work record of one tile, written by the dispatch: expert, first position
// in the expert-sorted pair list, pairs (0 past the last tile).
struct TileRec { int e, pos0, n, pad; };

// Work unit of a multi-row workgroup: tiles are dealt to the XCDs
// round-robin (tile t to XCD t % 8, so empty tiles spread evenly) and the
// bpt row blocks of one tile follow each other on that XCD, so the tile's
// activations (or h) are fetched into one L2 and re-read from there.
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

__device__ __forceinline__ u32 dword_of(const u32x4& c, int i) {
  return i == 0 ? c.x : (i == 1 ? c.y : (i == 2 ? c.z : c.w));
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr f32x4 ZERO4 = {0.f, 0.f, 0.f, 0.f};

// Materializes accumulators in registers at this point. Where the final
// value is stored only under a condition, the compiler otherwise sinks the
// whole fp32 epilogue chain (every sub-block's MFMA result kept live) into
// the conditional store, which spilled hundreds of registers.
template <int N = 1>
__device__ __forceinline__ void pin(f32x4* acc) {
#pragma unroll
  for (int j = 0; j < N; ++j) asm volatile("" : "+v"(acc[j]));
}

// ------------------------------------------------------------------ MXFP4 operands
// The eight weights of one code dword, converted with the block's scale to
// exact bf16 values, natural K order.
__device__ __forceinline__ bf16x8 fp4x8_bf16(u32 v, float scale) {
  u32x4 o;
  o.x = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0));
  o.y = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1));
  o.z = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2));
  o.w = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3));
  return __builtin_bit_cast(bf16x8, o);
}

// ------------------------------------------------------------------ 4-bit super-block operands
// The eight codes of one dword as exact bf16 values q, in unpack order
// (elements 0,2,4,6,1,3,5,7 of the dword's eight): the masked low and high
// nibbles, read as FP8 E4M3 bytes and converted with scale 2^9 (q exactly).
__device__ __forceinline__ bf16x8 codes8_bf16(u32 v) {
  const u32 lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
  u32x4 o;
  o.x = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false));   // (q0, q2)
  o.y = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true));    // (q4, q6)
  o.z = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false));   // (q1, q3)
  o.w = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true));    // (q5, q7)
  return __builtin_bit_cast(bf16x8, o);
}

// Eight bf16 values (16 bytes, natural order) in unpack order.
__device__ __forceinline__ u32x4 unpack_order(const u32x4& v) {
  u32x4 o;
  o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);   // (e0, e2)
  o.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);   // (e4, e6)
  o.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);   // (e1, e3)
  o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);   // (e5, e7)
  return o;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// bf16 (1, ..., 1): B operand of the MFMA that sums each A row.
__device__ __forceinline__ bf16x8 ones8() {
  const u32 one2 = 0x3F803F80u;
  return __builtin_bit_cast(bf16x8, u32x4{one2, one2, one2, one2});
}

// 4x4 transpose of code dwords over the four 16-lane groups: on entry lane
// group g holds the 16-byte chunk (dwords 0..3) of sub-block s_g; on exit
// dword s of lane group g holds dword g of sub-block s_s, so one MFMA on
// dword s covers exactly sub-block s_s (its 32 K values spread over the
// lane groups as the MFMA layout wants). permlane16_swap exchanges the odd
// 16-lane rows of its first operand with the even rows of its second,
// permlane32_swap the upper half of the first with the lower half of the
// second (checked on the box).
__device__ __forceinline__ void transpose4(u32x4& c) {
  const auto a = __builtin_amdgcn_permlane16_swap(c.x, c.y, false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(c.z, c.w, false, false);
  const auto e = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
  const auto f = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
  c = u32x4{e[0], f[0], e[1], f[1]};
}

// A value held per lane group g (v_g) gathered into every lane: out[s] = v_s.
__device__ __forceinline__ void allgather4(float v, float* out) {
  const u32 x = __builtin_bit_cast(u32, v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);   // (v0 v0 v2 v2), (v1 v1 v3 v3)
  const auto b = __builtin_amdgcn_permlane32_swap(a[0], a[0], false, false);   // v0, v2
  const auto c = __builtin_amdgcn_permlane32_swap(a[1], a[1], false, false);   // v1, v3
  // as_f32 takes the element by value: a bit cast of the vector element
  // itself read element 0 for both (checked on the box)
  out[0] = as_f32(b[0]);
  out[1] = as_f32(c[0]);
  out[2] = as_f32(b[1]);
  out[3] = as_f32(c[1]);
}

// Sub-block affines (a = d*sc, b = dmin*m) of four consecutive sub-blocks of
// one weight row: lane group g decodes sub-block sb_own (the chunk it loaded)
// from its super-block header, then every lane gets all four.
struct Affine4 { float a[4], b[4]; };
__device__ __forceinline__ Affine4 affine4(const u32x4& hdr, int sb_own) {
  const Affine af = header_affine(hdr, sb_own & 7);
  Affine4 r;
  allgather4(af.a, r.a);
  allgather4(af.b, r.b);
  return r;
}

// acc += a (A·q) - b (A·1) over one sub-block: P = A·q on the MFMA from zero,
// S = A·1 given, the affine in fp32.
__device__ __forceinline__ void q4k_step(f32x4& acc, const bf16x8& A, u32 codes, float a, float b, const f32x4& S) {
  const f32x4 P = mfma(A, codes8_bf16(codes), ZERO4);
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = fmaf(a, P[q], fmaf(-b, S[q], acc[q]));
}

// The same for h given as two bf16 planes (A = Ahi + Alo).
__device__ __forceinline__ void q4k_step2(f32x4& acc, const bf16x8& Ahi, const bf16x8& Alo, u32 codes, float a,
                                          float b, const f32x4& S) {
  const bf16x8 B = codes8_bf16(codes);
  const f32x4 P = mfma(Alo, B, mfma(Ahi, B, ZERO4));
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = fmaf(a, P[q], fmaf(-b, S[q], acc[q]));
}

// Position of intermediate row f in a 4-bit super-block h row: unpack order
// within each group of 8 (the down kernels' A operand order).
__device__ __forceinline__ int nib_pos(int e) { return (e >> 1) + 4 * (e & 1); }

// h = hv stored as bf16 hi and lo planes (lo plane hlo elements after hi).
__device__ __forceinline__ void store_h(uint16_t* hb, size_t hlo, float hv) {
  const uint16_t hi = float_to_bf16_rne(hv);
  hb[0] = hi;
  hb[hlo] = float_to_bf16_rne(hv - bf16_bits_to_float(hi));
}

template <int FMT>
__device__ __forceinline__ size_t h_index(size_t pos, int I, int f) {
  return pos * I + (FMT == FMT_MXFP4 ? f : (f & ~7) + nib_pos(f & 7));
}

// ------------------------------------------------------------------ gate/up, one 16-pair block
// Workgroup = one tile of at most 16 pairs x 16 row pairs (intermediate rows
// f0 .. f0+15); wave w takes K range [w*H/4, (w+1)*H/4), G = H/512 groups of
// 128 K; lane (row r = l%16, kg = l/16) loads the 16-byte code chunk of
// block 4m + kg of group m (MXFP4: with its scale byte; super-blocks: then
// transposed so that each MFMA covers one sub-block). The four partial
// products are added in wave order through LDS, then act(gate, up) goes to h
// at the pairs' sorted positions.
template <int G, int FMT>
__global__ __launch_bounds__(BLOCK) void gateup_g16_kernel(
    const uint8_t* __restrict__ gu, size_t gu_expert_bytes, int rp_bytes, int H, int I, int k,
    const uint16_t* __restrict__ x, const int32_t* __restrict__ pairs, const TileRec* __restrict__ tiles,
    uint16_t* __restrict__ hb, int act, size_t hlo) {
  constexpr bool MX = FMT == FMT_MXFP4;
  // MXFP4: one scale byte per group; super-blocks: one header per two groups
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
  const int sb0 = w * 4 * G;                    // first 32-block of the wave's K range
  // token of tile row l%16 first: loads complete in order, so the activation
  // loads, which wait on it, must not queue behind the weights. Rows past
  // the tile's pairs repeat its last row (their outputs are not stored), so
  // every load is unconditional.
  const int tok = pairs[tr.pos0 + min(lane & 15, tr.n - 1)] / k;
  __builtin_amdgcn_sched_barrier(0);
  // weights: row f0 + r; gate codes at 0, up codes at H/2, gate headers at H, up headers after them
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
      const int sbi = sb0 + 4 * b + kg;
      hg[b] = rec[H + sbi];
      hu[b] = rec[H + H / MXK + sbi];
    } else {
      const int sup = (sb0 + 8 * b) >> 3;
      hg[b] = *reinterpret_cast<const u32x4*>(rec + H + QHDR * sup);
      hu[b] = *reinterpret_cast<const u32x4*>(rec + H + H / 16 + QHDR * sup);
    }
  }
  // activations: MXFP4 lane group kg holds block 4m + kg whole (natural
  // order); super-blocks: 8 values of each sub-block 4m + i (K positions of
  // its lane group after the transpose)
  u32x4 xr[G][4];
#pragma unroll
  for (int m = 0; m < G; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xr[m][i] = *reinterpret_cast<const u32x4*>(
          x + (size_t)tok * H + (MX ? 32 * (sb0 + 4 * m + kg) + 8 * i : 32 * (sb0 + 4 * m + i) + 8 * kg));
  __builtin_amdgcn_sched_barrier(0);            // every load is in flight before the first use
  f32x4 accg = ZERO4, accu = ZERO4;
  if constexpr (MX) {
#pragma unroll
    for (int m = 0; m < G; ++m) {
      const float sg = e8m0_scale(hg[m]), su = e8m0_scale(hu[m]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 a = as_bf16x8(xr[m][i]);
        accg = mfma(a, fp4x8_bf16(dword_of(cg[m], i), sg), accg);
        accu = mfma(a, fp4x8_bf16(dword_of(cu[m], i), su), accu);
      }
    }
  } else {
    const bf16x8 one = ones8();
#pragma unroll
    for (int m = 0; m < G; ++m) {
      transpose4(cg[m]);
      transpose4(cu[m]);
      const Affine4 ag = affine4(hg[m >> 1], sb0 + 4 * m + kg), au = affine4(hu[m >> 1], sb0 + 4 * m + kg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 a = as_bf16x8(unpack_order(xr[m][i]));
        const f32x4 S = mfma(a, one, ZERO4);
        q4k_step(accg, a, dword_of(cg[m], i), ag.a[i], ag.b[i], S);
        q4k_step(accu, a, dword_of(cu[m], i), au.a[i], au.b[i], S);
      }
      pin(&accg);
      pin(&accu);
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
  if (tt < tr.n) {
    const int ln = rr + 16 * (tt >> 2), q = tt & 3;
    const float g = ((red[0][0][q][ln] + red[1][0][q][ln]) + red[2][0][q][ln]) + red[3][0][q][ln];
    const float u = ((red[0][1][q][ln] + red[1][1][q][ln]) + red[2][1][q][ln]) + red[3][1][q][ln];
    store_h(hb + h_index<FMT>((size_t)tr.pos0 + tt, I, f0 + rr), hlo, gate_act(g, u, act));
  }
}

// ------------------------------------------------------------------ gate/up, multi-row
// Multi-row gate/up (tiles of more than 16 pairs, and 16-pair tiles above a
// few pairs per expert): workgroup = one tile x 16*NW row pairs (f0 ..
// f0 + 16 NW), wave w the K range [w H/4, (w+1) H/4) for all NW row blocks;
// the tile's pairs 16 at a time, each activation slice loaded once and used
// for the NW blocks' gate and up MFMAs, so the activations are read
// I/(16 NW) times per tile instead of I/16. The four partial products are
// added in wave order through LDS, as in the one-block kernel.
template <int G, int NW, int FMT>
__global__ __launch_bounds__(BLOCK) void gateup_g16m_kernel(
    const uint8_t* gu, size_t gu_expert_bytes, int rp_bytes, int H, int I, int k,
    const uint16_t* x, const int32_t* pairs, const TileRec* __restrict__ tiles,
    uint16_t* __restrict__ hb, int act, size_t hlo, int ntiles) {
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
  // the activations of a 16-pair block come at the end of a dependent chain
  // (token ids, then activations): the first block's ids leave before the
  // weights, its activations as soon as the ids arrive (before the code
  // transposes wait for the weights), and each later block's ids and
  // activations while the block before it is reduced and stored
  int pid = pairs[tr.pos0 + min(lane & 15, min(16, tr.n) - 1)];
  u32x4 xr[G][4];
  auto load_x = [&](int tok) {
#pragma unroll
    for (int m = 0; m < G; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xr[m][i] = *reinterpret_cast<const u32x4*>(
            x + (size_t)tok * H + (MX ? 32 * (sb0 + 4 * m + kg) + 8 * i : 32 * (sb0 + 4 * m + i) + 8 * kg));
  };
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
  // compiler fences (no instruction): the loads above stay above, instead
  // of being sunk to their first uses behind the code transposes
  asm volatile("" ::: "memory");
  load_x(pid / k);
  asm volatile("" ::: "memory");
  if constexpr (!MX) {
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
      for (int m = 0; m < G; ++m) { transpose4(cg[j][m]); transpose4(cu[j][m]); }
  }
  const bf16x8 one = ones8();
  for (int b0 = 0; b0 < tr.n; b0 += 16) {
    const int nb = min(16, tr.n - b0);
    const bool more = b0 + 16 < tr.n;
    // the next block's token ids
    if (more) pid = pairs[tr.pos0 + b0 + 16 + min(lane & 15, min(16, tr.n - b0 - 16) - 1)];
    // the codes stay the live state across blocks, converted again per block
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
      for (int m = 0; m < G; ++m) asm volatile("" : "+v"(cg[j][m]), "+v"(cu[j][m]));
    f32x4 accg[NW], accu[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) accg[j] = accu[j] = ZERO4;
#pragma unroll
    for (int m = 0; m < G; ++m) {
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 a = as_bf16x8(xr[m][i]);
#pragma unroll
          for (int j = 0; j < NW; ++j) {
            accg[j] = mfma(a, fp4x8_bf16(dword_of(cg[j][m], i), e8m0_scale(sg[j][m])), accg[j]);
            accu[j] = mfma(a, fp4x8_bf16(dword_of(cu[j][m], i), e8m0_scale(su[j][m])), accu[j]);
          }
        }
      } else {
        Affine4 ag[NW], au[NW];
#pragma unroll
        for (int j = 0; j < NW; ++j) {
          ag[j] = affine4(sg[j][m >> 1], sb0 + 4 * m + kg);
          au[j] = affine4(su[j][m >> 1], sb0 + 4 * m + kg);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 a = as_bf16x8(unpack_order(xr[m][i]));
          const f32x4 S = mfma(a, one, ZERO4);
#pragma unroll
          for (int j = 0; j < NW; ++j) {
            q4k_step(accg[j], a, dword_of(cg[j][m], i), ag[j].a[i], ag[j].b[i], S);
            q4k_step(accu[j], a, dword_of(cu[j][m], i), au[j].a[i], au[j].b[i], S);
          }
        }
        pin<NW>(accg);
        pin<NW>(accu);
      }
    }
    // the next block's activations, now that this block's are consumed
    if (more) load_x(pid / k);
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
        store_h(hb + h_index<FMT>((size_t)tr.pos0 + b0 + tt, I, f0 + 16 * j + rr), hlo, gate_act(g, u, act));
      }
    }
    if (b0 + 16 < tr.n) __syncthreads();        // red is rewritten by the next block
  }
}

// ------------------------------------------------------------------ MXFP4 gate/up, rows split over the waves
// MXFP4 gate/up on tiles of more than 16 pairs between 6 and 12 pairs per
// expert: workgroup = one tile x 64 row pairs (wave w rows f0 + 16w .. + 15,
// gate and up) over the whole K = H with its codes held in registers; each
// 16-pair block of activations is staged in LDS once for the four waves
// (rows padded by 16 bytes), so a tile's activations are read I/64 times
// and no partial sums cross waves.
template <int GK>   // GK = H/128 groups of 128 K
__global__ __launch_bounds__(BLOCK, 2) void gateup_g16r_kernel(
    const uint8_t* gu, size_t gu_expert_bytes, int rp_bytes, int H, int I, int k,
    const uint16_t* x, const int32_t* pairs, const TileRec* __restrict__ tiles,
    uint16_t* __restrict__ hb, int act, size_t hlo, int ntiles) {
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
  // the first block's token ids leave before the weights (the activations
  // they address end the longest dependent chain); every thread loads one,
  // in bounds, so the load is not conditional and its wait covers it alone
  int tk = pairs[tr.pos0 + min(tid & 15, min(16, tr.n) - 1)];
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
  asm volatile("" ::: "memory");    // the loads above stay above (not sunk to their uses)
  // one 16-pair block; tkv: this thread's token id of the block (the
  // first block's was loaded before the weights, the later ones' are
  // loaded unconditionally in their own loop, so no wait drains the loads
  // in flight)
  auto block = [&](int b0, int tkv) {
    const int nb = min(16, tr.n - b0);
    if (tid < 16) tok_s[tid] = tkv / k;
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
    f32x4 accg = ZERO4, accu = ZERO4;
#pragma unroll
    for (int m = 0; m < GK; ++m) {
      const float scg = e8m0_scale(sg[m]), scu = e8m0_scale(su[m]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&xs[lane & 15][32 * (4 * m + kg) + 8 * i]);
        accg = mfma(a, fp4x8_bf16(dword_of(cg[m], i), scg), accg);
        accu = mfma(a, fp4x8_bf16(dword_of(cu[m], i), scu), accu);
      }
    }
    // D[tt][rr]: tile row tt = 4 kg + q, row rr = lane % 16
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tt = 4 * kg + q;
      if (tt < nb)
        store_h(hb + h_index<FMT_MXFP4>((size_t)tr.pos0 + b0 + tt, I, f0 + r), hlo, gate_act(accg[q], accu[q], act));
    }
    // the codes and scale bytes stay the live state across blocks,
    // converted again per block (pinned after their use, so the first block
    // waits for them only where it converts them)
#pragma unroll
    for (int m = 0; m < GK; ++m) asm volatile("" : "+v"(cg[m]), "+v"(cu[m]), "+v"(sg[m]), "+v"(su[m]));
    if (b0 + 16 < tr.n) __syncthreads();          // xs and tok_s are rewritten by the next block
  };
  block(0, tk);
  for (int b0 = 16; b0 < tr.n; b0 += 16) block(b0, pairs[tr.pos0 + b0 + min(tid & 15, min(16, tr.n - b0) - 1)]);
}

// ------------------------------------------------------------------ gate/up, K outermost
// Gate/up above 12 pairs per expert (tiles of up to 128 pairs), K outermost:
// workgroup = one tile x 64 row pairs (wave w: rows f0 + 16w .. + 15, gate
// and up). K runs in chunks of 128: the tile's activations for the chunk are
// staged in LDS (rows padded by 16 bytes; super-blocks: each 8-group in
// unpack order) while the next chunk is loaded into registers, and each wave
// converts its code slices once per chunk and feeds every 16-pair block of
// the tile from that one conversion, with one accumulator pair per block.
// Super-block sub-blocks: one MFMA of P = A·q per block and sub-block, one of
// S = A·1 per block and sub-block (shared by gate and up), the affine in
// fp32.
constexpr int KCH = 128;
template <int NBR, int MT, int FMT>   // NBR = 16-pair blocks this tile fills (the MFMAs run unconditionally)
__device__ __forceinline__ void g16k_body(const uint8_t* __restrict__ rec, int H, int I, const uint16_t* __restrict__ x,
                                          const TileRec& tr, uint16_t* __restrict__ hb, int act, size_t hlo,
                                          int f0, uint16_t (*xs)[KCH + 8], const int* tok_s) {
  constexpr bool MX = FMT == FMT_MXFP4;
  constexpr int CPR = KCH / 8, NST = 16 * NBR * CPR / BLOCK;
  static_assert(NST * BLOCK == 16 * NBR * CPR || NBR < 2, "staging split");
  constexpr int NSTX = NST > 0 ? NST : 1;
  using Hdr = std::conditional_t<MX, u32, u32x4>;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int r = lane & 15, kg = lane >> 4;
  // staging unit c = tid + BLOCK q: row c / CPR, 16-byte column c % CPR.
  // The row guards below always hold (the units cover exactly 16 NBR rows);
  // they stay because without them the compiler schedules the staging so
  // that the kernel needs more registers (fewer waves per SIMD).
  u32x4 st[NSTX];
  auto load_x = [&](int c0) {
#pragma unroll
    for (int q = 0; q < NSTX; ++q) {
      const int c = tid + BLOCK * q, row = c / CPR;
      if (row < 16 * NBR)
        st[q] = *reinterpret_cast<const u32x4*>(x + (size_t)tok_s[row] * H + c0 + 8 * (c % CPR));
    }
  };
  u32x4 cg, cu;
  Hdr sg, su;
  auto load_codes = [&](int c0) {
    const int sbi = c0 / MXK + kg;
    cg = *reinterpret_cast<const u32x4*>(rec + 16 * sbi);
    cu = *reinterpret_cast<const u32x4*>(rec + H / 2 + 16 * sbi);
    if constexpr (MX) {
      sg = rec[H + sbi];
      su = rec[H + H / MXK + sbi];
    } else {
      sg = *reinterpret_cast<const u32x4*>(rec + H + QHDR * (c0 / QK));
      su = *reinterpret_cast<const u32x4*>(rec + H + H / 16 + QHDR * (c0 / QK));
    }
  };
  f32x4 accg[NBR], accu[NBR];
#pragma unroll
  for (int b = 0; b < NBR; ++b) accg[b] = accu[b] = ZERO4;
  const bf16x8 one = ones8();
  load_x(0);
  load_codes(0);
  for (int c0 = 0; c0 < H; c0 += KCH) {
    if (c0) __syncthreads();                        // the previous chunk's reads of xs are done
#pragma unroll
    for (int q = 0; q < NSTX; ++q) {
      const int c = tid + BLOCK * q, row = c / CPR;
      if (row < 16 * NBR) *reinterpret_cast<u32x4*>(&xs[row][8 * (c % CPR)]) = MX ? st[q] : unpack_order(st[q]);
    }
    __syncthreads();
    u32x4 ncg = cg, ncu = cu;
    const Hdr nsg = sg, nsu = su;
    const int sb_own = c0 / MXK + kg;
    if (c0 + KCH < H) {
      load_x(c0 + KCH);
      load_codes(c0 + KCH);
    }
    if constexpr (MX) {
      const float scg = e8m0_scale(nsg), scu = e8m0_scale(nsu);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 bg = fp4x8_bf16(dword_of(ncg, i), scg);
        const bf16x8 bu = fp4x8_bf16(dword_of(ncu, i), scu);
#pragma unroll
        for (int b = 0; b < NBR; ++b) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&xs[16 * b + r][32 * kg + 8 * i]);
          accg[b] = mfma(a, bg, accg[b]);
          accu[b] = mfma(a, bu, accu[b]);
        }
      }
    } else {
      transpose4(ncg);
      transpose4(ncu);
      const Affine4 ag = affine4(nsg, sb_own), au = affine4(nsu, sb_own);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 bg = codes8_bf16(dword_of(ncg, i));
        const bf16x8 bu = codes8_bf16(dword_of(ncu, i));
#pragma unroll
        for (int b = 0; b < NBR; ++b) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&xs[16 * b + r][32 * i + 8 * kg]);
          const f32x4 S = mfma(a, one, ZERO4);
          const f32x4 Pg = mfma(a, bg, ZERO4), Pu = mfma(a, bu, ZERO4);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            accg[b][q] = fmaf(ag.a[i], Pg[q], fmaf(-ag.b[i], S[q], accg[b][q]));
            accu[b][q] = fmaf(au.a[i], Pu[q], fmaf(-au.b[i], S[q], accu[b][q]));
          }
        }
      }
      pin<NBR>(accg);
      pin<NBR>(accu);
    }
  }
  // D[tt][rr] of block b: pair 16 b + tt, tt = 4 kg + q; row rr = lane % 16
#pragma unroll
  for (int b = 0; b < NBR; ++b) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = 16 * b + 4 * kg + q;
      const float hv = gate_act(accg[b][q], accu[b][q], act);
      if (p < tr.n) store_h(hb + h_index<FMT>((size_t)tr.pos0 + p, I, f0 + r), hlo, hv);
    }
  }
}

template <int NB, int FMT>   // up to 16 NB pairs per tile
__global__ __launch_bounds__(BLOCK, 2) void gateup_g16k_kernel(
    const uint8_t* __restrict__ gu, size_t gu_expert_bytes, int rp_bytes, int H, int I, int k,
    const uint16_t* __restrict__ x, const int32_t* __restrict__ pairs, const TileRec* __restrict__ tiles,
    uint16_t* __restrict__ hb, int act, size_t hlo, int ntiles) {
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
  if (NB >= 8 && nblk > 4) g16k_body<8, MT, FMT>(rec, H, I, x, tr, hb, act, hlo, f0, xs, tok_s);
  else if (nblk > 2) g16k_body<4, MT, FMT>(rec, H, I, x, tr, hb, act, hlo, f0, xs, tok_s);
  else if (nblk > 1) g16k_body<2, MT, FMT>(rec, H, I, x, tr, hb, act, hlo, f0, xs, tok_s);
  else g16k_body<1, MT, FMT>(rec, H, I, x, tr, hb, act, hlo, f0, xs, tok_s);
}

// ------------------------------------------------------------------ down, one 16-pair block
// Down: workgroup = one tile x 64 output rows, wave w rows n0 .. n0+15 over
// the whole K = I (GD = I/128 groups); A = h from its two bf16 planes (two
// MFMAs per slice). Rows go to ypair at the pair index t*k + s.
template <int GD, int FMT>
__global__ __launch_bounds__(BLOCK) void down_g16_kernel(
    const uint8_t* __restrict__ dn, size_t dn_expert_bytes, int drow_bytes, int H, int I,
    const int32_t* __restrict__ pairs, const TileRec* __restrict__ tiles, const uint16_t* __restrict__ hb,
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
  // h of tile row t = l%16; rows past the tile's pairs repeat its last row
  // (their outputs are not stored), so the loads are unconditional
  const uint16_t* hp = hb + (size_t)(tr.pos0 + min(lane & 15, tr.n - 1)) * I;
  // output pair indices of this lane's four accumulator rows (tile rows 4*kg .. 4*kg+3)
  int pr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) pr[q] = 4 * kg + q < tr.n ? pairs[tr.pos0 + 4 * kg + q] : -1;
  f32x4 acc = ZERO4;
  if constexpr (MX) {
#pragma unroll
    for (int m = 0; m < GD; ++m) {
      const float sc = e8m0_scale(hd[m]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t* a = hp + 32 * (4 * m + kg) + 8 * i;
        const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(a), alo = *reinterpret_cast<const bf16x8*>(a + hlo);
        const bf16x8 b = fp4x8_bf16(dword_of(cd[m], i), sc);
        acc = mfma(alo, b, mfma(ahi, b, acc));
      }
    }
  } else {
    const bf16x8 one = ones8();
#pragma unroll
    for (int m = 0; m < GD; ++m) {
      transpose4(cd[m]);
      const Affine4 af = affine4(hd[m >> 1], 4 * m + kg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t* a = hp + 32 * (4 * m + i) + 8 * kg;
        const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(a), alo = *reinterpret_cast<const bf16x8*>(a + hlo);
        const f32x4 S = mfma(alo, one, mfma(ahi, one, ZERO4));
        q4k_step2(acc, ahi, alo, dword_of(cd[m], i), af.a[i], af.b[i], S);
      }
      pin(&acc);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (pr[q] >= 0) ypair[(size_t)pr[q] * H + n0 + r] = acc[q];
}

// ------------------------------------------------------------------ down, multi-row
// Down on tiles of more than 16 pairs (and 16-pair tiles above a few pairs
// per expert): workgroup = one tile x 4*NW*16 output rows, wave w the NW
// blocks of 16 rows from n0 = (256*NW/4)*fb + 16*NW*w over the whole K = I;
// the tile's pairs 16 at a time, each 16-pair block of h (both planes)
// staged in LDS once for the four waves (rows padded by 16 bytes against
// bank conflicts) and used for all NW row blocks, so h is read H/(64 NW)
// times per tile instead of H/16.
template <int GD, int NW, int FMT>
__global__ __launch_bounds__(BLOCK) void down_g16m_kernel(
    const uint8_t* dn, size_t dn_expert_bytes, int drow_bytes, int H, int I,
    const int32_t* pairs, const TileRec* __restrict__ tiles, const uint16_t* hb,
    float* __restrict__ ypair, size_t hlo, int ntiles) {
  constexpr bool MX = FMT == FMT_MXFP4;
  constexpr int NH = MX ? GD : (GD + 1) / 2;
  using Hdr = std::conditional_t<MX, u32, u32x4>;
  constexpr int IK = 128 * GD, LS = IK + 8, CPR = IK / 8;
  __shared__ __align__(16) uint16_t hs[2][16][LS];
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
  // a 16-pair block's h rows (staged in LDS) and pair ids: thread -> one
  // (plane, row) and every TPR-th 16-byte column of it
  constexpr int TPR = BLOCK / (2 * 16), NQ = CPR / TPR;
  static_assert(CPR % TPR == 0, "h staging split");
  const int prw = tid / TPR, pl = prw / 16, hrow = prw % 16, col0 = tid % TPR;
  u32x4 st[NQ];
  int pr[4];
  auto load_block = [&](int b0) {
    const int nb = min(16, tr.n - b0);
    const uint16_t* src = hb + (pl ? hlo : 0) + (size_t)(tr.pos0 + b0 + min(hrow, nb - 1)) * I + 8 * col0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) st[q] = *reinterpret_cast<const u32x4*>(src + 8 * TPR * q);
#pragma unroll
    for (int q = 0; q < 4; ++q) pr[q] = pairs[tr.pos0 + b0 + min(4 * kg + q, nb - 1)];
  };
  auto stage_block = [&]() {
#pragma unroll
    for (int q = 0; q < NQ; ++q) *reinterpret_cast<u32x4*>(&hs[pl][hrow][8 * col0 + 8 * TPR * q]) = st[q];
  };
  // the first block's h and pair ids leave first, then the weights; h goes
  // to LDS as soon as it arrives, ahead of the code transposes that wait for
  // the weights (the fences keep the compiler from sinking the loads to
  // their uses)
  load_block(0);
  asm volatile("" ::: "memory");
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
  asm volatile("" ::: "memory");
  stage_block();
  if constexpr (!MX) {
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
      for (int m = 0; m < GD; ++m) transpose4(cd[j][m]);
  }
  const bf16x8 one = ones8();
  for (int b0 = 0; b0 < tr.n; b0 += 16) {
    const int nb = min(16, tr.n - b0);
    // the codes stay the live state across blocks, converted again per block
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
      for (int m = 0; m < GD; ++m) asm volatile("" : "+v"(cd[j][m]));
    if (b0 > 0) {
      load_block(b0);
      stage_block();
    }
    __syncthreads();
    f32x4 acc[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) acc[j] = ZERO4;
#pragma unroll
    for (int m = 0; m < GD; ++m) {
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint16_t* a = &hs[0][lane & 15][32 * (4 * m + kg) + 8 * i];
          const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(a);
          const bf16x8 alo = *reinterpret_cast<const bf16x8*>(a + 16 * LS);   // the lo plane
#pragma unroll
          for (int j = 0; j < NW; ++j) {
            const bf16x8 b = fp4x8_bf16(dword_of(cd[j][m], i), e8m0_scale(sc[j][m]));
            acc[j] = mfma(alo, b, mfma(ahi, b, acc[j]));
          }
        }
      } else {
        Affine4 af[NW];
#pragma unroll
        for (int j = 0; j < NW; ++j) af[j] = affine4(sc[j][m >> 1], 4 * m + kg);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint16_t* a = &hs[0][lane & 15][32 * (4 * m + i) + 8 * kg];
          const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(a);
          const bf16x8 alo = *reinterpret_cast<const bf16x8*>(a + 16 * LS);
          const f32x4 S = mfma(alo, one, mfma(ahi, one, ZERO4));
#pragma unroll
          for (int j = 0; j < NW; ++j) q4k_step2(acc[j], ahi, alo, dword_of(cd[j][m], i), af[j].a[i], af[j].b[i], S);
        }
        pin<NW>(acc);
      }
    }
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (4 * kg + q < nb) ypair[(size_t)pr[q] * H + n0 + 16 * j + r] = acc[j][q];
    if (b0 + 16 < tr.n) __syncthreads();          // hs is rewritten by the next block
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

// ------------------------------------------------------------------ launchers
// rows: 0 one row block per gate/up workgroup and per down wave; 1 the
// multi-row kernels (2 row blocks per gate/up wave, 2 or 4 per down wave), which
// read a tile's activations and h fewer times but run fewer workgroups; 2
// (above 6 pairs per expert) MXFP4 gate/up splits rows over the waves; 3
// (above 12 pairs per expert) gate/up runs K outermost and reuses each
// converted code slice for all of a tile's 16-pair blocks.
template <int G, int GD, int FMT>
static hipError_t launch_g16_f(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* pairs,
                               const TileRec* tiles, int ntiles, uint16_t* hb, float* ypair, size_t hlo, int rows,
                               hipStream_t s) {
  constexpr int NWG = 2;                         // row blocks per wave of the multi-row gate/up
  if (rows == 3 && d.I % 64 == 0)
    hipLaunchKernelGGL((gateup_g16k_kernel<8, FMT>), dim3(tile_unit_grid(ntiles, d.I / 64)), dim3(BLOCK), 0, s,
                       layer + d.gu_off, d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.k, x, pairs, tiles, hb,
                       d.act, hlo, ntiles);
  else if (FMT == FMT_MXFP4 && rows == 2 && d.I % 64 == 0)
    hipLaunchKernelGGL((gateup_g16r_kernel<4 * G>), dim3(tile_unit_grid(ntiles, d.I / 64)), dim3(BLOCK), 0, s,
                       layer + d.gu_off, d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.k, x, pairs, tiles, hb,
                       d.act, hlo, ntiles);
  else if (rows)
    hipLaunchKernelGGL((gateup_g16m_kernel<G, NWG, FMT>), dim3(tile_unit_grid(ntiles, d.I / (16 * NWG))), dim3(BLOCK),
                       0, s, layer + d.gu_off, d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.k, x, pairs, tiles, hb,
                       d.act, hlo, ntiles);
  else
    hipLaunchKernelGGL((gateup_g16_kernel<G, FMT>), dim3(ntiles * (d.I / 16)), dim3(BLOCK), 0, s, layer + d.gu_off,
                       d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.k, x, pairs, tiles, hb, d.act, hlo);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // row blocks per wave of the multi-row down: 4 for MXFP4; 2 for
  // super-blocks, whose affine epilogue needs more registers (239 -> 143,
  // two -> three waves per SIMD: 3-6 % faster from 32 to 1024 tokens)
  constexpr int NW = FMT == FMT_Q4K ? 2 : 4;
  if (rows && d.H % (64 * NW) == 0) {
    hipLaunchKernelGGL((down_g16m_kernel<GD, NW, FMT>), dim3(tile_unit_grid(ntiles, d.H / (64 * NW))), dim3(BLOCK), 0, s,
                       layer + d.dn_off, d.dn_expert_bytes, (int)d.drow_bytes, d.H, d.I, pairs, tiles, hb, ypair, hlo,
                       ntiles);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((down_g16_kernel<GD, FMT>), dim3(ntiles * (d.H / 64)), dim3(BLOCK), 0, s, layer + d.dn_off,
                     d.dn_expert_bytes, (int)d.drow_bytes, d.H, d.I, pairs, tiles, hb, ypair, hlo);
  return hipGetLastError();
}

template <int G, int GD>
static hipError_t launch_g16(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* pairs,
                             const TileRec* tiles, int ntiles, uint16_t* hb, float* ypair, size_t hlo, int rows,
                             hipStream_t s) {
  if (d.fmt == FMT_MXFP4)
    return launch_g16_f<G, GD, FMT_MXFP4>(d, layer, x, pairs, tiles, ntiles, hb, ypair, hlo, rows, s);
  return launch_g16_f<G, GD, FMT_Q4K>(d, layer, x, pairs, tiles, ntiles, hb, ypair, hlo, rows, s);
}

template <int G>
static hipError_t launch_g16_i(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* pairs,
                               const TileRec* tiles, int ntiles, uint16_t* hb, float* ypair, size_t hlo, int rows,
                               hipStream_t s) {
  switch (d.I) {
    case 256: return launch_g16<G, 2>(d, layer, x, pairs, tiles, ntiles, hb, ypair, hlo, rows, s);
    case 512: return launch_g16<G, 4>(d, layer, x, pairs, tiles, ntiles, hb, ypair, hlo, rows, s);
    case 768: return launch_g16<G, 6>(d, layer, x, pairs, tiles, ntiles, hb, ypair, hlo, rows, s);
    case 1024: return launch_g16<G, 8>(d, layer, x, pairs, tiles, ntiles, hb, ypair, hlo, rows, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace grouped

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

// Pairs per tile: 16 up to one pair per expert, 64 up to 16 and 128 beyond,
// walked 16 at a time by the multi-block kernels (measured on the
// Qwen3-30B-A3B-shaped layer with MXFP4 weights: at 41 / 96 / 128 tokens
// 108 / 122 / 126 us against 123 / 151 / 166 us on 16-pair tiles).
int g16_mt(const Layout& d, int T) {
  const long long P = (long long)T * d.k;
  return P <= d.E ? 16 : (P <= 16LL * d.E ? 64 : 128);
}

int g16_max_tiles(const Layout& d, int T) {
  const int P = T * d.k, mt = g16_mt(d, T);
  return (P + mt - 1) / mt + (P < d.E ? P : d.E);
}

hipError_t launch_g16_ffn(const Layout& d, const uint8_t* layer, const uint16_t* x, const float* w,
                          const int32_t* pairs, const void* tiles, uint16_t* hb, float* ypair, float* out, int T,
                          hipStream_t s) {
  using namespace grouped;
  if (!g16_supported(d)) return hipErrorInvalidValue;
  if (T <= 0) return hipSuccess;
  const TileRec* tr = static_cast<const TileRec*>(tiles);
  const int nt = g16_max_tiles(d, T);
  // h's bf16 lo plane follows the hi plane (scratch holds 4 bytes per value)
  const size_t hlo = (size_t)T * d.k * d.I;
  const long long P = (long long)T * d.k;
  const int rows = P > 12LL * d.E ? 3 : (P > 6LL * d.E ? 2 : (g16_mt(d, T) > 16 ? 1 : 0));
  hipError_t e;
  switch (d.H) {
    case 512: e = launch_g16_i<1>(d, layer, x, pairs, tr, nt, hb, ypair, hlo, rows, s); break;
    case 1024: e = launch_g16_i<2>(d, layer, x, pairs, tr, nt, hb, ypair, hlo, rows, s); break;
    default: e = launch_g16_i<4>(d, layer, x, pairs, tr, nt, hb, ypair, hlo, rows, s); break;
  }
  if (e != hipSuccess) return e;
  return launch_combine(d, ypair, w, out, T, s);
}

}  // namespace qmoe

// gfx950 kernels of the expert-major GEMV path for small token batches.
//
// Between one token and a batch large enough to fill MFMA tiles, each routed
// expert carries only a few tokens. The per-token GEMV would stream such an
// expert once per token; the grouped MFMA GEMM would pad each expert's few
// tokens to a 32-row tile and walk K in a dependent loop. Here every weight
// row of every routed expert is streamed once, straight into registers, and
// used for all the tokens routed to that expert. The tokens are grouped by
// expert on the device (dispatch lists). This is the same one-pass expert
// read as the pages' batched prefill (sparkinfer README, MoE-bandwidth item
// and kernel table), sized for batches that are too small to use MFMA.
//
// A wave owns RW = (64 / LPR) * U rows of one expert; LPR lanes share a row,
// each lane owning fixed 32-weight sub-blocks of it, so the lane's slices of
// the tokens' activations (NT tokens at a time) stay in registers for all
// its rows. The arithmetic is that of the per-token kernels: gate/up take
// bf16 activations against codes made exact bf16 values 128 + q, down takes
// fp32 h against the exactly converted codes; products and sums are fp32, so
// h keeps its full range and precision. The 2*U*NT
// (gate/up) or U*NT (down) partial sums of a lane are reduced over the LPR
// lanes of its row by a transposed butterfly: at each level a lane keeps one
// half of its values and swaps the other half with its partner, so after
// log2(count) levels each lane holds one finished sum instead of every lane
// holding every sum.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moe_device.h"

namespace qmoe {
namespace egemv {

// Butterfly levels in the order used, as the lane bit that separates the two
// partners: the half-row mirror (lane ^ 7) is a valid partner only while all
// lanes of the group still hold the same value indices, so it goes first and
// splits on bit 2; then lane ^ 1, lane ^ 2 (quad permutes), lane ^ 8 (row
// rotate by 8), lane ^ 16 (swizzle within 32 lanes) and lane ^ 32.
__host__ __device__ constexpr int level_bit(int lv) { return lv == 0 ? 2 : (lv == 1 ? 0 : (lv == 2 ? 1 : lv)); }

template <int LV>
__device__ __forceinline__ float partner(float v) {
  if constexpr (LV == 0) return dpp_mov<0x141>(v);        // row_half_mirror
  else if constexpr (LV == 1) return dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
  else if constexpr (LV == 2) return dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  else if constexpr (LV == 3) return dpp_mov<0x128>(v);   // row_ror:8
  else if constexpr (LV == 4)
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));  // xor 16
  else return __shfl_xor(v, 32, WAVE);
}

// One level with N values per lane: transposed (N >= 2) or a plain sum.
template <int LV, int N>
__device__ __forceinline__ void tstep(float* v) {
  if constexpr (N >= 2) {
    const bool b = ((threadIdx.x & (WAVE - 1)) >> level_bit(LV)) & 1;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float keep = b ? v[2 * i + 1] : v[2 * i];
      const float send = b ? v[2 * i] : v[2 * i + 1];
      v[i] = keep + partner<LV>(send);
    }
  } else {
    v[0] += partner<LV>(v[0]);
  }
}

__host__ __device__ constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }
__host__ __device__ constexpr int count_at(int V, int lv) { return (V >> lv) > 0 ? (V >> lv) : 1; }

// Sums each of the V values over the 2^LG lanes of a lane group (V <= 2^LG,
// both powers of two); returns the lane's finished sum, that of value
// tsum_index<V>(lane). Must be called with the whole wave active.
template <int V, int LG>
__device__ __forceinline__ float tsum(float* v) {
  static_assert((V & (V - 1)) == 0 && V <= (1 << LG), "V must be a power of two within the lane group");
  if constexpr (LG > 0) tstep<0, count_at(V, 0)>(v);
  if constexpr (LG > 1) tstep<1, count_at(V, 1)>(v);
  if constexpr (LG > 2) tstep<2, count_at(V, 2)>(v);
  if constexpr (LG > 3) tstep<3, count_at(V, 3)>(v);
  if constexpr (LG > 4) tstep<4, count_at(V, 4)>(v);
  if constexpr (LG > 5) tstep<5, count_at(V, 5)>(v);
  return v[0];
}

// Index of the value whose sum lane `lane` holds after tsum<V, LG>: bit i of
// the index is the lane bit split at level i (the first log2(V) levels).
template <int V>
__device__ __forceinline__ int tsum_index(int lane) {
  int idx = 0;
#pragma unroll
  for (int lv = 0; lv < ilog2(V); ++lv) idx |= ((lane >> level_bit(lv)) & 1) << lv;
  return idx;
}

// The lanes of a group holding the same sum differ only in the bits of the
// plain levels; the one with those bits clear writes it.
template <int V, int LG>
__device__ __forceinline__ bool tsum_owner(int lane) {
  bool own = true;
#pragma unroll
  for (int lv = ilog2(V); lv < LG; ++lv) own = own && !((lane >> level_bit(lv)) & 1);
  return own;
}

// Slot record written by the dispatch: expert, first expert-sorted pair
// position, pair count (0 for slots past the last routed expert).
struct SlotDesc { int e, pos0, n, pad; };

// ------------------------------------------------------------------ gate/up + SiLU
// Workgroup: 4 waves on rows [r0, r0 + 4*RW) of the expert in slot a, all of
// its routed pairs, NT at a time; h[pos * I + r] = SiLU(G_e[r]·x_t) *
// (U_e[r]·x_t) (fp32) for the pair at expert-sorted position pos, t its token.
template <int IPL, int LPR, int U, int NT, int FMT>
__global__ __launch_bounds__(BLOCK) void gateup_egemv_kernel(
    const uint8_t* gu, size_t gu_expert_bytes, int rp_bytes, int H, int I, int k,
    const uint16_t* x, const int32_t* pairs, const SlotDesc* __restrict__ slots,
    float* __restrict__ hbuf, int act) {
  constexpr int LG = ilog2(LPR), RPS = WAVE / LPR, RW = RPS * U, V = 2 * U * NT;
  static_assert((1 << LG) == LPR, "LPR must be a power of two");
  const int bpe = I / (4 * RW);                 // workgroups per expert
  const SlotDesc sd = slots[blockIdx.x / bpe];  // workgroup-uniform
  if (sd.n == 0) return;                        // past the last routed expert
  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = __builtin_amdgcn_readfirstlane((int)threadIdx.x / WAVE);
  const int r0 = ((int)(blockIdx.x % bpe) * 4 + wid) * RW;
  const int pos0 = sd.pos0, n = sd.n;
  const int rho = lane / LPR, lam = lane % LPR;
  // tokens of the first chunk before the weights: the activation loads wait
  // on them, and a wait for a later load would also wait for the weights.
  // Every one in bounds (slots past the expert's pairs reload its last), so
  // no load is conditional and that wait covers these loads alone.
  int t0[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    int pt = pos0 + min(tt, n - 1);
    asm volatile("" : "+s"(pt));    // opaque: no load made conditional on pt == pos0
    t0[tt] = pairs[pt] / k;
  }
  const uint8_t* base = gu + (size_t)sd.e * gu_expert_bytes;
  const int half = H / 2;                 // code bytes per matrix row
  const int hdr = H;                      // headers (MXFP4: scale bytes) start after both code areas
  const int nb = H / QK;
  // per lane and row: the sub-block's 16-byte header, or its E8M0 scale byte
  using Hdr = std::conditional_t<FMT == FMT_MXFP4, u32, u32x4>;
  u32x4 cg[U][IPL], cu[U][IPL];
  Hdr hg[U][IPL], hu[U][IPL];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint8_t* rp = base + (size_t)(r0 + u * RPS + rho) * rp_bytes;
#pragma unroll
    for (int q = 0; q < IPL; ++q) {
      const int j = lam + LPR * q;
      cg[u][q] = load_nt(rp + 16 * j);
      cu[u][q] = load_nt(rp + half + 16 * j);
      if constexpr (FMT == FMT_MXFP4) {
        hg[u][q] = __builtin_nontemporal_load(rp + hdr + j);
        hu[u][q] = __builtin_nontemporal_load(rp + hdr + H / MXK + j);
      } else {
        hg[u][q] = load_nt(rp + hdr + QHDR * (j >> 3));
        hu[u][q] = load_nt(rp + hdr + QHDR * nb + QHDR * (j >> 3));
      }
    }
  }
  // compiler fence: the loads above stay above, issued together (not sunk
  // to their uses)
  asm volatile("" ::: "memory");
  for (int c0 = 0; c0 < n; c0 += NT) {
    const int nv = min(NT, n - c0);             // tokens present in this chunk (wave-uniform)
    u32 X[NT][IPL][16];
    float S[NT][IPL];
    // every token's activations loaded (slots past the chunk's pairs reload
    // its last token, in bounds), so no load is conditional
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      {
        const int t = c0 == 0 ? t0[tt] : pairs[pos0 + c0 + min(tt, nv - 1)] / k;
#pragma unroll
        for (int q = 0; q < IPL; ++q) {
          const uint16_t* xp = x + (size_t)t * H + 32 * (lam + LPR * q);
          if constexpr (FMT == FMT_MXFP4) {
            // natural pair order, no sums needed
            u32x4 r[4];
            load_x_raw(xp, r);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              X[tt][q][4 * m] = r[m].x; X[tt][q][4 * m + 1] = r[m].y;
              X[tt][q][4 * m + 2] = r[m].z; X[tt][q][4 * m + 3] = r[m].w;
            }
            S[tt][q] = 0.f;
          } else {
            S[tt][q] = load_x_pairs(xp, X[tt][q]);
          }
        }
      }
    }
    float v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int q = 0; q < IPL; ++q) {
        if constexpr (FMT == FMT_MXFP4) {
          const float sg = e8m0_scale(hg[u][q]), su = e8m0_scale(hu[u][q]);
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            if (tt < nv) {
              v[2 * (u * NT + tt)] = fmaf(sg, dot_fp4_bf16(cg[u][q], X[tt][q]), v[2 * (u * NT + tt)]);
              v[2 * (u * NT + tt) + 1] = fmaf(su, dot_fp4_bf16(cu[u][q], X[tt][q]), v[2 * (u * NT + tt) + 1]);
            }
          }
        } else {
          const int jj = (lam + LPR * q) & 7;
          const Affine ag = header_affine(hg[u][q], jj);
          const Affine au = header_affine(hu[u][q], jj);
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            if (tt < nv) {
              const float Ag = dot_codes_bf16(cg[u][q], X[tt][q]);
              const float Au = dot_codes_bf16(cu[u][q], X[tt][q]);
              v[2 * (u * NT + tt)] += ag.a * Ag - (128.f * ag.a + ag.b) * S[tt][q];
              v[2 * (u * NT + tt) + 1] += au.a * Au - (128.f * au.a + au.b) * S[tt][q];
            }
          }
        }
      }
    }
    const float s = tsum<V, LG>(v);
    // the other matrix of the same (row, token) differs in index bit 0, i.e.
    // in lane bit level_bit(0) = 2
    const float o = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, s), 0x101F));
    const int idx = tsum_index<V>(lane);
    const int u = (idx >> 1) / NT, tt = (idx >> 1) % NT;
    if (tsum_owner<V, LG>(lane) && !(idx & 1) && tt < nv) {
      hbuf[(size_t)(pos0 + c0 + tt) * I + r0 + u * RPS + rho] = gate_act(s, o, act);
    }
    // the codes and headers (scale bytes) stay raw across chunks: converted
    // and decoded in each chunk, not ahead of the first chunk's activation
    // loads (and without the registers of converted copies)
#pragma unroll
    for (int u2 = 0; u2 < U; ++u2)
#pragma unroll
      for (int q = 0; q < IPL; ++q)
        asm volatile("" : "+v"(cg[u2][q]), "+v"(cu[u2][q]), "+v"(hg[u2][q]), "+v"(hu[u2][q]));
  }
}

// ------------------------------------------------------------------ down
// Workgroup: 4 waves on output features [n0, n0 + 4*RW) of the expert in
// slot a; one 32-code sub-block of the row per lane (lanes with j >= I/32
// hold nothing); ypair[p * H + f] = D_e[f]·h_p for each of the expert's pairs
// p = t*k + s, with fp32 h (32 values per lane and token, NT tokens at a
// time).
template <int LPR, int U, int NT, int FMT>
__global__ __launch_bounds__(BLOCK) void down_egemv_kernel(
    const uint8_t* dn, size_t dn_expert_bytes, int drow_bytes, int H, int I,
    const int32_t* pairs, const SlotDesc* __restrict__ slots, const float* hbuf,
    float* __restrict__ ypair) {
  constexpr int LG = ilog2(LPR), RPS = WAVE / LPR, RW = RPS * U, V = U * NT;
  static_assert((1 << LG) == LPR, "LPR must be a power of two");
  const int bpe = H / (4 * RW);
  const SlotDesc sd = slots[blockIdx.x / bpe];
  if (sd.n == 0) return;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = __builtin_amdgcn_readfirstlane((int)threadIdx.x / WAVE);
  const int n0 = ((int)(blockIdx.x % bpe) * 4 + wid) * RW;
  const int pos0 = sd.pos0, n = sd.n;
  const int rho = lane / LPR, j = lane % LPR;
  const bool has = j < I / 32;
  const uint8_t* base = dn + (size_t)sd.e * dn_expert_bytes;
  // the first chunk's h and pair ids before the weights: a wait for a later
  // load would also wait for the weights. Every load in bounds (lanes past
  // the row read its first block, slots past the expert's pairs its last
  // pair), so none is conditional and no wait drains the loads in flight.
  const int jh = has ? j : 0;
  u32x4 hq[NT][8];
  int pq[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    int pt = pos0 + min(tt, n - 1);
    asm volatile("" : "+s"(pt));    // opaque: no load made conditional on pt == pos0
#pragma unroll
    for (int g = 0; g < 8; ++g) hq[tt][g] = load16(hbuf + (size_t)pt * I + 32 * jh + 4 * g);
    pq[tt] = pairs[pt];
  }
  using Hdr = std::conditional_t<FMT == FMT_MXFP4, u32, u32x4>;
  u32x4 cd[U];
  Hdr hd[U];
  const int hdr = I / 2 + QHDR * (jh >> 3);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint8_t* row = base + (size_t)(n0 + u * RPS + rho) * drow_bytes;
    cd[u] = load_nt(row + 16 * jh);
    if constexpr (FMT == FMT_MXFP4) hd[u] = (u32)__builtin_nontemporal_load(row + I / 2 + jh);
    else hd[u] = load_nt(row + hdr);
  }
  // compiler fence: the loads above stay above, issued together (not sunk
  // to their uses behind the per-token branches)
  asm volatile("" ::: "memory");
  // lanes past the row contribute nothing: zero codes (and, for MXFP4, scale
  // code 0, factor 0)
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!has) {
      cd[u] = u32x4{0u, 0u, 0u, 0u};
      if constexpr (FMT == FMT_MXFP4) hd[u] = 0u;
      else hd[u] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  for (int c0 = 0; c0 < n; c0 += NT) {
    const int nv = min(NT, n - c0);
    float X[NT][32];
    float S[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      if (tt < nv) {
        const float* hp = hbuf + (size_t)(pos0 + c0 + tt) * I + 32 * jh;
        float s = 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const u32x4 r = c0 == 0 ? hq[tt][g] : load16(hp + 4 * g);
          X[tt][4 * g + 0] = as_f32(r.x); X[tt][4 * g + 1] = as_f32(r.y);
          X[tt][4 * g + 2] = as_f32(r.z); X[tt][4 * g + 3] = as_f32(r.w);
        }
        if constexpr (FMT != FMT_MXFP4) {          // the super-block min term needs sum(h)
#pragma unroll
          for (int c = 0; c < 32; ++c) s += X[tt][c];
        }
        S[tt] = s;
      }
    }
    float v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (FMT == FMT_MXFP4) {
        // a lane past the row has scale code 0 (factor 0) and zero codes
        const float sc = e8m0_scale(hd[u]);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          if (tt < nv) v[u * NT + tt] = sc * dot_fp4_f32(cd[u], X[tt]);
      } else {
        const Affine af = header_affine(hd[u], j & 7);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          if (tt < nv) v[u * NT + tt] = fmaf(af.a, dot_codes_f32(cd[u], X[tt]), -af.b * S[tt]);
      }
    }
    const float s = tsum<V, LG>(v);
    const int idx = tsum_index<V>(lane);
    const int u = idx / NT, tt = idx % NT;
    if (tsum_owner<V, LG>(lane) && tt < nv) {
      int p = pairs[pos0 + c0 + min(tt, nv - 1)];
      if (c0 == 0) {
        // the first chunk's pair ids, loaded up front
#pragma unroll
        for (int q = 0; q < NT; ++q)
          if (tt == q) p = pq[q];
      }
      ypair[(size_t)p * H + n0 + u * RPS + rho] = s;
    }
  }
}

template <int IPL, int LPR, int U, int NT, int FMT>
static hipError_t gateup_go(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* pairs,
                            const SlotDesc* slots, float* hbuf, int nslots, hipStream_t s) {
  constexpr int RW = (WAVE / LPR) * U;
  static_assert(RW <= 64, "four waves of RW rows must divide a multiple of 256");
  const long long blocks = (long long)nslots * (d.I / (4 * RW));
  hipLaunchKernelGGL((gateup_egemv_kernel<IPL, LPR, U, NT, FMT>), dim3((unsigned)blocks), dim3(BLOCK), 0, s,
                     layer + d.gu_off, d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.k, x, pairs, slots, hbuf,
                     d.act);
  return hipGetLastError();
}

template <int LPR, int U, int NT, int FMT>
static hipError_t down_go(const Layout& d, const uint8_t* layer, const int32_t* pairs, const SlotDesc* slots,
                          const float* hbuf, float* ypair, int nslots, hipStream_t s) {
  constexpr int RW = (WAVE / LPR) * U;
  static_assert(RW <= 64, "four waves of RW rows must divide a multiple of 256");
  const long long blocks = (long long)nslots * (d.H / (4 * RW));
  hipLaunchKernelGGL((down_egemv_kernel<LPR, U, NT, FMT>), dim3((unsigned)blocks), dim3(BLOCK), 0, s, layer + d.dn_off,
                     d.dn_expert_bytes, (int)d.drow_bytes, d.H, d.I, pairs, slots, hbuf, ypair);
  return hipGetLastError();
}

// Token chunk NT of the gate/up kernel: 2 while the routed experts average
// at most 2 pairs (fewer registers, more waves in flight), else 4; the down
// kernel, whose fp32 h takes 32 registers per token, walks 2 at a time.
template <int NT, int FMT>
static hipError_t egemv_go(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* pairs,
                           const SlotDesc* slots, float* hbuf, float* ypair, int nslots, hipStream_t s) {
  hipError_t e;
  // gate/up: the per-token kernel's lane mapping of a hidden-size row
  switch (d.H) {
    case 256: e = gateup_go<1, 8, 2, 2, FMT>(d, layer, x, pairs, slots, hbuf, nslots, s); break;
    case 512: e = gateup_go<1, 16, 2, NT, FMT>(d, layer, x, pairs, slots, hbuf, nslots, s); break;
    case 1024: e = gateup_go<1, 32, 4, NT, FMT>(d, layer, x, pairs, slots, hbuf, nslots, s); break;
    case 2048: e = gateup_go<1, 64, 4, NT, FMT>(d, layer, x, pairs, slots, hbuf, nslots, s); break;
    case 3072: e = gateup_go<3, 32, 1, 1, FMT>(d, layer, x, pairs, slots, hbuf, nslots, s); break;
    case 4096: e = gateup_go<2, 64, 2, 2, FMT>(d, layer, x, pairs, slots, hbuf, nslots, s); break;
    case 6144: e = gateup_go<3, 64, 1, 1, FMT>(d, layer, x, pairs, slots, hbuf, nslots, s); break;
    case 8192: e = gateup_go<4, 64, 1, 1, FMT>(d, layer, x, pairs, slots, hbuf, nslots, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  // down: a power-of-two lane group covering the I/32 sub-blocks of a row
  const int nsb = d.I / 32;
  if (nsb <= 8) return down_go<8, 2, 2, FMT>(d, layer, pairs, slots, hbuf, ypair, nslots, s);
  if (nsb <= 16) return down_go<16, 4, 2, FMT>(d, layer, pairs, slots, hbuf, ypair, nslots, s);
  if (nsb <= 32) return down_go<32, 4, 2, FMT>(d, layer, pairs, slots, hbuf, ypair, nslots, s);
  return down_go<64, 4, 2, FMT>(d, layer, pairs, slots, hbuf, ypair, nslots, s);
}

}  // namespace egemv

bool egemv_supported(const Layout& d) { return d.I <= 2048; }

hipError_t launch_egemv_ffn(const Layout& d, const uint8_t* layer, const uint16_t* x, const float* w,
                            const int32_t* pairs, const void* slot_desc, float* hbuf, float* ypair, float* out,
                            int T, hipStream_t s) {
  using namespace egemv;
  if (!egemv_supported(d)) return hipErrorInvalidValue;
  if (T <= 0) return hipSuccess;
  const int P = T * d.k;
  const int nslots = P < d.E ? P : d.E;     // routed experts, at most
  const SlotDesc* slots = static_cast<const SlotDesc*>(slot_desc);
  hipError_t e;
  if (d.fmt == FMT_MXFP4)
    e = P <= 2 * d.E ? egemv_go<2, FMT_MXFP4>(d, layer, x, pairs, slots, hbuf, ypair, nslots, s)
                     : egemv_go<4, FMT_MXFP4>(d, layer, x, pairs, slots, hbuf, ypair, nslots, s);
  else
    e = P <= 2 * d.E ? egemv_go<2, FMT_Q4K>(d, layer, x, pairs, slots, hbuf, ypair, nslots, s)
                     : egemv_go<4, FMT_Q4K>(d, layer, x, pairs, slots, hbuf, ypair, nslots, s);
  if (e != hipSuccess) return e;
  return launch_combine(d, ypair, w, out, T, s);
}

}  // namespace qmoe

// gfx950 kernels of the single-stream (per-token) path: router GEMV, top-k
// routing, dequant-on-read gate/up GEMV with SiLU(gate)*up, dequant-on-read
// down GEMV with the routing-weighted combine, residual + RMSNorm, and the
// on-device expert dispatch lists.
//
// The expert GEMVs follow the pages' decode design goal -- experts stay
// resident as 4-bit super-blocks and are dequantized on read, so the bytes per
// token are the encoded weight bytes (sparkinfer README, opening paragraph and
// the MoE-bandwidth item; kernel table: decode GEMV, fused quantized MoE
// expert FFN, GGUF dequant). Their shape on CDNA4 is our own: one wave64 owns
// whole weight rows, each lane owns fixed 32-weight sub-blocks of every row it
// touches, so its slice of the activation vector and that slice's sum stay in
// registers for all rows; weights are streamed with 128-bit non-temporal loads
// and the sub-block affine (d*sc*q - dmin*m) is applied once per sub-block:
//   sum_i (a*q_i - b) x_i = a * sum_i q_i x_i - b * sum_i x_i.
// Gate/up use the exact trick bf16(128 + q) = 0x4300 | q, so two codes per
// v_dot2_f32_bf16 against the bf16 activations, with 128*sum(x) removed after.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <type_traits>

#include "moe_device.h"
#include "moe_timeline.h"

namespace qmoe {

// ------------------------------------------------------------------ top-k
// Order-preserving map fp32 -> u32 (a > b  <=>  key(a) > key(b) for non-NaN).
__device__ __forceinline__ u32 order_key(float f) {
  const u32 b = __builtin_bit_cast(u32, f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// LDS workspace of wave_topk (one per wave that runs it).
struct TopkSmem {
  unsigned long long ckey[16];     // selected keys (order_key(logit) << 32 | ~id), id order
  float cval[16];                  // their logits
  float val[16];                   // selected logits, descending
  int32_t sid[16];                 // selected ids, descending logit (equal logits: lower id first)
  float sw[16];                    // softmax over the selection
};

// Orders the LDS accesses of one wave (the LDS serves a wave's requests in
// program order; this keeps the compiler from moving them across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Top-k of E <= 64*NC logits by one wave (k <= 16 <= E; descending, equal
// logits -> lower id first), in three steps that a caller may separate:
// topk_threshold, topk_select (the selection, in id order, into sm.ckey /
// sm.cval) and topk_rank (its order, into sm.sid / sm.val, and optionally
// the softmax restricted to the selection into sm.sw). Lane l holds the
// logits of ids l + 64c (c < NC) as order keys (a > b <=> key(a) > key(b)),
// and key 0 for ids >= E.
//
// topk_threshold: a threshold T is built bit by bit from the top: a bit stays
// set when at least k keys reach the prefix with it set (compare masks +
// popcount per 64 keys); the search stops early once exactly k keys reach T.
// After a full search T is the k-th largest key; after an early stop the keys
// reaching T are exactly the k largest.
template <int NC>
__device__ __forceinline__ u32 topk_threshold(const u32 (&key)[4], int k) {
  u32 thr = 0u;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const u32 cand = thr | (1u << b);
    // all compares first, into masks of their own, so their latencies
    // overlap before the counts read them
    unsigned long long m[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) m[c] = __builtin_amdgcn_uicmp(key[c], cand, 35);   // 35: unsigned >=
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) cnt += __popcll(m[c]);
    if (cnt >= k) {
      thr = cand;
      if (cnt == k) break;
    }
  }
  return thr;
}

// topk_select: every key above T is selected and keys equal to T fill the
// remaining places in id order; ids >= E are never selected. The selection
// is stored in id order: sm.ckey[p] = key << 32 | ~id (distinct, a larger
// value means a higher logit or, on equal logits, a lower id), sm.cval[p]
// its logit, p < k. No wait on the stores: the caller orders them.
template <int NC>
__device__ __forceinline__ void topk_select(const u32 (&key)[4], const float (&v)[4], int E, int k, u32 thr,
                                            TopkSmem& sm) {
  const int lane = threadIdx.x & (WAVE - 1);
  const unsigned long long below = lane ? (~0ull >> (WAVE - lane)) : 0ull;
  // the selection's compares up front, into masks of their own: keys above
  // T, and keys equal to T among ids < E
  unsigned long long gtm[NC], eqm[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int nv = E - WAVE * c;                   // ids < E in this group of 64
    const unsigned long long vm = nv >= WAVE ? ~0ull : (nv > 0 ? (1ull << nv) - 1 : 0ull);
    gtm[c] = __builtin_amdgcn_uicmp(key[c], thr, 34);          // 34: unsigned >
    eqm[c] = __builtin_amdgcn_uicmp(key[c], thr, 32) & vm;     // 32: ==
  }
  int gt = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) gt += __popcll(gtm[c]);
  const int need = k - gt;                         // >= 1 places left for keys equal to T
  int ties_before = 0, base = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int id = lane + WAVE * c;
    const unsigned long long em = eqm[c];
    const bool eq = (em >> lane) & 1ull;
    const bool sel = ((gtm[c] >> lane) & 1ull) || (eq && ties_before + __popcll(em & below) < need);
    ties_before += __popcll(em);
    // without keys equal to T in the group the selection is the keys above it
    const unsigned long long sm_mask = em ? __ballot(sel) : gtm[c];
    if (sel) {
      const int pos = base + __popcll(sm_mask & below);
      sm.ckey[pos] = ((unsigned long long)key[c] << 32) | (u32)~(u32)id;
      sm.cval[pos] = v[c];
    }
    base += __popcll(sm_mask);
  }
}

// topk_rank: the rank of a selected key is the number of selected keys
// above it; only the k selected keys are compared, against each other.
// Reads the selection topk_select stored (visible to this wave).
__device__ __forceinline__ void topk_rank(int k, bool want_weights, TopkSmem& sm) {
  const int lane = threadIdx.x & (WAVE - 1);
  if (lane < k) {
    const unsigned long long mk = sm.ckey[lane];
    int r = 0;
    for (int j = 0; j < k; ++j) r += sm.ckey[j] > mk ? 1 : 0;
    sm.sid[r] = (int32_t)~(u32)mk;
    sm.val[r] = sm.cval[lane];
  }
  wave_lds_sync();
  if (want_weights && lane < k) {
    // every lane forms the denominator in the same order
    const float l0 = sm.val[0];
    float den = 0.f;
    for (int j = 0; j < k; ++j) den += __expf(sm.val[j] - l0);
    sm.sw[lane] = __expf(sm.val[lane] - l0) / den;
  }
  wave_lds_sync();
}

// The rank of selection entry p (id order) among the k selected: every
// lane reads all 16 entries at once and counts those above entry p.
__device__ __forceinline__ int topk_entry_rank(const TopkSmem& sm, int p, int k) {
  unsigned long long c[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) c[j] = sm.ckey[j];
  const unsigned long long mine = sm.ckey[p];
  int r = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) r += (j < k && c[j] > mine) ? 1 : 0;
  return r;
}

template <int NC>
__device__ void wave_topk(const float* __restrict__ lg, int E, int k, bool want_weights, TopkSmem& sm) {
  const int lane = threadIdx.x & (WAVE - 1);
  float v[4];
  u32 key[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int id = lane + WAVE * c;
    v[c] = (c < NC && id < E) ? lg[id] : 0.f;
    key[c] = (c < NC && id < E) ? order_key(v[c]) : 0u;
  }
  const u32 thr = topk_threshold<NC>(key, k);
  topk_select<NC>(key, v, E, k, thr, sm);
  wave_lds_sync();
  topk_rank(k, want_weights, sm);
}

__device__ __forceinline__ void wave_topk_any(const float* __restrict__ lg, int E, int k, bool want_weights,
                                              TopkSmem& sm) {
  if (E <= WAVE) wave_topk<1>(lg, E, k, want_weights, sm);
  else if (E <= 2 * WAVE) wave_topk<2>(lg, E, k, want_weights, sm);
  else if (E <= 3 * WAVE) wave_topk<3>(lg, E, k, want_weights, sm);
  else wave_topk<4>(lg, E, k, want_weights, sm);
}

// One wave per token.
__global__ __launch_bounds__(WAVE) void topk_kernel(const float* __restrict__ logits, int32_t* __restrict__ ids,
                                                    float* __restrict__ w, int E, int k, int T) {
  __shared__ TopkSmem sm;
  const int t = blockIdx.x;
  wave_topk_any(logits + (size_t)t * E, E, k, true, sm);
  if (threadIdx.x < k) {
    ids[(size_t)t * k + threadIdx.x] = sm.sid[threadIdx.x];
    w[(size_t)t * k + threadIdx.x] = sm.sw[threadIdx.x];
  }
}

// ------------------------------------------------------------------ residual + RMSNorm
// Element order shared by the standalone norm kernel and the router prologue
// (so both produce the same bits): thread tid owns the 4-element chunks
// starting at 4*(tid + 256c); the sum of squares is accumulated chunk by
// chunk, then reduced over the wave (butterfly) and over the 4 waves.
// One barrier: a caller that reduces again uses another part array, and
// reuses one only after a later reduction's barrier (by then every wave has
// read it).
__device__ __forceinline__ float block_sum4(float v, float* part) {
  v = group_sum<WAVE>(v);
  if ((threadIdx.x & (WAVE - 1)) == 0) part[threadIdx.x / WAVE] = v;
  __syncthreads();
  return (part[0] + part[1]) + (part[2] + part[3]);
}

// ------------------------------------------------------------------ router GEMV
// One block per expert row; the 256 threads split the hidden dimension
// (4 consecutive fp32 weights each per chunk). Tokens loop inside with the
// weight slice held in registers. Block reduction in a fixed order.
// With NORM the block first forms its input as x = bf16(RMSNorm(x_in +
// y_prev)) (the stacked-layer epilogue of the previous layer, recomputed by
// every block) and block 0 stores it to x_out. A token's x and y loads are
// issued together, before either is waited for.
template <int CH, bool NORM>  // chunks of 4 weights per thread: H = CH * 1024
__global__ __launch_bounds__(BLOCK) void router_kernel(const float* __restrict__ wr, const uint16_t* __restrict__ x,
                                                       const float* __restrict__ y_prev, uint16_t* __restrict__ x_out,
                                                       float eps, float* __restrict__ logits, int E, int H,
                                                       int T QMOE_TL_PARAMS) {
  // the norm's and the dot's reductions use one part array each (without the
  // norm, tokens alternate between the two)
  __shared__ float part[2][BLOCK / WAVE];
  QMOE_TL_SCOPE(wr, 0);
  // every kernel argument in registers before the first load (the compiler
  // otherwise fetches them in dependent batches, each a scalar round trip)
  asm volatile("" ::"s"(wr), "s"(x), "s"(y_prev), "s"(x_out), "s"(eps), "s"(logits), "s"(E), "s"(H), "s"(T));
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  float w[CH][4];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wr + (size_t)e * H + 4 * (tid + BLOCK * c)));
    w[c][0] = as_f32(v.x); w[c][1] = as_f32(v.y); w[c][2] = as_f32(v.z); w[c][3] = as_f32(v.w);
  }
  // T >= 1 (the launcher skips empty batches), so the first token's loads
  // are not held behind a test of T
  for (int t = 0;;) {
    uint2 xq[CH];
    u32x4 yq[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      xq[c] = *reinterpret_cast<const uint2*>(x + (size_t)t * H + 4 * (tid + BLOCK * c));
      if constexpr (NORM) yq[c] = load16(y_prev + (size_t)t * H + 4 * (tid + BLOCK * c));
    }
    __builtin_amdgcn_sched_barrier(0);
    float xv[CH][4];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint2 q = xq[c];
      xv[c][0] = bf16_bits_to_float(q.x & 0xFFFFu); xv[c][1] = bf16_bits_to_float(q.x >> 16);
      xv[c][2] = bf16_bits_to_float(q.y & 0xFFFFu); xv[c][3] = bf16_bits_to_float(q.y >> 16);
    }
    if constexpr (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const u32x4 q = yq[c];
        xv[c][0] += as_f32(q.x); xv[c][1] += as_f32(q.y); xv[c][2] += as_f32(q.z); xv[c][3] += as_f32(q.w);
#pragma unroll
        for (int i = 0; i < 4; ++i) ss = fmaf(xv[c][i], xv[c][i], ss);
      }
      const float inv = 1.0f / sqrtf(block_sum4(ss, part[0]) / (float)H + eps);
      QMOE_TL_MARK(5);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        uint16_t b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          b[i] = float_to_bf16_rne(xv[c][i] * inv);
          xv[c][i] = bf16_bits_to_float(b[i]);
        }
        if (e == 0)
          *reinterpret_cast<uint2*>(x_out + (size_t)t * H + 4 * (tid + BLOCK * c)) =
              make_uint2((u32)b[0] | ((u32)b[1] << 16), (u32)b[2] | ((u32)b[3] << 16));
      }
    }
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(w[c][i], xv[c][i], acc);
    const float tot = block_sum4(acc, part[NORM ? 1 : (t & 1)]);
    if (tid == 0) logits[(size_t)t * E + e] = tot;
    if (++t >= T) break;
  }
}

// ------------------------------------------------------------------ gate/up GEMV
// Wave work unit: RPS*U consecutive intermediate rows of one (token, slot);
// RPS = 64/LPR rows per step, LPR lanes per row, IPL sub-blocks per lane.
// h[(t*k + s)*I + r] = SiLU(G_e[r]·x_t) * (U_e[r]·x_t).
// Fused routing, after a wave's weight loads have left: the output row of
// its slot (selection entry p, T == 1) is the entry's rank; wave 0 of block 0
// also ranks the whole selection, forms the softmax over it and publishes
// ids and weights in rank order.
__device__ __forceinline__ int fused_rank_publish(TopkSmem& sm, int p, int k, int wid, int32_t* __restrict__ ids_out,
                                                  float* __restrict__ w_out) {
  const int r = topk_entry_rank(sm, p, k);
  if (blockIdx.x == 0 && blockIdx.y == 0 && wid == 0) {
    topk_rank(k, true, sm);
    const int lane = threadIdx.x & (WAVE - 1);
    if (lane < k) {
      ids_out[lane] = sm.sid[lane];
      w_out[lane] = sm.sw[lane];
    }
  }
  return r;
}

// ACT: the gate activation as a template argument, so the epilogue on this
// kernel's critical path carries no branch. FMT: the weight encoding; with
// MXFP4 a lane's sub-block is one 32-code block with its E8M0 scale byte.
template <int IPL, int LPR, int U, int ACT, int FMT, int NWB>
__global__ __launch_bounds__(NWB * WAVE) void gateup_kernel(
    const uint8_t* __restrict__ gu, size_t gu_expert_bytes, int rp_bytes, int H, int I, int E, int k,
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids_in, const float* __restrict__ logits,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, float* __restrict__ h, int T,
    int fused_topk QMOE_TL_PARAMS) {
  constexpr int RPS = WAVE / LPR;
  __shared__ TopkSmem s_topk;
  QMOE_TL_SCOPE(gu, 1);
  // the kernel arguments the first loads need, in registers at once (the
  // compiler otherwise fetches the logits pointer only after testing
  // fused_topk, a second scalar round trip)
  asm volatile("" ::"s"(logits), "s"(E), "s"(fused_topk), "s"(x), "s"(H), "s"(k));
  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = threadIdx.x / WAVE;
  // fused routing (T == 1): wave 0's logit loads leave first (every one in
  // bounds, so the search waits for them alone)
  float lv[4];
  u32 lk[4];
  if (fused_topk && wid == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int id = lane + WAVE * c;
      lv[c] = logits[(u32)(id < E ? id : E - 1)];
    }
  }
  // grid (I / (4 * RPS * U), k, T): no division stands before a load
  const int t = blockIdx.z;
  const int ts = t * k + blockIdx.y;                      // t*k + s
  const int r0 = (blockIdx.x * NWB + wid) * (RPS * U);
  const int rho = lane / LPR, lam = lane % LPR;
  // the expert stride in registers and the lane's row offsets (bytes from
  // the expert's base; an expert spans less than 4 GiB) formed before the
  // routing, so only the expert's base is left to form after it
  size_t geb = gu_expert_bytes;
  float* hout = h;
  asm volatile("" : "+s"(geb), "+s"(hout));
  const int half = H / 2;                 // code bytes per matrix row
  const int hdr = H / 2 * 2;              // headers start after both code areas
  // per row and sub-block: gate codes, up codes, gate header, up header
  // (super-blocks) or gate codes, up codes, gate scale, up scale (MXFP4)
  u32 off[U][IPL][4];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const u32 ro = (u32)(r0 + u * RPS + rho) * (u32)rp_bytes;
#pragma unroll
    for (int q = 0; q < IPL; ++q) {
      const u32 j = lam + LPR * q;
      off[u][q][0] = ro + 16 * j;
      off[u][q][1] = ro + half + 16 * j;
      if constexpr (FMT == FMT_MXFP4) {
        off[u][q][2] = ro + hdr + j;
        off[u][q][3] = ro + hdr + H / MXK + j;
      } else {
        off[u][q][2] = ro + hdr + QHDR * (j >> 3);
        off[u][q][3] = ro + hdr + QHDR * (H / QK) + QHDR * (j >> 3);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) asm volatile("" : "+v"(off[u][q][m]));
    }
  }
  // the activation slice does not depend on the routing: load it next so
  // its round trip overlaps the routing's (super-blocks: its pairing and
  // sums wait until the weight loads have left, below)
  u32 X[IPL][16];
  float S[IPL];
  u32x4 xr[IPL][4];
#pragma unroll
  for (int q = 0; q < IPL; ++q) {
    const int j = lam + LPR * q;
    load_x_raw(x + (size_t)t * H + 32 * j, xr[q]);
    if constexpr (FMT == FMT_MXFP4) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        X[q][4 * m] = xr[q][m].x; X[q][4 * m + 1] = xr[q][m].y;
        X[q][4 * m + 2] = xr[q][m].z; X[q][4 * m + 3] = xr[q][m].w;
      }
      S[q] = 0.f;
    }
  }
  if (fused_topk) {
    // T == 1: wave 0 of every block derives the same selection from the
    // logits, in id order; a wave's slot is an entry of it. Only the
    // threshold search and the selection stand before the weight loads: the
    // order of the selection (where a slot's output row goes) is taken after
    // they have left, and so is block 0's publication of the routing.
    if (wid == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) lk[c] = lane + WAVE * c < E ? order_key(lv[c]) : 0u;
      if (E <= WAVE) topk_select<1>(lk, lv, E, k, topk_threshold<1>(lk, k), s_topk);
      else if (E <= 2 * WAVE) topk_select<2>(lk, lv, E, k, topk_threshold<2>(lk, k), s_topk);
      else if (E <= 3 * WAVE) topk_select<3>(lk, lv, E, k, topk_threshold<3>(lk, k), s_topk);
      else topk_select<4>(lk, lv, E, k, topk_threshold<4>(lk, k), s_topk);
    }
    __syncthreads();
    QMOE_TL_MARK(5);
  }
  // the selection entry is read unconditionally (any in-bounds entry when
  // not fused), so the routing read stays an LDS read
  const unsigned long long sel_key = s_topk.ckey[ts < 16 ? ts : 0];
  const int e = fused_topk ? (int)~(u32)sel_key : ids_in[ts];
  int hrow = ts;                          // output row of h: t*k + rank of the slot
  const uint8_t* base = gu + (size_t)e * geb;
  if constexpr (FMT == FMT_MXFP4) {
    // scale bytes: gate's H/32, then up's
    u32x4 cg[U][IPL], cu[U][IPL];
    u32 sg[U][IPL], su[U][IPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int q = 0; q < IPL; ++q) {
        cg[u][q] = load_nt(base + off[u][q][0]);
        cu[u][q] = load_nt(base + off[u][q][1]);
        sg[u][q] = __builtin_nontemporal_load(base + off[u][q][2]);
        su[u][q] = __builtin_nontemporal_load(base + off[u][q][3]);
      }
    }
    if (fused_topk) {
      __builtin_amdgcn_sched_barrier(0);
      hrow = fused_rank_publish(s_topk, ts, k, wid, ids_out, w_out);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float pg = 0.f, pu = 0.f;
#pragma unroll
      for (int q = 0; q < IPL; ++q) {
        pg = fmaf(e8m0_scale(sg[u][q]), dot_fp4_bf16(cg[u][q], X[q]), pg);
        pu = fmaf(e8m0_scale(su[u][q]), dot_fp4_bf16(cu[u][q], X[q]), pu);
      }
      pg = group_sum<LPR>(pg);
      pu = group_sum<LPR>(pu);
      if (u == 0) QMOE_TL_MARK(6);
      if (lam == 0) hout[(size_t)hrow * I + r0 + u * RPS + rho] = gate_act(pg, pu, ACT);
    }
    return;
  }
  u32x4 cg[U][IPL], cu[U][IPL], hg[U][IPL], hu[U][IPL];
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int q = 0; q < IPL; ++q) {
      cg[u][q] = load_nt(base + off[u][q][0]);
      cu[u][q] = load_nt(base + off[u][q][1]);
      hg[u][q] = load_nt(base + off[u][q][2]);
      hu[u][q] = load_nt(base + off[u][q][3]);
    }
    if (u == 0) {
      // the activation pairing and sums after the first row's loads have
      // left, so they overlap its round trip instead of delaying its start,
      // and before the later rows' loads (the empty asm keeps the compiler
      // from sinking them below the routing epilogue)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < IPL; ++q) {
        S[q] = x_pairs(xr[q], X[q]);
        asm volatile("" : "+v"(S[q]));
#pragma unroll
        for (int m = 0; m < 16; ++m) asm volatile("" : "+v"(X[q][m]));
      }
    }
  }
  if (fused_topk) hrow = fused_rank_publish(s_topk, ts, k, wid, ids_out, w_out);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float pg = 0.f, pu = 0.f;
#pragma unroll
    for (int q = 0; q < IPL; ++q) {
      const int jj = (lam + LPR * q) & 7;
      const Affine ag = header_affine(hg[u][q], jj);
      const Affine au = header_affine(hu[u][q], jj);
      const float Ag = dot_codes_bf16(cg[u][q], X[q]);
      const float Au = dot_codes_bf16(cu[u][q], X[q]);
      pg += ag.a * Ag - (128.f * ag.a + ag.b) * S[q];
      pu += au.a * Au - (128.f * au.a + au.b) * S[q];
    }
    pg = group_sum<LPR>(pg);
    pu = group_sum<LPR>(pu);
    if (u == 0) QMOE_TL_MARK(6);
    if (lam == 0) hout[(size_t)hrow * I + r0 + u * RPS + rho] = gate_act(pg, pu, ACT);
  }
}

// ------------------------------------------------------------------ down GEMV + combine
// Items of an output row: (slot s, sub-block j) for s < k, j < I/32, i.e.
// G = k*I/32 <= 64*NW items. A block of NW waves (4, or 8 when G > 256)
// computes R consecutive output rows of one token; wave w takes the
// contiguous item range [w*IW, (w+1)*IW), IW = ceil(G/NW) <= 64, one item
// per lane, for all R rows, so a lane loads its 32 values of h once (fp32,
// straight into registers) and one 16-byte code chunk and header per row.
// The routing is read directly, so the weight loads leave as soon as the
// expert ids arrive. The wave partials of a row are added in wave order. h stays fp32: the codes are converted exactly
// and every product and sum is an fp32 operation, so h keeps its full range
// and precision.
// y[t*H + n] = sum_s w_s * D_{e_s}[n]·h_{t,s}. With MXFP4 weights an item's
// 32 codes share one E8M0 scale byte.
template <int R, int FMT, int NW>
__global__ __launch_bounds__(NW * WAVE) void down_kernel(
    const uint8_t* __restrict__ dn, size_t dn_expert_bytes, int drow_bytes, int H, int I, int k,
    const int32_t* __restrict__ ids, const float* __restrict__ wts, const float* __restrict__ h,
    float* __restrict__ y, int T, u32 nsb_inv QMOE_TL_PARAMS) {
  __shared__ float part[NW][R];
  QMOE_TL_SCOPE(dn, 2);
  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = threadIdx.x / WAVE;
  // grid (H / R, T): no division stands before a load
  const int t = blockIdx.y;
  const int n0 = blockIdx.x * R;
  const int nsb = I / 32;
  const int G = k * nsb;
  const int IW = (G + NW - 1) / NW;
  const int i = wid * IW + lane;
  const bool valid = lane < IW && i < G;
  // an idle lane takes the item of the wave's last busy lane, so every load
  // below is in bounds and none is conditional: the weight loads then wait
  // for the expert id alone, not for h and ws as well (a conditional load
  // makes the compiler drain every load in flight). An idle lane's ws and h
  // are zeroed where they are used, and its loads hit lines already fetched.
  const int ic = min(wid * IW + min(lane, IW - 1), G - 1);
  // ic / nsb as a multiply by nsb_inv = ceil(2^32 / nsb): exact for every
  // ic < 2^32 / nsb (here ic < 512), the rounding error staying below 1/nsb
  const int s = (int)__umulhi((u32)ic, nsb_inv);
  const int j = ic - s * nsb;
  const int e = ids[(size_t)t * k + s];
  const float ws_raw = wts[(size_t)t * k + s];
  u32x4 hr[8];
  const float* hp = h + ((size_t)t * k + s) * I + 32 * j;
#pragma unroll
  for (int c = 0; c < 8; ++c) hr[c] = load16(hp + 4 * c);
  const uint8_t* row0 = dn + (size_t)e * dn_expert_bytes + (size_t)n0 * drow_bytes;
  using Hdr = std::conditional_t<FMT == FMT_MXFP4, u32, u32x4>;
  u32x4 cd[R];
  Hdr hd[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint8_t* row = row0 + (size_t)r * drow_bytes;
    cd[r] = load_nt(row + 16 * j);
    if constexpr (FMT == FMT_MXFP4) hd[r] = __builtin_nontemporal_load(row + I / 2 + j);
    else hd[r] = load_nt(row + I / 2 + QHDR * (j >> 3));
  }
  // every weight load in flight before the first use of h
  __builtin_amdgcn_sched_barrier(0);
  const float ws = valid ? ws_raw : 0.f;
  float hv[32];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    hv[4 * c] = valid ? as_f32(hr[c].x) : 0.f; hv[4 * c + 1] = valid ? as_f32(hr[c].y) : 0.f;
    hv[4 * c + 2] = valid ? as_f32(hr[c].z) : 0.f; hv[4 * c + 3] = valid ? as_f32(hr[c].w) : 0.f;
  }
  float p[R];
  if constexpr (FMT == FMT_MXFP4) {
#pragma unroll
    for (int r = 0; r < R; ++r) p[r] = group_sum<WAVE>(ws * (e8m0_scale(hd[r]) * dot_fp4_f32(cd[r], hv)));
  } else {
    float S = 0.f;                                 // sum of the sub-block's h (the min term)
#pragma unroll
    for (int c = 0; c < 32; ++c) S += hv[c];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const Affine a = header_affine(hd[r], j & 7);
      p[r] = group_sum<WAVE>(ws * fmaf(a.a, dot_codes_f32(cd[r], hv), -a.b * S));
    }
  }
  QMOE_TL_MARK(6);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) part[wid][r] = p[r];
  }
  __syncthreads();
  if (threadIdx.x < R) {
    const int r = threadIdx.x;
    float acc = ((part[0][r] + part[1][r]) + part[2][r]) + part[3][r];
#pragma unroll
    for (int w = 4; w < NW; ++w) acc += part[w][r];
    y[(size_t)t * H + n0 + r] = acc;
  }
}

// ------------------------------------------------------------------ standalone residual + RMSNorm
// One block per token: v = x + y (fp32), x_next = bf16(v / sqrt(mean(v^2) + eps)),
// in the element order of the router prologue (H a multiple of 4). xn may be
// x itself (a one-layer stack writes the next step's input in place): every
// element is read by the thread that writes it, and the first pass's reads
// complete before the block barrier inside the sum, so x and xn are not
// declared restrict.
__global__ __launch_bounds__(BLOCK) void resid_norm_kernel(const uint16_t* x, const float* __restrict__ y, uint16_t* xn,
                                                           int H, float eps QMOE_TL_PARAMS) {
  __shared__ float part[BLOCK / WAVE];
  QMOE_TL_SCOPE(nullptr, 3);
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  float ss = 0.f;
  for (int c = 0; 4 * (tid + BLOCK * c) < H; ++c) {
    const int i0 = 4 * (tid + BLOCK * c);
    const uint2 q = *reinterpret_cast<const uint2*>(x + (size_t)t * H + i0);
    const u32x4 yv = load16(y + (size_t)t * H + i0);
    const float v0 = bf16_bits_to_float(q.x & 0xFFFFu) + as_f32(yv.x);
    const float v1 = bf16_bits_to_float(q.x >> 16) + as_f32(yv.y);
    const float v2 = bf16_bits_to_float(q.y & 0xFFFFu) + as_f32(yv.z);
    const float v3 = bf16_bits_to_float(q.y >> 16) + as_f32(yv.w);
    ss = fmaf(v0, v0, ss); ss = fmaf(v1, v1, ss); ss = fmaf(v2, v2, ss); ss = fmaf(v3, v3, ss);
  }
  const float inv = 1.0f / sqrtf(block_sum4(ss, part) / (float)H + eps);
  for (int c = 0; 4 * (tid + BLOCK * c) < H; ++c) {
    const int i0 = 4 * (tid + BLOCK * c);
    const uint2 q = *reinterpret_cast<const uint2*>(x + (size_t)t * H + i0);
    const u32x4 yv = load16(y + (size_t)t * H + i0);
    const u32 b0 = float_to_bf16_rne((bf16_bits_to_float(q.x & 0xFFFFu) + as_f32(yv.x)) * inv);
    const u32 b1 = float_to_bf16_rne((bf16_bits_to_float(q.x >> 16) + as_f32(yv.y)) * inv);
    const u32 b2 = float_to_bf16_rne((bf16_bits_to_float(q.y & 0xFFFFu) + as_f32(yv.z)) * inv);
    const u32 b3 = float_to_bf16_rne((bf16_bits_to_float(q.y >> 16) + as_f32(yv.w)) * inv);
    *reinterpret_cast<uint2*>(xn + (size_t)t * H + i0) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
  }
}

// ------------------------------------------------------------------ dispatch lists
// Exclusive scans of a and b over threads 0..255 of the block (threads past
// 255 take part in the calls but their results are unspecified); totals in
// tot_a / tot_b. Wave inclusive scans (shfl_up), then the four wave totals
// through LDS. Every thread of the block must call it.
__device__ __forceinline__ void excl_scan256x2(int a, int b, int& ea, int& eb, int& tot_a, int& tot_b, int* wsum) {
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wid = tid / WAVE;
  int ia = a, ib = b;
#pragma unroll
  for (int dl = 1; dl < WAVE; dl <<= 1) {
    const int ta = __shfl_up(ia, dl, WAVE), tb = __shfl_up(ib, dl, WAVE);
    if (lane >= dl) { ia += ta; ib += tb; }
  }
  if (tid < 4 * WAVE && lane == WAVE - 1) { wsum[wid] = ia; wsum[4 + wid] = ib; }
  __syncthreads();
  int ba = 0, bb = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (w < wid) { ba += wsum[w]; bb += wsum[4 + w]; }
  ea = ba + ia - a;
  eb = bb + ib - b;
  tot_a = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  tot_b = (wsum[4] + wsum[5]) + (wsum[6] + wsum[7]);
}

// One wave's group of up to 64 consecutive pairs p (lanes in order; act:
// the lane holds a pair, routed to expert e): each pair goes to
// pairs[base[e] + its rank among the group's pairs of e], ranks from ballots
// over the 8 bits of e (no atomics, so the order is p's), and base[e] moves
// past the group's pairs of e. base: the wave's own row of first positions.
__device__ __forceinline__ void place_group(int p, bool act, int e, int* base, int32_t* __restrict__ pairs) {
  const int lane = threadIdx.x & (WAVE - 1);
  unsigned long long same = __ballot(act);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const unsigned long long bal = __ballot(act && ((e >> b) & 1));
    same &= ((e >> b) & 1) ? bal : ~bal;
  }
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (WAVE - lane));
  const int rank = __popcll(same & below);
  const int n = __popcll(same);
  int b0 = 0;
  if (act) b0 = base[e];
  __builtin_amdgcn_wave_barrier();
  if (act) pairs[b0 + rank] = p;
  if (act && rank == n - 1) base[e] = b0 + n;
  __builtin_amdgcn_wave_barrier();
}

// Single block of 1024 threads (16 waves). counts[e] = #pairs routed to e,
// offsets = exclusive scan (E+1 entries), pairs = pair indices p = t*k+s
// ordered by (expert, p), and (slots given) the batched paths' work list:
// one record {e, first pair position, pairs} per tile of mt pairs in expert
// order, then zero records up to max_slots.
// Deterministic: ranks come from ballots, not from the order of atomics.
// NPL: a wave's ids are read NPL per lane at a time, all loads in flight
// before the first use (32 for large P; 1, the plain loop, for small P,
// where the unrolled form cost ~2 us).
constexpr int DISP_THREADS = 1024;
constexpr int DISP_WAVES = DISP_THREADS / WAVE;
template <int NPL>
__global__ __launch_bounds__(DISP_THREADS) void dispatch_kernel(const int32_t* __restrict__ ids, int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets, int32_t* __restrict__ pairs,
                                                                int4* __restrict__ slots, int E, int P, int mt,
                                                                int max_slots) {
  __shared__ int cnt[DISP_WAVES][256];
  __shared__ int wsum[8];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wid = tid / WAVE;
  for (int i = tid; i < DISP_WAVES * 256; i += DISP_THREADS) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int chunk = (P + DISP_WAVES - 1) / DISP_WAVES;
  const int p0 = wid * chunk, p1 = min(P, p0 + chunk);
  if constexpr (NPL == 1) {
    for (int p = p0 + lane; p < p1; p += WAVE) atomicAdd(&cnt[wid][ids[p]], 1);
  } else {
    for (int sb = p0; sb < p1; sb += WAVE * NPL) {
      int ev[NPL];
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int p = sb + WAVE * j + lane;
        ev[j] = p < p1 ? ids[p] : -1;
      }
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (ev[j] >= 0) atomicAdd(&cnt[wid][ev[j]], 1);
    }
  }
  __syncthreads();
  // thread e: its expert's column over the waves (exclusive within the expert)
  int tot = 0;
  if (tid < E) {
    for (int w = 0; w < DISP_WAVES; ++w) { const int c = cnt[w][tid]; cnt[w][tid] = tot; tot += c; }
  }
  const int tiles = tid < E ? (tot + mt - 1) / mt : 0;
  int ex_tot, ex_tiles, all_tot, all_tiles;
  excl_scan256x2(tid < E ? tot : 0, tiles, ex_tot, ex_tiles, all_tot, all_tiles, wsum);
  if (tid < E) {
    counts[tid] = tot;
    offsets[tid] = ex_tot;
    if (slots)
      for (int q = 0; q < tiles; ++q) slots[ex_tiles + q] = make_int4(tid, ex_tot + q * mt, min(mt, tot - q * mt), 0);
    for (int w = 0; w < DISP_WAVES; ++w) cnt[w][tid] += ex_tot;
  }
  if (tid == 0) offsets[E] = all_tot;
  if (slots)
    for (int i = all_tiles + tid; i < max_slots; i += DISP_THREADS) slots[i] = make_int4(0, 0, 0, 0);
  __syncthreads();
  // cnt[w][e] is now the first output slot of wave w's pairs for expert e;
  // pairs in increasing p (groups of 64 in order, lanes in order)
  auto place = [&](int p, bool act, int e) { place_group(p, act, e, cnt[wid], pairs); };
  if constexpr (NPL == 1) {
    for (int pb = p0; pb < p1; pb += WAVE) {
      const int p = pb + lane;
      const bool act = p < p1;
      place(p, act, act ? ids[p] : -1);
    }
  } else {
    for (int sb = p0; sb < p1; sb += WAVE * NPL) {
      int ev[NPL];
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int p = sb + WAVE * j + lane;
        ev[j] = p < p1 ? ids[p] : -1;
      }
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        if (sb + WAVE * j >= p1) break;               // wave-uniform
        const int p = sb + WAVE * j + lane;
        place(p, p < p1, ev[j]);
      }
    }
  }
}

// The same lists for large batches, over many workgroups: the pairs in
// chunks of DISP_CHUNK in pair order, one workgroup of 4 waves per chunk
// (wave w: the chunk's w-th quarter, in groups of 64). dispatch_hist_kernel
// counts each chunk's pairs per expert (part[c][e]). dispatch_place_kernel
// gives each wave, for every expert, the first output position of its pairs
// (the exclusive scan of the experts' totals, plus the pairs of that expert
// in the chunks and waves before it) and places them with place_group, so
// the lists are identical to dispatch_kernel's; workgroup 0 also writes
// counts, offsets and the work list.
__global__ __launch_bounds__(BLOCK) void dispatch_hist_kernel(const int32_t* __restrict__ ids,
                                                              int32_t* __restrict__ part, int E, int P) {
  static_assert(BLOCK == 256 && DISP_CHUNK % BLOCK == 0, "one histogram entry per thread, whole groups");
  __shared__ int hist[256];
  const int tid = threadIdx.x;
  hist[tid] = 0;
  __syncthreads();
  const int p0 = (int)blockIdx.x * DISP_CHUNK, p1 = min(P, p0 + DISP_CHUNK);
  constexpr int G = DISP_CHUNK / BLOCK;
  int ev[G];
  // every load in bounds (slots past the chunk reload its last pair, then
  // count nothing), so none is conditional and they are in flight together
#pragma unroll
  for (int j = 0; j < G; ++j) ev[j] = ids[min(p0 + tid + BLOCK * j, p1 - 1)];
#pragma unroll
  for (int j = 0; j < G; ++j)
    if (p0 + tid + BLOCK * j < p1) atomicAdd(&hist[ev[j]], 1);
  __syncthreads();
  if (tid < E) part[(size_t)blockIdx.x * E + tid] = hist[tid];
}

__global__ __launch_bounds__(BLOCK) void dispatch_place_kernel(const int32_t* __restrict__ ids,
                                                               const int32_t* __restrict__ part,
                                                               int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ pairs, int4* __restrict__ slots,
                                                               int E, int P, int nchunks, int mt, int max_slots) {
  constexpr int NW = BLOCK / WAVE, G = DISP_CHUNK / BLOCK;   // waves; groups of 64 per wave
  __shared__ int cnt[NW][256];
  __shared__ int wsum[8];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wid = tid / WAVE;
  const int c = (int)blockIdx.x;
  const int p0 = c * DISP_CHUNK, p1 = min(P, p0 + DISP_CHUNK);
  const int pw = p0 + wid * (DISP_CHUNK / NW);              // the wave's quarter
  int ev[G];
  // every load in bounds (slots past the chunk reload its last pair and are
  // then marked empty), so none is conditional and they are in flight together
#pragma unroll
  for (int j = 0; j < G; ++j) ev[j] = ids[min(pw + WAVE * j + lane, p1 - 1)];
#pragma unroll
  for (int j = 0; j < G; ++j)
    if (pw + WAVE * j + lane >= p1) ev[j] = -1;
  // thread e: expert e's total and its pairs in the chunks before this one,
  // the chunks' counts read 16 at a time (all 16 loads in flight)
  int tot = 0, before = 0;
  const int te = tid < E ? tid : 0;
  for (int i0 = 0; i0 < nchunks; i0 += 16) {
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = part[(size_t)min(i0 + u, nchunks - 1) * E + te];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int n = i0 + u < nchunks ? v[u] : 0;
      tot += n;
      before += i0 + u < c ? n : 0;
    }
  }
  if (tid >= E) tot = before = 0;
  for (int i = tid; i < NW * 256; i += BLOCK) (&cnt[0][0])[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < G; ++j)
    if (ev[j] >= 0) atomicAdd(&cnt[wid][ev[j]], 1);
  __syncthreads();
  const int tiles = tid < E ? (tot + mt - 1) / mt : 0;
  int ex_tot, ex_tiles, all_tot, all_tiles;
  excl_scan256x2(tid < E ? tot : 0, tiles, ex_tot, ex_tiles, all_tot, all_tiles, wsum);
  if (c == 0) {
    if (tid < E) {
      counts[tid] = tot;
      offsets[tid] = ex_tot;
      if (slots)
        for (int q = 0; q < tiles; ++q) slots[ex_tiles + q] = make_int4(tid, ex_tot + q * mt, min(mt, tot - q * mt), 0);
    }
    if (tid == 0) offsets[E] = all_tot;
    if (slots)
      for (int i = all_tiles + tid; i < max_slots; i += BLOCK) slots[i] = make_int4(0, 0, 0, 0);
  }
  // cnt[w][e]: first output position of wave w's pairs of expert e
  if (tid < E) {
    int base = ex_tot + before;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int n = cnt[w][tid];
      cnt[w][tid] = base;
      base += n;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < G; ++j) {
    if (pw + WAVE * j >= p1) break;                           // wave-uniform
    place_group(pw + WAVE * j + lane, ev[j] >= 0, ev[j], cnt[wid], pairs);
  }
}

// ------------------------------------------------------------------ launchers

static hipError_t launch_router_big(const Layout& d, const float* wr, const uint16_t* x, const float* y_prev,
                                    uint16_t* x_out, float* logits, int T, hipStream_t s) {
  const int CH = d.H / 1024;
  dim3 grid(d.E), block(BLOCK);
  if (T <= 0) return hipSuccess;           // the kernel takes at least one token
#define QMOE_ROUTER(C)                                                                                        \
  if (y_prev)                                                                                                 \
    hipLaunchKernelGGL((router_kernel<C, true>), grid, block, 0, s, wr, x, y_prev, x_out, d.eps, logits, d.E, d.H, \
                       T QMOE_TL_ARGS);                                                                            \
  else                                                                                                        \
    hipLaunchKernelGGL((router_kernel<C, false>), grid, block, 0, s, wr, x, y_prev, x_out, d.eps, logits, d.E, d.H, \
                       T QMOE_TL_ARGS)
  switch (CH) {
    case 1: QMOE_ROUTER(1); break;
    case 2: QMOE_ROUTER(2); break;
    case 3: QMOE_ROUTER(3); break;
    case 4: QMOE_ROUTER(4); break;
    case 6: QMOE_ROUTER(6); break;
    case 8: QMOE_ROUTER(8); break;
    default: return hipErrorInvalidValue;
  }
#undef QMOE_ROUTER
  return hipGetLastError();
}

bool router_has_norm_prologue(const Layout& d) {
  const int CH = d.H / 1024;
  return d.H % 1024 == 0 && (CH == 1 || CH == 2 || CH == 3 || CH == 4 || CH == 6 || CH == 8);
}

hipError_t launch_router_norm(const Layout& d, const float* wr, const uint16_t* x_prev, const float* y_prev,
                              uint16_t* x_out, float* logits, int T, hipStream_t s) {
  if (!router_has_norm_prologue(d)) return hipErrorInvalidValue;
  return launch_router_big(d, wr, x_prev, y_prev, x_out, logits, T, s);
}

// Router for hidden sizes that are not a multiple of 1024: wave per row.
__global__ __launch_bounds__(BLOCK) void router_small_kernel(const float* __restrict__ wr, const uint16_t* __restrict__ x,
                                                             float* __restrict__ logits, int E, int H, int T) {
  const int e = blockIdx.x * (BLOCK / WAVE) + threadIdx.x / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  if (e >= E) return;
  for (int t = 0; t < T; ++t) {
    float acc = 0.f;
    for (int i = lane; i < H; i += WAVE) acc = fmaf(wr[(size_t)e * H + i], bf16_bits_to_float(x[(size_t)t * H + i]), acc);
    acc = group_sum<WAVE>(acc);
    if (lane == 0) logits[(size_t)t * E + e] = acc;
  }
}

hipError_t launch_router(const Layout& d, const float* wr, const uint16_t* x, float* logits, int T, hipStream_t s) {
  if (router_has_norm_prologue(d)) return launch_router_big(d, wr, x, nullptr, nullptr, logits, T, s);
  hipLaunchKernelGGL(router_small_kernel, dim3((d.E + 3) / 4), dim3(BLOCK), 0, s, wr, x, logits, d.E, d.H, T);
  return hipGetLastError();
}

hipError_t launch_topk(const Layout& d, const float* logits, int32_t* ids, float* w, int T, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3(T), dim3(WAVE), 0, s, logits, ids, w, d.E, d.k, T);
  return hipGetLastError();
}

// Grid dimensions past x hold at most this many blocks; longer batches are
// launched in chunks of tokens.
constexpr int GRID_YZ_MAX = 65535;

template <int IPL, int LPR, int U, int ACT, int FMT, int NWB>
static void gateup_launch(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* ids,
                          const float* logits, int32_t* ids_out, float* w_out, float* h, int T, bool fused,
                          hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int RPS = WAVE / LPR;
  const dim3 grid(d.I / (NWB * RPS * U), d.k, T);
  if (ev0 || ev1) {
    // measurement launch: the events bracket this kernel's execution
    hipExtLaunchKernelGGL((gateup_kernel<IPL, LPR, U, ACT, FMT, NWB>), grid, dim3(NWB * WAVE), 0, s, ev0, ev1,
                          0, layer + d.gu_off, d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.E, d.k, x, ids, logits,
                          ids_out, w_out, h, T, fused ? 1 : 0 QMOE_TL_ARGS);
    return;
  }
  hipLaunchKernelGGL((gateup_kernel<IPL, LPR, U, ACT, FMT, NWB>), grid, dim3(NWB * WAVE), 0, s,
                     layer + d.gu_off, d.gu_expert_bytes, (int)d.rp_bytes, d.H, d.I, d.E, d.k, x, ids, logits,
                     ids_out, w_out, h, T, fused ? 1 : 0 QMOE_TL_ARGS);
}

template <int IPL, int LPR, int U, int ACT, int FMT>
static void gateup_go_act(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* ids,
                          const float* logits, int32_t* ids_out, float* w_out, float* h, int T, bool fused,
                          hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int RPS = WAVE / LPR;
  if (T <= 0) return;
  if (T > GRID_YZ_MAX) {   // per-token path only (fused routing and timed launches are single tokens)
    for (int t0 = 0; t0 < T; t0 += GRID_YZ_MAX)
      gateup_go_act<IPL, LPR, U, ACT, FMT>(d, layer, x + (size_t)t0 * d.H, ids + (size_t)t0 * d.k, logits, ids_out,
                                           w_out, h + (size_t)t0 * d.k * d.I, min(GRID_YZ_MAX, T - t0), false, s,
                                           nullptr, nullptr);
    return;
  }
  // a block's NWB waves take NWB * RPS * U consecutive rows of one (token,
  // slot); I is a multiple of 256, so every block of four waves is full.
  // One token with I a multiple of 12 * RPS * U: twelve waves per block, so
  // the k * I / (RPS * U) wave units of a 768-row layer at top-8 fill the
  // 256 CUs with one block each, and each CU searches the routing once
  // instead of once per block
  if (T == 1 && d.I % (12 * RPS * U) == 0 && d.k * d.I / (12 * RPS * U) <= 256) {
    gateup_launch<IPL, LPR, U, ACT, FMT, 12>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused, s, ev0, ev1);
    return;
  }
  gateup_launch<IPL, LPR, U, ACT, FMT, 4>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused, s, ev0, ev1);
}

template <int IPL, int LPR, int U>
static void gateup_go(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* ids, const float* logits,
                      int32_t* ids_out, float* w_out, float* h, int T, bool fused, hipStream_t s, hipEvent_t ev0,
                      hipEvent_t ev1) {
  if (d.fmt == FMT_MXFP4) {
    switch (d.act) {
      case 1: gateup_go_act<IPL, LPR, U, 1, FMT_MXFP4>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused, s, ev0, ev1); break;
      case 2: gateup_go_act<IPL, LPR, U, 2, FMT_MXFP4>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused, s, ev0, ev1); break;
      default: gateup_go_act<IPL, LPR, U, 0, FMT_MXFP4>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused, s, ev0, ev1); break;
    }
    return;
  }
  switch (d.act) {
    case 1: gateup_go_act<IPL, LPR, U, 1, FMT_Q4K>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused, s, ev0, ev1); break;
    case 2: gateup_go_act<IPL, LPR, U, 2, FMT_Q4K>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused, s, ev0, ev1); break;
    default: gateup_go_act<IPL, LPR, U, 0, FMT_Q4K>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused, s, ev0, ev1); break;
  }
}

hipError_t launch_gateup(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* ids,
                         const float* logits, int32_t* ids_out, float* w_out, float* h, int T, bool fused_topk,
                         hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int nsb = d.H / 32;
  // rows per wave unit must divide I (a multiple of 256): RPS*U <= 256
  if (nsb == 96) {
    // 96 sub-blocks: 32 lanes per row with three each, two rows per step
    gateup_go<3, 32, 2>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused_topk, s, ev0, ev1);
  } else if (nsb >= 64 && nsb % 64 == 0) {
    switch (nsb / 64) {
      // hidden 2048: 32-lane half waves with two sub-blocks each, two rows
      // per step and one step per wave (one row per 64-lane wave with two
      // steps was 1.8 % slower per decode step, 4 % with MXFP4 weights)
      case 1: gateup_go<2, 32, 1>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused_topk, s, ev0, ev1); break;
      case 2: gateup_go<2, 64, 2>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused_topk, s, ev0, ev1); break;
      case 3: gateup_go<3, 64, 1>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused_topk, s, ev0, ev1); break;
      case 4: gateup_go<4, 64, 1>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused_topk, s, ev0, ev1); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (nsb) {
      case 8: gateup_go<1, 8, 2>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused_topk, s, ev0, ev1); break;
      case 16: gateup_go<1, 16, 2>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused_topk, s, ev0, ev1); break;
      case 32: gateup_go<1, 32, 2>(d, layer, x, ids, logits, ids_out, w_out, h, T, fused_topk, s, ev0, ev1); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_down(const Layout& d, const uint8_t* layer, const int32_t* ids, const float* w, const float* h,
                       float* y, int T, hipStream_t s) {
  // rows per workgroup (and load phases) by encoding, from same-box A/B of
  // the 48-layer decode step: super-blocks 4 rows in one phase (8 rows in
  // two phases of 4: 0.6 % slower; 2 rows: 14 %), MXFP4 8 rows (4: 2 % slower)
  constexpr int RQ = 4, RM = 8;              // both divide every supported H
  const int G = d.k * (d.I / 32);
  if (G > 8 * WAVE || d.H % RM) return hipErrorInvalidValue;
  if (T <= 0) return hipSuccess;
  if (T > GRID_YZ_MAX) {
    for (int t0 = 0; t0 < T; t0 += GRID_YZ_MAX) {
      const hipError_t e = launch_down(d, layer, ids + (size_t)t0 * d.k, w + (size_t)t0 * d.k,
                                       h + (size_t)t0 * d.k * d.I, y + (size_t)t0 * d.H, min(GRID_YZ_MAX, T - t0), s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int nsb = d.I / 32;                  // >= 8
  const u32 nsb_inv = (u32)((0x100000000ull + nsb - 1) / nsb);
  // four waves cover up to 256 items of a row, eight up to 512
#define QMOE_DOWN(NW)                                                                                              \
  if (d.fmt == FMT_MXFP4)                                                                                          \
    hipLaunchKernelGGL((down_kernel<RM, FMT_MXFP4, NW>), dim3(d.H / RM, T), dim3(NW * WAVE), 0, s,                 \
                       layer + d.dn_off, d.dn_expert_bytes, (int)d.drow_bytes, d.H, d.I, d.k, ids, w, h, y, T,     \
                       nsb_inv QMOE_TL_ARGS);                                                                      \
  else                                                                                                             \
    hipLaunchKernelGGL((down_kernel<RQ, FMT_Q4K, NW>), dim3(d.H / RQ, T), dim3(NW * WAVE), 0, s,                   \
                       layer + d.dn_off, d.dn_expert_bytes, (int)d.drow_bytes, d.H, d.I, d.k, ids, w, h, y, T,     \
                       nsb_inv QMOE_TL_ARGS)
  if (G > 4 * WAVE) {
    QMOE_DOWN(8);
  } else {
    QMOE_DOWN(4);
  }
#undef QMOE_DOWN
  return hipGetLastError();
}

hipError_t launch_resid_norm(const Layout& d, const uint16_t* x, const float* y, uint16_t* x_next, int T, hipStream_t s) {
  hipLaunchKernelGGL(resid_norm_kernel, dim3(T), dim3(BLOCK), 0, s, x, y, x_next, d.H, d.eps QMOE_TL_ARGS);
  return hipGetLastError();
}

hipError_t launch_dispatch(const Layout& d, const int32_t* ids, int32_t* counts, int32_t* offsets, int32_t* pairs, int T,
                           hipStream_t s, int mt, void* slots, int max_slots, int32_t* part) {
  if (mt < 1) return hipErrorInvalidValue;
  // the slot records must cover every tile: at most ceil(T*k / mt) + min(E, T*k)
  const int P = T * d.k;
  if (slots && max_slots < (P + mt - 1) / mt + (P < d.E ? P : d.E)) return hipErrorInvalidValue;
  if (part && P > DISP_MULTI_MIN) {
    const int nchunks = (P + DISP_CHUNK - 1) / DISP_CHUNK;   // part holds nchunks x E counts
    hipLaunchKernelGGL(dispatch_hist_kernel, dim3(nchunks), dim3(BLOCK), 0, s, ids, part, d.E, P);
    hipLaunchKernelGGL(dispatch_place_kernel, dim3(nchunks), dim3(BLOCK), 0, s, ids, part, counts, offsets, pairs,
                       static_cast<int4*>(slots), d.E, P, nchunks, mt, slots ? max_slots : 0);
  } else if (P > 4 * DISP_THREADS)
    hipLaunchKernelGGL((dispatch_kernel<32>), dim3(1), dim3(DISP_THREADS), 0, s, ids, counts, offsets, pairs,
                       static_cast<int4*>(slots), d.E, P, mt, slots ? max_slots : 0);
  else
    hipLaunchKernelGGL((dispatch_kernel<1>), dim3(1), dim3(DISP_THREADS), 0, s, ids, counts, offsets, pairs,
                       static_cast<int4*>(slots), d.E, P, mt, slots ? max_slots : 0);
  return hipGetLastError();
}

// The batched paths' work list from given dispatch offsets (E+1 entries),
// as the dispatch kernel writes it. One block of 256 threads.
__global__ __launch_bounds__(BLOCK) void work_list_kernel(const int32_t* __restrict__ offsets, int4* __restrict__ slots,
                                                         int E, int mt, int max_slots) {
  __shared__ int wsum[8];
  const int tid = threadIdx.x;
  const int n = tid < E ? offsets[tid + 1] - offsets[tid] : 0;
  const int units = (n + mt - 1) / mt;
  int ex, ex2, tot, tot2;
  excl_scan256x2(units, 0, ex, ex2, tot, tot2, wsum);
  if (tid < E)
    for (int q = 0; q < units; ++q) slots[ex + q] = make_int4(tid, offsets[tid] + q * mt, min(mt, n - q * mt), 0);
  for (int i = tot + tid; i < max_slots; i += BLOCK) slots[i] = make_int4(0, 0, 0, 0);
}

hipError_t launch_work_list(const Layout& d, const int32_t* offsets, int T, int mt, void* slots, int max_slots,
                            hipStream_t s) {
  if (!slots || mt < 1) return hipErrorInvalidValue;
  const int P = T * d.k;
  if (max_slots < (P + mt - 1) / mt + (P < d.E ? P : d.E)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(work_list_kernel, dim3(1), dim3(BLOCK), 0, s, offsets, static_cast<int4*>(slots), d.E, mt,
                     max_slots);
  return hipGetLastError();
}

}  // namespace qmoe

#ifdef QMOE_TIMELINE
namespace qmoe {
__device__ unsigned long long tl_rec[TL_SLOTS][TL_WGS][TL_FIELDS];
const uint8_t* tl_host_base = nullptr;
float tl_host_inv = 0.f;
}  // namespace qmoe

extern "C" int moe_timeline_setup(const void* layer0, unsigned long long layer_bytes) {
  if (!layer0 || layer_bytes == 0) return (int)hipErrorInvalidValue;
  qmoe::tl_host_base = static_cast<const uint8_t*>(layer0);
  qmoe::tl_host_inv = (float)(256.0 / (double)layer_bytes);
  return (int)hipSuccess;
}

extern "C" int moe_timeline_reset(void) {
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(qmoe::tl_rec));
  if (e == hipSuccess) e = hipMemset(p, 0, sizeof(qmoe::tl_rec));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  return (int)e;
}

extern "C" int moe_timeline_read(unsigned long long* host) {
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpyFromSymbol(host, HIP_SYMBOL(qmoe::tl_rec), sizeof(qmoe::tl_rec));
  return (int)e;
}
#endif

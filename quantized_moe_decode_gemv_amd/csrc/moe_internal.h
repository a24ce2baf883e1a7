// Internal layout and launcher declarations shared by the C-ABI layer and the
// kernels. Not part of the public ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "../../include/moe.h"

namespace qmoe {

constexpr int QK = 256;            // weights per super-block
constexpr int QBYTES = 144;        // bytes per super-block
constexpr int QHDR = 16;           // header bytes (d, dmin, 12 bytes of 6-bit fields)
constexpr int QCODES = 128;        // code bytes
constexpr int MXK = 32;            // weights per MXFP4 block
constexpr int MXBYTES = 17;        // bytes per MXFP4 block (E8M0 scale, 16 code bytes)
constexpr int FMT_Q4K = 0, FMT_MXFP4 = 1;
constexpr size_t HEADER_BYTES = 4096;
constexpr uint64_t BLOB_MAGIC = 0x31424F4C42454F4DULL;  // "MOEBLOB1" little-endian
constexpr uint32_t BLOB_VERSION = 1;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Device layout of one layer (all offsets from the layer base, 256-aligned):
//   router   fp32 [E][H]
//   gate/up  per expert, per intermediate row r, one "row pair" record:
//            [gate codes H/2 B][up codes H/2 B][gate headers H/256*16 B][up headers H/256*16 B]
//            (codes of super-block b, sub-block j' at byte 128*b + 16*j'; canonical nibble order)
//   down     per expert, per output row n: [codes I/2 B][headers I/256*16 B]
// With MXFP4 weights the headers are the E8M0 scale bytes, one per 32-weight
// block (block b's 16 code bytes at 16*b, its scale at scales + b), and each
// record is padded to a multiple of 16 bytes.
struct Layout {
  int H, E, k, I, L, maxT;
  int act;                      // gate activation: 0 SiLU, 1 squared ReLU, 2 clamped SwiGLU
  int fmt;                      // FMT_Q4K or FMT_MXFP4
  uint32_t flags;
  float eps;
  int nbH, nbI;                 // super-blocks per gate/up row and per down row
  size_t rp_bytes;              // gate/up row-pair record
  size_t gu_expert_bytes;
  size_t drow_bytes;            // down row record
  size_t dn_expert_bytes;
  size_t router_off, gu_off, dn_off, layer_bytes;

  void init(const moe_config& c) {
    H = c.hidden; E = c.n_experts; k = c.top_k; I = c.inter; L = c.n_layers; maxT = c.max_tokens;
    flags = c.flags; eps = c.rms_eps;
    act = (c.flags & MOE_FLAG_ACT_RELU2) ? 1 : ((c.flags & MOE_FLAG_ACT_SWIGLU_OAI) ? 2 : 0);
    fmt = (c.flags & MOE_FLAG_WEIGHTS_MXFP4) ? FMT_MXFP4 : FMT_Q4K;
    nbH = H / QK; nbI = I / QK;
    if (fmt == FMT_MXFP4) {
      rp_bytes = align_up((size_t)H + H / MXK * 2, 16);
      drow_bytes = align_up((size_t)I / 2 + I / MXK, 16);
    } else {
      rp_bytes = (size_t)2 * nbH * QBYTES;
      drow_bytes = (size_t)nbI * QBYTES;
    }
    gu_expert_bytes = (size_t)I * rp_bytes;
    dn_expert_bytes = (size_t)H * drow_bytes;
    router_off = 0;
    gu_off = align_up((size_t)E * H * 4, 256);
    dn_off = align_up(gu_off + (size_t)E * gu_expert_bytes, 256);
    layer_bytes = align_up(dn_off + (size_t)E * dn_expert_bytes, 256);
  }
};

struct BlobHeader {
  uint64_t magic;
  uint32_t version;
  int32_t hidden, n_experts, top_k, inter, n_layers;
  uint64_t layer_bytes;
  uint64_t header_bytes;
  int32_t weight_format;        // FMT_Q4K or FMT_MXFP4
};

// Dispatch over many workgroups above DISP_MULTI_MIN routed pairs, one per
// DISP_CHUNK pairs.
constexpr int DISP_CHUNK = 1024;
constexpr int DISP_MULTI_MIN = 4096;

// Scratch carve-up for T tokens (offsets 256-aligned).
struct Scratch {
  size_t logits, ids, w, h, counts, offsets, pairs, slots, part, hbuf, ypair, total;
  void init(const Layout& d, int T) {
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes, 256); return r; };
    logits = take((size_t)T * d.E * 4);
    ids = take((size_t)T * d.k * 4);
    w = take((size_t)T * d.k * 4);
    h = take((size_t)T * d.k * d.I * 4);
    counts = take((size_t)d.E * 4);
    offsets = take((size_t)(d.E + 1) * 4);
    pairs = take((size_t)T * d.k * 4);
    // work records {expert, first pair, pairs}: one per routed expert, or per 16-pair tile
    slots = take((size_t)((T * d.k + 15) / 16 + d.E) * 16);
    // per-chunk expert counts of the multi-workgroup dispatch
    part = take((size_t)((T * d.k + DISP_CHUNK - 1) / DISP_CHUNK) * d.E * 4);
    // batched paths only (T > 1): h in expert-sorted pair order, 4 bytes per
    // value (fp32 on the expert-major GEMV, bf16 hi and lo planes on the MFMA
    // tiles), and one fp32 output row per pair
    hbuf = take(T > 1 ? (size_t)T * d.k * d.I * 4 : 0);
    ypair = take(T > 1 ? (size_t)T * d.k * d.H * 4 : 0);
    total = o;
  }
};

// ---------------------------------------------------------------- launchers
// All return hipSuccess or the launch error. Pointers are device pointers.
hipError_t launch_router(const Layout& d, const float* wr, const uint16_t* x, float* logits, int T,
                         hipStream_t s);
// Router whose input is formed as bf16(RMSNorm(x_prev + y_prev)) inside the
// kernel (stored to x_out by block 0); available when router_has_norm_prologue.
bool router_has_norm_prologue(const Layout& d);
hipError_t launch_router_norm(const Layout& d, const float* wr, const uint16_t* x_prev, const float* y_prev,
                              uint16_t* x_out, float* logits, int T, hipStream_t s);
hipError_t launch_topk(const Layout& d, const float* logits, int32_t* ids, float* w, int T, hipStream_t s);
// ids/w given (fused_topk == false), or computed per block from logits (T == 1 only).
hipError_t launch_gateup(const Layout& d, const uint8_t* layer, const uint16_t* x, const int32_t* ids,
                         const float* logits, int32_t* ids_out, float* w_out, float* h, int T,
                         bool fused_topk, hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_down(const Layout& d, const uint8_t* layer, const int32_t* ids, const float* w,
                       const float* h, float* y, int T, hipStream_t s);
hipError_t launch_resid_norm(const Layout& d, const uint16_t* x, const float* y, uint16_t* x_next, int T,
                             hipStream_t s);
// Batched-path work lists, written by the dispatch or, from given dispatch
// lists, by launch_work_list: slot records {expert, first pair position,
// pairs}, one per tile of mt pairs of every expert in expert order (mt = T*k:
// one per routed expert), followed by {0, 0, 0} records up to max_slots (at
// least ceil(T*k / mt) + min(E, T*k)).
// part: scratch for the per-chunk counts of the multi-workgroup dispatch
// (ceil(T*k / DISP_CHUNK) x E int32), used above DISP_MULTI_MIN pairs; null:
// the single-workgroup dispatch at every size.
hipError_t launch_dispatch(const Layout& d, const int32_t* ids, int32_t* counts, int32_t* offsets,
                           int32_t* pairs, int T, hipStream_t s, int mt = 1, void* slots = nullptr, int max_slots = 0,
                           int32_t* part = nullptr);
hipError_t launch_work_list(const Layout& d, const int32_t* offsets, int T, int mt, void* slots, int max_slots,
                            hipStream_t s);

// MFMA tiles of 16, 64 or 128 pairs (T > 1; hidden 512, 1024 or 2048, inter
// <= 1024); tiles = slot records of g16_mt pairs. hb: h as bf16 hi and lo
// planes (T*k*I values each).
bool g16_supported(const Layout& d);
int g16_mt(const Layout& d, int T);
int g16_max_tiles(const Layout& d, int T);
hipError_t launch_g16_ffn(const Layout& d, const uint8_t* layer, const uint16_t* x, const float* w,
                          const int32_t* pairs, const void* tiles, uint16_t* hb, float* ypair, float* out, int T,
                          hipStream_t s);
// out[t] = sum_s w[t][s] * ypair[t*k + s], slot order
hipError_t launch_combine(const Layout& d, const float* ypair, const float* w, float* out, int T, hipStream_t s);

// expert-major GEMV path (T > 1, few pairs per expert); slots from the dispatch
bool egemv_supported(const Layout& d);
hipError_t launch_egemv_ffn(const Layout& d, const uint8_t* layer, const uint16_t* x, const float* w,
                            const int32_t* pairs, const void* slots, float* hbuf, float* ypair, float* out,
                            int T, hipStream_t s);

}  // namespace qmoe

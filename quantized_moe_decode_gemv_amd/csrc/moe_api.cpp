// C ABI of the quantized MoE expert FFN: plan, size queries, host-side
// packing of canonical 4-bit super-blocks into the device layout, argument
// validation and kernel launches. No device allocation, no synchronisation,
// no host reads of device memory.
#include <stdlib.h>
#include <string.h>

#include <new>

#include "moe_internal.h"

using namespace qmoe;

struct moe_plan {
  Layout d;
};

static bool cfg_ok(const moe_config* c) {
  if (!c) return false;
  const int H = c->hidden, E = c->n_experts, k = c->top_k, I = c->inter;
  if (H <= 0 || H % QK || E < 1 || E > 256 || k < 1 || k > 16 || k > E || I <= 0 || I % QK) return false;
  if (c->n_layers < 1 || c->max_tokens < 1 || !(c->rms_eps >= 0.0f)) return false;
  // device index arithmetic over (token, slot, row) runs in 32 bits
  if ((long long)c->max_tokens * k * (H > I ? H : I) >= (1LL << 31)) return false;
  // gate/up lane mapping: hidden/32 sub-blocks per row either fill a
  // power-of-two lane group (256, 512, 1024), half waves with two per lane
  // (2048), whole waves (2048 * {2..4}) or three per lane of 32-lane groups
  // (3072)
  const bool h_ok = H == 256 || H == 512 || H == 1024 || H == 3072 || (H % 2048 == 0 && H / 2048 <= 4);
  if (!h_ok) return false;
  // down: k * inter/32 items per output row, one per lane of at most 8 waves
  if ((long long)k * (I / 32) > 512) return false;
  const uint32_t force = c->flags & (MOE_FLAG_FORCE_GEMV | MOE_FLAG_FORCE_GROUPED | MOE_FLAG_FORCE_EXPERT_GEMV);
  const uint32_t act = c->flags & (MOE_FLAG_ACT_RELU2 | MOE_FLAG_ACT_SWIGLU_OAI);
  const uint32_t fmt = c->flags & MOE_FLAG_WEIGHTS_MXFP4;
  if (c->flags & ~(force | act | fmt)) return false;
  // the MFMA tiles: hidden 512, 1024 or 2048, inter <= 1024
  if ((force & MOE_FLAG_FORCE_GROUPED) && !((H == 512 || H == 1024 || H == 2048) && I <= 1024)) return false;
  if (force & (force - 1)) return false;          // at most one path may be forced
  if (act & (act - 1)) return false;              // at most one activation
  // expert-major GEMV: one 32-code sub-block of a down row per lane of a wave
  if ((force & MOE_FLAG_FORCE_EXPERT_GEMV) && I > 2048) return false;
  return true;
}

extern "C" int moe_is_supported(const moe_config* cfg) { return cfg_ok(cfg) ? 1 : 0; }

extern "C" int moe_plan_create(const moe_config* cfg, moe_plan** out) {
  if (!out) return MOE_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (!cfg) return MOE_ERR_INVALID_ARGUMENT;
  if (!cfg_ok(cfg)) return MOE_ERR_UNSUPPORTED;
  moe_plan* p = new (std::nothrow) moe_plan;
  if (!p) return MOE_ERR_INVALID_ARGUMENT;
  p->d.init(*cfg);
  *out = p;
  return MOE_OK;
}

extern "C" void moe_plan_destroy(moe_plan* plan) { delete plan; }

extern "C" size_t moe_header_bytes(const moe_plan* plan) { return plan ? HEADER_BYTES : 0; }
extern "C" size_t moe_layer_bytes(const moe_plan* plan) { return plan ? plan->d.layer_bytes : 0; }
extern "C" size_t moe_blob_bytes(const moe_plan* plan) {
  return plan ? HEADER_BYTES + (size_t)plan->d.L * plan->d.layer_bytes : 0;
}
extern "C" size_t moe_layer_offset(const moe_plan* plan, int32_t layer) {
  if (!plan || layer < 0 || layer >= plan->d.L) return 0;
  return HEADER_BYTES + (size_t)layer * plan->d.layer_bytes;
}
extern "C" size_t moe_scratch_bytes(const moe_plan* plan, int32_t T) {
  if (!plan || T < 0 || T > plan->d.maxT) return 0;
  Scratch s;
  s.init(plan->d, T);
  return s.total;
}

// ---------------------------------------------------------------- packing
extern "C" int moe_pack_header(const moe_plan* plan, void* dst_host) {
  if (!plan || !dst_host) return MOE_ERR_INVALID_ARGUMENT;
  memset(dst_host, 0, HEADER_BYTES);
  BlobHeader h;
  memset(&h, 0, sizeof(h));
  h.magic = BLOB_MAGIC;
  h.version = BLOB_VERSION;
  h.hidden = plan->d.H;
  h.n_experts = plan->d.E;
  h.top_k = plan->d.k;
  h.inter = plan->d.I;
  h.n_layers = plan->d.L;
  h.layer_bytes = plan->d.layer_bytes;
  h.header_bytes = HEADER_BYTES;
  h.weight_format = plan->d.fmt;
  memcpy(dst_host, &h, sizeof(h));
  return MOE_OK;
}

extern "C" int moe_blob_check(const moe_plan* plan, const void* header_host) {
  if (!plan || !header_host) return MOE_ERR_INVALID_ARGUMENT;
  BlobHeader h;
  memcpy(&h, header_host, sizeof(h));
  const Layout& d = plan->d;
  if (h.magic != BLOB_MAGIC || h.version != BLOB_VERSION || h.hidden != d.H || h.n_experts != d.E ||
      h.inter != d.I || h.n_layers != d.L || h.layer_bytes != d.layer_bytes || h.header_bytes != HEADER_BYTES ||
      h.weight_format != d.fmt)
    return MOE_ERR_BLOB_MISMATCH;
  return MOE_OK;
}

// canonical block -> (16-byte header, 128 code bytes) and back
static inline void split_block(const uint8_t* blk, uint8_t* hdr, uint8_t* codes) {
  memcpy(hdr, blk, QHDR);
  memcpy(codes, blk + QHDR, QCODES);
}
static inline void join_block(const uint8_t* hdr, const uint8_t* codes, uint8_t* blk) {
  memcpy(blk, hdr, QHDR);
  memcpy(blk + QHDR, codes, QCODES);
}

// MXFP4 rows: canonical [scale][16 code bytes] blocks <-> [codes][scales]
// scale codes 2..252: every weight, and every scaled pair the MFMA tiles
// convert, is then a normal bf16 (or zero)
static bool mx_scale_ok(uint8_t e) { return e >= 2 && e <= 252; }

static int pack_mx_layer(const Layout& d, const uint8_t* gate, const uint8_t* up, const uint8_t* down,
                         uint8_t* dst) {
  const int nbH = d.H / MXK, nbI = d.I / MXK;
  for (int e = 0; e < d.E; ++e) {
    for (int r = 0; r < d.I; ++r) {
      uint8_t* rp = dst + d.gu_off + (size_t)e * d.gu_expert_bytes + (size_t)r * d.rp_bytes;
      for (int m = 0; m < 2; ++m) {          // gate, up
        const uint8_t* src = (m ? up : gate) + ((size_t)e * d.I + r) * nbH * MXBYTES;
        uint8_t* codes = rp + (size_t)m * d.H / 2;
        uint8_t* scales = rp + d.H + (size_t)m * nbH;
        for (int b = 0; b < nbH; ++b) {
          if (!mx_scale_ok(src[(size_t)b * MXBYTES])) return MOE_ERR_INVALID_ARGUMENT;
          scales[b] = src[(size_t)b * MXBYTES];
          memcpy(codes + (size_t)b * 16, src + (size_t)b * MXBYTES + 1, 16);
        }
      }
    }
    for (int n = 0; n < d.H; ++n) {
      const uint8_t* src = down + ((size_t)e * d.H + n) * nbI * MXBYTES;
      uint8_t* row = dst + d.dn_off + (size_t)e * d.dn_expert_bytes + (size_t)n * d.drow_bytes;
      for (int b = 0; b < nbI; ++b) {
        if (!mx_scale_ok(src[(size_t)b * MXBYTES])) return MOE_ERR_INVALID_ARGUMENT;
        row[d.I / 2 + b] = src[(size_t)b * MXBYTES];
        memcpy(row + (size_t)b * 16, src + (size_t)b * MXBYTES + 1, 16);
      }
    }
  }
  return MOE_OK;
}

static void unpack_mx_layer(const Layout& d, const uint8_t* src, uint8_t* gate, uint8_t* up, uint8_t* down) {
  const int nbH = d.H / MXK, nbI = d.I / MXK;
  for (int e = 0; e < d.E; ++e) {
    for (int r = 0; r < d.I; ++r) {
      const uint8_t* rp = src + d.gu_off + (size_t)e * d.gu_expert_bytes + (size_t)r * d.rp_bytes;
      for (int m = 0; m < 2; ++m) {
        uint8_t* out = (m ? up : gate) + ((size_t)e * d.I + r) * nbH * MXBYTES;
        const uint8_t* codes = rp + (size_t)m * d.H / 2;
        const uint8_t* scales = rp + d.H + (size_t)m * nbH;
        for (int b = 0; b < nbH; ++b) {
          out[(size_t)b * MXBYTES] = scales[b];
          memcpy(out + (size_t)b * MXBYTES + 1, codes + (size_t)b * 16, 16);
        }
      }
    }
    for (int n = 0; n < d.H; ++n) {
      uint8_t* out = down + ((size_t)e * d.H + n) * nbI * MXBYTES;
      const uint8_t* row = src + d.dn_off + (size_t)e * d.dn_expert_bytes + (size_t)n * d.drow_bytes;
      for (int b = 0; b < nbI; ++b) {
        out[(size_t)b * MXBYTES] = row[d.I / 2 + b];
        memcpy(out + (size_t)b * MXBYTES + 1, row + (size_t)b * 16, 16);
      }
    }
  }
}

extern "C" int moe_pack_layer(const moe_plan* plan, const uint8_t* gate, const uint8_t* up, const uint8_t* down,
                              const float* router, void* dst_host) {
  if (!plan || !gate || !up || !down || !router || !dst_host) return MOE_ERR_INVALID_ARGUMENT;
  const Layout& d = plan->d;
  uint8_t* dst = static_cast<uint8_t*>(dst_host);
  memset(dst, 0, d.layer_bytes);
  memcpy(dst + d.router_off, router, (size_t)d.E * d.H * 4);
  if (d.fmt == FMT_MXFP4) return pack_mx_layer(d, gate, up, down, dst);
  const size_t grow = (size_t)d.nbH * QBYTES;   // canonical bytes of one gate/up row
  const size_t drow = (size_t)d.nbI * QBYTES;   // canonical bytes of one down row
  for (int e = 0; e < d.E; ++e) {
    for (int r = 0; r < d.I; ++r) {
      const uint8_t* g = gate + ((size_t)e * d.I + r) * grow;
      const uint8_t* u = up + ((size_t)e * d.I + r) * grow;
      uint8_t* rp = dst + d.gu_off + (size_t)e * d.gu_expert_bytes + (size_t)r * d.rp_bytes;
      uint8_t* gcodes = rp;
      uint8_t* ucodes = rp + (size_t)d.nbH * QCODES;
      uint8_t* ghdr = rp + (size_t)2 * d.nbH * QCODES;
      uint8_t* uhdr = ghdr + (size_t)d.nbH * QHDR;
      for (int b = 0; b < d.nbH; ++b) {
        split_block(g + (size_t)b * QBYTES, ghdr + (size_t)b * QHDR, gcodes + (size_t)b * QCODES);
        split_block(u + (size_t)b * QBYTES, uhdr + (size_t)b * QHDR, ucodes + (size_t)b * QCODES);
      }
    }
    for (int n = 0; n < d.H; ++n) {
      const uint8_t* s = down + ((size_t)e * d.H + n) * drow;
      uint8_t* row = dst + d.dn_off + (size_t)e * d.dn_expert_bytes + (size_t)n * d.drow_bytes;
      for (int b = 0; b < d.nbI; ++b)
        split_block(s + (size_t)b * QBYTES, row + (size_t)d.nbI * QCODES + (size_t)b * QHDR, row + (size_t)b * QCODES);
    }
  }
  return MOE_OK;
}

extern "C" int moe_unpack_layer(const moe_plan* plan, const void* src_host, uint8_t* gate, uint8_t* up,
                                uint8_t* down, float* router) {
  if (!plan || !src_host || !gate || !up || !down || !router) return MOE_ERR_INVALID_ARGUMENT;
  const Layout& d = plan->d;
  const uint8_t* src = static_cast<const uint8_t*>(src_host);
  memcpy(router, src + d.router_off, (size_t)d.E * d.H * 4);
  if (d.fmt == FMT_MXFP4) {
    unpack_mx_layer(d, src, gate, up, down);
    return MOE_OK;
  }
  const size_t grow = (size_t)d.nbH * QBYTES;
  const size_t drow = (size_t)d.nbI * QBYTES;
  for (int e = 0; e < d.E; ++e) {
    for (int r = 0; r < d.I; ++r) {
      uint8_t* g = gate + ((size_t)e * d.I + r) * grow;
      uint8_t* u = up + ((size_t)e * d.I + r) * grow;
      const uint8_t* rp = src + d.gu_off + (size_t)e * d.gu_expert_bytes + (size_t)r * d.rp_bytes;
      const uint8_t* gcodes = rp;
      const uint8_t* ucodes = rp + (size_t)d.nbH * QCODES;
      const uint8_t* ghdr = rp + (size_t)2 * d.nbH * QCODES;
      const uint8_t* uhdr = ghdr + (size_t)d.nbH * QHDR;
      for (int b = 0; b < d.nbH; ++b) {
        join_block(ghdr + (size_t)b * QHDR, gcodes + (size_t)b * QCODES, g + (size_t)b * QBYTES);
        join_block(uhdr + (size_t)b * QHDR, ucodes + (size_t)b * QCODES, u + (size_t)b * QBYTES);
      }
    }
    for (int n = 0; n < d.H; ++n) {
      uint8_t* s = down + ((size_t)e * d.H + n) * drow;
      const uint8_t* row = src + d.dn_off + (size_t)e * d.dn_expert_bytes + (size_t)n * d.drow_bytes;
      for (int b = 0; b < d.nbI; ++b)
        join_block(row + (size_t)d.nbI * QCODES + (size_t)b * QHDR, row + (size_t)b * QCODES, s + (size_t)b * QBYTES);
    }
  }
  return MOE_OK;
}

// ---------------------------------------------------------------- device calls
static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static int common_checks(const moe_plan* plan, const void* blob, int32_t layer, int32_t T, void* scratch,
                         size_t scratch_bytes, Scratch* sc) {
  if (!plan || !blob || !aligned(blob, 256)) return MOE_ERR_INVALID_ARGUMENT;
  if (layer < 0 || layer >= plan->d.L) return MOE_ERR_INVALID_ARGUMENT;
  if (T < 0 || T > plan->d.maxT) return MOE_ERR_INVALID_ARGUMENT;
  sc->init(plan->d, T);
  if (T > 0) {
    if (!scratch || !aligned(scratch, 256)) return MOE_ERR_INVALID_ARGUMENT;
    if (scratch_bytes < sc->total) return MOE_ERR_SCRATCH_TOO_SMALL;
  }
  return MOE_OK;
}

static const uint8_t* layer_ptr(const moe_plan* plan, const void* blob, int32_t layer) {
  return static_cast<const uint8_t*>(blob) + HEADER_BYTES + (size_t)layer * plan->d.layer_bytes;
}

// Path choice by the host-known token count T. The per-token GEMV streams
// every routed expert once per token; the expert-major GEMV and the MFMA
// tiles stream each routed expert once per batch, the former with the tokens
// of an expert held in registers, the latter as GEMMs on tiles of 16, 64 or
// 128 pairs, which pay off once experts carry several pairs. The switches
// are in routed pairs per expert, P/E with P = T*k. Measured per call (route
// + FFN) on the Qwen3-30B-A3B-shaped layer, T = 4..32: the per-token GEMV
// is ahead while P < E (T <= 15; MXFP4 weights: P <= E, T <= 16) and the
// tiles beyond, with the expert-major GEMV behind one of the two at every T
// (e.g. T = 8: 53.0 / 59.5 / 63.7 us, T = 16: 87.3 / 92.2 / 83.4 us; MXFP4
// T = 20: 86.5 / 114.8 / 80.9 us). Shapes without the tiles take the
// expert-major GEMV from P/E = 1/2 (its reads per batch against the
// per-token GEMV's per token), or the per-token GEMV where that does not
// apply either.
enum class Path { Gemv, ExpertGemv, Tiles };
static Path choose_path(const moe_plan* plan, int32_t T) {
  const Layout& d = plan->d;
  if (T < 2 || (d.flags & MOE_FLAG_FORCE_GEMV)) return Path::Gemv;
  if (d.flags & MOE_FLAG_FORCE_GROUPED) return Path::Tiles;       // cfg_ok: the shape has the tiles
  if (d.flags & MOE_FLAG_FORCE_EXPERT_GEMV) return Path::ExpertGemv;
  const long long P = (long long)T * d.k, E = d.E;
  if (g16_supported(d)) return (d.fmt == FMT_MXFP4 ? P <= E : P < E) ? Path::Gemv : Path::Tiles;
  if (2 * P < E || !egemv_supported(d)) return Path::Gemv;
  return Path::ExpertGemv;
}

// Work list of each batched path in scratch: one record per MFMA tile, or
// one record per routed expert.
struct WorkList {
  void* slots;
  int mt, max_slots;
};
static WorkList work_list(const Layout& d, Path p, int32_t T, uint8_t* scr, const Scratch& sc) {
  if (p == Path::Tiles) return {scr + sc.slots, g16_mt(d, T), g16_max_tiles(d, T)};
  const int P = T * d.k;
  return {scr + sc.slots, P, 1 + (P < d.E ? P : d.E)};
}

// lists_ready: the dispatch kernel already wrote the work list into scratch.
static int batched_impl(const moe_plan* plan, Path path, const uint8_t* L, const uint16_t* x, int32_t T, const float* w,
                        const int32_t* offsets, const int32_t* pairs, float* out, uint8_t* scr, const Scratch& sc,
                        hipStream_t stream, bool lists_ready = false) {
  const Layout& d = plan->d;
  const WorkList wl = work_list(d, path, T, scr, sc);
  if (!lists_ready && launch_work_list(d, offsets, T, wl.mt, wl.slots, wl.max_slots, stream) != hipSuccess)
    return MOE_ERR_HIP;
  float* ypair = reinterpret_cast<float*>(scr + sc.ypair);
  hipError_t e;
  if (path == Path::ExpertGemv)
    e = launch_egemv_ffn(d, L, x, w, pairs, wl.slots, reinterpret_cast<float*>(scr + sc.hbuf), ypair, out, T, stream);
  else
    e = launch_g16_ffn(d, L, x, w, pairs, wl.slots, reinterpret_cast<uint16_t*>(scr + sc.hbuf), ypair, out, T, stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

static int route_impl(const moe_plan* plan, const uint8_t* L, const uint16_t* x, const float* logits, int32_t T,
                      int32_t* ids, float* w, int32_t* counts, int32_t* offsets, int32_t* pairs, uint8_t* scr,
                      const Scratch& sc, hipStream_t stream) {
  const Layout& d = plan->d;
  const float* lg = logits;
  if (!lg) {
    float* tmp = reinterpret_cast<float*>(scr + sc.logits);
    if (launch_router(d, reinterpret_cast<const float*>(L + d.router_off), x, tmp, T, stream) != hipSuccess)
      return MOE_ERR_HIP;
    lg = tmp;
  }
  if (launch_topk(d, lg, ids, w, T, stream) != hipSuccess) return MOE_ERR_HIP;
  if (counts && launch_dispatch(d, ids, counts, offsets, pairs, T, stream, 1, nullptr, 0,
                                reinterpret_cast<int32_t*>(scr + sc.part)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

extern "C" int moe_route(const moe_plan* plan, const void* blob, int32_t layer, const uint16_t* x_bf16,
                         const float* logits, int32_t T, const moe_route_out* out, void* scratch,
                         size_t scratch_bytes, hipStream_t stream) {
  Scratch sc;
  int st = common_checks(plan, blob, layer, T, scratch, scratch_bytes, &sc);
  if (st) return st;
  if (!out || !out->topk_ids || !out->topk_w) return MOE_ERR_INVALID_ARGUMENT;
  const bool lists = out->counts || out->offsets || out->pairs;
  if (lists && !(out->counts && out->offsets && out->pairs)) return MOE_ERR_INVALID_ARGUMENT;
  if (!logits && (!x_bf16 || !aligned(x_bf16, 16))) return MOE_ERR_INVALID_ARGUMENT;
  if (logits && !aligned(logits, 4)) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  return route_impl(plan, layer_ptr(plan, blob, layer), x_bf16, logits, T, out->topk_ids, out->topk_w,
                    lists ? out->counts : nullptr, out->offsets, out->pairs, static_cast<uint8_t*>(scratch), sc,
                    stream);
}

extern "C" int moe_expert_ffn(const moe_plan* plan, const void* blob, int32_t layer, const uint16_t* x_bf16,
                              int32_t T, const moe_route_out* r, float* out, void* scratch, size_t scratch_bytes,
                              hipStream_t stream) {
  Scratch sc;
  int st = common_checks(plan, blob, layer, T, scratch, scratch_bytes, &sc);
  if (st) return st;
  if (!r || !r->topk_ids || !r->topk_w || !x_bf16 || !aligned(x_bf16, 16) || !out || !aligned(out, 16))
    return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  const Layout& d = plan->d;
  const uint8_t* L = layer_ptr(plan, blob, layer);
  uint8_t* scr = static_cast<uint8_t*>(scratch);
  float* h = reinterpret_cast<float*>(scr + sc.h);
  Path path = choose_path(plan, T);
  if (path != Path::Gemv && (!r->offsets || !r->pairs)) {
    // without dispatch lists only the per-token path can run, and only if
    // no batched path was forced
    if (d.flags & (MOE_FLAG_FORCE_GROUPED | MOE_FLAG_FORCE_EXPERT_GEMV)) return MOE_ERR_INVALID_ARGUMENT;
    path = Path::Gemv;
  }
  if (path != Path::Gemv)
    return batched_impl(plan, path, L, x_bf16, T, r->topk_w, r->offsets, r->pairs, out, scr, sc, stream);
  if (launch_gateup(d, L, x_bf16, r->topk_ids, nullptr, nullptr, nullptr, h, T, false, stream) != hipSuccess)
    return MOE_ERR_HIP;
  if (launch_down(d, L, r->topk_ids, r->topk_w, h, out, T, stream) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

// Router + expert FFN for one layer. With y_prev the layer input is formed
// inside the router kernel as bf16(RMSNorm(x_in + y_prev)) and stored to
// x_formed; otherwise x_in is the layer input. lists: the caller's dispatch
// lists (counts, offsets, pairs) to fill, or nullptr for scratch.
static int forward_impl(const moe_plan* plan, const void* blob, int32_t layer, const uint16_t* x_in,
                        const float* y_prev, uint16_t* x_formed, int32_t T, float* out, uint16_t* x_next,
                        int32_t* ids, float* w, uint8_t* scr, const Scratch& sc, hipStream_t stream,
                        const moe_route_out* lists = nullptr) {
  const Layout& d = plan->d;
  const uint8_t* L = layer_ptr(plan, blob, layer);
  float* lg = reinterpret_cast<float*>(scr + sc.logits);
  float* h = reinterpret_cast<float*>(scr + sc.h);
  const float* wr = reinterpret_cast<const float*>(L + d.router_off);
  const uint16_t* x = x_in;
  if (y_prev) {
    if (launch_router_norm(d, wr, x_in, y_prev, x_formed, lg, T, stream) != hipSuccess) return MOE_ERR_HIP;
    x = x_formed;
  } else if (launch_router(d, wr, x_in, lg, T, stream) != hipSuccess) {
    return MOE_ERR_HIP;
  }
  const bool fused = (T == 1);
  if (!fused && launch_topk(d, lg, ids, w, T, stream) != hipSuccess) return MOE_ERR_HIP;
  const Path path = choose_path(plan, T);
  int32_t* counts = lists ? lists->counts : reinterpret_cast<int32_t*>(scr + sc.counts);
  int32_t* offsets = lists ? lists->offsets : reinterpret_cast<int32_t*>(scr + sc.offsets);
  int32_t* pairs = lists ? lists->pairs : reinterpret_cast<int32_t*>(scr + sc.pairs);
  if (path != Path::Gemv) {
    const WorkList wl = work_list(d, path, T, scr, sc);
    if (launch_dispatch(d, ids, counts, offsets, pairs, T, stream, wl.mt, wl.slots, wl.max_slots,
                        reinterpret_cast<int32_t*>(scr + sc.part)) != hipSuccess)
      return MOE_ERR_HIP;
    const int st = batched_impl(plan, path, L, x, T, w, offsets, pairs, out, scr, sc, stream, true);
    if (st) return st;
  } else {
    if (launch_gateup(d, L, x, ids, lg, ids, w, h, T, fused, stream) != hipSuccess) return MOE_ERR_HIP;
    if (launch_down(d, L, ids, w, h, out, T, stream) != hipSuccess) return MOE_ERR_HIP;
    // the per-token path needs no dispatch lists; build them when asked for
    if (lists && launch_dispatch(d, ids, counts, offsets, pairs, T, stream, 1, nullptr, 0,
                                 reinterpret_cast<int32_t*>(scr + sc.part)) != hipSuccess)
      return MOE_ERR_HIP;
  }
  if (x_next && launch_resid_norm(d, x, out, x_next, T, stream) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

extern "C" int moe_forward(const moe_plan* plan, const void* blob, int32_t layer, const uint16_t* x_bf16, int32_t T,
                           float* out, uint16_t* x_next, const moe_route_out* route_out, void* scratch,
                           size_t scratch_bytes, hipStream_t stream) {
  Scratch sc;
  int st = common_checks(plan, blob, layer, T, scratch, scratch_bytes, &sc);
  if (st) return st;
  if (!x_bf16 || !aligned(x_bf16, 16) || !out || !aligned(out, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (x_next && !aligned(x_next, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (route_out && (!route_out->topk_ids || !route_out->topk_w)) return MOE_ERR_INVALID_ARGUMENT;
  const bool lists = route_out && (route_out->counts || route_out->offsets || route_out->pairs);
  if (lists && !(route_out->counts && route_out->offsets && route_out->pairs)) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  uint8_t* scr = static_cast<uint8_t*>(scratch);
  int32_t* ids = route_out ? route_out->topk_ids : reinterpret_cast<int32_t*>(scr + sc.ids);
  float* w = route_out ? route_out->topk_w : reinterpret_cast<float*>(scr + sc.w);
  return forward_impl(plan, blob, layer, x_bf16, nullptr, nullptr, T, out, x_next, ids, w, scr, sc, stream,
                      lists ? route_out : nullptr);
}

// ---------------------------------------------------------------- stacked decode step
extern "C" int moe_stack_step(const moe_plan* plan, const void* blob, uint16_t* xs, float* ys, int32_t* ids, float* w,
                              int32_t T, void* scratch, size_t scratch_bytes, hipStream_t stream) {
  Scratch sc;
  int st = common_checks(plan, blob, 0, T, scratch, scratch_bytes, &sc);
  if (st) return st;
  if (!xs || !ys || !aligned(xs, 16) || !aligned(ys, 16) || (!ids) != (!w)) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  const Layout& d = plan->d;
  uint8_t* scr = static_cast<uint8_t*>(scratch);
  const size_t xstride = (size_t)T * d.H, rstride = (size_t)T * d.k;
  // The epilogue of layer l (x_{l+1} = bf16(RMSNorm(x_l + y_l))) runs inside
  // layer l+1's router kernel when that kernel supports it; the last layer's
  // epilogue, which feeds the next step, runs as its own kernel.
  const bool fold = router_has_norm_prologue(d);
  for (int l = 0; l < d.L; ++l) {
    int32_t* li = ids ? ids + l * rstride : reinterpret_cast<int32_t*>(scr + sc.ids);
    float* lw = w ? w + l * rstride : reinterpret_cast<float*>(scr + sc.w);
    uint16_t* xl = xs + l * xstride;
    float* yl = ys + l * xstride;
    const bool folded_in = fold && l > 0;
    const bool last = (l == d.L - 1);
    uint16_t* x_next = (!fold || last) ? xs + ((l + 1) % d.L) * xstride : nullptr;
    st = forward_impl(plan, blob, l, folded_in ? xl - xstride : xl, folded_in ? yl - xstride : nullptr, xl, T, yl,
                      x_next, li, lw, scr, sc, stream);
    if (st) return st;
  }
  return MOE_OK;
}

struct moe_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

extern "C" int moe_graph_capture_step(const moe_plan* plan, const void* blob, uint16_t* xs, float* ys, int32_t* ids,
                                      float* w, int32_t T, void* scratch, size_t scratch_bytes, hipStream_t stream,
                                      moe_graph** out) {
  if (!out) return MOE_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (!stream) return MOE_ERR_INVALID_ARGUMENT;  // the legacy default stream cannot be captured
  Scratch sc;
  int st = common_checks(plan, blob, 0, T, scratch, scratch_bytes, &sc);
  if (st) return st;
  if (T < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal) != hipSuccess) return MOE_ERR_HIP;
  st = moe_stack_step(plan, blob, xs, ys, ids, w, T, scratch, scratch_bytes, stream);
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(stream, &g);
  if (st || e != hipSuccess || !g) {
    if (g) hipGraphDestroy(g);
    return st ? st : MOE_ERR_HIP;
  }
  hipGraphExec_t x = nullptr;
  if (hipGraphInstantiate(&x, g, nullptr, nullptr, 0) != hipSuccess) {
    hipGraphDestroy(g);
    return MOE_ERR_HIP;
  }
  moe_graph* mg = new (std::nothrow) moe_graph{g, x};
  if (!mg) {
    hipGraphExecDestroy(x);
    hipGraphDestroy(g);
    return MOE_ERR_INVALID_ARGUMENT;
  }
  *out = mg;
  return MOE_OK;
}

extern "C" int moe_graph_launch(const moe_graph* g, hipStream_t stream) {
  if (!g) return MOE_ERR_INVALID_ARGUMENT;
  return hipGraphLaunch(g->exec, stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" void moe_graph_destroy(moe_graph* g) {
  if (!g) return;
  hipGraphExecDestroy(g->exec);
  hipGraphDestroy(g->graph);
  delete g;
}

extern "C" int moe_profile_gate_up(const moe_plan* plan, const void* blob, int32_t layer, const uint16_t* x_bf16,
                                   int32_t T, void* scratch, size_t scratch_bytes, hipEvent_t start, hipEvent_t stop,
                                   hipStream_t stream) {
  Scratch sc;
  int st = common_checks(plan, blob, layer, T, scratch, scratch_bytes, &sc);
  if (st) return st;
  if (!x_bf16 || !aligned(x_bf16, 16) || !start || !stop) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  const Layout& d = plan->d;
  const uint8_t* L = layer_ptr(plan, blob, layer);
  uint8_t* scr = static_cast<uint8_t*>(scratch);
  int32_t* ids = reinterpret_cast<int32_t*>(scr + sc.ids);
  float* w = reinterpret_cast<float*>(scr + sc.w);
  float* lg = reinterpret_cast<float*>(scr + sc.logits);
  float* h = reinterpret_cast<float*>(scr + sc.h);
  // same launches as moe_forward up to and including the gate/up kernel
  if (launch_router(d, reinterpret_cast<const float*>(L + d.router_off), x_bf16, lg, T, stream) != hipSuccess)
    return MOE_ERR_HIP;
  const bool fused = (T == 1);
  if (!fused && launch_topk(d, lg, ids, w, T, stream) != hipSuccess) return MOE_ERR_HIP;
  if (launch_gateup(d, L, x_bf16, ids, lg, ids, w, h, T, fused, stream, start, stop) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

extern "C" const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_BLOB_MISMATCH: return "weight blob does not match the plan";
    case MOE_ERR_SCRATCH_TOO_SMALL: return "scratch buffer too small";
    case MOE_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

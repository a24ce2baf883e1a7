/*
 * moe.h -- C ABI of the MI355X (gfx950) quantized mixture-of-experts expert FFN.
 *
 * What it computes (sparkinfer README: opening paragraph, "deeper
 * MoE-bandwidth specialization" item and the kernel/moe rows of the layout
 * table; sparkinfer CuTe-DSL README, "moe" paragraph and "Using it"):
 * for each token x (bf16, length hidden),
 *   logits = W_r x                        (router GEMV, fp32 weights)
 *   ids    = the top_k largest logits      (descending; equal -> lower id)
 *   w_s    = softmax over the selected logits (softmax renormalised on top-k)
 *   y      = sum_s w_s * D_{ids_s} ( SiLU(G_{ids_s} x) * (U_{ids_s} x) )
 * with every expert matrix G, U [inter x hidden] and D [hidden x inter] kept
 * resident as 4-bit super-blocks (256 weights = 144 bytes: fp16 d, fp16 dmin,
 * eight 6-bit sub-block scales and mins, 4-bit codes; weight =
 * d*sc_j*q - dmin*m_j) and dequantized on read. Optionally the stacked-layer
 * epilogue x_next = bf16(RMSNorm(x + y)) (weight 1, eps from the config).
 *
 * Conventions for every entry point:
 *  - Pointers named *_host are host memory; every other buffer pointer is
 *    device memory owned by the caller. The library never allocates, frees,
 *    synchronises or reads device memory on the host; device calls only
 *    enqueue kernels on `stream` and are safe to capture into a hipGraph.
 *  - Device buffers must be 16-byte aligned; the blob 256-byte aligned.
 *  - Return value: MOE_OK (0) or a negative moe_status. Errors are detected
 *    on the host before any launch (nothing is enqueued then), except
 *    MOE_ERR_HIP, which reports a failed launch. Faults inside kernels surface
 *    at the caller's next synchronisation.
 *  - T == 0 is valid and enqueues nothing.
 *  - Inputs must be finite (not checked).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = -1,
  MOE_ERR_UNSUPPORTED = -2,
  MOE_ERR_BLOB_MISMATCH = -3,
  MOE_ERR_SCRATCH_TOO_SMALL = -4,
  MOE_ERR_HIP = -5,
};

/* Routing/FFN path choice for moe_expert_ffn and moe_forward (moe_config.flags,
 * at most one of them). T = 1 always takes the per-token GEMV. Without a flag
 * the choice goes by routed pairs per expert, P/E = T*top_k/n_experts. Shapes
 * with the MFMA tiles (grouped GEMMs on tiles of 16, 64 or 128 routed pairs of
 * one expert; hidden 512, 1024 or 2048 and inter <= 1024): the per-token GEMV
 * (each routed expert streamed once per token) below P/E = 1 (MXFP4 weights:
 * up to 1), the tiles beyond. Other shapes: the per-token GEMV below 1/2,
 * beyond it the expert-major GEMV (each routed expert streamed once, its
 * tokens held in registers; needs inter <= 2048), which the flag below also
 * selects for any shape. Every path computes with exact operands and fp32
 * accumulation (h in fp32, or as bf16 hi + lo planes on the tiles), so the
 * results agree to fp32-level rounding over the whole input range. */
#define MOE_FLAG_FORCE_GEMV 0x1u         /* per-token dequant-on-read GEMV for every T */
#define MOE_FLAG_FORCE_GROUPED 0x2u      /* MFMA tiles for every T >= 2 (tile size by P/E); shapes with the tiles only */
#define MOE_FLAG_FORCE_EXPERT_GEMV 0x4u  /* expert-major GEMV for every T >= 2; needs inter <= 2048 */

/* Gate activation h = act(g, u) of the expert FFN (at most one flag; default
 * SiLU(g) * u). The pages name SiLU, ReLU2 and SwiGLU-OAI activations for the
 * fused MoE (sparkinfer CuTe-DSL README, "moe" paragraph) without formulas;
 * the readings used: */
#define MOE_FLAG_ACT_RELU2 0x8u          /* max(g, 0)^2 * u */
#define MOE_FLAG_ACT_SWIGLU_OAI 0x10u    /* g' * sigmoid(1.702 g') * (u' + 1), g' = min(g, 7), u' = clamp(u, -7, 7) */

/* Expert weight encoding (default: 144-byte 4-bit super-blocks of 256
 * weights). MXFP4: the pages' FP4 experts with bf16 activations and inline
 * dequant (sparkinfer CuTe-DSL README, "moe" paragraph), in 17-byte blocks of
 * 32 weights: one E8M0 scale byte e (2^(e-127)), then 16 bytes of FP4 E2M1
 * codes, element 2i in the low nibble of byte 1+i. The packer accepts scale
 * codes 2..252 (2^-125 .. 2^125). The paths and force flags are those
 * above. */
#define MOE_FLAG_WEIGHTS_MXFP4 0x20u

typedef struct moe_config {
  int32_t hidden;      /* H: 256, 512, 1024, 3072 or a multiple of 2048 up to 8192 */
  int32_t n_experts;   /* E: 1..256 */
  int32_t top_k;       /* k: 1..min(E, 16) */
  int32_t inter;       /* I: expert intermediate size, multiple of 256, with top_k*inter/32 <= 512 */
  int32_t n_layers;    /* layers held in one blob, >= 1 */
  int32_t max_tokens;  /* largest T any call will pass, >= 1, with max_tokens*top_k*max(hidden, inter) < 2^31 */
  uint32_t flags;      /* MOE_FLAG_* */
  float rms_eps;       /* RMSNorm epsilon of the stacked-layer epilogue, >= 0 */
} moe_config;

typedef struct moe_plan moe_plan;

/* 1 if the configuration is supported, else 0. No side effects. (Every op
 * of the pages' kernel library exports such a query: sparkinfer (formerly
 * b12x) README, the paragraph after "Using it".) */
int moe_is_supported(const moe_config* cfg);

/* Host-only. Validates cfg and builds an immutable plan (host allocation).
 * *out is set to NULL on error (MOE_ERR_UNSUPPORTED for a configuration
 * moe_is_supported refuses). Thread-safe to use concurrently once made.
 * The plan step of the pages' plan / bind / run split: the plan is host-side
 * and may allocate, the device calls below never do (sparkinfer (formerly
 * b12x) README, "Using it" and the paragraph after it). */
int moe_plan_create(const moe_config* cfg, moe_plan** out);
void moe_plan_destroy(moe_plan* plan);

/* Pure size queries (0 on a NULL plan or T out of range). moe_scratch_bytes
 * sizes the one device workspace a call needs for T tokens, as the pages'
 * plans report their scratch (sparkinfer (formerly b12x) README, "Using it":
 * scratch_specs). */
size_t moe_blob_bytes(const moe_plan* plan);          /* header + n_layers * layer bytes */
size_t moe_header_bytes(const moe_plan* plan);        /* blob header (4096) */
size_t moe_layer_bytes(const moe_plan* plan);         /* one packed layer */
size_t moe_layer_offset(const moe_plan* plan, int32_t layer);  /* byte offset of a layer in the blob */
size_t moe_scratch_bytes(const moe_plan* plan, int32_t T);     /* device scratch for T tokens */

/* ---------------------------------------------------------------- packing
 * The weights are prepared once per model, as the pages' fused MoE prepares
 * its experts (sparkinfer (formerly b12x) README, "Using it": plan_weights /
 * prepare_weights), and stay resident in the 4-bit encoding that is
 * dequantized on read (sparkinfer README, "Deeper MoE-bandwidth
 * specialization" bullet).
 * Canonical input: for one layer, gate_host and up_host are
 * [E][inter][hidden/K] blocks, down_host is [E][hidden][inter/K] blocks
 * (K = 256 and 144-byte blocks, or with MOE_FLAG_WEIGHTS_MXFP4 K = 32 and
 * 17-byte blocks), router_host is fp32 [E][hidden]; all row-major, host
 * memory, read only. The device layout written to dst_host (moe_layer_bytes,
 * host memory owned by the caller) is private to the library; the caller
 * copies it to blob + moe_layer_offset(layer). moe_pack_layer returns
 * MOE_ERR_INVALID_ARGUMENT for an MXFP4 scale code outside 2..252.
 */
int moe_pack_header(const moe_plan* plan, void* dst_host);
int moe_pack_layer(const moe_plan* plan, const uint8_t* gate_host, const uint8_t* up_host,
                   const uint8_t* down_host, const float* router_host, void* dst_host);
/* Inverse of moe_pack_layer (host-only; used to verify the layout). */
int moe_unpack_layer(const moe_plan* plan, const void* src_host, uint8_t* gate_host, uint8_t* up_host,
                     uint8_t* down_host, float* router_host);
/* Checks a host copy of the blob header against the plan:
 * MOE_OK or MOE_ERR_BLOB_MISMATCH. */
int moe_blob_check(const moe_plan* plan, const void* header_host);

/* ---------------------------------------------------------------- device calls
 * Buffers for routing results. topk_ids int32 [T][k] and topk_w fp32 [T][k]
 * are always written. counts int32 [E], offsets int32 [E+1] and pairs int32
 * [T*k] (pair index t*k+s, ordered by expert, then token, then slot) are the
 * on-device dispatch lists; they may be NULL (all three together) when not
 * wanted.
 */
typedef struct moe_route_out {
  int32_t* topk_ids;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* pairs;
} moe_route_out;

/* Router for T tokens of layer `layer`: the pages' sync-free MoE router and
 * expert dispatch, with the expert counts computed on the device and no host
 * readback, so it can be captured in a graph (sparkinfer README, repository
 * layout table, moe/ row). If logits is NULL the logits are the router GEMV
 * of x_bf16 ([T][hidden] bf16) with the layer's fp32 router weights;
 * otherwise logits (fp32 [T][E], device) are used and x_bf16 is ignored (may
 * be NULL). out->topk_ids/topk_w receive the top_k experts (descending logit,
 * equal logits to the lower id) and their softmax restricted to the
 * selection; with the three list pointers set, also counts, offsets and
 * pairs. Errors: MOE_ERR_INVALID_ARGUMENT for a NULL or misaligned buffer,
 * a partial set of list pointers, a layer or T out of range;
 * MOE_ERR_SCRATCH_TOO_SMALL. */
int moe_route(const moe_plan* plan, const void* blob, int32_t layer, const uint16_t* x_bf16,
              const float* logits, int32_t T, const moe_route_out* out, void* scratch,
              size_t scratch_bytes, hipStream_t stream);

/* Expert FFN and weighted sum for T tokens given routing results r: the
 * pages' fused MoE consumes top-k ids and weights computed outside it
 * (sparkinfer (formerly b12x) README, "Using it": fused_moe bound with
 * topk_weights and topk_ids; the kernel table's fused quantized MoE expert
 * FFN in the sparkinfer README's layout table). x_bf16: [T][hidden] bf16;
 * r->topk_ids, r->topk_w: [T][k]; out: fp32 [T][hidden], written in full.
 * The batched paths read the dispatch lists (r->offsets, r->pairs, as
 * moe_route writes them); without them the per-token GEMV path runs, unless
 * a batched path is forced, which is then MOE_ERR_INVALID_ARGUMENT. */
int moe_expert_ffn(const moe_plan* plan, const void* blob, int32_t layer, const uint16_t* x_bf16,
                   int32_t T, const moe_route_out* r, float* out, void* scratch, size_t scratch_bytes,
                   hipStream_t stream);

/* Router + expert FFN for T tokens, the whole MoE block of one layer as the
 * pages' decode runs it (sparkinfer README, opening paragraph and layout
 * table: router, dispatch and fused quantized expert FFN): out = y (fp32
 * [T][hidden]). If x_next is
 * not NULL it also writes x_next = bf16(RMSNorm(x + y)) ([T][hidden] bf16),
 * the input of the next stacked layer; x_next may be x itself. route_out may
 * be NULL; if given, topk_ids and topk_w receive the routing, and its
 * dispatch lists (counts, offsets, pairs: all three, or none) the on-device
 * lists, whichever path runs. Routing comes from the router GEMV. */
int moe_forward(const moe_plan* plan, const void* blob, int32_t layer, const uint16_t* x_bf16,
                int32_t T, float* out, uint16_t* x_next, const moe_route_out* route_out,
                void* scratch, size_t scratch_bytes, hipStream_t stream);

/* moe_forward for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same launches and results, with the workspace taken from a device array
 * the library holds, MOE_STATIC_SCRATCH_BYTES per GPU, instead of a caller
 * buffer. It calls no allocating routine; the array's device address is
 * looked up once per GPU, on the first call with that GPU current. Returns
 * MOE_ERR_SCRATCH_TOO_SMALL when moe_scratch_bytes(plan, T) exceeds the
 * array (about 145 tokens of the Qwen3-30B-A3B-shaped layer), otherwise as
 * moe_forward. Every call on a GPU shares that GPU's array: calls that may
 * overlap on one GPU (different streams without ordering, several host
 * threads) race and must be serialised by the caller. No kernel reads the
 * workspace before writing it in the same call, so nothing is cleared. */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
int moe_forward_static_scratch(const moe_plan* plan, const void* blob, int32_t layer, const uint16_t* x_bf16,
                               int32_t T, float* out, uint16_t* x_next, const moe_route_out* route_out,
                               hipStream_t stream);

/* One decode step of the whole stack for T tokens (the greedy bs=1 decode
 * the pages time: sparkinfer README, opening paragraph): for l = 0..n_layers-1,
 * moe_forward(layer l, x = xs[l], out = ys[l], x_next = xs[(l+1) % n_layers]),
 * so the last layer's normalised output becomes the next step's layer-0
 * input. xs: bf16 [n_layers][T][hidden]; ys: fp32 [n_layers][T][hidden];
 * ids/w: int32/fp32 [n_layers][T][k] routing record, both or neither (NULL).
 * Routing of every layer comes from its router GEMV. */
int moe_stack_step(const moe_plan* plan, const void* blob, uint16_t* xs, float* ys, int32_t* ids, float* w,
                   int32_t T, void* scratch, size_t scratch_bytes, hipStream_t stream);

/* A decode step captured once as a hipGraph and replayed per token (the
 * pages' CUDA-graph decode: sparkinfer README, repository layout table,
 * runtime/ row). Capture
 * is a set-up call (like plan creation: it may allocate runtime resources)
 * and needs a non-default `stream`; it records moe_stack_step with exactly
 * these buffers, which must stay alive and in place for the graph's life.
 * moe_graph_launch enqueues one step on `stream`. */
typedef struct moe_graph moe_graph;
int moe_graph_capture_step(const moe_plan* plan, const void* blob, uint16_t* xs, float* ys, int32_t* ids,
                           float* w, int32_t T, void* scratch, size_t scratch_bytes, hipStream_t stream,
                           moe_graph** out);
int moe_graph_launch(const moe_graph* graph, hipStream_t stream);
void moe_graph_destroy(moe_graph* graph);

/* Measurement hook (for benchmarks and profilers; not graph-capturable):
 * enqueues the launches moe_forward makes for the same arguments up to and
 * including the gate/up GEMV kernel (router GEMV, routing, then
 * h = SiLU(G x) * (U x) for every routed (token, slot), into scratch), with
 * the caller's HIP events start/stop recorded around the gate/up kernel's
 * execution only (hipExtLaunchKernel). start and stop must be valid events. */
int moe_profile_gate_up(const moe_plan* plan, const void* blob, int32_t layer, const uint16_t* x_bf16,
                        int32_t T, void* scratch, size_t scratch_bytes, hipEvent_t start, hipEvent_t stop,
                        hipStream_t stream);

/* Static description of a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */

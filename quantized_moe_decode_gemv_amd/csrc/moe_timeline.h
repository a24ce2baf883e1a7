// In-kernel timeline stamps of the decode kernels, compiled only into the
// profiling build of the library (-DQMOE_TIMELINE, libqmoe_timeline.so);
// in the product build every macro here expands to nothing.
//
// Each launch of an instrumented kernel owns a slot, 4 * layer + kind (kind
// 0 router, 1 gate/up, 2 down, 3 the stand-alone residual + RMSNorm), where
// the layer is found from the kernel's weight pointer: (pointer - base) *
// (1 / layer_bytes), with base and 256 / layer_bytes passed as two extra kernel
// arguments (QMOE_TL_PARAMS / QMOE_TL_ARGS) from the values
// moe_timeline_setup stored on the host, so the instrumentation adds no
// memory round trip before a kernel's own loads. A graph keeps the values it
// was captured with: call moe_timeline_setup before capturing. Per slot and
// workgroup (the first TL_WGS workgroups, by linear index) the record holds
//   [0] s_memrealtime (100 MHz) when thread 0 starts (its first instruction),
//   [1..4] s_memrealtime when each of the four waves leaves the kernel,
//   [5], [6] two marks a kernel sets at points of its own.
// Host exports of the profiling build (extern "C", return hipError_t as int):
//   moe_timeline_setup(const void* layer0, unsigned long long layer_bytes)
//   moe_timeline_reset()                 zeroes every record
//   moe_timeline_read(unsigned long long* host)   copies TL_SLOTS*TL_WGS*8 words
// Launches whose pointer falls outside the layers, and workgroups past
// TL_WGS, record nothing.
#pragma once

#ifdef QMOE_TIMELINE
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {
constexpr int TL_LAYERS = 64, TL_SLOTS = 4 * TL_LAYERS, TL_WGS = 1024, TL_FIELDS = 8;
extern __device__ unsigned long long tl_rec[TL_SLOTS][TL_WGS][TL_FIELDS];
extern const uint8_t* tl_host_base;     // set by moe_timeline_setup
extern float tl_host_inv;               // 256 / layer_bytes

__device__ inline int tl_slot(const void* p, int kind, const uint8_t* b, float inv) {
  if (kind == 3) return 3;
  if (!b || (const uint8_t*)p < b) return -1;
  // in units of 256 bytes (inv = 256 / layer_bytes)
  const unsigned long long d = (unsigned long long)((const uint8_t*)p - b) >> 8;
  if (d >> 32) return -1;
  // a kernel's weight pointer lies less than 3/4 of a layer past its layer's
  // start; the product's error (< 64 * 2^-22, plus the truncated bytes) is
  // far below the 1/8 added
  const int layer = (int)((float)(unsigned)d * inv + 0.125f);
  return layer < TL_LAYERS ? 4 * layer + kind : -1;
}

// the workgroup's linear index (x fastest, then y, then z)
__device__ inline unsigned tl_wg() { return blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z); }

struct TLScope {
  int slot;
  unsigned wg;
  // the start is read before anything else and stored once the slot is known
  __device__ TLScope(const void* p, int kind, const uint8_t* b, float inv) {
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    slot = tl_slot(p, kind, b, inv);
    wg = tl_wg();
    if (threadIdx.x == 0 && slot >= 0 && wg < TL_WGS) tl_rec[slot][wg][0] = t0;
  }
  // wave w's exit goes to field 1 + w % 4 as a maximum, so blocks of more
  // than four waves keep their last exit (the clock only grows, so a later
  // replay's stamps also replace an earlier one's)
  __device__ ~TLScope() {
    if ((threadIdx.x & 63) == 0 && slot >= 0 && wg < TL_WGS)
      atomicMax(&tl_rec[slot][wg][1 + (threadIdx.x / 64) % 4], __builtin_amdgcn_s_memrealtime());
  }
  __device__ void mark(int field) const {
    if (threadIdx.x == 0 && slot >= 0 && wg < TL_WGS)
      tl_rec[slot][wg][field] = __builtin_amdgcn_s_memrealtime();
  }
};
}  // namespace qmoe

#define QMOE_TL_PARAMS , const uint8_t *qmoe_tl_b, float qmoe_tl_inv
#define QMOE_TL_ARGS , qmoe::tl_host_base, qmoe::tl_host_inv
#define QMOE_TL_SCOPE(ptr, kind) const qmoe::TLScope qmoe_tl_scope_((ptr), (kind), qmoe_tl_b, qmoe_tl_inv)
#define QMOE_TL_MARK(field) qmoe_tl_scope_.mark(field)
#else
#define QMOE_TL_PARAMS
#define QMOE_TL_ARGS
#define QMOE_TL_SCOPE(ptr, kind)
#define QMOE_TL_MARK(field) \
  do {                     \
  } while (0)
#endif

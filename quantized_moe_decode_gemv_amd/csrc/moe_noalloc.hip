// Allocation-free variant of moe_forward: the same launches on a device
// workspace the library holds itself, a file-scope device array of
// MOE_STATIC_SCRATCH_BYTES per GPU, so that callers that cannot allocate
// (code under graph capture, tight serving loops) need no scratch buffer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

namespace {

// The workspace. In host code this name stands for the device symbol, not a
// device address: host code uses only the address hipGetSymbolAddress
// returns for the current device (each GPU holds its own copy).
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
void* g_ptr[MAX_DEVICES];
hipError_t g_err[MAX_DEVICES];
std::once_flag g_once[MAX_DEVICES];

// The current device's address of the workspace, looked up once per device
// (with that device current) on its first call.
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return MOE_ERR_HIP;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = p;
  });
  if (g_err[dev] != hipSuccess || !g_ptr[dev]) return MOE_ERR_HIP;
  *out = g_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_static_scratch(const moe_plan* plan, const void* blob, int32_t layer,
                                          const uint16_t* x_bf16, int32_t T, float* out, uint16_t* x_next,
                                          const moe_route_out* route_out, hipStream_t stream) {
  if (!plan) return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = moe_scratch_bytes(plan, T);
  if (T < 0 || (T > 0 && need == 0)) return MOE_ERR_INVALID_ARGUMENT;   // T beyond the plan's max_tokens
  if (need > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_SCRATCH_TOO_SMALL;
  void* p = nullptr;
  const int st = device_scratch(&p);
  if (st) return st;
  return moe_forward(plan, blob, layer, x_bf16, T, out, x_next, route_out, p, MOE_STATIC_SCRATCH_BYTES, stream);
}

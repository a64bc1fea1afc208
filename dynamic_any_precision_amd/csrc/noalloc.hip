// The whole layer for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// moe_layer on a workspace that is a static device array of this library
// instead of a caller-provided buffer.
//
// The array lives in the library's code object; each GPU the library runs on
// holds its own copy until the process ends.  Its device address is looked
// up once per device (hipGetSymbolAddress, with that device current, on the
// first call made on it) and cached; host code passes that address, never the
// array's name, to the kernels.  Nothing here allocates.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_anyprec.h"
#include "kernels.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB: decode batches up to 256 tokens (Qwen3-30B-A3B shape)
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's scratch array (looked up once per device).
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t moe_layer_static_scratch_bytes(void) { return kScratchBytes; }

moe_status moe_layer_static(const moe_expert_bank* routed, const moe_expert_bank* shared, const uint16_t* x,
                            int32_t T, int32_t top_k, const float* w_router, const float* logit_bias,
                            int32_t renorm_topk, int32_t b_lo, float target_avg_bits, int32_t* topk_idx,
                            float* topk_gate, uint8_t* bits, float* y, int32_t accumulate, void* stream) {
  const size_t need = moe_layer_workspace_bytes(routed, shared, T, top_k);
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (T > 0 && need > 0) {
    const hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) return static_cast<moe_status>(moe::record_hip_error(e));
  }
  // need == 0 means invalid arguments: moe_layer reports which
  return moe_layer(routed, shared, x, T, top_k, w_router, logit_bias, renorm_topk, b_lo, target_avg_bits, topk_idx,
                   topk_gate, bits, y, accumulate, ws, ws ? kScratchBytes : 0, stream);
}

}  // extern "C"

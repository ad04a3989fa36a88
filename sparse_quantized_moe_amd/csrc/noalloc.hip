// moesq_moe_ffn_noalloc: the MoE FFN of moesq_moe_ffn with its workspace in a library-owned device
// array instead of a caller buffer, for callers that cannot allocate device memory (code under graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable: every GPU the library runs on holds its own copy
// (kNoAllocScratchBytes, until the process ends), at its own address. In host code the variable's
// name is only a stand-in, so the device address is looked up once per device, with that device
// current (hipGetSymbolAddress), and that address is what the launches receive. Every call on one
// GPU shares that GPU's array and finds the previous call's contents there; no kernel of the FFN
// needs the workspace cleared (each region is written before it is read), and calls that overlap in
// time on one GPU race on the array.
#include <cstdio>
#include <mutex>

#include "moesq.h"
#include "moesq_internal.h"

namespace {

constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch` (looked up on first use), or an error.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t moesq_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

moesq_status moesq_moe_ffn_noalloc(const void* x, int64_t T, int32_t H, const int32_t* topk_ids,
                                   const float* topk_weights, int32_t k, const moesq_weights* w13,
                                   const moesq_weights* w2, const float* a13_global, const float* a2_global,
                                   float* out, uint32_t flags, hipStream_t stream) {
  const moesq_status s =
      moesq::validate_ffn_args(x, T, H, topk_ids, topk_weights, k, w13, w2, a13_global, a2_global, out);
  if (s != MOESQ_OK || T == 0) return s;
  const uint32_t f = (flags & ~MOESQ_FLAG_FUSED) | MOESQ_FLAG_UNFUSED;
  moesq_ffn_layout L;
  moesq_moe_ffn_layout(T, H, w2->K, k, w13->E, f, &L);
  if (L.total > kNoAllocScratchBytes) {
    char msg[160];
    std::snprintf(msg, sizeof msg, "moe_ffn_noalloc: the call needs %zu bytes of workspace, the static scratch holds %zu",
                  L.total, kNoAllocScratchBytes);
    return moesq::report(MOESQ_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) {
    char msg[160];
    std::snprintf(msg, sizeof msg, "moe_ffn_noalloc: scratch address: %s", hipGetErrorString(e));
    return moesq::report(MOESQ_ERR_HIP, msg);
  }
  return moesq_moe_ffn(x, T, H, topk_ids, topk_weights, k, w13, w2, a13_global, a2_global, out, ws,
                       kNoAllocScratchBytes, f, stream);
}

}  // extern "C"

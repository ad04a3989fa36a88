// MoE router on the GPU: per token, softmax over the E expert logits, the k most probable experts
// (equal probability: the lower expert id first, listed by decreasing probability) and their
// weights, renormalized over the k picks or not. The model cards keep this router (`mlp.gate`) in
// BF16 ahead of the compressed routed experts (model card "Qwen3.5-397B-A17B-P48NVFP4-MoESQ",
// "Compression details": what is left in BF16); the selection rule is the usual softmax top-k.
//
// Softmax is strictly increasing, so the k most probable experts are the k largest logits: the
// selection compares the logits themselves (exact, in fp32; bf16 inputs convert exactly), and only
// the weights are computed, in fp32.
#include "moesq_device.h"
#include "moesq_internal.h"

namespace moesq {

// Selection keys: a logit's bits mapped to an unsigned integer of the same order (-0 folded into +0,
// so equal values tie), above the expert id inverted, so the largest key is the largest logit and,
// among equal logits, the lowest id. bf16 logits need 16 bits of value and E <= 1024 needs 10 of id,
// so their key is 32 bits; fp32 logits take a 64-bit key.
__device__ __forceinline__ uint32_t order_bits32(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_order_bits32(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <bool F32>
struct RouterKey;
template <>
struct RouterKey<false> {
  using T = uint32_t;
  static __device__ T make(float v, int e) { return (order_bits32(v) & 0xFFFF0000u) | (0xFFFFu - (uint32_t)e); }
  static __device__ int id(T k) { return (int)(0xFFFFu - (k & 0xFFFFu)); }
  static __device__ float value(T k) { return from_order_bits32(k & 0xFFFF0000u); }
  static __device__ T shfl_xor(T k, int off) { return (T)__shfl_xor((int)k, off); }
};
template <>
struct RouterKey<true> {
  using T = unsigned long long;
  static __device__ T make(float v, int e) { return ((T)order_bits32(v) << 32) | (0xFFFFFFFFull - (T)e); }
  static __device__ int id(T k) { return (int)(0xFFFFFFFFull - (k & 0xFFFFFFFFull)); }
  static __device__ float value(T k) { return from_order_bits32((uint32_t)(k >> 32)); }
  static __device__ T shfl_xor(T k, int off) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)k, off), hi = (uint32_t)__shfl_xor((int)(uint32_t)(k >> 32), off);
    return ((T)hi << 32) | lo;
  }
};

// One wave per token; lane l holds the keys of experts l, l + 64, ... (EPL of them). Each of the k
// rounds takes the wave's largest key; the lane that holds it clears it (0 is below every key).
template <bool F32, int EPL>
__global__ __launch_bounds__(256) void k_route_topk(const void* __restrict__ logits, int64_t T, int E, int k,
                                                    int renormalize, int* __restrict__ ids, float* __restrict__ wts) {
  using Key = RouterKey<F32>;
  using KT = typename Key::T;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[EPL];
  KT key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      const int64_t i = t * E + e;
      v[j] = F32 ? static_cast<const float*>(logits)[i]
                 : __uint_as_float((uint32_t) static_cast<const uint16_t*>(logits)[i] << 16);
      key[j] = Key::make(v[j], e);
    } else {
      v[j] = -__builtin_inff();
      key[j] = 0;
    }
  }
  float m = v[0];
#pragma unroll
  for (int j = 1; j < EPL; ++j) m = __builtin_fmaxf(m, v[j]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  int my_id = 0;
  float my_v = 0.0f;
  for (int r = 0; r < k; ++r) {
    KT b = key[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) b = key[j] > b ? key[j] : b;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const KT o = Key::shfl_xor(b, off);
      b = o > b ? o : b;
    }
    const int bi = Key::id(b);
    if (lane == (bi & 63)) {
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (j == (bi >> 6)) key[j] = 0;
    }
    if (lane == r) {
      my_id = bi;
      my_v = Key::value(b);
    }
  }
  // weights: exp(l - max) over the picks (renormalized) or over all experts (softmax)
  const float ex = lane < k ? expf(my_v - m) : 0.0f;
  float s = 0.0f;
  if (renormalize) {
    s = ex;
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + 64 * j < E) s += expf(v[j] - m);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane < k) {
    ids[t * k + lane] = my_id;
    wts[t * k + lane] = ex / s;
  }
}

template <bool F32>
static void launch_route_topk_t(const void* logits, int64_t T, int E, int k, int renorm, int* ids, float* wts,
                                hipStream_t stream) {
  const unsigned grid = (unsigned)((T + 3) / 4);
  if (E <= 64) k_route_topk<F32, 1><<<grid, 256, 0, stream>>>(logits, T, E, k, renorm, ids, wts);
  else if (E <= 128) k_route_topk<F32, 2><<<grid, 256, 0, stream>>>(logits, T, E, k, renorm, ids, wts);
  else if (E <= 256) k_route_topk<F32, 4><<<grid, 256, 0, stream>>>(logits, T, E, k, renorm, ids, wts);
  else if (E <= 512) k_route_topk<F32, 8><<<grid, 256, 0, stream>>>(logits, T, E, k, renorm, ids, wts);
  else k_route_topk<F32, 16><<<grid, 256, 0, stream>>>(logits, T, E, k, renorm, ids, wts);
}

void launch_route_topk(const void* logits, bool f32, int64_t T, int E, int k, bool renormalize, int* ids,
                       float* wts, hipStream_t stream) {
  if (T <= 0) return;
  if (f32) launch_route_topk_t<true>(logits, T, E, k, renormalize ? 1 : 0, ids, wts, stream);
  else launch_route_topk_t<false>(logits, T, E, k, renormalize ? 1 : 0, ids, wts, stream);
}

}  // namespace moesq

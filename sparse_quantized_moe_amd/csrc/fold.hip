// Load-time fold of the gate/up global ratio into the up projection's block scales.
//
// The model cards ("Qwen3.8-Flash-Next-P48NVFP4-MoESQ", the note under "Compression details";
// "Qwen3-30B-A3B-P48NVFP4-MoESQ", the note after the evaluation table) store separate fp32 globals for
// the gate and up halves of an expert and fold their ratio into the block scales when the layer is
// loaded, so that one global serves both halves. Here the gate's global is kept for both, and each up
// scale byte s becomes the E4M3 byte nearest to e4m3(s) * r (ties to even, saturating at 448), with
// r = g_up / g_gate rounded to fp32; a zero scale stays zero.
//
// For one expert the new byte depends on the old byte only, so a workgroup first fills a 128-entry
// table in LDS (one exact fp64 rounding per entry: e4m3(s) has 4 significant bits and r 24, so the
// product is exact in fp64), then streams its slab of up scales through the table with 16-byte loads
// and stores. The table is 32 dwords, one per LDS bank, so lookups never conflict. A second launch
// sets g_up = g_gate once every workgroup has read the old value.
#include "moesq_device.h"
#include "moesq_internal.h"

namespace moesq {

namespace {

constexpr int kFoldThreads = 256;
constexpr int kFoldVecsPerThread = 4;   // 16-byte vectors per thread: 16 KB of scales per workgroup

// E4M3FN byte of the non-negative double v: nearest, ties to even, saturating at 448. v is split
// into its binade [2^e, 2^(e+1)) (e >= -6; below 2^-6 the subnormal step 2^-9 applies) and rounded
// to 3 fraction bits with rint (ties to even, and an even rounded mantissa is an even byte, since the
// exponent field sits above bit 2); a mantissa that rounds up to 2 carries into the next binade.
__device__ __forceinline__ uint32_t e4m3_nearest_f64(double v) {
  if (!(v < 448.0)) return 0x7Eu;                                        // also +inf and NaN
  if (v < 0x1p-6) return (uint32_t)__builtin_rint(v * 512.0);           // 0..8 (8 = 2^-6, byte 0x08)
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const int e = (int)((u >> 52) & 0x7FFu) - 1023;                       // -6..8
  const double mant = __longlong_as_double((long long)((u & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull));
  const uint32_t m = (uint32_t)__builtin_rint((mant - 1.0) * 8.0);      // 0..8, exact scaling
  const uint32_t c = ((uint32_t)(e + 7) << 3) + m;
  return c < 0x7Eu ? c : 0x7Eu;
}

// Fold table of one expert: byte b (0..127) -> its folded byte; 0 stays 0 and 0x7F (NaN, not a
// scale) is left as it is. r = fp32(g_up / g_gate): the fp64 quotient of two fp32 values rounded to
// fp32 is the correctly rounded fp32 quotient (53 >= 2 * 24 + 2 bits).
__device__ __forceinline__ uint32_t fold_entry(uint32_t b, float g_gate, float g_up) {
  if (b == 0u || b == 0x7Fu) return b;
  const double r = (double)(float)((double)g_up / (double)g_gate);
  return e4m3_nearest_f64((double)e4m3_value(b) * r);
}

// grid (slabs per expert, E). Each workgroup rewrites slab blockIdx.x of expert blockIdx.y's up
// scales, a contiguous region of `region` bytes starting at scale + (2e + 1) * region. VEC16: region
// is a multiple of 16 bytes and the tensor 16-byte aligned; otherwise one byte per thread and step.
template <bool VEC16>
__global__ __launch_bounds__(kFoldThreads) void k_fold_scales(uint8_t* __restrict__ scale, const float* __restrict__ global,
                                                             int64_t region) {
  __shared__ uint32_t s_lut[32];
  const int e = blockIdx.y;
  if (threadIdx.x < 32) {
    const float gg = global[2 * e], gu = global[2 * e + 1];
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= fold_entry(4 * threadIdx.x + i, gg, gu) << (8 * i);
    s_lut[threadIdx.x] = w;
  }
  __syncthreads();
  const uint8_t* lut = reinterpret_cast<const uint8_t*>(s_lut);
  uint8_t* up = scale + (2 * (int64_t)e + 1) * region;
  auto map = [&](uint32_t b) -> uint32_t { return b < 0x80u ? (uint32_t)lut[b] : b; };
  if constexpr (VEC16) {
    const int64_t nvec = region >> 4;
    int64_t v = ((int64_t)blockIdx.x * kFoldVecsPerThread) * kFoldThreads + threadIdx.x;
    u32x4 in[kFoldVecsPerThread];
#pragma unroll
    for (int i = 0; i < kFoldVecsPerThread; ++i)
      if (v + i * kFoldThreads < nvec) in[i] = reinterpret_cast<const u32x4*>(up)[v + i * kFoldThreads];
#pragma unroll
    for (int i = 0; i < kFoldVecsPerThread; ++i) {
      if (v + i * kFoldThreads >= nvec) break;
      uint32_t w[4] = {in[i].x, in[i].y, in[i].z, in[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = map(w[j] & 255u) | map((w[j] >> 8) & 255u) << 8 | map((w[j] >> 16) & 255u) << 16 |
               map(w[j] >> 24) << 24;
      reinterpret_cast<u32x4*>(up)[v + i * kFoldThreads] = u32x4{w[0], w[1], w[2], w[3]};
    }
  } else {
    const int64_t base = (int64_t)blockIdx.x * kFoldVecsPerThread * 16 * kFoldThreads;
    for (int i = threadIdx.x; i < kFoldVecsPerThread * 16 * kFoldThreads; i += kFoldThreads) {
      const int64_t o = base + i;
      if (o < region) up[o] = (uint8_t)map(up[o]);
    }
  }
}

__global__ void k_fold_globals(float* __restrict__ global, int E) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) global[2 * e + 1] = global[2 * e];
}

}  // namespace

void launch_fold_gate_up(uint8_t* scale, float* global, int E, int N, int K, hipStream_t stream) {
  const int64_t region = (int64_t)(N / 2) * (K / 32);
  const int64_t slab = (int64_t)kFoldVecsPerThread * 16 * kFoldThreads;
  const dim3 grid((unsigned)((region + slab - 1) / slab), (unsigned)E);
  if (region % 16 == 0 && (reinterpret_cast<uintptr_t>(scale) & 15u) == 0)
    k_fold_scales<true><<<grid, kFoldThreads, 0, stream>>>(scale, global, region);
  else
    k_fold_scales<false><<<grid, kFoldThreads, 0, stream>>>(scale, global, region);
  k_fold_globals<<<(E + 255) / 256, 256, 0, stream>>>(global, E);
}

}  // namespace moesq

// Throughput probes, so a roofline can be quoted against the rate this GPU sustains as well as against
// the published peak: the instruction the grouped GEMMs are built on, v_smfmac_f32_16x16x64_f16, and a
// plain read stream from HBM (the decode GEMMs read their weights and write little).
//
// smfmac probe:
// Each wave runs the GEMMs' own issue pattern: 4 sparse operands x 8 dense operands, 32 independent
// accumulators (the most a wave of the prefill GEMM keeps), and stores its accumulators at the end, so
// nothing is folded away. Two workgroups per CU give every SIMD two waves, as in the GEMMs.
#include "moesq_device.h"
#include "moesq_internal.h"

namespace moesq {

constexpr int kProbeA = 4, kProbeB = 8;

__global__ __launch_bounds__(256) void k_probe_smfmac(float* __restrict__ sink, int iters) {
  f16x8 a[kProbeA];
  f16x16 b[kProbeB];
  int idx[kProbeA];
#pragma unroll
  for (int r = 0; r < kProbeA; ++r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[r][i] = (f16)(0.001f * (float)(threadIdx.x + i + r));
    idx[r] = 0x4E4E4E4E ^ r;
  }
#pragma unroll
  for (int t = 0; t < kProbeB; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) b[t][i] = (f16)(0.002f * (float)((int)threadIdx.x - i - t));
  f32x4 acc[kProbeA][kProbeB];
#pragma unroll
  for (int r = 0; r < kProbeA; ++r)
#pragma unroll
    for (int t = 0; t < kProbeB; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < kProbeB; ++t)
#pragma unroll
      for (int r = 0; r < kProbeA; ++r)
        acc[r][t] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(a[r], b[t], acc[r][t], idx[r], 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < kProbeA; ++r)
#pragma unroll
    for (int t = 0; t < kProbeB; ++t) s += acc[r][t][0] + acc[r][t][1] + acc[r][t][2] + acc[r][t][3];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

int64_t launch_probe_smfmac(int blocks, int iters, float* sink, hipStream_t stream) {
  k_probe_smfmac<<<blocks, 256, 0, stream>>>(sink, iters);
  return (int64_t)blocks * 4 * iters * kProbeA * kProbeB;
}

// Read probe: 16-byte loads in a grid-stride loop (2048 workgroups of 512 threads, the fastest
// configuration of a sweep on MI355X), folded into one word per thread that is stored only if it
// equals a constant, so no load can be removed and almost nothing is written.
constexpr int kReadBlocks = 2048, kReadThreads = 512;

__global__ __launch_bounds__(kReadThreads) void k_probe_read(const u32x4* __restrict__ src, int64_t nvec,
                                                             uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    const u32x4 w = src[v];
    acc ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

void launch_probe_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  k_probe_read<<<kReadBlocks, kReadThreads, 0, stream>>>(static_cast<const u32x4*>(src), bytes >> 4, sink);
}

}  // namespace moesq

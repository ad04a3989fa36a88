// Throughput probe of the instruction the grouped GEMMs are built on, v_smfmac_f32_16x16x64_f16, so a
// roofline can be quoted against the rate this GPU sustains as well as against the published peak.
// Each wave keeps 8 independent accumulator chains (enough to cover the instruction's latency) and
// stores its accumulators at the end, so nothing is folded away.
#include "moesq_device.h"
#include "moesq_internal.h"

namespace moesq {

constexpr int kProbeChains = 8;

__global__ __launch_bounds__(256) void k_probe_smfmac(float* __restrict__ sink, int iters) {
  f16x8 a;
  f16x16 b;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (f16)(0.001f * (float)(threadIdx.x + i));
#pragma unroll
  for (int i = 0; i < 16; ++i) b[i] = (f16)(0.002f * (float)((int)threadIdx.x - i));
  f32x4 acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j)
      acc[j] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, b, acc[j], 0x4444, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

int64_t launch_probe_smfmac(int blocks, int iters, float* sink, hipStream_t stream) {
  k_probe_smfmac<<<blocks, 256, 0, stream>>>(sink, iters);
  return (int64_t)blocks * 4 * iters * kProbeChains;
}

}  // namespace moesq

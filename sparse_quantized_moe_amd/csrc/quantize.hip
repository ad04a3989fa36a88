// NVFP4 activation quantizer, weight compression (paired-4:8 prune + NVFP4 + pair-bitmask pack) and
// the storage codec kernels, for gfx950.
//
// Activation quantization (model cards, "Compression details": NVFP4 activations with dynamic
// per-32 group scales and an FP32 global stored per expert linear): for each 32-group of a row,
// amax -> E4M3 scale = RNE(amax / (6 g)) -> E2M1 codes = RNE(x / (s g)), exact decisions
// (moesq_device.h). One thread owns one 32-group: it reads 64 B (bf16) or 128 B (fp32), writes 16 B
// of codes and 1 scale byte; the pass is HBM-bound.
#include "moesq_device.h"
#include "moesq_internal.h"

namespace moesq {

// ---------------------------------------------------------------------------------------------
// Activation quantizer
// ---------------------------------------------------------------------------------------------
struct QuantArgs {
  const void* x;
  int64_t rows;
  int K;
  int64_t stride;          // elements between rows of x
  const int* src_row;      // source row of x per row (NULL = identity)
  const int* offsets;      // [E+1]: rows offsets[e] .. offsets[e+1]-1 use global[e] (binary search)
  int E;
  const float* global;
  uint8_t* codes;
  uint8_t* scales;
};

template <bool F32>
__device__ __forceinline__ void load_group(const void* x, int64_t off, float v[32]) {
  if (F32) {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(x) + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 w = p[i];
      v[4 * i + 0] = __uint_as_float(w.x); v[4 * i + 1] = __uint_as_float(w.y);
      v[4 * i + 2] = __uint_as_float(w.z); v[4 * i + 3] = __uint_as_float(w.w);
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 w = p[i];
      uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(a[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(a[j] & 0xFFFF0000u);
      }
    }
  }
}

// Quantize 32 values with global g: writes 16 code bytes and returns the scale byte. fp32 inputs take
// the hardware conversion with its exact fallback; bf16 inputs (few significant bits, so quotients
// often sit right on a boundary) take the one-test snap encoding.
template <bool F32>
__device__ __forceinline__ uint32_t quantize_group(const float v[32], float g, u32x4& out) {
  float amax = 0.0f;
  uint32_t mb = 0;   // largest magnitude bit pattern: >= 0x7F800000 iff some value is not finite
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    if (!F32) mb = __builtin_elementwise_max(mb, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  }
  const int sc = scale_code(amax, g);
  const float s = e4m3_value(sc);
  if (F32) {
    const Nvfp4Recip rc = nvfp4_recip(s, g);
    out.x = nvfp4_codes<8>(v, s, g, rc);
    out.y = nvfp4_codes<8>(v + 8, s, g, rc);
    out.z = nvfp4_codes<8>(v + 16, s, g, rc);
    out.w = nvfp4_codes<8>(v + 24, s, g, rc);
  } else {
    const Nvfp4Snap sn = nvfp4_snap(s, g, mb < 0x7F800000u);
    out.x = nvfp4_codes_snap<8>(v, s, g, sn);
    out.y = nvfp4_codes_snap<8>(v + 8, s, g, sn);
    out.z = nvfp4_codes_snap<8>(v + 16, s, g, sn);
    out.w = nvfp4_codes_snap<8>(v + 24, s, g, sn);
  }
  return (uint32_t)sc;
}

template <bool F32, bool OFFSETS>
__global__ __launch_bounds__(256) void k_quantize(QuantArgs a) {
  const int G = a.K >> 5;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = gid / G;
  const int grp = (int)(gid - r * G);
  if (r >= a.rows) return;
  const int64_t src = a.src_row ? a.src_row[r] : r;
  float g;
  if (OFFSETS) {
    int lo = 0, hi = a.E;                         // largest e with offsets[e] <= r
    if (r >= a.offsets[a.E] || r < a.offsets[0]) return;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.offsets[mid] <= r) lo = mid; else hi = mid;
    }
    g = a.global[lo];
  } else {
    g = a.global[0];
  }
  float v[32];
  load_group<F32>(a.x, src * a.stride + (int64_t)grp * 32, v);
  u32x4 out;
  const uint32_t sc = quantize_group<F32>(v, g, out);
  *reinterpret_cast<u32x4*>(a.codes + r * (a.K >> 1) + grp * 16) = out;
  a.scales[r * G + grp] = (uint8_t)sc;
}

void launch_quantize(const void* x, bool f32, int64_t rows, int K, int64_t stride, const int* src_row,
                     const int* offsets, int E, const float* global, uint8_t* codes, uint8_t* scales,
                     hipStream_t stream) {
  QuantArgs a{x, rows, K, stride, src_row, offsets, E, global, codes, scales};
  const int64_t n = rows * (K >> 5);
  if (n == 0) return;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (f32) {
    if (offsets) k_quantize<true, true><<<grid, 256, 0, stream>>>(a);
    else k_quantize<true, false><<<grid, 256, 0, stream>>>(a);
  } else {
    if (offsets) k_quantize<false, true><<<grid, 256, 0, stream>>>(a);
    else k_quantize<false, false><<<grid, 256, 0, stream>>>(a);
  }
}

// ---------------------------------------------------------------------------------------------
// Weight compression: dense fp32 [N, K] -> pair-bitmask NVFP4 (synthetic-layer recipe).
// Prune: in each 8-K chunk keep the two pairs with the largest a*a + b*b (float64, no fused
// multiply-add), ties to the lower pair index. Global: fp32(amax of the kept values) / 2688.
// Then the NVFP4 rule above with that global; pruned pairs are byte 0x00; the mask names the kept
// pairs (model card "Sparse storage layout": 2 kept bytes of every 4 in K order, one nibble per
// 4-byte chunk, bit i = byte i kept, the lower-K chunk in the low nibble).
// ---------------------------------------------------------------------------------------------

// Kept-pair nibble of one 8-K chunk.
__device__ __forceinline__ uint32_t prune_chunk(const float w[8]) {
  double sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double a = (double)w[2 * i], b = (double)w[2 * i + 1];
    sc[i] = __dadd_rn(__dmul_rn(a, a), __dmul_rn(b, b));
  }
  // first: largest score, lowest index on ties; second: largest among the rest
  int i0 = 0;
#pragma unroll
  for (int i = 1; i < 4; ++i) if (sc[i] > sc[i0]) i0 = i;
  int i1 = i0 == 0 ? 1 : 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) if (i != i0 && sc[i] > sc[i1]) i1 = i;
  return (1u << i0) | (1u << i1);
}

__device__ __forceinline__ void load8(const float* p, float w[8]) {
  const u32x4 a = reinterpret_cast<const u32x4*>(p)[0];
  const u32x4 b = reinterpret_cast<const u32x4*>(p)[1];
  w[0] = __uint_as_float(a.x); w[1] = __uint_as_float(a.y); w[2] = __uint_as_float(a.z); w[3] = __uint_as_float(a.w);
  w[4] = __uint_as_float(b.x); w[5] = __uint_as_float(b.y); w[6] = __uint_as_float(b.z); w[7] = __uint_as_float(b.w);
}

__global__ void k_fill_u32(uint32_t* p, uint32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// amax of the kept values; one thread per 8-K chunk, block max, one atomicMax per block on the
// fp32 bits (non-negative floats order like their bit patterns).
__global__ __launch_bounds__(256) void k_compress_amax(const float* w, int64_t N, int K, uint32_t* amax_bits) {
  __shared__ float red[256];
  const int64_t chunks = N * (K >> 3);
  float m = 0.0f;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * blockDim.x) {
    float v[8];
    load8(w + c * 8, v);
    const uint32_t keep = prune_chunk(v);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (keep & (1u << i)) m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(v[2 * i]), __builtin_fabsf(v[2 * i + 1])));
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = __builtin_fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(amax_bits, __float_as_uint(red[0]));
}

// global = fp32(amax) / 2688 (IEEE division), in place over the amax bits.
__global__ void k_compress_global(uint32_t* slot) {
  const float amax = __uint_as_float(*slot);
  *reinterpret_cast<float*>(slot) = amax / 2688.0f;
}

// One thread per 32-K group (4 chunks): prune, scale, codes, pack.
__global__ __launch_bounds__(256) void k_compress_quant(const float* w, int64_t N, int K, const float* global,
                                                        uint8_t* packed, uint8_t* mask, uint8_t* scale) {
  const int G = K >> 5;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= N * G) return;
  const int64_t n = gid / G;
  const int grp = (int)(gid - n * G);
  const float g = *global;
  float v[32];
  uint32_t keep[4];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    load8(w + n * K + (int64_t)grp * 32 + c * 8, v + 8 * c);
    keep[c] = prune_chunk(v + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (keep[c] & (1u << i))
        amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(v[8 * c + 2 * i]), __builtin_fabsf(v[8 * c + 2 * i + 1])));
  }
  const int sc = g > 0.0f ? scale_code(amax, g) : 0;
  const float s = e4m3_value(sc);
  uint32_t kept_bytes[2] = {0, 0};
  uint32_t nib = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int slot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (keep[c] & (1u << i)) {
        const uint32_t byte = nvfp4_code(v[8 * c + 2 * i], s, g) | (nvfp4_code(v[8 * c + 2 * i + 1], s, g) << 4);
        const int pos = 2 * c + slot;                 // kept byte index within the group (0..7)
        kept_bytes[pos >> 2] |= byte << (8 * (pos & 3));
        ++slot;
      }
    }
    nib |= keep[c] << (4 * c);
  }
  uint8_t* pk = packed + n * (K >> 2) + (int64_t)grp * 8;
  reinterpret_cast<uint32_t*>(pk)[0] = kept_bytes[0];
  reinterpret_cast<uint32_t*>(pk)[1] = kept_bytes[1];
  *reinterpret_cast<uint16_t*>(mask + n * (K >> 4) + (int64_t)grp * 2) = (uint16_t)nib;
  scale[n * G + grp] = (uint8_t)sc;
}

void launch_compress(const float* w, int64_t N, int K, uint8_t* packed, uint8_t* mask, uint8_t* scale,
                     float* global, hipStream_t stream) {
  uint32_t* slot = reinterpret_cast<uint32_t*>(global);
  k_fill_u32<<<1, 64, 0, stream>>>(slot, 0u, 1);
  const int64_t chunks = N * (K >> 3);
  int blocks = (int)((chunks + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  k_compress_amax<<<blocks, 256, 0, stream>>>(w, N, K, slot);
  k_compress_global<<<1, 1, 0, stream>>>(slot);
  const int64_t groups = N * (K >> 5);
  if (groups) k_compress_quant<<<(unsigned)((groups + 255) / 256), 256, 0, stream>>>(w, N, K, global, packed, mask, scale);
}

// ---------------------------------------------------------------------------------------------
// Storage codec: validate, unpack (sparse -> dense packed NVFP4) and pack (dense -> sparse).
// One thread per 4-byte chunk pair (one mask byte).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t popc4(uint32_t q) { return __builtin_popcount(q & 15u); }

__global__ void k_validate(const uint8_t* mask, int64_t nbytes, int* bad) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int b = 0;
  if (i < nbytes) {
    const uint32_t m = mask[i];
    b = (popc4(m) != 2) + (popc4(m >> 4) != 2);
  }
  // wave reduction then one atomic per wave
  for (int off = 32; off > 0; off >>= 1) b += __shfl_xor(b, off);
  if ((threadIdx.x & 63) == 0 && b) atomicAdd(bad, b);
}

// Unpack: mask byte j covers chunks 2j, 2j+1 = packed bytes 4j..4j+3 -> dense bytes 8j..8j+7.
__global__ void k_unpack(const uint8_t* packed, const uint8_t* mask, int64_t nbytes, uint8_t* dense, int* bad) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= nbytes) return;
  const uint32_t m = mask[j];
  const uint32_t kept = *reinterpret_cast<const uint32_t*>(packed + 4 * j);
  uint32_t out[2] = {0, 0};
  int b = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t q = (m >> (4 * h)) & 15u;
    if (popc4(q) != 2) { ++b; continue; }
    const uint32_t kb = kept >> (16 * h);
    int slot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (q & (1u << i)) { out[h] |= ((kb >> (8 * slot)) & 255u) << (8 * i); ++slot; }
  }
  reinterpret_cast<uint32_t*>(dense + 8 * j)[0] = out[0];
  reinterpret_cast<uint32_t*>(dense + 8 * j)[1] = out[1];
  if (b) atomicAdd(bad, b);
}

// Pack with the canonical rule: kept = nonzero bytes; a chunk with fewer than two is completed with
// its lowest-index zero bytes; a chunk with more than two is counted in *bad (and packs its first two).
__global__ void k_pack(const uint8_t* dense, int64_t nbytes, uint8_t* packed, uint8_t* mask, int* bad) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= nbytes) return;
  const uint32_t d[2] = {reinterpret_cast<const uint32_t*>(dense + 8 * j)[0], reinterpret_cast<const uint32_t*>(dense + 8 * j)[1]};
  uint32_t kept = 0, m = 0;
  int b = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t q = 0;
    int n = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) if ((d[h] >> (8 * i)) & 255u) { q |= 1u << i; ++n; }
    if (n > 2) { ++b; n = 0; q = 0; for (int i = 0; i < 4 && n < 2; ++i) if ((d[h] >> (8 * i)) & 255u) { q |= 1u << i; ++n; } }
    for (int i = 0; i < 4 && n < 2; ++i) if (!(q & (1u << i))) { q |= 1u << i; ++n; }
    int slot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (q & (1u << i)) { kept |= ((d[h] >> (8 * i)) & 255u) << (16 * h + 8 * slot); ++slot; }
    m |= q << (4 * h);
  }
  *reinterpret_cast<uint32_t*>(packed + 4 * j) = kept;
  mask[j] = (uint8_t)m;
  if (b) atomicAdd(bad, b);
}

void launch_validate(const uint8_t* mask, int64_t nbytes, int* bad, hipStream_t stream) {
  k_fill_u32<<<1, 64, 0, stream>>>(reinterpret_cast<uint32_t*>(bad), 0u, 1);
  if (nbytes) k_validate<<<(unsigned)((nbytes + 255) / 256), 256, 0, stream>>>(mask, nbytes, bad);
}

void launch_unpack(const uint8_t* packed, const uint8_t* mask, int64_t nbytes, uint8_t* dense, int* bad, hipStream_t stream) {
  k_fill_u32<<<1, 64, 0, stream>>>(reinterpret_cast<uint32_t*>(bad), 0u, 1);
  if (nbytes) k_unpack<<<(unsigned)((nbytes + 255) / 256), 256, 0, stream>>>(packed, mask, nbytes, dense, bad);
}

void launch_pack(const uint8_t* dense, int64_t nbytes, uint8_t* packed, uint8_t* mask, int* bad, hipStream_t stream) {
  k_fill_u32<<<1, 64, 0, stream>>>(reinterpret_cast<uint32_t*>(bad), 0u, 1);
  if (nbytes) k_pack<<<(unsigned)((nbytes + 255) / 256), 256, 0, stream>>>(dense, nbytes, packed, mask, bad);
}

void launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t stream) {
  if (n) k_fill_u32<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(p, v, n);
}

}  // namespace moesq

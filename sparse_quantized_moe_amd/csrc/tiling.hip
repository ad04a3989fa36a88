// Load-time re-tiling of pair-bitmask weights into the kernels' own layout and back.
//
// The model cards ("Sparse storage layout") note that the serving stack rebuilds each layer into the
// GEMM kernel's own layout at load time; here that layout keeps the same bytes, reordered so that one
// 256-K step of a 16-row tile is one contiguous 1408-byte record (1024 B kept bytes, 256 B index
// codes, 128 B scales, each in lane order): the kept-byte nibbles of each smfmac are pre-arranged
// into operand order, and each mask nibble is replaced by the position code of its two kept pairs,
// which the kernels use as the sparse index with no table. A wave then reads each of its fragments
// with fully coalesced loads.
#include "moesq_device.h"
#include "moesq_internal.h"

namespace moesq {

// One thread per (record, lane): record = (tile, step) of all experts' tiles, lane = (row, quarter).
__global__ __launch_bounds__(256) void k_prepare(const uint8_t* __restrict__ packed, const uint8_t* __restrict__ mask,
                                                 const uint8_t* __restrict__ scale, int64_t tiles, int K,
                                                 uint8_t* __restrict__ tiled) {
  const int steps = K >> 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rec = gid >> 6;
  if (rec >= tiles * steps) return;
  const int lane = (int)(gid & 63);
  const int64_t tile = rec / steps;
  const int ss = (int)(rec - tile * steps);
  const int64_t row = tile * 16 + (lane & 15);   // row over all experts (expert-major, N % 16 == 0)
  const int q = lane >> 4;
  const int64_t k0 = (int64_t)ss * 256 + 64 * q;
  const u32x4 pk = *reinterpret_cast<const u32x4*>(packed + row * (K >> 2) + (k0 >> 2));
  const uint32_t mk = *reinterpret_cast<const uint32_t*>(mask + row * (K >> 4) + (k0 >> 4));
  const uint16_t sc = *reinterpret_cast<const uint16_t*>(scale + row * (K >> 5) + (k0 >> 5));
  uint8_t* r = tiled + rec * kTileRecordBytes;
  u32x4 t;
  t.x = kept_to_tiled(pk.x); t.y = kept_to_tiled(pk.y); t.z = kept_to_tiled(pk.z); t.w = kept_to_tiled(pk.w);
  *reinterpret_cast<u32x4*>(r + 16 * lane) = t;
  const uint32_t code = mask_to_code_byte(mk & 255u) | mask_to_code_byte((mk >> 8) & 255u) << 8 |
                        mask_to_code_byte((mk >> 16) & 255u) << 16 | mask_to_code_byte(mk >> 24) << 24;
  *reinterpret_cast<uint32_t*>(r + kTileCodeOffset + 4 * lane) = code;
  *reinterpret_cast<uint16_t*>(r + kTileScaleOffset + 2 * lane) = sc;
}

__global__ __launch_bounds__(256) void k_unprepare(const uint8_t* __restrict__ tiled, int64_t tiles, int K,
                                                   uint8_t* __restrict__ packed, uint8_t* __restrict__ mask,
                                                   uint8_t* __restrict__ scale) {
  const int steps = K >> 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rec = gid >> 6;
  if (rec >= tiles * steps) return;
  const int lane = (int)(gid & 63);
  const int64_t tile = rec / steps;
  const int ss = (int)(rec - tile * steps);
  const int64_t row = tile * 16 + (lane & 15);
  const int q = lane >> 4;
  const int64_t k0 = (int64_t)ss * 256 + 64 * q;
  const uint8_t* r = tiled + rec * kTileRecordBytes;
  const u32x4 t = *reinterpret_cast<const u32x4*>(r + 16 * lane);
  u32x4 pk;
  pk.x = tiled_to_kept(t.x); pk.y = tiled_to_kept(t.y); pk.z = tiled_to_kept(t.z); pk.w = tiled_to_kept(t.w);
  *reinterpret_cast<u32x4*>(packed + row * (K >> 2) + (k0 >> 2)) = pk;
  const uint32_t code = *reinterpret_cast<const uint32_t*>(r + kTileCodeOffset + 4 * lane);
  *reinterpret_cast<uint32_t*>(mask + row * (K >> 4) + (k0 >> 4)) =
      code_to_mask_byte(code & 255u) | code_to_mask_byte((code >> 8) & 255u) << 8 |
      code_to_mask_byte((code >> 16) & 255u) << 16 | code_to_mask_byte(code >> 24) << 24;
  *reinterpret_cast<uint16_t*>(scale + row * (K >> 5) + (k0 >> 5)) = *reinterpret_cast<const uint16_t*>(r + kTileScaleOffset + 2 * lane);
}

size_t tiled_bytes(int E, int N, int K) { return (size_t)E * (N / 16) * (K / 256) * kTileRecordBytes; }

void launch_prepare(const uint8_t* packed, const uint8_t* mask, const uint8_t* scale, int E, int N, int K,
                    uint8_t* tiled, hipStream_t stream) {
  const int64_t tiles = (int64_t)E * (N / 16);
  const int64_t threads = tiles * (K / 256) * 64;
  if (threads) k_prepare<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(packed, mask, scale, tiles, K, tiled);
}

void launch_unprepare(const uint8_t* tiled, int E, int N, int K, uint8_t* packed, uint8_t* mask, uint8_t* scale,
                      hipStream_t stream) {
  const int64_t tiles = (int64_t)E * (N / 16);
  const int64_t threads = tiles * (K / 256) * 64;
  if (threads) k_unprepare<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(tiled, tiles, K, packed, mask, scale);
}

}  // namespace moesq

// Stable token->expert permutation for the grouped GEMM, on one workgroup of 8 waves.
//
// The pairs p = t*k + j of the router's top-k ids are grouped by expert, stable in p (the grouped
// GEMM of model card "Qwen3.5-397B-A17B-P48NVFP4-MoESQ" runs one GEMM per expert over its rows).
// Two passes over tiles of 512 tokens: (1) per-expert counts with LDS atomics, then exclusive scans
// into offsets[E+1] and the m-block prefix tile_offsets[E+1]; (2) per tile, each wave of 64 tokens
// marks the experts of its lanes in a 64-bit LDS mask per expert; a pair's row is
//   running_base[e] + (pairs of e in earlier waves of the tile) + popcount(mask[e] & lanes below),
// which is the stable order because a token holds each expert at most once. A tile that holds a
// duplicate id inside one token's row is ranked serially by one thread (same order, slower).
// Ids outside [-1, E) are dropped like -1 and counted in status[0].
#include "moesq_device.h"
#include "moesq_internal.h"

namespace moesq {

constexpr int kPermThreads = 512;
constexpr int kPermWaves = kPermThreads / 64;

// Exclusive scan in place of a[0..n) (LDS), returns the total. tmp: kPermThreads ints of LDS.
__device__ int block_exclusive_scan(int* a, int n, int* tmp) {
  const int tid = threadIdx.x;
  const int per = (n + kPermThreads - 1) / kPermThreads;
  const int s0 = tid * per;
  const int s1 = s0 + per < n ? s0 + per : n;
  int sum = 0;
  for (int i = s0; i < s1; ++i) sum += a[i];
  tmp[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kPermThreads; off <<= 1) {
    const int v = tid >= off ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += v;
    __syncthreads();
  }
  int base = tmp[tid] - sum;
  const int total = tmp[kPermThreads - 1];
  for (int i = s0; i < s1; ++i) {
    const int v = a[i];
    a[i] = base;
    base += v;
  }
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kPermThreads) void k_permute(const int* __restrict__ ids, int64_t T, int k, int E,
                                                          int* counts, int* offsets, int* sorted, int* inv,
                                                          int* tile_offsets, int bm, int* status) {
  extern __shared__ __align__(16) uint8_t smem[];
  unsigned long long* wmask = reinterpret_cast<unsigned long long*>(smem);    // [waves][E]
  int* wbase = reinterpret_cast<int*>(wmask + kPermWaves * E);               // [waves][E]
  int* cnt = wbase + kPermWaves * E;                                          // [E] counts, then running base
  int* tcnt = cnt + E;                                                        // [E] m-blocks per expert
  __shared__ int tmp[kPermThreads];
  __shared__ int s_bad, s_dup;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < E; e += kPermThreads) cnt[e] = 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // pass 1: counts
  for (int64_t t0 = 0; t0 < T; t0 += kPermThreads) {
    const int64_t t = t0 + tid;
    if (t < T) {
      for (int j = 0; j < k; ++j) {
        const int e = ids[t * k + j];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
        else if (e != -1) atomicAdd(&s_bad, 1);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermThreads) {
    counts[e] = cnt[e];
    tcnt[e] = bm > 0 ? (cnt[e] + bm - 1) / bm : 0;
  }
  __syncthreads();
  const int total = block_exclusive_scan(cnt, E, tmp);
  const int ttotal = block_exclusive_scan(tcnt, E, tmp);
  for (int e = tid; e < E; e += kPermThreads) {
    offsets[e] = cnt[e];
    if (bm > 0) tile_offsets[e] = tcnt[e];
  }
  if (tid == 0) {
    offsets[E] = total;
    if (bm > 0) tile_offsets[E] = ttotal;
  }

  // pass 2: ranks
  for (int64_t t0 = 0; t0 < T; t0 += kPermThreads) {
    for (int i = tid; i < kPermWaves * E; i += kPermThreads) wmask[i] = 0ull;
    if (tid == 0) s_dup = 0;
    __syncthreads();
    const int64_t t = t0 + tid;
    const bool valid = t < T;
    if (valid) {
      for (int j = 0; j < k; ++j) {
        const int e = ids[t * k + j];
        if (e < 0 || e >= E) continue;
        atomicOr(&wmask[wv * E + e], 1ull << lane);
        for (int j2 = 0; j2 < j; ++j2)
          if (ids[t * k + j2] == e) s_dup = 1;
      }
    }
    __syncthreads();
    if (s_dup) {
      if (tid == 0) {
        const int64_t t1 = t0 + kPermThreads < T ? t0 + kPermThreads : T;
        for (int64_t tt = t0; tt < t1; ++tt)
          for (int j = 0; j < k; ++j) {
            const int e = ids[tt * k + j];
            if (e < 0 || e >= E) { inv[tt * k + j] = -1; continue; }
            const int r = cnt[e]++;
            sorted[r] = (int)(tt * k + j);
            inv[tt * k + j] = r;
          }
      }
      __syncthreads();
      continue;
    }
    for (int e = tid; e < E; e += kPermThreads) {
      int run = cnt[e];
      for (int w = 0; w < kPermWaves; ++w) {
        wbase[w * E + e] = run;
        run += __builtin_popcountll(wmask[w * E + e]);
      }
      cnt[e] = run;
    }
    __syncthreads();
    if (valid) {
      const unsigned long long below = (1ull << lane) - 1ull;
      for (int j = 0; j < k; ++j) {
        const int e = ids[t * k + j];
        if (e < 0 || e >= E) { inv[t * k + j] = -1; continue; }
        const int r = wbase[wv * E + e] + __builtin_popcountll(wmask[wv * E + e] & below);
        sorted[r] = (int)(t * k + j);
        inv[t * k + j] = r;
      }
    }
    __syncthreads();
  }
  if (tid == 0) status[0] = s_bad;
}

static size_t permute_lds_bytes(int E) {
  return (size_t)kPermWaves * E * 8 + (size_t)kPermWaves * E * 4 + (size_t)2 * E * 4;
}

void launch_permute(const int* ids, int64_t T, int k, int E, int* counts, int* offsets, int* sorted, int* inv,
                    int* tile_offsets, int bm, int* status, hipStream_t stream) {
  const size_t lds = permute_lds_bytes(E);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_permute), hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)permute_lds_bytes(1024));
    attr_set = true;
  }
  k_permute<<<1, kPermThreads, lds, stream>>>(ids, T, k, E, counts, offsets, sorted, inv, tile_offsets, bm, status);
}

// tile_offsets[e] = sum_{e' < e} ceil(count_e' / bm), from offsets.
__global__ __launch_bounds__(kPermThreads) void k_tile_offsets(const int* offsets, int E, int bm, int* tile_offsets) {
  __shared__ int a[1025];
  __shared__ int tmp[kPermThreads];
  for (int e = threadIdx.x; e < E; e += kPermThreads) {
    const int c = offsets[e + 1] - offsets[e];
    a[e] = c > 0 ? (c + bm - 1) / bm : 0;
  }
  __syncthreads();
  const int total = block_exclusive_scan(a, E, tmp);
  for (int e = threadIdx.x; e < E; e += kPermThreads) tile_offsets[e] = a[e];
  if (threadIdx.x == 0) tile_offsets[E] = total;
}

void launch_tile_offsets(const int* offsets, int E, int bm, int* tile_offsets, hipStream_t stream) {
  k_tile_offsets<<<1, kPermThreads, 0, stream>>>(offsets, E, bm, tile_offsets);
}

}  // namespace moesq

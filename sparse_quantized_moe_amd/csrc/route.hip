// Routing front of the MoE FFN: the stable token -> expert permutation and the NVFP4 quantization of
// every (token, expert) pair's activation row, in one launch when the tokens fit one tile.
//
// Permutation (the grouped GEMM of model card "Qwen3.5-397B-A17B-P48NVFP4-MoESQ" runs one GEMM per
// expert over that expert's rows): pairs p = t*k + j are grouped by expert, stable in p. Tokens are cut
// into tiles of 512, one workgroup each. Inside a tile every wave of 64 tokens sets, per expert, the
// bits of its lanes in a 64-bit LDS mask, and the rank of a pair inside the tile is
//   (pairs of e in earlier waves of the tile) + popcount(mask[e] & lanes below).
// That is the stable order because a token names each expert at most once; a tile holding a token
// that names an expert twice (detected by the mask bit being set already) is ranked serially by one
// thread instead, giving the same order. The row of a pair is then
//   offsets[e] + (pairs of e in earlier tiles) + rank in the tile.
// With one tile, its workgroup also scans and scatters. With several, a scan kernel and a scatter
// kernel follow. Ids outside [-1, E) are dropped like -1 and counted in status[0].
//
// Quantization (model card "Compression details": NVFP4 activations with per-32 scales and an FP32
// global stored per expert linear): row p of the codes is NVFP4(x[t], a_global[ids[p]]) in pair order,
// so it does not wait for the permutation; the GEMM reads row sorted[r] for its r-th row. A thread
// loads one 32-group of a token once, takes its amax once and encodes it for a run of that token's
// experts.
#include <mutex>

#include "moesq_device.h"
#include "moesq_internal.h"

namespace moesq {

constexpr int kRouteThreads = 512;
constexpr int kRouteWaves = kRouteThreads / 64;

// Exclusive scan in place of a[0..n) (LDS) by the whole workgroup; returns the total.
__device__ int route_block_scan(int* a, int n, int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (n + kRouteThreads - 1) / kRouteThreads;
  const int s0 = tid * per < n ? tid * per : n;
  const int s1 = s0 + per < n ? s0 + per : n;
  int sum = 0;
  for (int i = s0; i < s1; ++i) sum += a[i];
  int v = sum;                                   // inclusive scan over the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) tmp[wv] = v;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < kRouteWaves; ++w) { const int x = tmp[w]; tmp[w] = run; run += x; }
    tmp[kRouteWaves] = run;
  }
  __syncthreads();
  int base = tmp[wv] + v - sum;
  const int total = tmp[kRouteWaves];
  for (int i = s0; i < s1; ++i) {
    const int x = a[i];
    a[i] = base;
    base += x;
  }
  __syncthreads();
  return total;
}

// Exclusive scans in place of a[0..n) and b[0..n) (LDS) in one pass; returns both totals.
__device__ int2 route_block_scan2(int* a, int* b, int n, int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (n + kRouteThreads - 1) / kRouteThreads;
  const int s0 = tid * per < n ? tid * per : n;
  const int s1 = s0 + per < n ? s0 + per : n;
  int sa = 0, sb = 0;
  for (int i = s0; i < s1; ++i) { sa += a[i]; sb += b[i]; }
  int va = sa, vb = sb;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ua = __shfl_up(va, off), ub = __shfl_up(vb, off);
    if (lane >= off) { va += ua; vb += ub; }
  }
  if (lane == 63) { tmp[wv] = va; tmp[kRouteWaves + 1 + wv] = vb; }
  __syncthreads();
  if (tid == 0) {
    int ra = 0, rb = 0;
    for (int w = 0; w < kRouteWaves; ++w) {
      const int xa = tmp[w], xb = tmp[kRouteWaves + 1 + w];
      tmp[w] = ra; tmp[kRouteWaves + 1 + w] = rb;
      ra += xa; rb += xb;
    }
    tmp[kRouteWaves] = ra;
    tmp[2 * kRouteWaves + 1] = rb;
  }
  __syncthreads();
  int ba = tmp[wv] + va - sa, bb = tmp[kRouteWaves + 1 + wv] + vb - sb;
  const int2 total = int2{tmp[kRouteWaves], tmp[2 * kRouteWaves + 1]};
  for (int i = s0; i < s1; ++i) {
    const int xa = a[i], xb = b[i];
    a[i] = ba; b[i] = bb;
    ba += xa; bb += xb;
  }
  __syncthreads();
  return total;
}

// One tile stages sorted and inv in LDS (written out contiguously afterwards) when they fit.
constexpr int kRouteStagePairs = 4096;

struct RouteArgs {
  const int* ids;            // [T*k]
  int64_t T;
  int k, E, ntiles;
  int* counts;               // [E]
  int* offsets;              // [E+1]
  int* tile_offsets;         // [E+1] prefix of ceil(count / bm), when bm > 0
  int bm;
  int* sorted;               // [T*k], live prefix offsets[E]
  int* inv;                  // [T*k]; holds the in-tile rank until the scatter
  int* status;               // [1]
  int* tile_counts;          // several tiles: [ntiles][E] counts, then [ntiles] dropped-id counts
  // quantization of the pairs' rows (qblocks = 0: none)
  const uint16_t* x;         // bf16 [T][H]
  int H;
  const float* a_global;     // [E]
  uint8_t* codes;            // [T*k][H/2]
  uint8_t* scales;           // [T*k][H/32]
  int qblocks;
  int kchunk;                // experts encoded per thread
};

// KMAX >= k: the token's ids live in registers (static indices), loaded together up front.
template <int KMAX>
__device__ void route_tile(const RouteArgs& a, int tile, uint8_t* smem) {
  const int E = a.E, k = a.k;
  unsigned long long* wmask = reinterpret_cast<unsigned long long*>(smem);   // [waves][E]
  int* wbase = reinterpret_cast<int*>(wmask + kRouteWaves * E);              // [waves][E]
  int* cnt = wbase + kRouteWaves * E;                                         // [E]
  int* tcnt = cnt + E;                                                        // [E]
  int* s_sorted = tcnt + E;                                                   // [T k] (one tile, staged)
  int* s_inv = s_sorted + kRouteStagePairs;                                   // [T k]
  __shared__ int tmp[2 * kRouteWaves + 2];
  __shared__ int s_bad, s_dup;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t t = (int64_t)tile * kRouteThreads + tid;
  const bool valid = t < a.T;
  const unsigned long long bit = 1ull << lane, below = bit - 1ull;

  int ids[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) ids[j] = (valid && j < k) ? a.ids[t * k + j] : -1;
  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) wmask[i] = 0ull;
  if (tid == 0) { s_bad = 0; s_dup = 0; }
  __syncthreads();
  if (valid) {
    // a token naming an expert twice is found by comparing its ids (the mask bits only say "some")
    int bad = 0, dup = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int e = ids[j];
      if (e < 0 || e >= E) { bad += e != -1; continue; }
      atomicOr(&wmask[wv * E + e], bit);
#pragma unroll
      for (int i = 0; i < j; ++i) dup |= ids[i] == e;
    }
    if (bad) atomicAdd(&s_bad, bad);
    if (dup) s_dup = 1;
  }
  __syncthreads();
  const bool serial = s_dup != 0;
  if (serial) {
    // a token names an expert twice: rank this tile by one thread, in pair order
    for (int e = tid; e < E; e += kRouteThreads) cnt[e] = 0;
    __syncthreads();
    if (tid == 0) {
      const int64_t t0 = (int64_t)tile * kRouteThreads;
      const int64_t t1 = t0 + kRouteThreads < a.T ? t0 + kRouteThreads : a.T;
      for (int64_t p = t0 * k; p < t1 * k; ++p) {
        const int e = a.ids[p];
        if (e >= 0 && e < E) a.inv[p] = cnt[e]++;
      }
    }
  } else {
    for (int e = tid; e < E; e += kRouteThreads) {
      int run = 0;
      for (int w = 0; w < kRouteWaves; ++w) {
        wbase[w * E + e] = run;
        run += __builtin_popcountll(wmask[w * E + e]);
      }
      cnt[e] = run;
    }
  }
  __syncthreads();
  // rank inside the tile of pair p (expert e) of this thread's token
  auto rank_of = [&](int64_t p, int e) -> int {
    return serial ? a.inv[p] : wbase[wv * E + e] + __builtin_popcountll(wmask[wv * E + e] & below);
  };
  if (a.ntiles > 1) {
    for (int e = tid; e < E; e += kRouteThreads) a.tile_counts[(int64_t)tile * E + e] = cnt[e];
    if (tid == 0) a.tile_counts[(int64_t)a.ntiles * E + tile] = s_bad;
    if (valid && !serial) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        const int64_t p = t * k + j;
        const int e = ids[j];
        if (j < k && e >= 0 && e < E) a.inv[p] = rank_of(p, e);
      }
    }
    return;
  }
  // one tile: counts, scans, then the scatter
  for (int e = tid; e < E; e += kRouteThreads) {
    a.counts[e] = cnt[e];
    tcnt[e] = a.bm > 0 ? (cnt[e] + a.bm - 1) / a.bm : 0;
  }
  __syncthreads();
  const int2 totals = route_block_scan2(cnt, tcnt, E, tmp);
  for (int e = tid; e < E; e += kRouteThreads) {
    a.offsets[e] = cnt[e];
    if (a.bm > 0) a.tile_offsets[e] = tcnt[e];
  }
  if (tid == 0) {
    a.offsets[E] = totals.x;
    if (a.bm > 0) a.tile_offsets[E] = totals.y;
    a.status[0] = s_bad;
  }
  if (a.bm > 0 && tid < kPrefillPools) prefill_pools(a.tile_offsets, E)[tid] = 0;
  // scatter: through LDS when the pairs fit (scattered LDS writes, then contiguous global writes),
  // else straight to memory
  const int64_t P = a.T * k;
  const bool staged = P <= kRouteStagePairs;
  if (valid) {
    // every rank first (reads only), then the writes; the two destinations are written by separate
    // code so that each store has a known address space (LDS or global, not flat)
    int rr[KMAX];
    if (serial) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        const int e = ids[j];
        rr[j] = (j < k && e >= 0 && e < E) ? cnt[e] + a.inv[t * k + j] : -1;
      }
    } else {   // LDS only: no wait on the global stores above
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        const int e = ids[j];
        rr[j] = (j < k && e >= 0 && e < E)
                    ? cnt[e] + wbase[wv * E + e] + (int)__builtin_popcountll(wmask[wv * E + e] & below)
                    : -1;
      }
    }
    auto scatter = [&](int* dst_sorted, int* dst_inv) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j >= k) continue;
        const int64_t p = t * k + j;
        dst_inv[p] = rr[j];
        if (rr[j] >= 0) dst_sorted[rr[j]] = (int)p;
      }
    };
    if (staged)
      scatter(s_sorted, s_inv);
    else
      scatter(a.sorted, a.inv);
  }
  if (staged) {
    __syncthreads();
    for (int i = tid; i < totals.x; i += kRouteThreads) a.sorted[i] = s_sorted[i];
    for (int i = tid; i < (int)P; i += kRouteThreads) a.inv[i] = s_inv[i];
  }
}

// Experts encoded per load of a token's values, at most.
constexpr int kQuantRun = 8;

// One item = (token t, run jc of its experts, 32-group grp); consecutive threads take consecutive
// groups of one token. The per-expert globals sit in LDS and a run's ids are loaded with the token's
// values, so an item costs one round trip to memory.
template <int KMAX>
__device__ __forceinline__ void route_quantize(const RouteArgs& a, int qb, float* s_g) {
  for (int e = threadIdx.x; e < a.E; e += kRouteThreads) s_g[e] = a.a_global[e];
  __syncthreads();
  const uint32_t G = (uint32_t)(a.H >> 5);
  const uint32_t nj = (uint32_t)((a.k + a.kchunk - 1) / a.kchunk);
  const uint32_t items = (uint32_t)a.T * nj * G;               // < 2^31 (checked by the host)
  for (uint32_t it = (uint32_t)qb * kRouteThreads + threadIdx.x; it < items; it += (uint32_t)a.qblocks * kRouteThreads) {
    const uint32_t tj = it / G;
    const uint32_t grp = it - tj * G;
    const uint32_t t = tj / nj;
    const int j0 = (int)(tj - t * nj) * a.kchunk;
    const int nrun = a.k - j0 < a.kchunk ? a.k - j0 : a.kchunk;
    const int64_t p0 = (int64_t)t * a.k + j0;
    int ids[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) ids[j] = j < nrun ? a.ids[p0 + j] : -1;
    const u32x4* src = reinterpret_cast<const u32x4*>(a.x + (int64_t)t * a.H + grp * 32);
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 w = src[i];
      const uint32_t b[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v[8 * i + 2 * h] = __uint_as_float(b[h] << 16);
        v[8 * i + 2 * h + 1] = __uint_as_float(b[h] & 0xFFFF0000u);
      }
    }
    float amax = 0.0f;
    uint32_t mb = 0;   // largest magnitude bit pattern: >= 0x7F800000 iff some value is not finite
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
      mb = __builtin_elementwise_max(mb, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    }
    const bool finite = mb < 0x7F800000u;
    // The codes and the scale of a group depend on its values and the expert's global only, so an
    // expert whose global has the same bits as the last one encoded reuses that encoding (layers
    // whose experts share one activation global encode each group once per run instead of once per
    // expert).
    bool have = false;
    uint32_t glast = 0u;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    int sc = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int e = ids[j];
      if (j >= nrun || e < 0 || e >= a.E) continue;
      const int64_t p = p0 + j;
      const float g = s_g[e];
      if (!have || __float_as_uint(g) != glast) {
        sc = scale_code(amax, g);
        const float s = e4m3_value(sc);
        const Nvfp4Snap sn = nvfp4_snap(s, g, finite);
#pragma unroll
        for (int h = 0; h < 4; ++h) w[h] = nvfp4_codes_snap<8>(v + 8 * h, s, g, sn);
        have = true;
        glast = __float_as_uint(g);
      }
      *reinterpret_cast<u32x4*>(a.codes + p * (a.H >> 1) + grp * 16) = u32x4{w[0], w[1], w[2], w[3]};
      a.scales[p * G + grp] = (uint8_t)sc;
    }
  }
}

template <int KMAX>
__global__ __launch_bounds__(kRouteThreads) void k_route(RouteArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  if ((int)blockIdx.x < a.ntiles) route_tile<KMAX>(a, blockIdx.x, smem);
  else route_quantize<(KMAX < kQuantRun ? KMAX : kQuantRun)>(a, blockIdx.x - a.ntiles, reinterpret_cast<float*>(smem));
}

// Several tiles: per expert, the exclusive prefix of the tile counts becomes each (tile, expert)'s
// global row base; counts, offsets, tile_offsets and status are written.
__global__ __launch_bounds__(kRouteThreads) void k_route_scan(RouteArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  int* cnt = reinterpret_cast<int*>(smem);      // [E]
  int* tcnt = cnt + a.E;                        // [E]
  __shared__ int tmp[kRouteWaves + 1];
  const int E = a.E, tid = threadIdx.x;
  // the tile counts of an expert are read kScanBatch at a time (independent loads, one round trip
  // per batch rather than per tile), then rewritten as exclusive prefixes
  constexpr int kScanBatch = 16;
  for (int e = tid; e < E; e += kRouteThreads) {
    int run = 0;
    for (int t0 = 0; t0 < a.ntiles; t0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) c[i] = t0 + i < a.ntiles ? a.tile_counts[(int64_t)(t0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) {
        if (t0 + i < a.ntiles) a.tile_counts[(int64_t)(t0 + i) * E + e] = run;
        run += c[i];
      }
    }
    cnt[e] = run;
    a.counts[e] = run;
    tcnt[e] = a.bm > 0 ? (run + a.bm - 1) / a.bm : 0;
  }
  __syncthreads();
  const int total = route_block_scan(cnt, E, tmp);
  const int ttotal = route_block_scan(tcnt, E, tmp);
  for (int e = tid; e < E; e += kRouteThreads) {
    a.offsets[e] = cnt[e];
    if (a.bm > 0) a.tile_offsets[e] = tcnt[e];
    for (int t0 = 0; t0 < a.ntiles; t0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) c[i] = t0 + i < a.ntiles ? a.tile_counts[(int64_t)(t0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        if (t0 + i < a.ntiles) a.tile_counts[(int64_t)(t0 + i) * E + e] = c[i] + cnt[e];
    }
  }
  if (a.bm > 0 && tid < kPrefillPools) prefill_pools(a.tile_offsets, E)[tid] = 0;
  if (tid == 0) {
    a.offsets[E] = total;
    if (a.bm > 0) a.tile_offsets[E] = ttotal;
    int bad = 0;
    for (int t = 0; t < a.ntiles; ++t) bad += a.tile_counts[(int64_t)a.ntiles * E + t];
    a.status[0] = bad;
  }
}

__global__ __launch_bounds__(256) void k_route_scatter(RouteArgs a) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= a.T * a.k) return;
  const int e = a.ids[p];
  if (e < 0 || e >= a.E) { a.inv[p] = -1; return; }
  const int64_t tile = (p / a.k) / kRouteThreads;
  const int r = a.tile_counts[tile * a.E + e] + a.inv[p];
  a.sorted[r] = (int)p;
  a.inv[p] = r;
}

size_t route_scratch_bytes(int64_t T, int E) {
  const int64_t ntiles = (T + kRouteThreads - 1) / kRouteThreads;
  return ntiles <= 1 ? 0 : (size_t)ntiles * (E + 1) * 4;
}

// masks and bases [waves][E], counts [2][E], then the staged sorted / inv of one tile
static size_t route_lds_bytes(int E) {
  return (size_t)kRouteWaves * E * 12 + (size_t)2 * E * 4 + (size_t)2 * kRouteStagePairs * 4;
}

void launch_route(const int* ids, int64_t T, int k, int E, int* counts, int* offsets, int* tile_offsets, int bm,
                  int* sorted, int* inv, int* status, void* scratch, const uint16_t* x, int H, const float* a_global,
                  uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  static std::once_flag attr;
  static hipError_t attr_err = hipSuccess;   // written once, inside call_once, read after it
  std::call_once(attr, [] {
    for (const void* f : {reinterpret_cast<const void*>(&k_route<8>), reinterpret_cast<const void*>(&k_route<16>),
                          reinterpret_cast<const void*>(&k_route<32>)}) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)route_lds_bytes(1024));
      if (e != hipSuccess && attr_err == hipSuccess) attr_err = e;
    }
  });
  if (attr_err != hipSuccess) {
    note_hip_error(attr_err);
    return;
  }
  RouteArgs a{};
  a.ids = ids; a.T = T; a.k = k; a.E = E;
  a.ntiles = T > 0 ? (int)((T + kRouteThreads - 1) / kRouteThreads) : 1;
  a.counts = counts; a.offsets = offsets; a.tile_offsets = tile_offsets; a.bm = bm;
  a.sorted = sorted; a.inv = inv; a.status = status;
  a.tile_counts = static_cast<int*>(scratch);
  if (x && T > 0) {
    // enough items to spread a small batch over the chip; a large one encodes all k experts per load
    const int64_t tg = T * (H >> 5);
    // (runs of at most kQuantRun experts, the quantizer's register budget)
    int64_t nj = (131072 + tg - 1) / tg;
    nj = nj < 1 ? 1 : (nj > k ? k : nj);
    if (nj < (k + kQuantRun - 1) / kQuantRun) nj = (k + kQuantRun - 1) / kQuantRun;
    a.kchunk = (int)((k + nj - 1) / nj);
    nj = (k + a.kchunk - 1) / a.kchunk;
    const int64_t qb = (tg * nj + kRouteThreads - 1) / kRouteThreads;
    a.qblocks = (int)(qb > 4096 ? 4096 : qb);
    a.x = x; a.H = H; a.a_global = a_global; a.codes = codes; a.scales = scales;
  }
  const dim3 grid((unsigned)(a.ntiles + a.qblocks));
  if (k <= 8) launch_kernel(k_route<8>, grid, dim3(kRouteThreads), route_lds_bytes(E), stream, a);
  else if (k <= 16) launch_kernel(k_route<16>, grid, dim3(kRouteThreads), route_lds_bytes(E), stream, a);
  else launch_kernel(k_route<32>, grid, dim3(kRouteThreads), route_lds_bytes(E), stream, a);
  if (a.ntiles > 1) {
    launch_kernel(k_route_scan, dim3(1), dim3(kRouteThreads), (size_t)2 * E * 4, stream, a);
    const int64_t P = T * k;
    launch_kernel(k_route_scatter, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, stream, a);
  }
}

// tile_offsets[e] = sum over e' < e of ceil(count_e' / bm), from offsets.
__global__ __launch_bounds__(kRouteThreads) void k_tile_offsets(const int* offsets, int E, int bm, int* tile_offsets) {
  __shared__ int c[1024];
  __shared__ int tmp[kRouteWaves + 1];
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    const int n = offsets[e + 1] - offsets[e];
    c[e] = n > 0 ? (n + bm - 1) / bm : 0;
  }
  __syncthreads();
  const int total = route_block_scan(c, E, tmp);
  for (int e = threadIdx.x; e < E; e += kRouteThreads) tile_offsets[e] = c[e];
  if (threadIdx.x == 0) tile_offsets[E] = total;
  if (threadIdx.x < kPrefillPools) prefill_pools(tile_offsets, E)[threadIdx.x] = 0;
}

void launch_tile_offsets(const int* offsets, int E, int bm, int* tile_offsets, hipStream_t stream) {
  k_tile_offsets<<<1, kRouteThreads, 0, stream>>>(offsets, E, bm, tile_offsets);
}

}  // namespace moesq

// Decode-size MoE FFN in one persistent launch: routing, gate/up GEMM, down GEMM and the top-k
// combine as four phases of one kernel, separated by grid barriers (between gate/up and down, by a
// wait on the same expert's workgroups only).
//
// What is computed is the unfused path's (route.hip, gemm.hip), step for step and bit for bit: the
// pairs' NVFP4 activation rows (model card "Qwen3.5-397B-A17B-P48NVFP4-MoESQ", "Compression
// details"), the grouped sparse GEMMs over the pair-bitmask weights ("Sparse storage layout"), the
// fused silu(gate) * up with its NVFP4 re-quantization, and the router-weighted sum over each
// token's k experts. The aim: at decode sizes each phase is short, and separate kernels leave memory
// idle between them (launch gaps) and at each start (a GEMM workgroup waits for its activations
// before its weight stream gets going). Here a phase's first weight loads go out before the barrier
// that guards its inputs, since weights depend on nothing. Measured on MI355X at 128 experts, top-8,
// hidden 2048, intermediate 768, 256 tokens, this path takes about 75 us against about 68 us for the
// separate launches: the per-item activation encoding and the barriers cost more than the overlap
// gains, so the library keeps the separate launches by default and this path is opt-in.
//
// Work split: one workgroup of 12 waves per (expert e, part). A part covers 12 waves x 32 gate/up
// columns of e and, in the down phase, a balanced share of e's output row-pairs; with 128 experts
// and I = 768 that is 256 workgroups, one per CU. Each workgroup finds e's rows itself from the
// router ids (stable compaction of the pairs with id e; the row base is the number of pairs with
// a smaller id), so no phase waits for a serial permutation pass.
//
// Barrier: per-workgroup arrival flags and a release word in the workspace, each holding (launch
// ticket << 32 | round), so they need no reset between launches and may hold anything before the
// first; every wait is bounded, and a wait that runs out sets an error word (tagged with the ticket)
// that makes every other workgroup leave too, and reports -1 in status[0].
#include <unistd.h>

#include <atomic>

#include "gemm_common.h"

namespace moesq {

constexpr int kFzWaves = 12;
constexpr int kFzThreads = kFzWaves * 64;
constexpr int kFzBMT = 32;                 // rows per m-block (2 token tiles)
constexpr int kFzTG = 2;
constexpr int kFzMaxPairs = 4096;          // T * k handled by the fused path
constexpr int kFzIdRounds = kFzMaxPairs / kFzThreads + 1;
constexpr int kFzMaxK = 2048;              // H and I
constexpr int kFzStageItems = (kFzBMT * (kFzMaxK / 32) + kFzThreads - 1) / kFzThreads;
constexpr int kFzDownRT = 2;
constexpr int kFzDownDepth = 6;
constexpr uint32_t kFzSpinLimit = 1u << 20;
constexpr int kFzMaxGrid = 1024;           // arrival flags in the sync area

struct FusedArgs {
  const uint16_t* x;            // bf16 [T][H]
  const int* ids;               // [T*k]
  const float* topk_weights;    // [T*k]
  const float* a13_global;      // [E]
  const float* a2_global;       // [E]
  const uint8_t* w13;           // tiled records of the gate|up weights
  const float* w13_global;      // [E][2]
  const uint8_t* w2;            // tiled records of the down weights
  const float* w2_global;       // [E]
  int T, H, I, k, E, parts;
  int* counts;                  // [E]
  int* offsets;                 // [E+1]
  int* sorted;                  // [T*k]
  int* inv;                     // [T*k]
  int* status;                  // [1]
  uint8_t* a13c;                // [T*k][H/2], pair order
  uint8_t* a13s;                // [T*k][H/32]
  uint8_t* a2c;                 // [T*k][I/2], sorted order
  uint8_t* a2s;                 // [T*k][I/32]
  float* D;                     // [T*k][H], sorted order
  float* out;                   // [T][H]
  unsigned long long* release;  // barrier release word
  unsigned* err;                // error word (ticket of the failed launch)
  unsigned long long* flags;    // [grid] arrival flags
  unsigned ticket;              // unique per launch, non-zero
  uint32_t spin_limit;          // polls before a barrier wait gives up
};

__host__ __device__ constexpr size_t fused_lds_bytes(int H, int I, int P) {
  return (size_t)kFzBMT * (2 * (H > I ? H : I) + 16) + (size_t)P * 4;
}

// Workgroup barrier that orders LDS only: a wave with global loads in flight does not wait for them
// (on CDNA one counter covers loads and stores, so a full fence would).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  asm volatile("" ::: "memory");                    // no global access moves across it either
}

// This wave's stores (device-coherent, see below) have all completed. The counter also covers loads,
// so it is called where the wave has none in flight that it would rather not wait for.
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Grid barrier `round` (1, 2, 3), run by the 64 lanes of wave 0 once every wave of the workgroup has
// completed its stores (stores_done and a workgroup barrier before). Everything one workgroup writes
// for another in this kernel is stored and loaded device-coherent (sc1: written through, read from
// the coherence point), so the barrier needs no cache write-back or invalidation: arrival is a store
// of (ticket, round) into the workgroup's own flag, wave 0 of workgroup 0 polls all flags and then
// stores (ticket, round) into the release word that everyone polls. No read-modify-write atomics, so
// no contention on one address; every word carries the launch ticket, so leftovers of earlier
// launches (or any initial contents) never count. Returns false if a wait ran out or another
// workgroup's did.
__device__ bool fz_grid_wait(const FusedArgs& a, unsigned round) {
  const int lane = threadIdx.x & 63;
  const unsigned long long tag = (unsigned long long)a.ticket << 32;
  const unsigned long long want = tag | round;
  auto failed = [&](uint32_t spins) {
    return spins >= a.spin_limit || __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.ticket;
  };
  auto reached = [&](unsigned long long v) { return (v & 0xFFFFFFFF00000000ull) == tag && v >= want; };
  bool ok = true;
  if (lane == 0) __hip_atomic_store(a.flags + blockIdx.x, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the bound is checked before each poll, so a limit of 0 gives up at once (the host's test hook)
  if (blockIdx.x == 0) {                              // the collector: every flag at this round
    for (uint32_t spins = 0;; ++spins) {
      if (__shfl(failed(spins) ? 1 : 0, 0)) { ok = false; break; }
      bool mine = true;
      for (unsigned b = lane; b < gridDim.x; b += 64)
        mine = mine && reached(__hip_atomic_load(a.flags + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (__all(mine)) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0 && ok) __hip_atomic_store(a.release, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (lane == 0) {
    if (ok) {
      for (uint32_t spins = 0;; ++spins) {
        if (failed(spins)) { ok = false; break; }
        if (reached(__hip_atomic_load(a.release, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) break;
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (!ok) {
      __hip_atomic_store(a.err, a.ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.status[0] = -1;
    }
  }
  asm volatile("" ::: "memory");
  return __shfl(ok ? 1 : 0, 0) != 0;
}

// Wait of the 64 lanes of wave 0 for the workgroups of expert e only (blocks e * parts .. e * parts +
// parts - 1, this one included) at `round`: arrival is the same flag store as in the grid barrier,
// and the wait polls just those flags, with the same bound and error word. The down phase reads
// nothing but its own expert's h rows, which only those workgroups write, so experts whose gate/up
// work is done go on streaming down weights while the grid's slowest experts finish theirs.
__device__ bool fz_expert_wait(const FusedArgs& a, unsigned round, int e) {
  const int lane = threadIdx.x & 63;
  const unsigned long long tag = (unsigned long long)a.ticket << 32;
  const unsigned long long want = tag | round;
  auto reached = [&](unsigned long long v) { return (v & 0xFFFFFFFF00000000ull) == tag && v >= want; };
  if (lane == 0) __hip_atomic_store(a.flags + blockIdx.x, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bool ok = true;
  for (uint32_t spins = 0;; ++spins) {
    const bool give_up =
        spins >= a.spin_limit || __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.ticket;
    if (__shfl(give_up ? 1 : 0, 0)) {
      ok = false;
      break;
    }
    bool mine = true;
    for (int b = lane; b < a.parts; b += 64)
      mine = mine && reached(__hip_atomic_load(a.flags + e * a.parts + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (__all(mine)) break;
    __builtin_amdgcn_s_sleep(1);
  }
  if (lane == 0 && !ok) {
    __hip_atomic_store(a.err, a.ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.status[0] = -1;
  }
  asm volatile("" ::: "memory");
  return __shfl(ok ? 1 : 0, 0) != 0;
}

// Full grid barrier for the whole workgroup: every wave's stores complete, wave 0 waits for the
// grid, the outcome is shared through LDS.
__device__ bool fz_barrier(const FusedArgs& a, unsigned round, int* s_flag) {
  stores_done();
  lds_barrier();
  if (threadIdx.x < 64) {
    const bool ok = fz_grid_wait(a, round);
    if (threadIdx.x == 0) *s_flag = ok ? 1 : 0;
  }
  lds_barrier();
  return *s_flag != 0;
}

// Staging of an m-block's activation rows (all of K) as exact f16 into LDS rows of RS bytes: rows
// n < mrows read activation row row_of(n), rows up to the token tiles read zeros. Item i = (32-K
// group q, row n), rows fastest so that the 8 lanes of an LDS write group hit 8 rows; the rows were
// written by other workgroups of this launch, so the loads are device-coherent. NT threads
// (the first NT of the workgroup) share the items, BATCH per thread at a time, each batch's loads
// all issued before the first is used.
template <int NT, int BATCH, class RowOf>
__device__ __forceinline__ void fz_stage(__amdgpu_buffer_rsrc_t c_rsrc, __amdgpu_buffer_rsrc_t s_rsrc, int K,
                                         int mrows, int ntiles, RowOf row_of, uint8_t* sB, int RS) {
  const int G = K >> 5, tid = threadIdx.x;
  const int items = kFzBMT * G;
  for (int i0 = 0; i0 < items; i0 += NT * BATCH) {
    u32x4 cv[BATCH];
    uint32_t sv[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int i = i0 + tid + j * NT;
      const int n = i % kFzBMT, q = i / kFzBMT;
      const bool live = n < mrows && q < G;
      const uint32_t ar = live ? (uint32_t)row_of(n) : 0u;
      cv[j] = __builtin_amdgcn_raw_buffer_load_b128(c_rsrc, live ? ar * (uint32_t)(K >> 1) + 16u * q : 0x80000000u, 0,
                                                    kCpolDevice);
      sv[j] = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, live ? ar * (uint32_t)G + q : 0x80000000u, 0, kCpolDevice);
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int i = i0 + tid + j * NT;
      const int n = i % kFzBMT, q = i / kFzBMT;
      if (n < ntiles * 16 && q < G) {
        const f16x2 s2 = scale_bcast_f16(sv[j]);
        u32x4 u4[4];
        act_group_kprime(cv[j], s2, u4);
#pragma unroll
        for (int h = 0; h < 4; ++h)
          *reinterpret_cast<u32x4*>(sB + n * RS + (4 * q + h) * 16) = u4[h];
      }
    }
  }
}

// The MFMAs of one 256-K super-step `gs` of weight fragment w against the staged rows; once the last
// word of w is decoded, w is reloaded through `reload` (a callable taking the fragment).
template <int RT, class Reload>
__device__ __forceinline__ void fz_step(const uint8_t* sB, int RS, int gs, int ntiles,
                                        WeightFrag<RT>& w, f32x4 (&acc)[RT][kFzTG], Reload reload) {
  const int lane = threadIdx.x & 63, nrow = lane & 15, qb = lane >> 4;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f16x8 A[RT];
    int idx[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const f16x2 sp = scale_pair_f16(w.sc[rt]);
      const f16x2 s2 = (t < 2) ? __builtin_shufflevector(sp, sp, 0, 0) : __builtin_shufflevector(sp, sp, 1, 1);
      A[rt] = weight_operand_tiled(frag_word(w.pk[rt], t), s2);
      idx[rt] = smfmac_index_of_codes(w.mk[rt], t);
    }
    if (t == 3) {
      slot_decoded<RT>(A, idx);
      reload(w);
    }
    const int c0 = 8 * (qb >> 1) + 2 * t + (qb & 1);
#pragma unroll
    for (int tt = 0; tt < kFzTG; ++tt) {
      if (tt < ntiles) {
        const uint8_t* bp = sB + (tt * 16 + nrow) * RS + (32 * gs + c0) * 16;
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(bp);
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(bp + 16 * 16);
        const f16x16 B = __builtin_bit_cast(f16x16, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt][tt] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(A[rt], B, acc[rt][tt], idx[rt], 0, 0);
      }
    }
  }
}

template <int RT>
__device__ __forceinline__ void fz_zero(f32x4 (&acc)[RT][kFzTG]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int tt = 0; tt < kFzTG; ++tt) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

__global__ __launch_bounds__(kFzThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_ffn_fused(FusedArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int H = a.H, I = a.I, k = a.k, E = a.E;
  const int P = a.T * k;
  const int RSmax = 2 * (H > I ? H : I) + 16;
  uint8_t* sB = smem;                                                    // [kFzBMT][RSmax] staging
  int* s_rows = reinterpret_cast<int*>(smem + kFzBMT * RSmax);           // [P]: pairs of expert e, in order
  __shared__ int s_wcnt[kFzWaves];
  __shared__ int s_sum[3];                                               // matches, smaller ids, dropped ids
  __shared__ float s_rw[kFzBMT];
  __shared__ int s_flag;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e = (int)blockIdx.x / a.parts, part = (int)blockIdx.x % a.parts;
  const int nthreads = (int)gridDim.x * kFzThreads;
  const int G13 = H >> 5;

  // per-phase GEMM descriptions (the shared epilogues and weight fragments take these)
  GemmParams gp{};
  gp.a_global = a.a13_global; gp.w_packed = a.w13; gp.w_global = a.w13_global; gp.E = E; gp.N = 2 * I; gp.K = H;
  gp.G = 2; gp.layout = 1; gp.h_codes = a.a2c; gp.h_scales = a.a2s; gp.h_global = a.a2_global;
  GemmParams dp{};
  dp.a_global = a.a2_global; dp.w_packed = a.w2; dp.w_global = a.w2_global; dp.E = E; dp.N = H; dp.K = I;
  dp.G = 1; dp.layout = 1; dp.out = a.D;

  // ---- the routing phase's loads go out first: router ids, the gate/up input globals, and the
  // token values of this thread's first quantization item
  int ep[kFzIdRounds];
#pragma unroll
  for (int j = 0; j < kFzIdRounds; ++j) {
    const int pidx = j * kFzThreads + tid;
    ep[j] = pidx < P ? a.ids[pidx] : -1;
  }
  const float gval = tid < E ? a.a13_global[tid] : 0.0f;
  const int it0 = (int)blockIdx.x * kFzThreads + tid;
  const bool item0 = it0 < P * G13;
  const int itc = item0 ? it0 : 0;                                        // an in-bounds item either way
  const int p0 = itc / G13;
  const int ex0 = item0 ? a.ids[p0] : -1;
  u32x4 xv0[4];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.x + (int64_t)(p0 / k) * H + (itc - p0 * G13) * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) xv0[i] = item0 ? src[i] : u32x4{0u, 0u, 0u, 0u};
  }
  // they return before the weight loads go out: issued together with the whole grid's weight
  // loads, they would wait behind those in the memory queues
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // ---- then the gate/up weight ring's first loads (they depend on nothing)
  const int gw = part * kFzWaves + wv;                                   // 32 gate/up columns per wave
  int wrow_g[4];
  const bool active_g = wave_rows<kEpiGateUp, 4>(2 * I, 0, gw, wrow_g);
  WeightPtrs<1, 4> wpg;
  wpg.init(gp, e, wrow_g, active_g, lane);
  const int nsg = H >> 8;
  WeightFrag<4> wg[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    wpg.load(d, wg[d], active_g && d < nsg);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- routing phase
  float* s_g = reinterpret_cast<float*>(sB);                             // staging area, free until then
  for (int i = tid; i < E; i += kFzThreads) s_g[i] = i == tid ? gval : a.a13_global[i];
  if (tid < 3) s_sum[tid] = 0;
  lds_barrier();
  {
    // NVFP4 codes of every pair's activation row (this workgroup's share of the (pair, 32-group)
    // items), the one-test snap encoding: bf16 inputs
    auto quantize_item = [&](int it, int p, int ex, const u32x4 (&xv)[4]) {
      if (ex < 0 || ex >= E) return;
      const int grp = it - p * G13;
      float v[32];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t b[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
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
      const float g = s_g[ex];
      const int sc = scale_code(amax, g);
      const float s = e4m3_value(sc);
      const Nvfp4Snap sn = nvfp4_snap(s, g, mb < 0x7F800000u);
      uint32_t w[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) w[h] = nvfp4_codes_snap<8>(v + 8 * h, s, g, sn);
      epi_store<kCpolDevice>(reinterpret_cast<u32x4*>(a.a13c), (int64_t)p * (H >> 5) + grp, u32x4{w[0], w[1], w[2], w[3]});
      epi_store<kCpolDevice>(a.a13s, (int64_t)p * G13 + grp, (uint8_t)sc);
    };
    if (item0) quantize_item(itc, p0, ex0, xv0);
    for (int it = it0 + nthreads; it < P * G13; it += nthreads) {   // larger batches
      const int p = it / G13;
      const u32x4* src = reinterpret_cast<const u32x4*>(a.x + (int64_t)(p / k) * H + (it - p * G13) * 32);
      u32x4 xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = src[i];
      quantize_item(it, p, a.ids[p], xv);
    }
    // rows of expert e: the pairs with id e in pair order; row base: pairs with a smaller valid id
    int base = 0, less = 0, bad = 0;
#pragma unroll
    for (int j = 0; j < kFzIdRounds; ++j) {
      const int pidx = j * kFzThreads + tid;
      const bool m = ep[j] == e;
      less += (ep[j] >= 0 && ep[j] < e) ? 1 : 0;
      bad += (pidx < P && (ep[j] < -1 || ep[j] >= E)) ? 1 : 0;
      const unsigned long long bal = __ballot(m);
      if (lane == 0) s_wcnt[wv] = __builtin_popcountll(bal);
      lds_barrier();
      int before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kFzWaves; ++w) {
        const int c = s_wcnt[w];
        before += w < wv ? c : 0;
        total += c;
      }
      if (m) s_rows[base + before + __builtin_popcountll(bal & ((1ull << lane) - 1ull))] = pidx;
      base += total;
      lds_barrier();
    }
    if (less) atomicAdd(&s_sum[1], less);
    if (bad) atomicAdd(&s_sum[2], bad);
    if (tid == 0) s_sum[0] = base;
    lds_barrier();
  }
  const int M = s_sum[0], row0 = s_sum[1];
  // routing outputs for the down phase, the combine and the caller: expert e's rows by its part 0
  if (part == 0) {
    for (int m = tid; m < M; m += kFzThreads) {
      const int p = s_rows[m];
      a.sorted[row0 + m] = p;
      epi_store<kCpolDevice>(a.inv, p, row0 + m);
    }
    if (tid == 0) {
      a.counts[e] = M;
      a.offsets[e] = row0;
      if (e == E - 1) a.offsets[E] = row0 + M;
    }
  }
  if (blockIdx.x == 0) {
    if (tid == 0) a.status[0] = s_sum[2];
#pragma unroll
    for (int j = 0; j < kFzIdRounds; ++j) {
      const int pidx = j * kFzThreads + tid;
      if (pidx < P && (ep[j] < 0 || ep[j] >= E)) epi_store<kCpolDevice>(a.inv, pidx, -1);
    }
  }
  bool ok = fz_barrier(a, 1, &s_flag);

  // ---- gate/up phase: h = silu(gate) * up of e's rows, NVFP4 with a2_global[e], sorted rows
  if (ok) {
    const EpiScalars es = epi_scalars<kEpiGateUp>(gp, e);
    const int RS = 2 * H + 16;
    const __amdgpu_buffer_rsrc_t c_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(a.a13c, (short)0, (int)((int64_t)P * (H >> 1)), kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t s_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(a.a13s, (short)0, (int)((int64_t)P * (H >> 5)), kBufferRsrcWord3);
    for (int m0 = 0; m0 < M; m0 += kFzBMT) {
      const int mrows = M - m0 < kFzBMT ? M - m0 : kFzBMT;
      const int ntiles = (mrows + 15) >> 4;
      if (m0 > 0) {                               // a further m-block streams the weights again
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          wpg.load(d, wg[d], active_g && d < nsg);
          __builtin_amdgcn_sched_barrier(0);
        }
        lds_barrier();                            // the previous m-block's readers are done
      }
      fz_stage<kFzThreads, kFzStageItems>(c_rsrc, s_rsrc, H, mrows, ntiles, [&](int n) { return s_rows[m0 + n]; },
                                          sB, RS);
      lds_barrier();
      f32x4 acc[4][kFzTG];
      fz_zero<4>(acc);
      int gs = 0;
      for (; gs + 2 <= nsg; gs += 2) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const int rl = gs + 2 + d;
          fz_step<4>(sB, RS, gs + d, ntiles, wg[d], acc,
                     [&](WeightFrag<4>& w) { wpg.load(rl, w, active_g && rl < nsg); });
        }
      }
      if (gs < nsg) fz_step<4>(sB, RS, gs, ntiles, wg[0], acc, [&](WeightFrag<4>&) {});
      if (active_g)
        gemm_epilogue<kEpiGateUp, kFzTG, 4, kCpolDevice>(gp, es, acc, row0, m0, mrows, 0, gw, wrow_g, s_rw, lane);
    }
  }

  // ---- down phase work: waves kDs..11 take row-pair groups gb + (wv - kDs), + kDw, ... of this
  // part's share [gb, ge) of the H / 32 groups of 2 row-tiles, records running group by group
  // (256 K each) through a ring of kFzDownDepth slots. Waves 0..kDs-1 stage the m-block's inputs
  // (their loads queue behind no weights), and wave 0 waits for the grid.
  constexpr int kDs = 4, kDw = kFzWaves - kDs;
  const int ngroups = H >> 5;
  const int gb = (int)(((int64_t)part * ngroups) / a.parts), ge = (int)(((int64_t)(part + 1) * ngroups) / a.parts);
  const int dw = wv - kDs;
  const int my_groups = (wv >= kDs && ge - gb > dw) ? (ge - gb - dw + kDw - 1) / kDw : 0;
  const int nsd = I >> 8;
  const int nrec = my_groups * nsd;
  auto down_rows = [&](int gi, int* wrow) {       // gi: the wave's group index
    const int r0 = (gb + dw + gi * kDw) * 32;
    wrow[0] = r0;
    wrow[1] = r0 + 16;
  };
  WeightFrag<kFzDownRT> wd[kFzDownDepth];
  auto load_rec = [&](int rec, WeightFrag<kFzDownRT>& w) {
    const bool live = rec < nrec;
    int wrow[2];
    down_rows(live ? rec / nsd : 0, wrow);
    WeightPtrs<1, kFzDownRT> wp;
    wp.init(dp, e, wrow, live, lane);
    wp.load(live ? rec % nsd : 0, w, live);
  };
  auto down_prologue = [&]() {
    if (wv >= kDs) {
#pragma unroll
      for (int d = 0; d < kFzDownDepth; ++d) {
        load_rec(d, wd[d]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  const EpiScalars esd = epi_scalars<kEpiDown>(dp, e);
  const int RSd = 2 * I + 16;
  const __amdgpu_buffer_rsrc_t c2_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(a.a2c, (short)0, (int)((int64_t)P * (I >> 1)), kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t s2_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(a.a2s, (short)0, (int)((int64_t)P * (I >> 5)), kBufferRsrcWord3);
  // waves 0..kDs-1: the m-block's router weights and h rows (written by the gate/up phase of e's parts)
  auto down_stage = [&](int m0, int mrows, int ntiles) {
    if (wv < kDs) {
      if (tid < kFzBMT) s_rw[tid] = tid < mrows ? a.topk_weights[s_rows[m0 + tid]] : 0.0f;
      fz_stage<kDs * 64, 4>(c2_rsrc, s2_rsrc, I, mrows, ntiles, [&](int n) { return row0 + m0 + n; }, sB, RSd);
    }
  };
  if (ok) {
    stores_done();                                // every wave's gate/up stores are complete
    lds_barrier();
    down_prologue();                              // the down weights stream from now on
    if (wv == 0) {
      const bool g = fz_expert_wait(a, 2, e);
      if (lane == 0) s_flag = g ? 1 : 0;
    }
    lds_barrier();
    ok = s_flag != 0;
    if (ok && M > 0) {
      const int mrows = M < kFzBMT ? M : kFzBMT;
      down_stage(0, mrows, (mrows + 15) >> 4);
    }
    lds_barrier();
  }

  // ---- down phase: D rows (sorted order) = a2_global[e] w2_global[e] router weight * h w2^T
  if (ok) {
    for (int m0 = 0; m0 < M; m0 += kFzBMT) {
      const int mrows = M - m0 < kFzBMT ? M - m0 : kFzBMT;
      const int ntiles = (mrows + 15) >> 4;
      if (m0 > 0) {                               // a further m-block: restage, stream the weights again
        lds_barrier();
        down_prologue();
        down_stage(m0, mrows, ntiles);
        lds_barrier();
      }
      f32x4 acc[kFzDownRT][kFzTG];
      fz_zero<kFzDownRT>(acc);
      // records rec = r0 + d on ring slot d; a group's epilogue follows its last super-step
      for (int r0 = 0; r0 < nrec; r0 += kFzDownDepth) {
#pragma unroll
        for (int d = 0; d < kFzDownDepth; ++d) {
          const int rec = r0 + d;
          if (rec < nrec) {
            const int rl = rec + kFzDownDepth;
            fz_step<kFzDownRT>(sB, RSd, rec % nsd, ntiles, wd[d], acc,
                               [&](WeightFrag<kFzDownRT>& w) { load_rec(rl, w); });
            if (rec % nsd == nsd - 1) {
              int wrow[2];
              down_rows(rec / nsd, wrow);
              gemm_epilogue<kEpiDown, kFzTG, kFzDownRT, kCpolDevice>(dp, esd, acc, row0, m0, mrows, 0, 0, wrow, s_rw,
                                                                     lane);
              fz_zero<kFzDownRT>(acc);
            }
          }
        }
      }
    }
  }
  ok = ok && fz_barrier(a, 3, &s_flag);

  // ---- combine: out[t] = sum over j of D[inv[t k + j]], j = 0 .. k-1
  if (ok) {
    const int H4 = H >> 2;
    const __amdgpu_buffer_rsrc_t inv_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.inv, (short)0, P * 4, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t d_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(a.D, (short)0, (int)((int64_t)P * H * 4), kBufferRsrcWord3);
    for (int it = (int)blockIdx.x * kFzThreads + tid; it < a.T * H4; it += nthreads) {
      const int t = it / H4, c = (it - t * H4) * 4;
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < k; j0 += 8) {         // 8 row indices, then their 8 rows, at a time
        int r[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          r[j] = j0 + j < k ? (int)__builtin_amdgcn_raw_buffer_load_b32(inv_rsrc, (uint32_t)(t * k + j0 + j) * 4u, 0,
                                                                        kCpolDevice)
                            : -1;
        f32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               d_rsrc, r[j] >= 0 ? (uint32_t)((r[j] * H + c) * 4) : 0x80000000u, 0,
                                               kCpolDevice));
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (r[j] >= 0) s += v[j];
      }
      *reinterpret_cast<f32x4*>(a.out + (int64_t)t * H + c) = s;
    }
  }
}

int fused_parts(int I) { return (I / 32 + kFzWaves - 1) / kFzWaves; }

bool fused_applicable(int64_t T, int H, int I, int k, int E) {
  if (H > kFzMaxK || I > kFzMaxK || T * k > kFzMaxPairs || T * k < 1) return false;
  const size_t lds = fused_lds_bytes(H, I, (int)(T * k));
  if (lds > kMaxLdsBytes - 1024) return false;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  static std::atomic<size_t> granted{0};   // always the same (largest) size, so racing first calls agree
  if (lds > granted.load(std::memory_order_relaxed)) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ffn_fused),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)fused_lds_bytes(kFzMaxK, kFzMaxK, kFzMaxPairs));
    if (e != hipSuccess) return false;          // the separate launches serve the call instead
    granted.store(fused_lds_bytes(kFzMaxK, kFzMaxK, kFzMaxPairs), std::memory_order_relaxed);
  }
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&k_ffn_fused), kFzThreads,
                                                   lds) != hipSuccess)
    return false;
  const int64_t grid = (int64_t)E * fused_parts(I);
  return grid <= (int64_t)per_cu * cus && grid <= kFzMaxGrid;
}

hipError_t launch_ffn_fused(const FusedLaunch& f, hipStream_t stream, unsigned* ticket_out) {
  // launch tickets: odd (so never zero), distinct per launch of this process, seeded by the process id
  static std::atomic<unsigned> next_ticket{(unsigned)(0x9E3779B9u * (unsigned)getpid()) | 1u};
  const unsigned ticket = next_ticket.fetch_add(2u, std::memory_order_relaxed);
  FusedArgs a{};
  a.x = f.x; a.ids = f.ids; a.topk_weights = f.topk_weights; a.a13_global = f.a13_global; a.a2_global = f.a2_global;
  a.w13 = f.w13; a.w13_global = f.w13_global; a.w2 = f.w2; a.w2_global = f.w2_global;
  a.T = (int)f.T; a.H = f.H; a.I = f.I; a.k = f.k; a.E = f.E; a.parts = fused_parts(f.I);
  a.counts = f.counts; a.offsets = f.offsets; a.sorted = f.sorted; a.inv = f.inv; a.status = f.status;
  a.a13c = f.a13c; a.a13s = f.a13s; a.a2c = f.a2c; a.a2s = f.a2s; a.D = f.D; a.out = f.out;
  a.release = reinterpret_cast<unsigned long long*>(f.sync);
  a.err = reinterpret_cast<unsigned*>(f.sync + kFusedErrOffset);
  a.flags = reinterpret_cast<unsigned long long*>(f.sync + 64);
  a.ticket = ticket;
  a.spin_limit = f.spin_limit >= 0 ? (uint32_t)f.spin_limit : kFzSpinLimit;
  *ticket_out = ticket;
  // A plain launch: the workgroups are all resident at once because each needs most of a CU's LDS
  // (at most one per CU) and the grid is no larger than the CU count times the occupancy the
  // runtime reports (fused_applicable). A cooperative launch, which would also check this, cost
  // about 19 us more per call on MI355X. Should other work hold CUs, the barrier waits end with
  // status -1 instead of hanging.
  launch_kernel(k_ffn_fused, dim3((unsigned)(a.E * a.parts)), dim3(kFzThreads), fused_lds_bytes(a.H, a.I, a.T * a.k), stream, a);
  return hipGetLastError();
}

}  // namespace moesq

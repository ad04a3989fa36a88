// Grouped paired-4:8 sparse NVFP4 GEMM on CDNA4 sparse MFMA (v_smfmac_f32_16x16x64_f16), gfx950.
//
// For each expert e and each of its rows r (a token routed to e): y[r, n] = sum_K xhat[r,K] w_e[n,K],
// with xhat, w the NVFP4 values (model card "Qwen3.5-397B-A17B-P48NVFP4-MoESQ", "Compression
// details"; the weights in pair-bitmask storage, "Sparse storage layout").
//
// Mapping onto the sparse MFMA. The weight is the structured-sparse operand A (16 weight rows x 64 K,
// stored as 16 x 32 kept values + a 2-bit position per kept value); the activations are the dense
// operand B (64 K x 16 tokens). In the K' order of moesq_device.h every 4-group holds exactly 2
// kept values, so the kept bytes of the pair-bitmask storage ARE the compressed operand (low nibbles
// for the even groups, high nibbles for the odd groups) and a chunk's mask nibble gives the index of
// both its groups (tiled weights carry that index code in place of the nibble).
// Dequantization is exact: e2m1 * e4m3 has <= 6 significant bits, so it is exact in f16, products
// of two such values are exact in fp32 and accumulation is in fp32. Global scales are applied in the
// fp32 epilogue.
//
// Lane data per 256-K super-step: lane (row = lane % 16, q = lane / 16) of a row-tile holds the 64
// contiguous K [64 q, 64 q + 64) of its weight row (16 B kept bytes, 4 B masks or index codes, 2 B
// scales; one load each), and smfmac t (t = 0..3) uses chunks 2t, 2t+1 of it. The sparse operand's lane q covers the
// MFMA's 8-K chunk positions {c0(q), c0(q) + 2} with c0 = 0, 4, 1, 5 for q = 0..3, so B lane qb must
// hold the local chunks 8*(qb/2) + 2t + (qb%2) and that + 16.
//
// Kernels:
//   * k_gemm_decode (small batches, any K): a workgroup owns one m-block (<= 32 rows of one expert)
//     and one n-block of weight rows; its activations are staged in LDS as exact f16 in the B-operand
//     order, 512 K at a time. Weights stream from HBM straight into registers, a few super-steps ahead.
//   * k_gemm_decode_nloop (small batches, K <= 1024, not gate/up): the whole K staged once; a
//     workgroup walks several n-blocks with its weight ring running across their boundaries.
//   * k_gemm_decode_stream (small batches, gate/up, tiled weights, K <= 2048): the whole K staged once
//     for 12 waves that each stream 32 intermediate columns.
//   * k_gemm_prefill (large batches): a workgroup owns 128 rows x 64 NWP weight rows (512 on tiled
//     weights); per 256-K step it dequantizes the activations into LDS as f16 and each wave reuses
//     every decoded weight fragment over up to 8 token tiles.
#include <atomic>

#include "gemm_common.h"

namespace moesq {

constexpr int kGemmThreads = 256;

// ---------------------------------------------------------------------------------------------
// Decode kernel
// ---------------------------------------------------------------------------------------------
constexpr int kDecTG = 2;                       // token tiles per m-block
constexpr int kDecBMT = kDecTG * 16;            // rows per m-block
constexpr int kDecTPR = kGemmThreads / kDecBMT; // staging threads per row
constexpr uint32_t kOutOfRange = 0x80000000u;   // a buffer offset past num_records: the load reads zero

// Staging geometry for a weight ring of DEPTH slots: one staged chunk = DEPTH 256-K super-steps.
template <int DEPTH>
struct DecGeom {
  static constexpr int KC = DEPTH * 256;                 // K staged in LDS at a time
  static constexpr int RS = KC * 2 + 16;                 // LDS bytes per token row (f16, +16 B skew)
  static constexpr int IPT = KC / 32 / kDecTPR;          // consecutive 32-K groups per staging thread
  static_assert(KC / 32 % kDecTPR == 0, "whole staging groups per thread");
  static constexpr size_t lds = (size_t)kDecBMT * RS + 512;
};

// Ring depth of a decode variant: gate/up waves (4 row-tiles) hold two weight super-steps in
// registers, the others (2 row-tiles) three.
__host__ __device__ constexpr int dec_depth(int rt) { return rt >= 4 ? 2 : 3; }

// Activation codes of one staged chunk, held in registers from one chunk ahead.
template <int IPT>
struct ActChunk {
  u32x4 v[IPT];
  uint32_t s[IPT];
};

// One workgroup per (expert, n-block): the expert comes straight from the block index. Experts with
// more than kDecBMT rows take further passes over the same (cache-resident) weights.
//
// Every global load in the K loop is a prefetch: weights stream through a register ring of DEPTH
// slots, each slot reloaded (DEPTH super-steps ahead) as soon as its last fragment word is decoded,
// and the activation codes of the next chunk are loaded into registers while the current one is
// used. vmcnt retires loads in order, so a synchronous load here would also wait for every weight
// load in flight; with only prefetches, and every load issued on every path, each wait counts
// exactly the loads issued after the data it needs.
template <int EPI, int LAYOUT, int RT>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_gemm_decode(GemmParams p) {
  constexpr int TG = kDecTG, BMT = kDecBMT, DEPTH = dec_depth(RT);
  using Geo = DecGeom<DEPTH>;
  constexpr int RS = Geo::RS, KC = Geo::KC, IPT = Geo::IPT;
  extern __shared__ __align__(16) uint8_t smem[];
  const int K = p.K;
  uint8_t* sB = smem;                                             // [BMT][RS] f16
  uint16_t* lut_idx = reinterpret_cast<uint16_t*>(smem + BMT * RS);   // [256]
  __shared__ int s_arow[BMT];                                     // activation row of each m-block row
  __shared__ float s_rw[BMT];                                     // router weight of each row (down)

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e = blockIdx.x, nb = blockIdx.y;
  const int row0 = p.offsets[e];
  const int M = p.offsets[e + 1] - row0;
  if (M <= 0) return;
  const EpiScalars es = epi_scalars<EPI>(p, e);
  if (LAYOUT == 0) lut_idx[tid] = (uint16_t)smfmac_index_of_mask_byte((uint32_t)tid);

  int wrow[RT];
  const bool active = wave_rows<EPI, RT>(p.N, nb, wv, wrow);
  WeightPtrs<LAYOUT, RT> wp;
  wp.init(p, e, wrow, active, lane);
  const int nsteps = K >> 8;
  const int nrow = lane & 15, qb = lane >> 4;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.a_codes), (short)0, (int)(p.rows * (K >> 1)), kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.a_scales), (short)0, (int)(p.rows * (K >> 5)), kBufferRsrcWord3);
  // staging map: thread -> row sn, 32-K groups sq0 .. sq0 + IPT - 1 of each chunk. Consecutive lanes
  // take consecutive rows, so each LDS write of 8 lanes hits 8 rows at one slot: with the 16 B row
  // skew that is 8 different bank groups.
  const int sn = tid % kDecBMT, sq0 = (tid / kDecBMT) * IPT;

  for (int m0 = 0; m0 < M; m0 += BMT) {
    const int mrows = M - m0 < BMT ? M - m0 : BMT;
    const int ntiles = (mrows + 15) >> 4;
    // every thread is past the previous m-block's last staging barrier, so s_arow is free
    __syncthreads();
    if (tid < BMT) {
      const int r = row0 + m0 + tid;
      s_arow[tid] = tid < mrows ? (p.a_rows ? p.a_rows[r] : r) : 0;
      if (EPI == kEpiDown) s_rw[tid] = tid < mrows ? row_weight(p, r) : 0.0f;
    }
    __syncthreads();
    // registers of the activation chunk [k0, k0 + kc): rows past the m-block and groups past the
    // chunk get an out-of-range offset and read zero (no branch, no zero fill)
    const bool srow_live = sn < mrows;
    const uint32_t ar = (uint32_t)s_arow[srow_live ? sn : 0];
    auto prefetch = [&](int k0, int kc, ActChunk<IPT>& ac) {
      const int quads = kc >> 5;
      const uint32_t cbase = ar * (uint32_t)(K >> 1) + (uint32_t)((k0 >> 1) + sq0 * 16);
      const uint32_t sbase = ar * (uint32_t)(K >> 5) + (uint32_t)((k0 >> 5) + sq0);
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        const bool live = srow_live && sq0 + j < quads;
        ac.v[j] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, live ? cbase + 16u * j : kOutOfRange, 0, 0);
        ac.s[j] = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, live ? sbase + j : kOutOfRange, 0, 0);
      }
    };
    // exact f16 values of the chunk into LDS in B-operand order (rows past the m-block as zeros,
    // groups past the chunk into positions no step reads)
    auto commit = [&](const ActChunk<IPT>& ac) {
      __syncthreads();
      if (sn < ntiles * 16) {
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
          const f16x2 s2 = scale_bcast_f16(ac.s[j]);
          u32x4 u4[4];
          act_group_kprime(ac.v[j], s2, u4);
#pragma unroll
          for (int h = 0; h < 4; ++h)                               // LDS unit 4 (sq0 + j) + h
            *reinterpret_cast<u32x4*>(sB + sn * RS + (4 * (sq0 + j) + h) * 16) = u4[h];
        }
      }
      __syncthreads();
    };
    f32x4 acc[RT][TG];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tt = 0; tt < TG; ++tt) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // MFMAs of one super-step (position ssl of its chunk) on weight fragment w; once the last word
    // of w is decoded, w is reloaded with super-step `reload` (< 0: none)
    auto step = [&](int ssl, WeightFrag<RT>& w, int reload) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f16x8 A[RT];
        int idx[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const f16x2 sp = scale_pair_f16(w.sc[rt]);
          const f16x2 s2 = (t < 2) ? __builtin_shufflevector(sp, sp, 0, 0) : __builtin_shufflevector(sp, sp, 1, 1);
          A[rt] = weight_operand_of<LAYOUT>(frag_word(w.pk[rt], t), s2);
          idx[rt] = sparse_index<LAYOUT>(w.mk[rt], t, lut_idx);
        }
        if (t == 3 && reload >= 0) {
          slot_decoded<RT>(A, idx);
          wp.load(reload, w, active && reload < nsteps);
        }
        const int c0 = 8 * (qb >> 1) + 2 * t + (qb & 1);
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
          if (tt < ntiles) {
            const uint8_t* bp = sB + (tt * 16 + nrow) * RS + (32 * ssl + c0) * 16;
            const u32x4 b0 = *reinterpret_cast<const u32x4*>(bp);
            const u32x4 b1 = *reinterpret_cast<const u32x4*>(bp + 16 * 16);
            const f16x16 B = __builtin_bit_cast(f16x16, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              acc[rt][tt] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(A[rt], B, acc[rt][tt], idx[rt], 0, 0);
          }
        }
      }
    };
    ActChunk<IPT> ac;
    prefetch(0, K < KC ? K : KC, ac);
    WeightFrag<RT> w[DEPTH];
    // slot by slot, in order: the loop's waits assume slot d's loads are older than slot d + 1's
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      wp.load(d, w[d], active && d < nsteps);
      __builtin_amdgcn_sched_barrier(0);
    }
    // One chunk per iteration, its DEPTH super-steps on the DEPTH ring slots.
    int gs = 0;
    for (; gs + DEPTH <= nsteps; gs += DEPTH) {
      const int k1 = (gs + DEPTH) * 256;
      commit(ac);
      prefetch(k1, K - k1 < KC ? K - k1 : KC, ac);
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) step(d, w[d], gs + DEPTH + d);
    }
    if (gs < nsteps) {                                            // a last, shorter chunk
      commit(ac);
#pragma unroll
      for (int d = 0; d < DEPTH - 1; ++d)
        if (gs + d < nsteps) step(d, w[d], -1);
    }
    if (active) gemm_epilogue<EPI, TG, RT>(p, es, acc, row0, m0, mrows, nb, wv, wrow, s_rw, lane);
  }
}

// ---------------------------------------------------------------------------------------------
// Decode kernel, one staged chunk: K == DEPTH * 256
// ---------------------------------------------------------------------------------------------
// A workgroup covers a range of n-blocks of one expert. The m-block's activations (all of K) are
// staged once and shared by every n-block, instead of once per n-block workgroup, and the weight
// ring runs on across n-block boundaries: while an n-block computes, the first super-steps of the
// next one are in flight, so its epilogue also runs under outstanding loads. Loads are issued on
// every path (past the last n-block as zero-reading out-of-range loads).
template <int EPI, int LAYOUT, int RT, int DEPTH>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_gemm_decode_nloop(
    GemmParams p, int nblocks) {
  constexpr int TG = kDecTG, BMT = kDecBMT;
  using Geo = DecGeom<DEPTH>;
  constexpr int RS = Geo::RS, IPT = Geo::IPT;
  extern __shared__ __align__(16) uint8_t smem[];
  const int K = p.K;                                              // == Geo::KC
  uint8_t* sB = smem;                                             // [BMT][RS] f16
  uint16_t* lut_idx = reinterpret_cast<uint16_t*>(smem + BMT * RS);   // [256]
  __shared__ int s_arow[BMT];
  __shared__ float s_rw[BMT];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e = blockIdx.x;
  const int nb0 = (int)(((int64_t)blockIdx.y * nblocks) / gridDim.y);
  const int nb1 = (int)(((int64_t)(blockIdx.y + 1) * nblocks) / gridDim.y);
  const int row0 = p.offsets[e];
  const int M = p.offsets[e + 1] - row0;
  if (M <= 0 || nb0 >= nb1) return;
  const EpiScalars es = epi_scalars<EPI>(p, e);
  if (LAYOUT == 0) lut_idx[tid] = (uint16_t)smfmac_index_of_mask_byte((uint32_t)tid);
  const int nrow = lane & 15, qb = lane >> 4;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.a_codes), (short)0, (int)(p.rows * (K >> 1)), kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.a_scales), (short)0, (int)(p.rows * (K >> 5)), kBufferRsrcWord3);
  const int sn = tid % kDecBMT, sq0 = (tid / kDecBMT) * IPT;      // staging map (as k_gemm_decode)

  for (int m0 = 0; m0 < M; m0 += BMT) {
    const int mrows = M - m0 < BMT ? M - m0 : BMT;
    const int ntiles = (mrows + 15) >> 4;
    __syncthreads();
    if (tid < BMT) {
      const int r = row0 + m0 + tid;
      s_arow[tid] = tid < mrows ? (p.a_rows ? p.a_rows[r] : r) : 0;
      if (EPI == kEpiDown) s_rw[tid] = tid < mrows ? row_weight(p, r) : 0.0f;
    }
    __syncthreads();
    ActChunk<IPT> ac;
    {
      const bool srow_live = sn < mrows;
      const uint32_t ar = (uint32_t)s_arow[srow_live ? sn : 0];
      const uint32_t cbase = ar * (uint32_t)(K >> 1) + (uint32_t)(sq0 * 16);
      const uint32_t sbase = ar * (uint32_t)(K >> 5) + (uint32_t)sq0;
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        ac.v[j] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, srow_live ? cbase + 16u * j : kOutOfRange, 0, 0);
        ac.s[j] = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, srow_live ? sbase + j : kOutOfRange, 0, 0);
      }
    }
    int wrow[RT];
    bool active = wave_rows<EPI, RT>(p.N, nb0, wv, wrow);
    WeightPtrs<LAYOUT, RT> wp;
    wp.init(p, e, wrow, active, lane);
    WeightFrag<RT> w[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      wp.load(d, w[d], active);
      __builtin_amdgcn_sched_barrier(0);
    }
    // stage the whole K once for all n-blocks of this m-block
    __syncthreads();
    if (sn < ntiles * 16) {
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        const f16x2 s2 = scale_bcast_f16(ac.s[j]);
        u32x4 u4[4];
        act_group_kprime(ac.v[j], s2, u4);
#pragma unroll
        for (int h = 0; h < 4; ++h)
          *reinterpret_cast<u32x4*>(sB + sn * RS + (4 * (sq0 + j) + h) * 16) = u4[h];
      }
    }
    __syncthreads();
    for (int nb = nb0; nb < nb1; ++nb) {
      int wrow_n[RT];
      const bool next = nb + 1 < nb1;
      const bool active_n = wave_rows<EPI, RT>(p.N, next ? nb + 1 : nb, wv, wrow_n) && next;
      WeightPtrs<LAYOUT, RT> wpn;
      wpn.init(p, e, wrow_n, active_n, lane);
      f32x4 acc[RT][TG];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          f16x8 A[RT];
          int idx[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const f16x2 sp = scale_pair_f16(w[d].sc[rt]);
            const f16x2 s2 = (t < 2) ? __builtin_shufflevector(sp, sp, 0, 0) : __builtin_shufflevector(sp, sp, 1, 1);
            A[rt] = weight_operand_of<LAYOUT>(frag_word(w[d].pk[rt], t), s2);
            idx[rt] = sparse_index<LAYOUT>(w[d].mk[rt], t, lut_idx);
          }
          if (t == 3) {                                             // the next n-block's step d
            slot_decoded<RT>(A, idx);
            wpn.load(d, w[d], active_n);
          }
          const int c0 = 8 * (qb >> 1) + 2 * t + (qb & 1);
#pragma unroll
          for (int tt = 0; tt < TG; ++tt) {
            if (tt < ntiles) {
              const uint8_t* bp = sB + (tt * 16 + nrow) * RS + (32 * d + c0) * 16;
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
      if (active) gemm_epilogue<EPI, TG, RT>(p, es, acc, row0, m0, mrows, nb, wv, wrow, s_rw, lane);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) wrow[rt] = wrow_n[rt];
      active = active_n;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Decode kernel, whole K staged (tiled weights, K <= kStreamMaxK)
// ---------------------------------------------------------------------------------------------
// One workgroup of kStreamWaves waves per (expert, column group): at the decode shapes the grid is
// one workgroup per CU, and the m-block's activations, all of K as exact f16 (32 rows x 2K bytes),
// are staged in LDS once and read by every wave. The weight ring's first loads go out before the
// staging, and the K loop has no barrier: each wave streams its own row-tiles through its register
// ring and runs its epilogue as soon as it is done, so the waves of a CU keep the loads in flight
// that one short-lived workgroup per n-block could not.
constexpr int kStreamWaves = 12;
constexpr int kStreamThreads = kStreamWaves * 64;
constexpr int kStreamMaxK = 2048;
constexpr int kStreamItems = (kDecBMT * (kStreamMaxK / 32) + kStreamThreads - 1) / kStreamThreads;  // staging items per thread

__host__ __device__ constexpr size_t stream_lds_bytes(int K) { return (size_t)kDecBMT * (K * 2 + 16); }

template <int EPI, int RT, int DEPTH>
__global__ __launch_bounds__(kStreamThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_gemm_decode_stream(GemmParams p) {
  constexpr int TG = kDecTG, BMT = kDecBMT;
  extern __shared__ __align__(16) uint8_t smem[];
  const int K = p.K, RS = K * 2 + 16;
  uint8_t* sB = smem;                                                     // [BMT][RS] f16
  __shared__ int s_arow[BMT];
  __shared__ float s_rw[BMT];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e = blockIdx.x;
  const int gw = (int)blockIdx.y * kStreamWaves + wv;                    // wave index in the expert
  const int row0 = p.offsets[e];
  const int M = p.offsets[e + 1] - row0;
  if (M <= 0) return;
  const EpiScalars es = epi_scalars<EPI>(p, e);
  int wrow[RT];
  const bool active = wave_rows<EPI, RT>(p.N, 0, gw, wrow);
  WeightPtrs<1, RT> wp;
  wp.init(p, e, wrow, active, lane);
  const int nsteps = K >> 8, G = K >> 5;
  const int nrow = lane & 15, qb = lane >> 4;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.a_codes), (short)0, (int)(p.rows * (K >> 1)), kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.a_scales), (short)0, (int)(p.rows * (K >> 5)), kBufferRsrcWord3);

  for (int m0 = 0; m0 < M; m0 += BMT) {
    const int mrows = M - m0 < BMT ? M - m0 : BMT;
    const int ntiles = (mrows + 15) >> 4;
    // the m-block's weight stream starts before its activations are staged
    WeightFrag<RT> w[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      wp.load(d, w[d], active && d < nsteps);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();                        // every wave is done with the previous m-block's LDS
    if (tid < BMT) {
      const int r = row0 + m0 + tid;
      s_arow[tid] = tid < mrows ? (p.a_rows ? p.a_rows[r] : r) : 0;
      if (EPI == kEpiDown) s_rw[tid] = tid < mrows ? row_weight(p, r) : 0.0f;
    }
    __syncthreads();
    // staging: item i = (32-K group q, row n), rows fastest so that the 8 lanes of an LDS write group
    // hit 8 rows; every load is issued before the first is used, rows past the m-block read zeros
    {
      u32x4 cv[kStreamItems];
      uint32_t sv[kStreamItems];
#pragma unroll
      for (int j = 0; j < kStreamItems; ++j) {
        const int i = tid + j * kStreamThreads;
        const int n = i % BMT, q = i / BMT;
        const bool live = n < mrows && q < G;
        const uint32_t ar = (uint32_t)s_arow[n];
        cv[j] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, live ? ar * (uint32_t)(K >> 1) + 16u * q : kOutOfRange, 0, 0);
        sv[j] = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, live ? ar * (uint32_t)G + q : kOutOfRange, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < kStreamItems; ++j) {
        const int i = tid + j * kStreamThreads;
        const int n = i % BMT, q = i / BMT;
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
    __syncthreads();
    f32x4 acc[RT][TG];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tt = 0; tt < TG; ++tt) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // super-step gs on weight fragment w; once its last word is decoded, w is reloaded with
    // super-step `reload` (< 0: none)
    auto step = [&](int gs, WeightFrag<RT>& w, int reload) {
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
        if (t == 3 && reload >= 0) {
          slot_decoded<RT>(A, idx);
          wp.load(reload, w, active && reload < nsteps);
        }
        const int c0 = 8 * (qb >> 1) + 2 * t + (qb & 1);
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
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
    };
    int gs = 0;
    for (; gs + DEPTH <= nsteps; gs += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) step(gs + d, w[d], gs + DEPTH + d);
    }
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d)
      if (gs + d < nsteps) step(gs + d, w[d], -1);
    if (active) gemm_epilogue<EPI, TG, RT>(p, es, acc, row0, m0, mrows, 0, gw, wrow, s_rw, lane);
  }
}

// ---------------------------------------------------------------------------------------------
// Prefill kernel
// ---------------------------------------------------------------------------------------------
constexpr int kPreTG = 8;
constexpr int kPreBMT = kPreTG * 16;
constexpr int kPreRowBytes = 256 * 2;          // one 256-K step of a token row in LDS (f16): 32 units of 16 B
constexpr int kPreLdsB = kPreBMT * kPreRowBytes;

// LDS byte offset of 16-byte unit u (0..31) of token row r in one staged step. The unit index is
// XOR-swizzled with the row's low five bits, so that both access patterns are free of LDS bank
// conflicts (measured on gfx950 with the hardware's conflict counter): the staging writes, where
// consecutive lanes write one unit of consecutive rows, and the MFMA operand reads, where the 16
// lanes of a quarter-wave read one unit of 16 consecutive rows and the quarters read units 0, 1, 8,
// 9 (+ 2t) of them. A plain row stride of 512 + 16 bytes costs about 4 extra cycles per read.
__device__ __forceinline__ uint32_t pre_lds_off(int row, int unit) {
  return (uint32_t)row * kPreRowBytes + ((uint32_t)(unit ^ (row & 31)) << 4);
}

// Work placement: consecutive workgroup ids go to the 8 XCDs in turn, and each XCD has its own L2.
// Workgroup L therefore takes item (L % 8) * per + L / 8 of the (m-block, n-block) work list, m-block
// major, where per = ceil(items / 8) for the live item count: each XCD walks a contiguous, balanced
// range of the list, so the n-blocks of one m-block (same activations) and consecutive m-blocks of
// one expert (same weights) run side by side on one L2 instead of being fetched by every XCD.
constexpr int kXcds = 8;
// The prefill items (m-block major) are dealt to the XCDs in contiguous shares of equal count, so
// that the items running at once on one XCD share activation rows and experts' weights in its L2,
// except the last 1 / kPrefillPoolDiv of them: workgroups past their XCD's share claim those from a
// counter, so XCDs whose shares cost less (routing skew makes items of 1 and of 8 token tiles) take
// more of them. On the 384-expert layer equal-count shares alone left the slowest XCD about 6 %
// behind the mean.
constexpr int kPrefillPoolDiv = 16;

// Waves per prefill workgroup (each 4 row-tiles of 16 weight rows) and the n-blocks they make. Both
// FFN GEMMs on tiled weights run 8 waves (512 weight rows, one workgroup per CU): each staged
// activation step then feeds twice the weight rows, which took the gate/up GEMM from 290 to 283 us on
// the 128-expert layer and from 513 to 486 us on the 512-expert layer. The plain store epilogue and
// the pair-bitmask layout keep 4 waves (two workgroups per CU): their larger register sets would spill
// at 8.
template <int EPI, int LAYOUT>
__host__ __device__ constexpr int prefill_waves() { return LAYOUT == 1 && EPI != kEpiStore ? 8 : 4; }

template <int EPI, int NWP>
__host__ __device__ constexpr int prefill_nblocks(int N) {
  return EPI == kEpiGateUp ? ((N >> 1) + 32 * NWP - 1) / (32 * NWP) : (N + 64 * NWP - 1) / (64 * NWP);
}

// What a prefill workgroup knows about its item once it has found it.
struct PrefillItem {
  int e, row0, m0, mrows;
  int gw;                 // wave index over the expert's weight rows
  uint32_t ar;            // activation row this thread stages (row 0 of the block when past the block)
  bool srow_live;
  EpiScalars es;
};

// The K loop and epilogue of one item for TGN token tiles (TGN = the item's live tiles, 1 to 8): every
// staged step's MFMAs run over all TGN tiles with no branch, so the operand reads of one tile are
// issued under the MFMAs of the previous one. Rows between the live rows and TGN * 16 hold
// whatever the LDS held; their accumulator columns are computed and never stored.
template <int EPI, int LAYOUT, int NWP, int TGN>
__device__ __forceinline__ void prefill_item(const GemmParams& p, const PrefillItem& it, uint8_t* sB,
                                             const uint16_t* lut, float* s_rw) {
  constexpr int SPR = NWP * 64 / kPreBMT;          // staging threads per row
  constexpr int GPT = 8 / SPR;                     // 32-K groups per staging thread and step
  static_assert(SPR * kPreBMT == NWP * 64 && (GPT == 4 || GPT == 2), "staging map");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int K = p.K;
  const int nsteps = K >> 8;
  const int nrow = lane & 15, qb = lane >> 4;
  const int row0 = it.row0, m0 = it.m0, mrows = it.mrows;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.a_codes), (short)0, (int)(p.rows * (K >> 1)), kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.a_scales), (short)0, (int)(p.rows * (K >> 5)), kBufferRsrcWord3);
  const int sn = tid % kPreBMT, sh = tid / kPreBMT;
  // staging: thread (row sn, part sh) converts groups GPT sh .. GPT sh + GPT - 1 of each step, i.e.
  // units 4 GPT sh + (4 j + h); 4 GPT sh and 4 j + h occupy different bits, so the swizzled offset is
  // a per-thread base XOR a constant
  const uint32_t wbase = (uint32_t)sn * kPreRowBytes + ((uint32_t)((4 * GPT * sh) ^ (sn & 31)) << 4);
  // operand reads: lane (nrow, qb) of tile tt reads units u0 + 2t and u0 + 2t + 16 of row tt 16 + nrow,
  // u0 = 8 (qb / 2) + qb % 2; with x = u0 ^ nrow (bits 0-3) the unit's swizzled index is
  // x ^ 2t ^ 16 ((tt & 1) ^ hi): per t a lane address, the rest immediate offsets
  const uint32_t x0 = (uint32_t)((8 * (qb >> 1) + (qb & 1)) ^ nrow);
  uint32_t roff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) roff[t] = (uint32_t)nrow * kPreRowBytes + ((x0 ^ (uint32_t)(2 * t)) << 4);

  int wrow[4];
  const bool active = wave_rows<EPI>(p.N, 0, it.gw, wrow);
  WeightPtrs<LAYOUT> wp;
  wp.init(p, it.e, wrow, active, lane);

  // down: the rows' router weights (topk_weights[sorted[r]], two dependent loads) are loaded under
  // the K loop's first steps and staged in LDS for the epilogue only
  int rw_pair = 0;
  float rw = 0.0f;
  const bool rw_live = EPI == kEpiDown && tid < mrows;
  auto rw_first = [&]() { if (rw_live) rw_pair = p.sorted[row0 + m0 + tid]; };
  auto rw_second = [&]() { if (rw_live) rw = p.topk_weights[rw_pair]; };

  struct Act { u32x4 v[GPT]; uint32_t s; };
  auto prefetch = [&](int gs, Act& ac) {
    const bool live = it.srow_live && gs < nsteps;
    const uint32_t cb = it.ar * (uint32_t)(K >> 1) + (uint32_t)(gs * 128 + sh * 16 * GPT);
#pragma unroll
    for (int j = 0; j < GPT; ++j)
      ac.v[j] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, live ? cb + 16u * j : kOutOfRange, 0, 0);
    const uint32_t so = live ? it.ar * (uint32_t)(K >> 5) + (uint32_t)(gs * 8 + sh * GPT) : kOutOfRange;
    if constexpr (GPT == 4) ac.s = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, so, 0, 0);
    else ac.s = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, so, 0, 0);
  };
  const bool stage_row = sn < ((mrows + 15) & ~15);           // rows of the live tiles (zeros past the block)
  auto commit = [&](const Act& ac) {
    __syncthreads();
    if (stage_row) {
#pragma unroll
      for (int j = 0; j < GPT; ++j) {
        const f16x2 sp = j < 2 ? scale_pair_f16<false>(ac.s) : scale_pair_f16<true>(ac.s);
        const f16x2 s2 = (j & 1) ? __builtin_shufflevector(sp, sp, 1, 1) : __builtin_shufflevector(sp, sp, 0, 0);
        u32x4 u4[4];
        act_group_kprime(ac.v[j], s2, u4);
#pragma unroll
        for (int h = 0; h < 4; ++h)
          *reinterpret_cast<u32x4*>(sB + (wbase ^ ((uint32_t)(4 * j + h) << 4))) = u4[h];
      }
    }
    __syncthreads();
  };

  f32x4 acc[4][TGN];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int tt = 0; tt < TGN; ++tt) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // operand reads of tile tt for smfmac t: units u and u + 16 of row tt 16 + nrow (bit 4 of the
  // swizzled index is (tt & 1) ^ half, an immediate offset)
  auto readB = [&](int t, int tt, u32x4 (&b)[2]) {
    const uint8_t* rb = sB + roff[t] + tt * 16 * kPreRowBytes;
    b[0] = *reinterpret_cast<const u32x4*>(rb + ((tt & 1) << 8));
    b[1] = *reinterpret_cast<const u32x4*>(rb + (((tt & 1) ^ 1) << 8));
  };
  auto decodeA = [&](const WeightFrag<>& w, int t, int rt, f16x8 (&A)[4], int (&idx)[4]) {
    const f16x2 sp = scale_pair_f16(w.sc[rt]);
    const f16x2 s2 = (t < 2) ? __builtin_shufflevector(sp, sp, 0, 0) : __builtin_shufflevector(sp, sp, 1, 1);
    A[rt] = weight_operand_of<LAYOUT>(frag_word(w.pk[rt], t), s2);
    idx[rt] = sparse_index<LAYOUT>(w.mk[rt], t, lut);
  };
  // One staged step, software-pipelined by hand: the operand reads run one tile ahead of the MFMAs
  // (two register sets), and a scheduling fence after each tile keeps that order (left alone, the
  // scheduler sinks the reads next to their MFMAs to save registers, and every tile waits out the
  // LDS latency). The weight operands of smfmac t are decoded before its tiles; the other wave of the
  // SIMD keeps the matrix unit busy meanwhile.
  auto step = [&](WeightFrag<>& w, int reload) {
    u32x4 bb[2][2];
    readB(0, 0, bb[0]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f16x8 A[4];
      int idx[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) decodeA(w, t, rt, A, idx);
      if (t == 3 && reload >= 0) {                   // the slot's last word is decoded: reload it
        slot_decoded<4>(A, idx);
        wp.load(reload, w, active && reload < nsteps);
      }
#pragma unroll
      for (int tt = 0; tt < TGN; ++tt) {
        const int cur = (t * TGN + tt) & 1;
        if (tt + 1 < TGN) readB(t, tt + 1, bb[cur ^ 1]);
        else if (t < 3) readB(t + 1, 0, bb[cur ^ 1]);
        const f16x16 B = __builtin_bit_cast(f16x16, __builtin_shufflevector(bb[cur][0], bb[cur][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          acc[rt][tt] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(A[rt], B, acc[rt][tt], idx[rt], 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  Act ac;
  prefetch(0, ac);
  WeightFrag<> w0, w1;
  wp.load(0, w0, active);
  __builtin_amdgcn_sched_barrier(0);
  wp.load(1, w1, active && nsteps > 1);
  __builtin_amdgcn_sched_barrier(0);
  int gs = 0;
  for (; gs + 2 <= nsteps; gs += 2) {
    commit(ac);
    prefetch(gs + 1, ac);
    if (gs == 0) rw_first();
    step(w0, gs + 2);
    commit(ac);
    prefetch(gs + 2, ac);
    if (gs == 0) rw_second();
    step(w1, gs + 3);
  }
  if (gs < nsteps) {                               // odd step count: the last step
    commit(ac);
    if (gs == 0) {                                 // a single step: the router weights now
      rw_first();
      rw_second();
    }
    step(w0, -1);
  }
  if constexpr (EPI == kEpiDown) {
    if (tid < kPreBMT) s_rw[tid] = rw;             // rows past the m-block: 0
    __syncthreads();
  }
  if (!active) return;
  gemm_epilogue<EPI, TGN>(p, it.es, acc, row0, m0, mrows, 0, it.gw, wrow, s_rw, lane);
}

// A workgroup owns one m-block (<= 128 rows of one expert) and 64 NWP weight rows; each wave keeps 4
// row-tiles x up to 8 token tiles of accumulators and reuses every decoded weight fragment over the
// token tiles. Per 256-K step the activations are converted to exact f16 in LDS; their codes are
// prefetched into registers one step ahead (NWP / 2 threads per row, each 256 / NWP bytes of codes
// and 16 / NWP scale bytes), and the weights run through a two-slot register ring reloaded right
// after decode, so every global load in the K loop is a prefetch issued on every path.
template <int EPI, int LAYOUT, int NWP>
__global__ __launch_bounds__(NWP * 64) __attribute__((amdgpu_waves_per_eu(LAYOUT == 1 ? 8 / NWP : 1))) void k_gemm_prefill(
    GemmParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* sB = smem;                              // [BMT] rows of one 256-K step, swizzled units
  uint16_t* lut = reinterpret_cast<uint16_t*>(smem + kPreLdsB);
  __shared__ int s_e;
  __shared__ int s_pool;                           // the claimed pooled item
  __shared__ int s_arow[kPreBMT];                  // activation row of each m-block row
  __shared__ float s_rw[kPreBMT];                  // router weight of each row (down)

  const int tid = threadIdx.x, wv = tid >> 6;
  const int nblocks = prefill_nblocks<EPI, NWP>(p.N);
  const int items = p.tile_offsets[p.E] * nblocks;
  const int pooled = items / kPrefillPoolDiv;
  const int shared_items = items - pooled;
  const int per = (shared_items + kXcds - 1) / kXcds;
  const int xcd = (int)(blockIdx.x % kXcds), xi = (int)(blockIdx.x / kXcds);
  const int share_end = (xcd + 1) * per < shared_items ? (xcd + 1) * per : shared_items;
  int w_item = xcd * per + xi;
  if (w_item >= share_end) {                       // past the XCD's share: the next pooled item
    // at most a quarter of the pool per XCD claims; the grid's other workgroups (sized for an upper
    // bound of the items) exit without touching the counter
    if (w_item - share_end >= (pooled + 3) / 4) return;
    if (tid == 0) s_pool = atomicAdd(prefill_pools(p.tile_offsets, p.E) + (EPI == kEpiDown ? 1 : 0), 1);
    __syncthreads();
    w_item = shared_items + s_pool;
    if (w_item >= items) return;
  }
  const int mb = w_item / nblocks, nb = w_item - mb * nblocks;
  if (LAYOUT == 0 && tid < 256) lut[tid] = (uint16_t)smfmac_index_of_mask_byte((uint32_t)tid);
  PrefillItem it;
  it.e = find_expert(p.tile_offsets, p.E, mb, &s_e);
  if (it.e < 0) return;
  it.row0 = p.offsets[it.e];
  const int M = p.offsets[it.e + 1] - it.row0;
  it.m0 = (mb - p.tile_offsets[it.e]) * kPreBMT;
  it.mrows = M - it.m0 < kPreBMT ? M - it.m0 : kPreBMT;
  if (tid < kPreBMT) {
    const int r = it.row0 + it.m0 + tid;
    s_arow[tid] = tid < it.mrows ? (p.a_rows ? p.a_rows[r] : r) : 0;
  }
  it.es = epi_scalars<EPI>(p, it.e);
  it.gw = nb * NWP + wv;
  const int sn = tid % kPreBMT;
  __syncthreads();                                 // s_arow
  it.srow_live = sn < it.mrows;
  it.ar = (uint32_t)s_arow[it.srow_live ? sn : 0];
  // one variant per live tile count: a last m-block of 5 to 7 tiles would spend 3/8 to 1/8 of a
  // rounded-up variant's MFMAs on rows past the block (on the 512-expert, top-10 prefill layer every
  // expert holds 54 to 112 rows, and rounding up to 4 or 8 tiles computed 44 % more tiles)
  switch ((it.mrows + 15) >> 4) {
    case 8: prefill_item<EPI, LAYOUT, NWP, 8>(p, it, sB, lut, s_rw); break;
    case 7: prefill_item<EPI, LAYOUT, NWP, 7>(p, it, sB, lut, s_rw); break;
    case 6: prefill_item<EPI, LAYOUT, NWP, 6>(p, it, sB, lut, s_rw); break;
    case 5: prefill_item<EPI, LAYOUT, NWP, 5>(p, it, sB, lut, s_rw); break;
    case 4: prefill_item<EPI, LAYOUT, NWP, 4>(p, it, sB, lut, s_rw); break;
    case 3: prefill_item<EPI, LAYOUT, NWP, 3>(p, it, sB, lut, s_rw); break;
    case 2: prefill_item<EPI, LAYOUT, NWP, 2>(p, it, sB, lut, s_rw); break;
    default: prefill_item<EPI, LAYOUT, NWP, 1>(p, it, sB, lut, s_rw); break;
  }
}

KernelEvents& kernel_events() {
  static thread_local KernelEvents ev;
  return ev;
}

int tactic_rows_per_mblock(int tactic) { return tactic == kTacticPrefill ? kPreBMT : kDecTG * 16; }

size_t gemm_lds_bytes(int tactic, int K) {
  (void)K;
  // the decode tactic's largest variant (the deepest ring)
  return tactic == kTacticPrefill ? (size_t)kPreLdsB + 512 : DecGeom<3>::lds;
}

// Every caller passes the same size for a given kernel, so concurrent first calls set the same value.
// Returns false (and notes the error for the entry point to report) if the attribute is refused; the
// caller then skips the launch.
template <class Kern>
static bool set_lds_attr(Kern* k, size_t lds) {
  static std::atomic<size_t> done{0};   // largest size already granted for this kernel
  if (lds > done.load(std::memory_order_relaxed)) {
    const hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) {
      note_hip_error(e);
      return false;
    }
    done.store(lds, std::memory_order_relaxed);
  }
  return true;
}

// Workgroups per expert of the one-chunk decode kernel, and the fewest n-blocks one covers: enough
// n-blocks per workgroup to stage the activations once for several of them and to hide each epilogue
// under the next n-block's loads (measured best: 4 workgroups per expert at 16 and at 32 n-blocks).
constexpr int kNloopGroups = 4;
constexpr int kNloopMinBlocks = 4;

template <int EPI, int LAYOUT, int RT, int DEPTH>
static void launch_nloop(const GemmParams& p, dim3 grid, int nblocks, hipStream_t stream) {
  const size_t lds = DecGeom<DEPTH>::lds;
  if (!set_lds_attr(&k_gemm_decode_nloop<EPI, LAYOUT, RT, DEPTH>, lds)) return;
  launch_kernel(k_gemm_decode_nloop<EPI, LAYOUT, RT, DEPTH>, grid, dim3(kGemmThreads), lds, stream, p, nblocks);
}

template <int EPI, int LAYOUT>
static void launch_decode(const GemmParams& p, hipStream_t stream) {
  // gate/up waves own 4 row-tiles (32 columns for the fused quantization); other linears stream
  // 2 row-tiles per wave, which keeps more, shorter streams in flight for short K
  constexpr int RT = EPI == kEpiGateUp ? 4 : 2;
  constexpr int DEPTH = dec_depth(RT);
  if constexpr (EPI == kEpiGateUp && LAYOUT == 1) {
    if (p.K <= kStreamMaxK) {
      const size_t lds = stream_lds_bytes(p.K);
      if (!set_lds_attr(&k_gemm_decode_stream<EPI, RT, DEPTH>, stream_lds_bytes(kStreamMaxK))) return;
      const int waves = (p.N >> 1) / 32;
      const int groups = (waves + kStreamWaves - 1) / kStreamWaves;
      launch_kernel(k_gemm_decode_stream<EPI, RT, DEPTH>, dim3((unsigned)p.E, (unsigned)groups), dim3(kStreamThreads), lds,
                    stream, p);
      return;
    }
  }
  const int nblocks = EPI == kEpiGateUp ? ((p.N >> 1) + 127) / 128 : (p.N + 64 * RT - 1) / (64 * RT);
  if constexpr (EPI != kEpiGateUp) {
    // K up to 1024: the whole K staged once and the ring holding one n-block's K (K / 256 slots)
    int per = (nblocks + kNloopGroups - 1) / kNloopGroups;
    per = per < kNloopMinBlocks ? kNloopMinBlocks : per;
    const int ny = (nblocks + per - 1) / per;
    const dim3 grid((unsigned)p.E, (unsigned)ny);
    switch (p.K) {
      case 256: launch_nloop<EPI, LAYOUT, RT, 1>(p, grid, nblocks, stream); return;
      case 512: launch_nloop<EPI, LAYOUT, RT, 2>(p, grid, nblocks, stream); return;
      case 768: launch_nloop<EPI, LAYOUT, RT, 3>(p, grid, nblocks, stream); return;
      case 1024: launch_nloop<EPI, LAYOUT, RT, 4>(p, grid, nblocks, stream); return;
      default: break;
    }
  }
  const size_t lds = DecGeom<DEPTH>::lds;
  if (!set_lds_attr(&k_gemm_decode<EPI, LAYOUT, RT>, lds)) return;
  launch_kernel(k_gemm_decode<EPI, LAYOUT, RT>, dim3((unsigned)p.E, (unsigned)nblocks), dim3(kGemmThreads), lds, stream, p);
}

template <int EPI, int LAYOUT>
static void launch_prefill(const GemmParams& p, hipStream_t stream) {
  const size_t lds = gemm_lds_bytes(kTacticPrefill, p.K);
  constexpr int NWP = prefill_waves<EPI, LAYOUT>();
  if (!set_lds_attr(&k_gemm_prefill<EPI, LAYOUT, NWP>, lds)) return;
  // an upper bound of the live m-blocks (each expert adds at most one partial m-block); the kernel
  // spreads the live items over the XCDs and the rest of the grid exits
  const int64_t mblocks = (p.rows + kPreBMT - 1) / kPreBMT + p.E;
  const int nblocks = prefill_nblocks<EPI, NWP>(p.N);
  // per XCD: its share of an upper bound of the live items, then enough workgroups to claim up to a
  // quarter of the pooled items (the rest of those find the pool empty and exit)
  const int64_t bound = mblocks * nblocks;
  const int64_t per_xcd = (bound + kXcds - 1) / kXcds + (bound + 4 * kPrefillPoolDiv - 1) / (4 * kPrefillPoolDiv);
  const int64_t grid = per_xcd * kXcds;
  launch_kernel(k_gemm_prefill<EPI, LAYOUT, NWP>, dim3((unsigned)grid), dim3(NWP * 64), lds, stream, p);
}

template <int EPI>
static void launch_epi(const GemmParams& p, int tactic, hipStream_t stream) {
  if (tactic == kTacticPrefill) {
    if (p.layout == 1) launch_prefill<EPI, 1>(p, stream); else launch_prefill<EPI, 0>(p, stream);
  } else {
    if (p.layout == 1) launch_decode<EPI, 1>(p, stream); else launch_decode<EPI, 0>(p, stream);
  }
}

void launch_grouped_gemm(const GemmParams& p, int epi, int tactic, hipStream_t stream) {
  if (p.rows <= 0) return;
  if (epi == kEpiStore) launch_epi<kEpiStore>(p, tactic, stream);
  else if (epi == kEpiGateUp) launch_epi<kEpiGateUp>(p, tactic, stream);
  else launch_epi<kEpiDown>(p, tactic, stream);
}

// ---------------------------------------------------------------------------------------------
// Top-k combine: out[t] = sum_j D[inv[t*k+j]] in j order (deterministic).
// ---------------------------------------------------------------------------------------------
// out[t] = sum over j of D[inv[t k + j]] in order j = 0 .. k-1 (pairs with inv < 0 skipped). The k
// row indices are loaded first and then all k rows at once. Every row is read once and the output
// written once, so both go through the non-temporal path: the pass then read its 3.76 GB of rows on
// the 384-expert layer in 0.75 instead of 0.85 ms, and the 128-expert one in 98 instead of 136 us.
template <int KMAX>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ D, const int* __restrict__ inv,
                                                 int64_t T, int k, int H, float* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int H4 = H >> 2;
  const int64_t t = gid / H4;
  if (t >= T) return;
  const int c = (int)(gid - t * H4) * 4;
  int r[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) r[j] = j < k ? inv[t * k + j] : -1;
  f32x4 v[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    v[j] = r[j] >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(D + (int64_t)r[j] * H + c))
                     : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (r[j] >= 0) s += v[j];
  __builtin_nontemporal_store(s, reinterpret_cast<f32x4*>(out + t * H + c));
}

void launch_combine(const float* D, const int* inv, int64_t T, int k, int H, float* out, hipStream_t stream) {
  const int64_t n = T * (H >> 2);
  if (!n) return;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (k <= 8) launch_kernel(k_combine<8>, dim3(grid), dim3(256), 0, stream, D, inv, T, k, H, out);
  else if (k <= 16) launch_kernel(k_combine<16>, dim3(grid), dim3(256), 0, stream, D, inv, T, k, H, out);
  else launch_kernel(k_combine<32>, dim3(grid), dim3(256), 0, stream, D, inv, T, k, H, out);
}

}  // namespace moesq

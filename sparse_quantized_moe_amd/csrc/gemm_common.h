// Pieces shared by the grouped sparse GEMM kernels: block -> (expert, m-block) lookup, per-lane
// weight fragments of the pair-bitmask storage, and the three epilogues.
#pragma once
#include "moesq_device.h"
#include "moesq_internal.h"

namespace moesq {

// Kept bytes, masks (tiled layout: index codes) and scales one lane needs for one 256-K super-step
// of RT row-tiles: 16 B of packed, 4 B of mask and 2 B of scale per row-tile (the lane's 64
// contiguous K of its row).
template <int RT = 4>
struct WeightFrag {
  u32x4 pk[RT];
  uint32_t mk[RT];
  uint32_t sc[RT];
};

// LAYOUT 0: pair-bitmask storage (three row-major tensors); LAYOUT 1: tiled records, one
// contiguous 1408-byte record per (16-row tile, 256-K step), so each load of a wave is coalesced.
template <int LAYOUT, int RT = 4>
struct WeightPtrs;

template <int RT>
struct WeightPtrs<0, RT> {
  const uint8_t* pk[RT];
  const uint8_t* mk[RT];
  const uint8_t* sc[RT];

  __device__ __forceinline__ void init(const GemmParams& p, int e, const int* wrow, bool active, int lane) {
    const int K = p.K, qa = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int64_t wr = (int64_t)e * p.N + (active ? wrow[rt] : 0) + (lane & 15);
      pk[rt] = p.w_packed + wr * (K >> 2) + 16 * qa;
      mk[rt] = p.w_mask + wr * (K >> 4) + 4 * qa;
      sc[rt] = p.w_scale + wr * (K >> 5) + 2 * qa;
    }
  }

  __device__ __forceinline__ void load(int gs, WeightFrag<RT>& w) const {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      w.pk[rt] = *reinterpret_cast<const u32x4*>(pk[rt] + 64 * gs);
      w.mk[rt] = *reinterpret_cast<const uint32_t*>(mk[rt] + 16 * gs);
      w.sc[rt] = *reinterpret_cast<const uint16_t*>(sc[rt] + 8 * gs);
    }
  }

  // live = false: zeros instead of a load
  __device__ __forceinline__ void load(int gs, WeightFrag<RT>& w, bool live) const {
    if (live) {
      load(gs, w);
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        w.pk[rt] = u32x4{0u, 0u, 0u, 0u};
        w.mk[rt] = 0u;
        w.sc[rt] = 0u;
      }
    }
  }
};

// A lane index whose record offsets (2, 4 or 16 bytes per lane) all lie at or past 2^31, beyond
// any buffer's num_records.
constexpr uint32_t kOutOfRangeLanes = 0x08000000u;

template <int RT>
struct WeightPtrs<1, RT> {
  __amdgpu_buffer_rsrc_t rsrc;  // the expert's records (wave-uniform, scalar registers)
  int tile_off[RT];             // byte offset of each row-tile's first record in the expert (uniform)
  uint32_t lane;                // lane offsets inside a record: 16 lane, 1024 + 4 lane, 1280 + 2 lane

  __device__ __forceinline__ void init(const GemmParams& p, int e, const int* wrow, bool active, int ln) {
    const int steps = p.K >> 8;
    const int64_t expert_bytes = (int64_t)(p.N >> 4) * steps * kTileRecordBytes;
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.w_packed) + e * expert_bytes, (short)0,
                                             (int)expert_bytes, kBufferRsrcWord3);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      tile_off[rt] = __builtin_amdgcn_readfirstlane(active ? (wrow[rt] >> 4) : 0) * steps * kTileRecordBytes;
    lane = (uint32_t)ln;
  }

  __device__ __forceinline__ void load(int gs, WeightFrag<RT>& w) const { load(gs, w, true); }

  // live = false: the same loads at an offset past the buffer, which read zeros without touching
  // memory (keeps the number of loads in flight the same on every path)
  __device__ __forceinline__ void load(int gs, WeightFrag<RT>& w, bool live) const {
    const uint32_t l = lane + (live ? 0u : kOutOfRangeLanes);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int soff = tile_off[rt] + gs * kTileRecordBytes;
      w.pk[rt] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, l * 16u, soff, 0);
      w.mk[rt] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, l * 4u + kTileCodeOffset, soff, 0);
      w.sc[rt] = __builtin_amdgcn_raw_buffer_load_b16(rsrc, l * 2u + kTileScaleOffset, soff, 0);
    }
  }
};

// Orders the reload of a weight ring slot after the last decode of its old contents: the (empty)
// statement consumes the decoded operands and is a memory barrier, so the slot's loads cannot be
// scheduled above it. Without it the scheduler hoists them, the old and new contents are live at
// once, and the register allocator rotates the ring through extra registers with copies that wait
// on loads still in flight.
template <int RT>
__device__ __forceinline__ void slot_decoded(const f16x8 (&A)[RT], const int (&idx)[RT]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) asm volatile("" ::"v"(A[rt]), "v"(idx[rt]) : "memory");
}

// Compressed sparse operand of smfmac t of a fragment word, in either layout.
template <int LAYOUT>
__device__ __forceinline__ f16x8 weight_operand_of(uint32_t word, f16x2 s2) {
  return LAYOUT == 0 ? weight_operand(word, s2) : weight_operand_tiled(word, s2);
}

// Sparse-index word of smfmac t of a row-tile's fragment word mk: through the LDS table of mask
// bytes (pair-bitmask layout) or by one byte permute of the record's code bytes (tiled layout).
template <int LAYOUT>
__device__ __forceinline__ int sparse_index(uint32_t mk, int t, const uint16_t* lut) {
  if constexpr (LAYOUT == 1) return smfmac_index_of_codes(mk, t);
  else return lut[(mk >> (8 * t)) & 255u];
}

__device__ __forceinline__ uint32_t frag_word(const u32x4& v, int t) {
  return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w;
}

// Weight rows of wave `wv` in n-block `nb`: RT row-tiles of 16 (n-blocks of 4 * 16 * RT rows).
// Gate/up (RT = 4): 32 intermediate columns, i.e. gate rows c..c+31 (tiles 0, 1) and up rows
// I+c..I+c+31 (tiles 2, 3), n-blocks of 128 columns.
template <int EPI, int RT = 4>
__device__ __forceinline__ bool wave_rows(int N, int nb, int wv_in, int* wrow) {
  const int wv = __builtin_amdgcn_readfirstlane(wv_in);
  if constexpr (EPI == kEpiGateUp) {
    static_assert(EPI != kEpiGateUp || RT == 4, "gate/up waves own 2 gate and 2 up tiles");
    const int I = N >> 1;
    const int hcol0 = nb * 128 + wv * 32;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) wrow[rt] = (rt < 2 ? 0 : I) + hcol0 + (rt & 1) * 16;
    return hcol0 < I;
  } else {
    const int r0 = (nb * 4 + wv) * 16 * RT;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) wrow[rt] = r0 + rt * 16;
    return r0 < N;
  }
}

// Expert of m-block `mb` (-1 past the last one), found by the whole workgroup in one pass.
__device__ __forceinline__ int find_expert(const int* tile_offsets, int E, int mb, int* s_e) {
  if (threadIdx.x == 0) *s_e = -1;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int a = tile_offsets[e], b = tile_offsets[e + 1];
    if (a <= mb && mb < b) *s_e = e;
  }
  __syncthreads();
  return *s_e;
}

// Per-expert scalars of the epilogue, read once at the start of a workgroup (uniform).
struct EpiScalars {
  float g0, g1;   // gate/up: activation x weight global of the gate and up halves; store/down: g0 for all rows
                  // (store with G = 2: g0 first half, g1 second half)
  float h_global; // gate/up: global of the h quantization
};

template <int EPI>
__device__ __forceinline__ EpiScalars epi_scalars(const GemmParams& p, int e) {
  EpiScalars es;
  const float ag = p.a_global[e];
  if (EPI == kEpiGateUp || (EPI == kEpiStore && p.G == 2)) {
    es.g0 = ag * p.w_global[2 * e];
    es.g1 = ag * p.w_global[2 * e + 1];
  } else {
    es.g0 = es.g1 = ag * p.w_global[e];
  }
  es.h_global = EPI == kEpiGateUp ? p.h_global[e] : 0.0f;
  return es;
}

// Router weight of row r of an m-block (down epilogue), staged in LDS with the m-block's rows.
__device__ __forceinline__ float row_weight(const GemmParams& p, int row) { return p.topk_weights[p.sorted[row]]; }

// Epilogues. Accumulator acc[rt][tt] of lane (n = lane & 15, q = lane >> 4) holds, for r = 0..3,
// weight row wrow[rt] + 4q + r and the m-block's token row tt*16 + n. s_rw: router weights of the
// m-block's rows (down only).
// Stores of the epilogues. CPOL 0: plain stores. Otherwise buffer stores with that cache policy
// (kCpolDevice: device-coherent, written through for readers in other workgroups of the same
// launch without a cache write-back); offsets are bytes from the buffer's base (< 2^31).
constexpr int kCpolDevice = 16;   // sc1

template <int CPOL, class T>
__device__ __forceinline__ void epi_store(T* base, int64_t idx, T v) {
  if constexpr (CPOL == 0) {
    base[idx] = v;
  } else {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, 0x7FFFFFFF, kBufferRsrcWord3);
    const uint32_t off = (uint32_t)(idx * (int64_t)sizeof(T));
    if constexpr (sizeof(T) == 16) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, CPOL);
    else if constexpr (sizeof(T) == 4) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, CPOL);
    else if constexpr (sizeof(T) == 2) __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), r, off, 0, CPOL);
    else __builtin_amdgcn_raw_buffer_store_b8(__builtin_bit_cast(uint8_t, v), r, off, 0, CPOL);
  }
}

template <int EPI, int TG, int RT = 4, int CPOL = 0>
__device__ __forceinline__ void gemm_epilogue(const GemmParams& p, const EpiScalars& es, f32x4 (&acc)[RT][TG],
                                              int row0, int m0, int mrows, int nb, int wv, const int* wrow,
                                              const float* s_rw, int lane) {
  const int N = p.N, ntok = lane & 15, qa = lane >> 4;
  if constexpr (EPI == kEpiGateUp) {
    // h = silu(gate) * up in fp32, then the NVFP4 quantization of h with the down input global:
    // the 32 columns of one scale group are the 8 values of each of the 4 lanes sharing ntok.
    const int I = N >> 1;
    const int hcol0 = nb * 128 + __builtin_amdgcn_readfirstlane(wv) * 32;
    const float g2 = es.h_global;
    const float inv6g2 = scale_code_inv(g2);
#pragma unroll
    for (int tt = 0; tt < TG; ++tt) {
      if (tt * 16 >= mrows) continue;
      const int n = tt * 16 + ntok;
      float h[2][4];
      float amax = 0.0f;
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gt = acc[half][tt][r] * es.g0;
          const float up = acc[2 + half][tt][r] * es.g1;
          // silu(gt) = gt / (1 + exp(-gt)), with the reciprocal instruction (1 ulp)
          const float hv = gt * up * __builtin_amdgcn_rcpf(1.0f + __expf(-gt));
          h[half][r] = hv;
          amax = __builtin_fmaxf(amax, __builtin_fabsf(hv));
        }
      amax = lane_max4(amax);
      const int scb = scale_code(amax, g2, inv6g2);
      const float s = e4m3_value(scb);
      if (n < mrows) {
        const int64_t row = row0 + m0 + n;
        const Nvfp4Recip rc = nvfp4_recip(s, g2);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint16_t v = (uint16_t)nvfp4_codes<4>(h[half], s, g2, rc);
          epi_store<CPOL>(reinterpret_cast<uint16_t*>(p.h_codes), (row * (I >> 1) + ((hcol0 + half * 16 + 4 * qa) >> 1)) >> 1, v);
        }
        if (qa == 0) epi_store<CPOL>(p.h_scales, row * (I >> 5) + (hcol0 >> 5), (uint8_t)scb);
      }
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < TG; ++tt) {
      if (tt * 16 >= mrows) continue;
      const int n = tt * 16 + ntok;
      if (n < mrows) {
        const int64_t row = row0 + m0 + n;
        const float gsc = EPI == kEpiDown ? es.g0 * s_rw[n] : es.g0;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int col = wrow[rt] + 4 * qa;
          const float gcol = (EPI == kEpiStore && col >= (N >> 1)) ? es.g1 : gsc;
          epi_store<CPOL>(reinterpret_cast<f32x4*>(p.out), (row * N + col) >> 2, acc[rt][tt] * gcol);
        }
      }
    }
  }
}

}  // namespace moesq

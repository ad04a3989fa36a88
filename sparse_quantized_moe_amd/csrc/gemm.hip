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
// for the even group, high nibbles for the odd group) and the mask nibble gives both groups' index.
// Dequantization is exact: e2m1 * e4m3 has <= 6 significant bits, so it is exact in f16, products
// of two such values are exact in fp32 and accumulation is in fp32. Global scales are applied in the
// fp32 epilogue.
//
// Work decomposition (one workgroup = 4 waves):
//   * a workgroup owns one m-block (up to TG*16 rows of one expert) and one n-block (256 weight rows;
//     for the fused gate|up epilogue 128 intermediate columns = their 128 gate and 128 up rows);
//   * each wave owns 4 row-tiles of 16 weight rows and streams their kept bytes, masks and scales
//     straight from HBM into registers (16 B + 4 B + 2 B per lane per 256 K, one load each),
//     prefetching the next 256 K while the current one is in the MFMAs;
//   * the m-block's activations are dequantized once per K-chunk into LDS in the B-operand order.
// Per 256 K a lane holds the contiguous 64 K [64 q, 64 q + 64) of its row (q = lane / 16); smfmac t
// (t = 0..3) takes chunks 2t, 2t+1 of it. The B lanes read the matching chunks from LDS.
//
// Tactics: "decode" (TG = 2: 32 rows per m-block, K-chunk 1024) streams each expert's weights once
// for small batches; "prefill" (TG = 8: 128 rows, K-chunk 256) reuses each decoded weight fragment
// over 8 token tiles.
#include "moesq_device.h"
#include "moesq_internal.h"

namespace moesq {

constexpr int kGemmThreads = 256;

template <int TG, int KC>
struct GemmShape {
  static constexpr int BMT = TG * 16;                 // rows (tokens) per m-block
  static constexpr int ROW_STRIDE = KC * 2 + 16;      // bytes per token row in LDS (+16 B skew)
  static constexpr int LDS_B = BMT * ROW_STRIDE;
};

template <int EPI, int TG, int KC>
__global__ __launch_bounds__(kGemmThreads) void k_grouped_gemm(GemmParams p) {
  using S = GemmShape<TG, KC>;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* sB = smem;
  uint16_t* lut = reinterpret_cast<uint16_t*>(smem + S::LDS_B);
  __shared__ int s_e;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int mb = blockIdx.x, nb = blockIdx.y;
  const int E = p.E, N = p.N, K = p.K;

  if (tid == 0) s_e = -1;
  __syncthreads();
  for (int e = tid; e < E; e += kGemmThreads) {
    const int a = p.tile_offsets[e], b = p.tile_offsets[e + 1];
    if (a <= mb && mb < b) s_e = e;
  }
  lut[tid] = (uint16_t)smfmac_index_of_mask_byte((uint32_t)tid);
  __syncthreads();
  const int e = s_e;
  if (e < 0) return;
  const int row0 = p.offsets[e];
  const int M = p.offsets[e + 1] - row0;
  const int m0 = (mb - p.tile_offsets[e]) * S::BMT;
  const int mrows = M - m0 < S::BMT ? M - m0 : S::BMT;

  // weight rows of this wave
  int wrow[4];
  bool active;
  if (EPI == kEpiGateUp) {
    const int I = N >> 1;
    const int hcol0 = nb * 128 + wv * 32;
    active = hcol0 < I;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) wrow[rt] = (rt < 2 ? 0 : I) + hcol0 + (rt & 1) * 16;
  } else {
    const int r0 = nb * 256 + wv * 64;
    active = r0 < N;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) wrow[rt] = r0 + rt * 16;
  }
  const int qa = lane >> 4;
  const uint8_t* pk_ptr[4];
  const uint8_t* mk_ptr[4];
  const uint8_t* sc_ptr[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int64_t wr = (int64_t)e * N + (active ? wrow[rt] + (lane & 15) : 0);
    pk_ptr[rt] = p.w_packed + wr * (K >> 2) + 16 * qa;
    mk_ptr[rt] = p.w_mask + wr * (K >> 4) + 4 * qa;
    sc_ptr[rt] = p.w_scale + wr * (K >> 5) + 2 * qa;
  }

  f32x4 acc[4][TG];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int tt = 0; tt < TG; ++tt) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = K >> 8;
  constexpr int SPC = KC / 256;          // super-steps per K-chunk
  u32x4 pk[4];
  uint32_t mk[4], sc[4];
  if (active) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      pk[rt] = *reinterpret_cast<const u32x4*>(pk_ptr[rt]);
      mk[rt] = *reinterpret_cast<const uint32_t*>(mk_ptr[rt]);
      sc[rt] = *reinterpret_cast<const uint16_t*>(sc_ptr[rt]);
    }
  }
  const int64_t a_row_bytes = K >> 1, a_row_scales = K >> 5;
  for (int gs = 0; gs < nsteps; ++gs) {
    const int ssl = gs % SPC;
    if (ssl == 0) {
      const int k0 = gs * 256;
      const int kc = K - k0 < KC ? K - k0 : KC;
      const int cpr = kc >> 3;               // chunks per row in this K-chunk
      __syncthreads();
      for (int i = tid; i < S::BMT * cpr; i += kGemmThreads) {
        const int n = i / cpr, c = i - n * cpr;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (n < mrows) {
          const int64_t ar = row0 + m0 + n;
          const uint32_t codes = *reinterpret_cast<const uint32_t*>(p.a_codes + ar * a_row_bytes + ((k0 >> 3) + c) * 4);
          const uint32_t sb = p.a_scales[ar * a_row_scales + ((k0 + 8 * c) >> 5)];
          const f16 s = e4m3_to_f16(sb);
          v = act_chunk_kprime(codes, f16x2{s, s});
        }
        *reinterpret_cast<u32x4*>(sB + n * S::ROW_STRIDE + c * 16) = v;
      }
      __syncthreads();
    }
    u32x4 pk_n[4];
    uint32_t mk_n[4], sc_n[4];
    if (active && gs + 1 < nsteps) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        pk_n[rt] = *reinterpret_cast<const u32x4*>(pk_ptr[rt] + 64 * (gs + 1));
        mk_n[rt] = *reinterpret_cast<const uint32_t*>(mk_ptr[rt] + 16 * (gs + 1));
        sc_n[rt] = *reinterpret_cast<const uint16_t*>(sc_ptr[rt] + 8 * (gs + 1));
      }
    }
    if (active) {
      const int nrow = lane & 15, qb = lane >> 4;
      const uint8_t* brow = sB + nrow * S::ROW_STRIDE + (32 * ssl + 8 * (qb >> 1) + (qb & 1)) * 16;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f16x8 A[4];
        int idx[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const uint32_t kept = t == 0 ? pk[rt].x : t == 1 ? pk[rt].y : t == 2 ? pk[rt].z : pk[rt].w;
          const f16 s = e4m3_to_f16((sc[rt] >> (8 * (t >> 1))) & 255u);
          A[rt] = weight_operand(kept, f16x2{s, s});
          idx[rt] = lut[(mk[rt] >> (8 * t)) & 255u];
        }
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
          if (tt * 16 < mrows) {
            const uint8_t* bp = brow + tt * 16 * S::ROW_STRIDE + 2 * t * 16;
            const u32x4 b0 = *reinterpret_cast<const u32x4*>(bp);
            const u32x4 b1 = *reinterpret_cast<const u32x4*>(bp + 16 * 16);
            const f16x16 B = __builtin_bit_cast(f16x16, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
              acc[rt][tt] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(A[rt], B, acc[rt][tt], idx[rt], 0, 0);
          }
        }
      }
    }
    if (active && gs + 1 < nsteps) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) { pk[rt] = pk_n[rt]; mk[rt] = mk_n[rt]; sc[rt] = sc_n[rt]; }
    }
  }
  if (!active) return;

  // ---- epilogues ----
  const int ntok = lane & 15;
  const float ag = p.a_global[e];
  if (EPI == kEpiGateUp) {
    const int I = N >> 1;
    const int hcol0 = nb * 128 + wv * 32;
    const float g_gate = ag * p.w_global[2 * e];
    const float g_up = ag * p.w_global[2 * e + 1];
    const float g2 = p.h_global[e];
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
          const float gt = acc[half][tt][r] * g_gate;
          const float up = acc[2 + half][tt][r] * g_up;
          const float hv = gt / (1.0f + __expf(-gt)) * up;
          h[half][r] = hv;
          amax = __builtin_fmaxf(amax, __builtin_fabsf(hv));
        }
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
      const int scb = scale_code(amax, g2);
      const float s = e4m3_value(scb);
      if (n < mrows) {
        const int64_t row = row0 + m0 + n;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint32_t c0 = nvfp4_code(h[half][0], s, g2), c1 = nvfp4_code(h[half][1], s, g2);
          const uint32_t c2 = nvfp4_code(h[half][2], s, g2), c3 = nvfp4_code(h[half][3], s, g2);
          const uint16_t v = (uint16_t)(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
          *reinterpret_cast<uint16_t*>(p.h_codes + row * (I >> 1) + ((hcol0 + half * 16 + 4 * qa) >> 1)) = v;
        }
        if (qa == 0) p.h_scales[row * (I >> 5) + (hcol0 >> 5)] = (uint8_t)scb;
      }
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < TG; ++tt) {
      if (tt * 16 >= mrows) continue;
      const int n = tt * 16 + ntok;
      if (n >= mrows) continue;
      const int64_t row = row0 + m0 + n;
      float gsc;
      if (EPI == kEpiDown) gsc = ag * p.w_global[e] * p.topk_weights[p.sorted[row]];
      else gsc = ag;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int col = wrow[rt] + 4 * qa;
        float gcol = gsc;
        if (EPI == kEpiStore) gcol = gsc * (p.G == 2 ? p.w_global[2 * e + (col >= (N >> 1) ? 1 : 0)] : p.w_global[e]);
        const f32x4 v = acc[rt][tt] * gcol;
        *reinterpret_cast<f32x4*>(p.out + row * N + col) = v;
      }
    }
  }
}

int tactic_rows_per_mblock(int tactic) { return tactic == kTacticPrefill ? 128 : 32; }

template <int EPI, int TG, int KC>
static void launch_variant(const GemmParams& p, hipStream_t stream) {
  using S = GemmShape<TG, KC>;
  const size_t lds = S::LDS_B + 512;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_grouped_gemm<EPI, TG, KC>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr = true;
  }
  const int64_t mblocks = (p.rows + S::BMT - 1) / S::BMT + p.E;
  const int nblocks = EPI == kEpiGateUp ? ((p.N >> 1) + 127) / 128 : (p.N + 255) / 256;
  if (mblocks <= 0 || nblocks <= 0) return;
  k_grouped_gemm<EPI, TG, KC><<<dim3((unsigned)mblocks, (unsigned)nblocks), kGemmThreads, lds, stream>>>(p);
}

void launch_grouped_gemm(const GemmParams& p, int epi, int tactic, hipStream_t stream) {
  if (tactic == kTacticPrefill) {
    if (epi == kEpiStore) launch_variant<kEpiStore, 8, 256>(p, stream);
    else if (epi == kEpiGateUp) launch_variant<kEpiGateUp, 8, 256>(p, stream);
    else launch_variant<kEpiDown, 8, 256>(p, stream);
  } else {
    if (epi == kEpiStore) launch_variant<kEpiStore, 2, 1024>(p, stream);
    else if (epi == kEpiGateUp) launch_variant<kEpiGateUp, 2, 1024>(p, stream);
    else launch_variant<kEpiDown, 2, 1024>(p, stream);
  }
}

// ---------------------------------------------------------------------------------------------
// Top-k combine: out[t] = sum_j D[inv[t*k+j]] in j order (deterministic).
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ D, const int* __restrict__ inv,
                                                 int64_t T, int k, int H, float* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int H4 = H >> 2;
  const int64_t t = gid / H4;
  if (t >= T) return;
  const int c = (int)(gid - t * H4) * 4;
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int r = inv[t * k + j];
    if (r >= 0) s += *reinterpret_cast<const f32x4*>(D + (int64_t)r * H + c);
  }
  *reinterpret_cast<f32x4*>(out + t * H + c) = s;
}

void launch_combine(const float* D, const int* inv, int64_t T, int k, int H, float* out, hipStream_t stream) {
  const int64_t n = T * (H >> 2);
  if (n) k_combine<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(D, inv, T, k, H, out);
}

}  // namespace moesq

// Device helpers of the MI355X (gfx950, wave64) paired-4:8 NVFP4 MoE kernels.
//
// Number formats (model card "Qwen3.5-397B-A17B-P48NVFP4-MoESQ", "Compression details"): NVFP4 is an
// E2M1 value per element, an FP8-E4M3 scale per 32 dense K and an FP32 global scale; the value of a
// code is e2m1(code) * e4m3(scale) * global.
//
// Exact decisions. Every rounding decision (the E4M3 scale of a 32-group and the E2M1 code of an
// element) is taken on the exact real quotient, with ties to even, by sign tests of single fused
// multiply-adds: sign(fma(-(b*s), g, |x|)) is the exact sign of |x| - b*s*g because b*s has at most
// 7 significant bits (exact in fp32) and the FMA rounds once. This holds for finite inputs and
// globals g >= 2^-90 (no underflow of the difference).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moesq {

typedef _Float16 f16;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) _Float16 f16x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// ---------------------------------------------------------------------------------------------
// E4M3FN (OCP FP8, bias 7, no infinities, 0x7F/0xFF NaN)
// ---------------------------------------------------------------------------------------------

// Non-negative finite E4M3 byte (0x00..0x7E) -> fp32, exact.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float normal = __uint_as_float(((e + 120u) << 23) | (m << 20));
  const float sub = (float)m * 0x1p-9f;
  return e ? normal : sub;
}

// Nearest E4M3 byte of fp32 v >= 0 (may be off by one step near a midpoint; callers fix it exactly).
// Selects only: the normal-range code (v = 1.f 2^e, 3 fraction bits rounded, a carry moving to the
// next binade), the subnormal code (steps of 2^-9) below 2^-6, and 0x7E from 448 up (NaN included).
__device__ __forceinline__ int e4m3_candidate(float v) {
  const uint32_t u = __float_as_uint(v);
  const int e = (int)((u >> 23) & 255u) - 127;
  const float mant = __uint_as_float((u & 0x007FFFFFu) | 0x3F800000u); // [1, 2)
  const int cn = ((e + 7) << 3) + (int)__builtin_rintf((mant - 1.0f) * 8.0f);
  const int cs = (int)__builtin_rintf(__builtin_fminf(v, 1.0f) * 512.0f);
  const int c = v < 0x1p-6f ? cs : (cn < 0x7E ? cn : 0x7E);
  return v < 448.0f ? c : 0x7E;
}

// Midpoint of E4M3 bytes c and c + 1 (0 <= c < 0x7E), exact in fp32: a normal byte's value plus half
// its step is the same bits with mantissa bit 19 set (the next byte, also in the next binade, is one
// full step up); below 2^-6 the step is 2^-9 and the midpoint (2c + 1) 2^-10.
__device__ __forceinline__ float e4m3_mid_up(uint32_t c) {
  const float normal = __uint_as_float((((c >> 3) + 120u) << 23) | ((c & 7u) << 20) | (1u << 19));
  const float sub = (float)(2u * c + 1u) * 0x1p-10f;
  return c >= 8u ? normal : sub;
}

// E4M3 byte of the exact quotient amax / (6 g): round to nearest, ties to even, saturating at 448.
// amax >= 0, g > 0, inv6g ~ 1 / (6 g) (a few ulps off is fine). The candidate from amax * inv6g is
// within one step of the answer; the midpoints m with its two neighbours are tested exactly with
// sign(fma(-(6m), g, amax)) (6m has <= 7 significant bits), with no branch.
__device__ __forceinline__ int scale_code(float amax, float g, float inv6g) {
  const int c = e4m3_candidate(amax * inv6g);
  const float dhi = __builtin_fmaf(-6.0f * e4m3_mid_up((uint32_t)c), g, amax);
  const float dlo = __builtin_fmaf(-6.0f * e4m3_mid_up((uint32_t)(c - 1)), g, amax);
  const bool odd = (c & 1) != 0;
  const bool up = (c < 0x7E) & ((dhi > 0.0f) | ((dhi == 0.0f) & odd));
  const bool down = (c > 0) & ((dlo < 0.0f) | ((dlo == 0.0f) & odd));
  return c + (int)up - (int)down;
}
__device__ __forceinline__ float scale_code_inv(float g) { return __builtin_amdgcn_rcpf(6.0f * g); }
__device__ __forceinline__ int scale_code(float amax, float g) { return scale_code(amax, g, scale_code_inv(g)); }

// E2M1 magnitude code (0..7) of the exact quotient ax / (s g): nearest, ties to even, saturating at 6.
// Boundaries 0.25 .75 1.25 1.75 2.5 3.5 5; a tie goes to the even code (strict '>' where the lower
// neighbour is even, '>=' where the upper one is). The code counts the boundaries ax passes, and as
// they increase it is found by a binary search: 1.75 decides bit 2, then 0.75 or 3.5 bit 1, then
// 0.25 / 1.25 / 2.5 / 5 bit 0. Each test is the exact sign of ax - B s g: B s is exact (few significant
// bits) and the FMA rounds once. s == 0 gives 0.
__device__ __forceinline__ uint32_t e2m1_code(float ax, float s, float g) {
  const bool h = __builtin_fmaf(-1.75f * s, g, ax) >= 0.0f;
  const bool m = __builtin_fmaf((h ? -3.5f : -0.75f) * s, g, ax) >= 0.0f;
  const float b0 = h ? (m ? -5.0f : -2.5f) : (m ? -1.25f : -0.25f);
  const bool l = __builtin_fmaf(b0 * s, g, ax) > 0.0f;
  const uint32_t c = (h ? 4u : 0u) | (m ? 2u : 0u) | (l ? 1u : 0u);
  return s == 0.0f ? 0u : c;
}

// 4-bit NVFP4 code of x for the group's scale value s and global g (sign bit copied from x).
__device__ __forceinline__ uint32_t nvfp4_code(float x, float s, float g) {
  return e2m1_code(__builtin_fabsf(x), s, g) | ((__float_as_uint(x) >> 28) & 8u);
}

// N consecutive NVFP4 codes by the exact comparisons alone, x[0] in the low nibble. For inputs with
// few significant bits (bf16) many quotients sit within an ulp of a boundary, and the fast path below
// would take its fallback in nearly every wave.
template <int N>
__device__ __forceinline__ uint32_t nvfp4_codes_exact(const float* x, float s, float g) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) w |= nvfp4_code(x[i], s, g) << (4 * i);
  return w;
}

// Fast exact codes. With sg = s g (one rounding), inv = v_rcp_f32(sg) (at most 1 ulp off) and
// r = x inv (one rounding), r is within 2^-22 relative of the exact quotient x / (s g), i.e. within
// 4 ulps of it, as long as sg and inv are normal numbers. The hardware conversion
// v_cvt_scalef32_pk_fp4_f32 (scale 1) rounds an fp32 value to nearest-even E2M1 with saturation at 6
// and keeps the sign (checked around every boundary against a host model), so its code equals the
// exact one unless a rounding boundary lies between r and the exact quotient. Every boundary
// (0.25 0.75 1.25 1.75 2.5 3.5 5) has at most 2 fraction bits, so that needs r within 4 ulps of such
// a value; nvfp4_near() flags r within 16 ulps (infinity and NaN included), and a word with a
// flagged value, or a group whose sg is zero or outside the normal range, takes the exact sign tests.
struct Nvfp4Recip {
  float inv;
  bool exact;  // sg zero, subnormal or too large for a normal reciprocal
};

__device__ __forceinline__ Nvfp4Recip nvfp4_recip(float s, float g) {
  const float sg = s * g;
  return {__builtin_amdgcn_rcpf(sg), !(sg >= 0x1p-126f && sg <= 0x1p125f)};
}

__device__ __forceinline__ bool nvfp4_near(float r) { return ((__float_as_uint(r) + 16u) & 0x1FFFFFu) < 32u; }

// N (2, 4, 6 or 8) consecutive NVFP4 codes, x[0] in the low nibble, for scale value s and global g;
// rc = nvfp4_recip(s, g). Equal to the codes of nvfp4_code().
template <int N>
__device__ __forceinline__ uint32_t nvfp4_codes(const float* x, float s, float g, Nvfp4Recip rc) {
  static_assert(N % 2 == 0 && N <= 8, "whole bytes of one word");
  float r[N];
  uint32_t nearest = 0xFFFFFFFFu;   // 0 iff some r is within 16 ulps of a boundary (nvfp4_near)
#pragma unroll
  for (int i = 0; i < N; ++i) {
    r[i] = x[i] * rc.inv;
    nearest = __builtin_elementwise_min(nearest, (__float_as_uint(r[i]) + 16u) & 0x1FFFE0u);
  }
  const bool near = rc.exact || nearest == 0u;
  // the byte selector of the conversion has to be a constant
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, r[0], r[1], 1.0f, 0);
  if constexpr (N >= 4) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[2], r[3], 1.0f, 1);
  if constexpr (N >= 6) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[4], r[5], 1.0f, 2);
  if constexpr (N >= 8) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[6], r[7], 1.0f, 3);
  if (near) w = nvfp4_codes_exact<N>(x, s, g);
  return w;
}

// Exact codes with one sign test per value and no branch on the data, for inputs with few significant
// bits (bf16), where nvfp4_codes() would fall back in nearly every wave. With inv4 = 4 rcp(s g),
// v4 = rint(|x| inv4) puts the quotient q = |x| / (s g) on a nearest multiple V = v4 / 4 of 1/4 (the
// product is within a few ulps of 4q), and d = fma(-(v4 s/4), g, |x|) has the exact sign of q - V
// (v4 s/4 has few significant bits; the FMA rounds once). Every E2M1 rounding boundary is a multiple
// of 1/4 and the next one is at least 1/2 away, so q lies within 1/8 and a few ulps of V, on the side
// that d gives, and shares its code with V moved one ulp to that side (with V itself when d = 0, where
// the conversion's ties-to-even is the rule's tie). The conversion (scale 1: nearest-even, saturating
// at 6, sign kept) encodes that value. Groups whose s g is zero or outside [2^-124, 2^125] (so that
// inv4 is finite and normal), or that hold a value that is not finite, take the exact tests.
struct Nvfp4Snap {
  float inv4;   // 4 rcp(s g)
  float s4;     // s / 4, exact
  bool exact;
};

__device__ __forceinline__ Nvfp4Snap nvfp4_snap(float s, float g, bool finite) {
  const float sg = s * g;
  return {4.0f * __builtin_amdgcn_rcpf(sg), 0.25f * s, !(finite && sg >= 0x1p-124f && sg <= 0x1p125f)};
}

template <int N>
__device__ __forceinline__ uint32_t nvfp4_codes_snap(const float* x, float s, float g, Nvfp4Snap sn) {
  static_assert(N % 2 == 0 && N <= 8, "whole bytes of one word");
  float r[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float a = __builtin_fabsf(x[i]);
    const float v4 = __builtin_rintf(a * sn.inv4);
    const uint32_t d = __float_as_uint(__builtin_fmaf(-(v4 * sn.s4), g, a));
    // + 1 for d > 0, - 1 for d < 0 (d is never -0: |x| - p rounds an exact zero to +0)
    const uint32_t vb = __float_as_uint(0.25f * v4) + (uint32_t)((int32_t)d >> 31) + ((0u - d) >> 31);
    r[i] = __uint_as_float(vb | (__float_as_uint(x[i]) & 0x80000000u));
  }
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, r[0], r[1], 1.0f, 0);
  if constexpr (N >= 4) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[2], r[3], 1.0f, 1);
  if constexpr (N >= 6) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[4], r[5], 1.0f, 2);
  if constexpr (N >= 8) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[6], r[7], 1.0f, 3);
  if (sn.exact) w = nvfp4_codes_exact<N>(x, s, g);
  return w;
}

// Maximum of v >= 0 over the four lanes l, l ^ 16, l ^ 32, l ^ 48 of a wave, in every one of them: a
// swap of odd and even 16-lane rows, then of the two 32-lane halves, each followed by a max (on the
// bit patterns, which order non-negative floats as their values).
__device__ __forceinline__ float lane_max4(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t m = a[0] > a[1] ? a[0] : a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(m, m, false, false);
  return __uint_as_float(b[0] > b[1] ? b[0] : b[1]);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// ---------------------------------------------------------------------------------------------
// Operand decode for v_smfmac_f32_16x16x64_f16.
//
// K' order. Paired-4:8 keeps two of the four pairs of every 8-K chunk, so the even elements of a
// chunk form a 4-group with exactly 2 kept elements, and so do its odd elements, at the same
// positions (the kept pair ids i0 < i1) in both: the structured 2:4 pattern of the sparse MFMA. The
// activations are laid out in the same K' order, which leaves every dot product unchanged.
// ---------------------------------------------------------------------------------------------

// Two fp4 codes of byte `sel` of w -> f16x2 (low nibble first), exact.
template <int SEL>
__device__ __forceinline__ f16x2 fp4x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

// lo16(a) | lo16(b) << 16  and  hi16(a) | hi16(b) << 16
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Operand order of one smfmac (16 K of a lane = two adjacent 8-K chunks c, c+1, c even): the four
// 4-groups of the 2:4 operand are (even K of c, even K of c+1, odd K of c, odd K of c+1). Both halves of a chunk
// then share one 2-bit position pair, so the index word of the smfmac is the byte
// code(c) | code(c+1) << 4 repeated in its two low bytes, code(q) = i0 | i1 << 2 for the nibble q
// whose set bits are i0 < i1.
//
// Dense side: the B operand reads, per lane, 16-byte LDS units holding [even K of c | even K of c+1]
// (unit c) and [odd K of c | odd K of c+1] (unit c+1) in f16.

// Dequantize the 32 codes of one 32-K group (4 chunks, low nibble = lower K) times its scale s (f16
// pair) into LDS units 0..3 of the group in B-operand order: u[2m] = even K of chunks 2m, 2m+1 and
// u[2m+1] = their odd K (each 4 + 4 f16 values, ascending K).
__device__ __forceinline__ void act_group_kprime(const u32x4& codes, f16x2 s2, u32x4 (&u)[4]) {
  const uint32_t c[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint32_t x = c[2 * m], y = c[2 * m + 1];
    const uint32_t d0 = as_u32(fp4x2_to_f16<0>(x) * s2), d1 = as_u32(fp4x2_to_f16<1>(x) * s2);
    const uint32_t d2 = as_u32(fp4x2_to_f16<2>(x) * s2), d3 = as_u32(fp4x2_to_f16<3>(x) * s2);
    const uint32_t e0 = as_u32(fp4x2_to_f16<0>(y) * s2), e1 = as_u32(fp4x2_to_f16<1>(y) * s2);
    const uint32_t e2 = as_u32(fp4x2_to_f16<2>(y) * s2), e3 = as_u32(fp4x2_to_f16<3>(y) * s2);
    u[2 * m] = u32x4{pack_lo(d0, d1), pack_lo(d2, d3), pack_lo(e0, e1), pack_lo(e2, e3)};
    u[2 * m + 1] = u32x4{pack_hi(d0, d1), pack_hi(d2, d3), pack_hi(e0, e1), pack_hi(e2, e3)};
  }
}

// Compressed A operand of one smfmac from one u32 of kept bytes: bytes (b0 b1) of chunk c and
// (b0' b1') of chunk c+1. Slots (lo b0, lo b1), (lo b0', lo b1'), (hi b0, hi b1), (hi b0', hi b1'),
// each times the block scale s (f16).
__device__ __forceinline__ f16x8 weight_operand(uint32_t kept, f16x2 s2) {
  const uint32_t c0 = as_u32(fp4x2_to_f16<0>(kept) * s2);
  const uint32_t c1 = as_u32(fp4x2_to_f16<1>(kept) * s2);
  const uint32_t c2 = as_u32(fp4x2_to_f16<2>(kept) * s2);
  const uint32_t c3 = as_u32(fp4x2_to_f16<3>(kept) * s2);
  u32x4 r;
  r.x = pack_lo(c0, c1);
  r.y = pack_lo(c2, c3);
  r.z = pack_hi(c0, c1);
  r.w = pack_hi(c2, c3);
  return __builtin_bit_cast(f16x8, r);
}

// Tiled layout: the 4 kept bytes (b0 b1)(b0' b1') of one smfmac rewritten as
// (lo b0 | lo b1 << 4, lo b0' | lo b1' << 4, hi b0 | hi b1 << 4, hi b0' | hi b1' << 4), so byte j
// converts straight to operand slots 2j, 2j+1.
__host__ __device__ inline uint32_t kept_to_tiled(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t x = lo | (lo >> 4);          // byte0 = lo b0 | lo b1 << 4, byte2 = lo b0' | lo b1' << 4
  const uint32_t y = hi | (hi >> 4);          // byte0 = hi b0 | hi b1 << 4, byte2 = hi b0' | hi b1' << 4
  return (x & 0xFFu) | (((x >> 16) & 0xFFu) << 8) | ((y & 0xFFu) << 16) | (((y >> 16) & 0xFFu) << 24);
}
__host__ __device__ inline uint32_t tiled_to_kept(uint32_t t) {
  uint32_t out = 0;
  for (int h = 0; h < 2; ++h) {                // h = 0: (b0 b1), h = 1: (b0' b1')
    const uint32_t X = (t >> (8 * h)) & 0xFFu, Y = (t >> (8 * h + 16)) & 0xFFu;
    const uint32_t b0 = (X & 15u) | ((Y & 15u) << 4), b1 = (X >> 4) | (Y & 0xF0u);
    out |= (b0 | (b1 << 8)) << (16 * h);
  }
  return out;
}

// Compressed A operand of one smfmac from one tiled u32: 4 conversions and 4 exact products.
__device__ __forceinline__ f16x8 weight_operand_tiled(uint32_t t, f16x2 s2) {
  u32x4 r;
  r.x = as_u32(fp4x2_to_f16<0>(t) * s2);
  r.y = as_u32(fp4x2_to_f16<1>(t) * s2);
  r.z = as_u32(fp4x2_to_f16<2>(t) * s2);
  r.w = as_u32(fp4x2_to_f16<3>(t) * s2);
  return __builtin_bit_cast(f16x8, r);
}

// Position code of a mask nibble: i0 | i1 << 2 for its lowest and highest set bits (the two kept
// pairs of a valid nibble), and its inverse. Nibbles without exactly two bits set are outside the
// format and do not survive the round trip.
__host__ __device__ inline uint32_t nibble_code(uint32_t q) {
  uint32_t i0 = 0, i1 = 0;
  for (uint32_t i = 0; i < 4; ++i)
    if (q & (1u << i)) i1 = i;
  for (int i = 3; i >= 0; --i)
    if (q & (1u << i)) i0 = (uint32_t)i;
  return i0 | (i1 << 2);
}
__host__ __device__ inline uint32_t code_nibble(uint32_t c) { return (1u << (c & 3u)) | (1u << (c >> 2)); }

// Code byte of a mask byte (its two chunks' nibbles, low nibble first) and back.
__host__ __device__ inline uint32_t mask_to_code_byte(uint32_t b) {
  return nibble_code(b & 15u) | (nibble_code((b >> 4) & 15u) << 4);
}
__host__ __device__ inline uint32_t code_to_mask_byte(uint32_t b) {
  return code_nibble(b & 15u) | (code_nibble((b >> 4) & 15u) << 4);
}

// Sparse-index word of one smfmac from the mask byte of its two chunks (pair-bitmask layout, through
// a 256-entry table) ...
__host__ __device__ inline uint32_t smfmac_index_of_mask_byte(uint32_t b) {
  const uint32_t y = mask_to_code_byte(b);
  return y | (y << 8);
}

// ... and from byte t of a word of code bytes (tiled layout), with one byte permute.
__device__ __forceinline__ int smfmac_index_of_codes(uint32_t codes, int t) {
  return (int)__builtin_amdgcn_perm(codes, codes, 0x0C0C0000u | ((uint32_t)t << 8) | (uint32_t)t);
}

// E4M3 scale bytes 0 and 1 (HI: 2 and 3) of sc as an f16 pair, by the hardware FP8 (E4M3FN) to f16
// conversion with unit scale: exact, since E4M3 lies inside f16's range and precision (checked for
// all 256 bytes on gfx950). A broadcast of one half folds into the consumer's op_sel.
template <bool HI = false>
__device__ __forceinline__ f16x2 scale_pair_f16(uint32_t sc) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, HI);
}

// f16 pair (v, v) of one E4M3 scale byte.
__device__ __forceinline__ f16x2 scale_bcast_f16(uint32_t b) {
  const f16x2 p = scale_pair_f16(b);
  return __builtin_shufflevector(p, p, 0, 0);
}

// Tiled weight record: 1408 bytes per (expert, 16-row tile, 256-K step).
constexpr int kTileRecordBytes = 1408;
constexpr int kTileCodeOffset = 1024;
constexpr int kTileScaleOffset = 1280;

// Word 3 of a raw buffer resource on gfx9-family targets (gfx950): no format conversion, no swizzle;
// an access past num_records bytes reads zero.
constexpr int kBufferRsrcWord3 = 0x00020000;

}  // namespace moesq

/*
 * moesq: paired-4:8 sparse NVFP4 (W4A4) MoE expert path for AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every pointer is a DEVICE pointer unless its comment says "host". Every call that takes a
 * hipStream_t is asynchronous on that stream: it validates its arguments on the host, enqueues its
 * kernels and returns; kernel faults surface at the caller's next synchronization (or inside the call
 * with MOESQ_FLAG_SYNC_CHECK). The library never allocates or frees device memory in these calls and
 * keeps no pointer after return; the caller owns every buffer, including workspaces, and keeps it
 * alive until the stream work is done. No C++ exception crosses this boundary. The calls keep no
 * global mutable state apart from a one-time kernel attribute set-up and thread-local values (the
 * text of moesq_last_error(), the profiling events of moesq_set_stage_events(), and inside a
 * moesq_moe_ffn call the events its kernels record), so they are reentrant.
 *
 * Errors: a synchronous argument check returns a negative moesq_status and enqueues nothing; a launch
 * failure (a kernel attribute that could not be set included) returns MOESQ_ERR_HIP with the HIP error
 * text in moesq_last_error().
 *
 * Storage format (model card "Qwen3.5-397B-A17B-P48NVFP4-MoESQ", section "Sparse storage layout",
 * table of stored tensors): per expert linear [out = N, in = K]
 *   packed u8 [N][K/4]   the 2 kept bytes of every 4-byte chunk of packed NVFP4, in K order;
 *   mask   u8 [N][K/16]  one nibble per 4-byte chunk, exactly 2 bits set, bit i = byte i kept,
 *                        the lower-K chunk in the low nibble;
 *   scale  u8 [N][K/32]  FP8-E4M3 (OCP, "FN") block scales, row-major ("linear layout");
 *   global f32           per-tensor scale, multiplicative: value = e2m1(code) * e4m3(scale) * global.
 * Packed NVFP4 holds two adjacent K per byte, the lower K in the low nibble. Activation NVFP4 (model
 * card "Compression details"): per 32 K an E4M3 scale = RNE(amax / (6 * global)) saturating at 448,
 * codes = RNE(x / (scale * global)) saturating at 6, ties to even, sign copied from x; global is the
 * FP32 "input_global_scale" stored per expert linear.
 */
#ifndef MOESQ_H_
#define MOESQ_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOESQ_ABI_VERSION 6
/* quantization_config marker "paired48_sparse": {"layout": "pair-bitmask", "version": 1} */
#define MOESQ_PAIR_BITMASK_VERSION 1

typedef enum {
  MOESQ_OK = 0,
  MOESQ_ERR_INVALID = -1,      /* a null pointer, a negative or inconsistent size, a bad enum */
  MOESQ_ERR_UNSUPPORTED = -2,  /* valid but outside what the kernels handle (a K not multiple of 256 ...) */
  MOESQ_ERR_WORKSPACE = -3,    /* workspace smaller than the size query returns */
  MOESQ_ERR_HIP = -4,          /* a HIP launch or synchronization failed; see moesq_last_error() */
  MOESQ_ERR_DEVICE = -5        /* (MOESQ_FLAG_SYNC_CHECK) a bounded device-side wait ran out: the
                                  outputs of the call are not valid; see moesq_last_error() */
} moesq_status;

typedef enum { MOESQ_BF16 = 0, MOESQ_F32 = 1 } moesq_dtype;

/* moe_ffn flags */
#define MOESQ_FLAG_SYNC_CHECK 1u    /* synchronize the stream before returning and report kernel errors */
#define MOESQ_FLAG_UNFUSED 2u       /* moe_ffn: separate launches even where the one-launch path applies */
#define MOESQ_FLAG_FUSED 4u         /* moe_ffn: the one-launch decode path wherever it applies */

/* Weight layouts.
 * MOESQ_LAYOUT_PAIR_BITMASK: the stored tensors packed / mask / scale as above, per expert.
 * MOESQ_LAYOUT_TILED: the same bytes re-tiled once at load time for the kernels (the model cards
 *   note that the serving stack rebuilds each layer into "the kernel's own layout" at load time):
 *   `packed` points to E * (N/16) * (K/256) records of 1408 bytes, ordered [expert][16-row tile]
 *   [256-K step]. Record lane l (row l % 16 of the tile, 64-K quarter q = l / 16 of the step) holds
 *   at 16*l the 16 kept bytes of its 64 K (every 4 bytes = two chunks (b0 b1)(b0' b1') rewritten as
 *   (lo b0 | lo b1 << 4, lo b0' | lo b1' << 4, hi b0 | hi b1 << 4, hi b0' | hi b1' << 4)), at
 *   1024 + 4*l its 4 mask bytes with each nibble replaced by the position code i0 | i1 << 2 of its
 *   two set bits i0 < i1, and at 1280 + 2*l its 2 scale bytes. mask and scale are unused (NULL).
 *   Requires K % 256 == 0 and N % 16 == 0; moesq_prepare_weights / moesq_unprepare_weights convert
 *   (exactly for masks whose nibbles have two bits set, as the format requires). */
#define MOESQ_LAYOUT_PAIR_BITMASK 0
#define MOESQ_LAYOUT_TILED 1

/* Weights of one linear of every expert. Host struct, read during the call only; its pointers are
 * device memory. Pair-bitmask layout: expert e's tensors start at e * N * (K/4), e * N * (K/16) and
 * e * N * (K/32). global [E][G]: G = 2 for a fused gate|up linear: rows [0, N/2) are gate_proj and
 * take global[e*2 + 0], rows [N/2, N) are up_proj and take global[e*2 + 1] (gate and up carry
 * separate global scales: model cards "Qwen3.8-Flash-Next-P48NVFP4-MoESQ" and
 * "Qwen3-30B-A3B-P48NVFP4-MoESQ"); G = 1 otherwise. Every pointer 16-byte aligned. */
typedef struct {
  const uint8_t *packed;   /* [E][N][K/4], or the tiled records */
  const uint8_t *mask;     /* [E][N][K/16] (pair-bitmask layout only) */
  const uint8_t *scale;    /* [E][N][K/32] (pair-bitmask layout only) */
  const float *global;     /* [E][G]       */
  int32_t E, N, K, G;
  int32_t layout;          /* MOESQ_LAYOUT_* */
} moesq_weights;

int moesq_abi_version(void);
const char *moesq_status_string(moesq_status s);           /* static string, host */
const char *moesq_last_error(void);                         /* thread-local text of the last failure, host */

/* NVFP4 quantization of activation rows (model card "Compression details", Activations row).
 *   x        [*][x_row_stride] bf16 or fp32 values; row r of the output reads x row src_row[r]
 *            (src_row NULL: row r).
 *   rows, K  output rows and K (K % 32 == 0; rows >= 0).
 *   expert_offsets [E+1] (optional): row r uses global[e] for offsets[e] <= r < offsets[e+1]; rows
 *            outside [offsets[0], offsets[E]) are not written. NULL: every row uses global[0].
 *   global   activation global scale(s) > 0 (finite, >= 2^-90 for exact rounding decisions).
 *   codes    [rows][K/2] out: two E2M1 codes per byte, lower K in the low nibble.
 *   scales   [rows][K/32] out: E4M3 bytes. x must be 16-byte aligned per row group. */
moesq_status moesq_quantize_act(const void *x, moesq_dtype x_dtype, int64_t rows, int32_t K,
                                int64_t x_row_stride, const int32_t *src_row,
                                const int32_t *expert_offsets, int32_t E, const float *global,
                                uint8_t *codes, uint8_t *scales, hipStream_t stream);

/* Stable grouping of the router's (token, slot) pairs p = t*k + j by expert id (model card
 * "Qwen3.5-397B-A17B-P48NVFP4-MoESQ": each token is routed to its top-k experts and the expert kernel
 * is a grouped GEMM, one GEMM per expert over the rows routed to it).
 *   topk_ids [T][k] int32 in [0, E), or -1 to drop the pair (ids outside [-1, E) are also dropped and
 *            counted in *status).
 *   counts [E], offsets [E+1] (exclusive prefix of counts), sorted [T*k] (the offsets[E] live pair ids
 *   in (expert, p) order; the tail is not written), inv [T*k] (row of pair p, -1 if dropped),
 *   status [1] int32 (count of ids outside [-1, E)). E in [1, 1024], k in [1, 32].
 *   workspace: moesq_permute_workspace_size(T, E) bytes of device scratch (0 for T <= 512, where
 *   workspace may be NULL). */
size_t moesq_permute_workspace_size(int64_t T, int32_t E);
moesq_status moesq_permute(const int32_t *topk_ids, int64_t T, int32_t k, int32_t E, int32_t *counts,
                           int32_t *offsets, int32_t *sorted, int32_t *inv, int32_t *status,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Grouped sparse GEMM (model card "Qwen3.5-397B-A17B-P48NVFP4-MoESQ": paired-4:8 sparse NVFP4
 * grouped GEMM over the routed experts): for each expert e and row r in [offsets[e], offsets[e+1]):
 *   out[r][n] = a_global[e] * wglobal(e, n) * sum_K e2m1(a)e4m3(a_scale) * e2m1(w)e4m3(w_scale)
 *   a_codes [rows][K/2], a_scales [rows][K/32] (as moesq_quantize_act writes them), a_global [E],
 *   expert_offsets [E+1] with offsets[E] <= rows, w: K % 256 == 0, N % 64 == 0, G in {1, 2}.
 *   out [rows][N] fp32: rows of an expert are overwritten, other rows are not written.
 *   workspace: moesq_grouped_gemm_workspace_size(E) bytes of device scratch. */
size_t moesq_grouped_gemm_workspace_size(int32_t E);
moesq_status moesq_grouped_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_global,
                                const int32_t *expert_offsets, int64_t rows, const moesq_weights *w,
                                float *out, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* MoE FFN of T tokens through the routed experts (model cards "Qwen3.5-397B-A17B-P48NVFP4-MoESQ" and
 * "Qwen3-30B-A3B-P48NVFP4-MoESQ", "Compression details": gate_proj, up_proj and down_proj of every
 * routed expert in W4A4 NVFP4 with paired-4:8 weights, activations quantized per expert linear):
 *   for each pair (t, j) with e = topk_ids[t][j] >= 0:
 *     a13 = NVFP4(x[t], a13_global[e]);  [gate | up] = a13 @ W13_e^T;  h = silu(gate) * up
 *     a2  = NVFP4(h, a2_global[e]);      y = a2 @ W2_e^T
 *     out[t] += topk_weights[t][j] * y          (sum over j in j order, fp32)
 *   x [T][H] bf16; topk_ids, topk_weights [T][k]; w13: N = 2I, K = H, G = 2; w2: N = H, K = I, G = 1;
 *   silu(v) = v / (1 + exp(-v)); h is kept in fp32 before its quantization.
 *   out [T][H] fp32, overwritten. H % 256 == 0, I % 256 == 0.
 *   workspace: moesq_moe_ffn_workspace_size(...) bytes. After the call (stream order) it holds the
 *   intermediates at the offsets moesq_moe_ffn_layout() reports: counts, offsets, sorted, inv (as
 *   moesq_permute writes them), the gate/up input codes+scales a13 in pair order (row p = t*k + j,
 *   rows of dropped pairs unwritten), the down input codes+scales a2 and the per-row down outputs
 *   (already times the router weight) in sorted order (row inv[p]); route_scratch is the
 *   permutation's scratch.
 *   Decode sizes (tiled weights, H and I <= 2048, T*k <= 4096, mean rows per expert <= 48, and one
 *   workgroup per (expert, 384 columns of I) resident at once) can run as one persistent launch with
 *   grid barriers (MOESQ_FLAG_FUSED; layout.fused = 1): same results and intermediates, except that
 *   tile_offsets and route_scratch are not written; `sync` is its barrier area (any initial
 *   contents). It assumes the device is not busy with other work holding CUs; if a barrier wait
 *   runs out (it should not), the outputs are not valid, status[0] may read -1, and a call with
 *   MOESQ_FLAG_SYNC_CHECK returns MOESQ_ERR_DEVICE (it reads the launch's own failure word, tagged
 *   with the launch, back from `sync` after the synchronization). Two fused calls on one workspace must not overlap in time.
 *   Limits: T*k*max(H, I)/2 < 2^31 (32-bit buffer offsets of the activation codes), else
 *   MOESQ_ERR_UNSUPPORTED. */
typedef struct {
  size_t counts, offsets, tile_offsets, sorted, inv, status;
  size_t a13_codes, a13_scales, a2_codes, a2_scales, down_rows, route_scratch, sync;
  size_t total;
  int32_t rows_per_mblock;   /* m-block size of the tactic the call uses */
  int32_t fused;             /* 1: a call with tiled weights runs as one persistent launch */
} moesq_ffn_layout;
moesq_status moesq_moe_ffn_layout(int64_t T, int32_t H, int32_t I, int32_t k, int32_t E, uint32_t flags,
                                  moesq_ffn_layout *layout /* host */);
size_t moesq_moe_ffn_workspace_size(int64_t T, int32_t H, int32_t I, int32_t k, int32_t E, uint32_t flags);
moesq_status moesq_moe_ffn(const void *x, int64_t T, int32_t H, const int32_t *topk_ids,
                           const float *topk_weights, int32_t k, const moesq_weights *w13,
                           const moesq_weights *w2, const float *a13_global, const float *a2_global,
                           float *out, void *workspace, size_t workspace_bytes, uint32_t flags,
                           hipStream_t stream);

/* The MoE FFN of moesq_moe_ffn without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation). The
 * workspace is a library-owned static device array of moesq_noalloc_scratch_bytes() bytes (64 MiB),
 * one per GPU the library runs on, held until the process ends; the call allocates and frees nothing.
 * Same arguments, results and intermediates (in that array) as moesq_moe_ffn with
 * MOESQ_FLAG_UNFUSED: the one-launch path is not used (MOESQ_FLAG_FUSED is ignored). Every call on a
 * GPU shares that GPU's array, which keeps the previous call's contents (no kernel of the FFN needs it
 * cleared): calls that overlap in time on one GPU race, and must not be made. Errors: those of
 * moesq_moe_ffn, plus MOESQ_ERR_WORKSPACE (nothing enqueued) when moesq_moe_ffn_workspace_size() of
 * the call exceeds the array (decode batches fit: at 128 experts, hidden 2048 and intermediate 768,
 * T*k up to about 6900 pairs), and MOESQ_ERR_HIP if the array's device address cannot be found. */
moesq_status moesq_moe_ffn_noalloc(const void *x, int64_t T, int32_t H, const int32_t *topk_ids,
                                   const float *topk_weights, int32_t k, const moesq_weights *w13,
                                   const moesq_weights *w2, const float *a13_global, const float *a2_global,
                                   float *out, uint32_t flags, hipStream_t stream);
size_t moesq_noalloc_scratch_bytes(void);

/* Router of the MoE layer (the step that feeds the permutation): per token t, softmax over the E
 * expert logits, the k most probable experts (equal probability: the lower expert id first), listed
 * by decreasing probability, and their weights: the probabilities renormalized over the k picks
 * (renormalize != 0) or the softmax probabilities themselves. The model cards keep this router
 * (`mlp.gate`) in BF16 ahead of the compressed experts (model card "Qwen3.5-397B-A17B-P48NVFP4-MoESQ",
 * "Compression details"); the softmax top-k rule is the usual one, the pages do not spell it out.
 *   logits [T][E] bf16 or fp32 (finite); topk_ids int32 [T][k], topk_weights fp32 [T][k] out.
 *   The picks compare the logits exactly; the weights are computed in fp32, within
 *   (2*S + log2(n) + n/64 + 16) * 2^-24 relative of the exact value (S: the token's max - min logit,
 *   n: the softmax terms, k or E). E <= 1024, 1 <= k <= min(E, 64); T = 0 is a no-op. Errors: a
 *   negative status for arguments out of range or a null pointer, nothing enqueued. */
moesq_status moesq_route_topk(const void *logits, moesq_dtype dtype, int64_t T, int32_t E, int32_t k,
                              int32_t renormalize, int32_t *topk_ids, float *topk_weights, hipStream_t stream);

/* Profiling aid: with events (host array of n >= 5 hipEvent_t created by the caller) set, every later
 * moesq_moe_ffn call on this host thread records events[0] on its stream before its first kernel and
 * events[1..4] after the routing (permutation and gate/up input quantization), the gate/up GEMM (with
 * the fused SiLU*up and down-input quantization), the down GEMM and the top-k combine. With n >= 13,
 * events[5 + 2i] and events[6 + 2i] are recorded by the kernels of stage i themselves (i = 0 routing,
 * 1 gate/up GEMM, 2 down GEMM, 3 combine) through their own dispatch (hipExtLaunchKernel): the stage's
 * first kernel records the start and its last kernel the end, so each pair times that stage's kernels
 * without the launch gap before them. On the one-launch path events[1..4] all follow the single
 * kernel, events[5..6] bracket it and events[7..12] are recorded right after it. NULL disables it.
 * The library keeps the pointer (thread-local) until it is reset; the caller keeps the array alive. */
moesq_status moesq_set_stage_events(hipEvent_t *events /* host */, int32_t n);

/* Failure-handling test hook: the number of polls after which a barrier wait of the one-launch decode
 * path (MOESQ_FLAG_FUSED) gives up, for later moesq_moe_ffn calls on this host thread (thread-local;
 * values above 2^32 - 1 are clamped). A negative value restores the default (2^20 polls, far beyond
 * any healthy wait). The bound is checked before each poll, so 0 makes every wait give up at once
 * while every workgroup still exits normally: the error path can be exercised without a stuck
 * device (the call then returns MOESQ_ERR_DEVICE with MOESQ_FLAG_SYNC_CHECK). */
moesq_status moesq_set_fused_spin_limit(int64_t polls);

/* Measurement aid: a throughput probe of v_smfmac_f32_16x16x64_f16, the instruction the grouped GEMMs
 * are built on, so rooflines can be quoted against the rate this GPU sustains besides the published
 * peak. Launches `blocks` workgroups of 4 waves, each wave issuing iters x 32 independent instructions
 * (4 sparse x 8 dense operands, the GEMMs' pattern; each 16 x 16 outputs over 64 dense K: 16384
 * multiply-adds on the kept half); time it with events on
 * `stream`. sink: blocks * 256 floats (device, written). *n_insts (host): instructions issued.
 * blocks >= 1, iters >= 1. */
moesq_status moesq_probe_smfmac(int32_t blocks, int32_t iters, float *sink, int64_t *n_insts /* host */,
                                hipStream_t stream);

/* Measurement aid: a read stream of `bytes` bytes from src (device, 16-byte aligned, bytes a positive
 * multiple of 16) with 16-byte loads over the whole GPU, the ceiling of kernels that read much and
 * write little; time it with events on `stream`. sink: one uint32 (device), written only if the
 * data's fold equals a fixed constant. */
moesq_status moesq_probe_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream);

/* Weight compression of a dense fp32 linear [N][K] into pair-bitmask NVFP4 (the synthetic-layer
 * recipe; model card "Compression details": paired 4:8 along K, 2 of every 4 pairs kept): in each
 * 8-K chunk keep the 2 pairs with the largest a*a + b*b (float64, ties to the lower pair),
 * global = fp32(amax of kept values) / 2688, then the NVFP4 rule above; pruned pairs are byte 0x00
 * and the mask names the kept pairs. global: 1 float out. K % 32 == 0. */
moesq_status moesq_compress_weights(const float *w, int64_t N, int32_t K, uint8_t *packed, uint8_t *mask,
                                    uint8_t *scale, float *global, hipStream_t stream);

/* Load-time re-tiling of pair-bitmask weights into MOESQ_LAYOUT_TILED and back (a permutation of
 * the same bytes, lossless both ways). src: a pair-bitmask moesq_weights (global is not touched);
 * tiled: moesq_tiled_bytes(E, N, K) bytes out (in). K % 256 == 0, N % 16 == 0. */
size_t moesq_tiled_bytes(int32_t E, int32_t N, int32_t K);
moesq_status moesq_prepare_weights(const moesq_weights *src /* host struct */, uint8_t *tiled, hipStream_t stream);
moesq_status moesq_unprepare_weights(const uint8_t *tiled, int32_t E, int32_t N, int32_t K, uint8_t *packed,
                                     uint8_t *mask, uint8_t *scale, hipStream_t stream);

/* Load-time fold of the gate/up global ratio into the block scales (model card
 * "Qwen3.8-Flash-Next-P48NVFP4-MoESQ", the note under "Compression details", and model card
 * "Qwen3-30B-A3B-P48NVFP4-MoESQ", the note after the evaluation table: gate and up carry separate
 * globals, and the serving loader folds their ratio into the block scales so that one global serves
 * both). In place on a fused gate|up linear in the pair-bitmask layout, before any re-tiling:
 *   scale  [E][N][K/32] E4M3 bytes, rows [0, N/2) gate, [N/2, N) up. Each up byte s in 0x01..0x7E
 *          becomes the E4M3 byte nearest to e4m3(s) * r (ties to even, saturating at 448),
 *          r = fp32(global[e][1] / global[e][0]); 0x00 and bytes that are not finite non-negative
 *          scales (0x7F and above) are left as they are. Gate rows are not touched.
 *   global [E][2] fp32, gate then up, positive: global[e][1] is set to global[e][0] afterwards.
 * N even, K % 32 == 0; E = 0 is a no-op. The result is lossy where a scale saturates or underflows.
 * Errors: a negative status for bad sizes or a null pointer, nothing enqueued. */
moesq_status moesq_fold_gate_up_globals(uint8_t *scale, float *global, int32_t E, int32_t N, int32_t K,
                                        hipStream_t stream);

/* Storage codec on whole tensors of `rows` rows of K (model card "Sparse storage layout": the encoding
 * is lossless).
 *   validate: *bad = number of chunk nibbles without exactly two bits set.
 *   unpack:   sparse -> dense packed NVFP4 [rows][K/2] (pruned bytes 0x00); a bad nibble is counted
 *             in *bad and its chunk written as zeros.
 *   pack:     dense -> sparse with the kept bytes = the nonzero ones, a chunk with fewer than two
 *             completed with its lowest-index zero bytes; a chunk with more than two is counted in
 *             *bad. K % 16 == 0 (K % 32 for whole mask bytes per row). bad: 1 int32. */
moesq_status moesq_validate_weights(const uint8_t *mask, int64_t rows, int32_t K, int32_t *bad,
                                    hipStream_t stream);
moesq_status moesq_unpack_pair_bitmask(const uint8_t *packed, const uint8_t *mask, int64_t rows, int32_t K,
                                       uint8_t *dense, int32_t *bad, hipStream_t stream);
moesq_status moesq_pack_pair_bitmask(const uint8_t *dense, int64_t rows, int32_t K, uint8_t *packed,
                                     uint8_t *mask, int32_t *bad, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOESQ_H_ */

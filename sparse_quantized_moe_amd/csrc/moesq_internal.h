// Host-side launchers shared between the kernel files and the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "moesq.h"

namespace moesq {

// Rows of x (gathered through src_row when given) quantized with global[0], or with global[e] for
// the rows offsets[e] .. offsets[e+1] when offsets is given.
void launch_quantize(const void* x, bool f32, int64_t rows, int K, int64_t stride, const int* src_row,
                     const int* offsets, int E, const float* global, uint8_t* codes, uint8_t* scales,
                     hipStream_t stream);
void launch_compress(const float* w, int64_t N, int K, uint8_t* packed, uint8_t* mask, uint8_t* scale,
                     float* global, hipStream_t stream);
void launch_validate(const uint8_t* mask, int64_t nbytes, int* bad, hipStream_t stream);
void launch_unpack(const uint8_t* packed, const uint8_t* mask, int64_t nbytes, uint8_t* dense, int* bad,
                   hipStream_t stream);
void launch_pack(const uint8_t* dense, int64_t nbytes, uint8_t* packed, uint8_t* mask, int* bad,
                 hipStream_t stream);
void launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t stream);

// Load-time re-tiling into the kernels' weight layout (see include/moesq.h, MOESQ_LAYOUT_TILED).
size_t tiled_bytes(int E, int N, int K);
void launch_prepare(const uint8_t* packed, const uint8_t* mask, const uint8_t* scale, int E, int N, int K,
                    uint8_t* tiled, hipStream_t stream);
void launch_fold_gate_up(uint8_t* scale, float* global, int E, int N, int K, hipStream_t stream);
void launch_unprepare(const uint8_t* tiled, int E, int N, int K, uint8_t* packed, uint8_t* mask, uint8_t* scale,
                      hipStream_t stream);

// Routing: counts[E], offsets[E+1], sorted[T*k] (live prefix), inv[T*k], tile_offsets[E+1] (prefix
// of ceil(count/bm) for the grouped GEMM's m-blocks, when bm > 0) and status[0] (number of ids
// outside [-1, E), which are dropped); with x (bf16 [T][H]) also the NVFP4 codes [T*k][H/2] and
// scales [T*k][H/32] of every live pair p, row p, with global a_global[ids[p]]. scratch holds
// route_scratch_bytes(T, E) bytes (none for T <= 512).
size_t route_scratch_bytes(int64_t T, int E);
void launch_route(const int* ids, int64_t T, int k, int E, int* counts, int* offsets, int* tile_offsets, int bm,
                  int* sorted, int* inv, int* status, void* scratch, const uint16_t* x, int H, const float* a_global,
                  uint8_t* codes, uint8_t* scales, hipStream_t stream);
// tile_offsets from offsets for m-blocks of bm rows.
void launch_tile_offsets(const int* offsets, int E, int bm, int* tile_offsets, hipStream_t stream);

// The prefill GEMMs hand the last items out through claim counters that follow the E + 1 m-block
// offsets: one for the GEMM of a plain or gate/up call, one for the down GEMM. Every launch that
// writes tile_offsets zeroes them, so tile_offsets needs E + 1 + kPrefillPools ints.
constexpr int kPrefillPools = 2;
__host__ __device__ inline int* prefill_pools(const int* tile_offsets, int E) {
  return const_cast<int*>(tile_offsets) + E + 1;
}

// Grouped sparse GEMM variants.
enum { kEpiStore = 0, kEpiGateUp = 1, kEpiDown = 2 };
enum { kTacticDecode = 0, kTacticPrefill = 1 };
int tactic_rows_per_mblock(int tactic);
// Dynamic LDS bytes of a GEMM workgroup of the tactic for reduction length K.
size_t gemm_lds_bytes(int tactic, int K);
constexpr size_t kMaxLdsBytes = 160 * 1024;

struct GemmParams {
  // B operand: activation codes [.][K/2], scales [.][K/32]; expert e owns GEMM rows offsets[e]..
  // offsets[e+1]-1, and GEMM row r reads activation row a_rows[r] (row r itself when a_rows is null)
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_global;     // [E]
  const int* offsets;        // [E+1]
  const int* tile_offsets;   // [E+1], m-blocks of tactic_rows_per_mblock rows
  const int* a_rows;         // [rows] or null
  int64_t rows;              // rows of A (upper bound of offsets[E])
  // weights, pair-bitmask storage [E][N][K/4], [E][N][K/16], [E][N][K/32], global [E][G]
  const uint8_t* w_packed;
  const uint8_t* w_mask;
  const uint8_t* w_scale;
  const float* w_global;
  int E, N, K, G;
  int layout;                // 0 pair-bitmask storage, 1 tiled records (w_packed only)
  // kEpiStore / kEpiDown: fp32 rows [rows][N]
  float* out;
  // kEpiGateUp: h = silu(gate) * up quantized with h_global[e] into h_codes [rows][N/4], h_scales [rows][N/64]
  uint8_t* h_codes;
  uint8_t* h_scales;
  const float* h_global;
  // kEpiDown: router weight of each sorted row = topk_weights[sorted[row]]
  const float* topk_weights;
  const int* sorted;
};
void launch_grouped_gemm(const GemmParams& p, int epi, int tactic, hipStream_t stream);

// Decode-size FFN in one persistent launch (ffn_fused.hip): tiled weights, H, I <= 2048,
// T*k <= 4096, and every (expert, part) workgroup resident at once.
struct FusedLaunch {
  const uint16_t* x;
  const int* ids;
  const float* topk_weights;
  const float* a13_global;
  const float* a2_global;
  const uint8_t* w13;
  const float* w13_global;
  const uint8_t* w2;
  const float* w2_global;
  int64_t T;
  int H, I, k, E;
  int* counts;
  int* offsets;
  int* sorted;
  int* inv;
  int* status;
  uint8_t* a13c;
  uint8_t* a13s;
  uint8_t* a2c;
  uint8_t* a2s;
  float* D;
  float* out;
  uint8_t* sync;      // kFusedSyncBytes of workspace: release word, error word, arrival flags (any contents)
  int64_t spin_limit;   // polls before a barrier wait gives up (negative: the default)
};
constexpr size_t kFusedSyncBytes = 64 + 8 * 1024;
bool fused_applicable(int64_t T, int H, int I, int k, int E);
// Enqueues the one-launch path; *ticket receives the launch's ticket, which the kernel writes into
// the error word (sync + kFusedErrOffset) if one of its barrier waits runs out.
hipError_t launch_ffn_fused(const FusedLaunch& f, hipStream_t stream, unsigned* ticket);
constexpr size_t kFusedErrOffset = 8;

// Router softmax top-k (router.hip): E <= 1024, 1 <= k <= min(E, 64).
void launch_route_topk(const void* logits, bool f32, int64_t T, int E, int k, bool renormalize, int* ids,
                       float* wts, hipStream_t stream);

// smfmac throughput probe (probe.hip): returns the number of instructions the launch issues.
int64_t launch_probe_smfmac(int blocks, int iters, float* sink, hipStream_t stream);
void launch_probe_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

// A host-side HIP failure met while preparing a launch (a kernel attribute that could not be set):
// the launch is skipped and the error is reported by the calling entry point (thread-local).
void note_hip_error(hipError_t e);
hipError_t take_hip_error();
// Records msg as this thread's moesq_last_error() text and returns s.
moesq_status report(moesq_status s, const char* msg);
// The argument checks of moesq_moe_ffn that do not involve its workspace (MOESQ_OK with T == 0: a
// no-op); they touch no device.
moesq_status validate_ffn_args(const void* x, int64_t T, int32_t H, const int32_t* topk_ids, const float* topk_weights,
                               int32_t k, const moesq_weights* w13, const moesq_weights* w2, const float* a13_global,
                               const float* a2_global, const float* out);

// out[t][:] = sum_j D[inv[t*k + j]][:] (rows with inv < 0 skipped), in j order.
void launch_combine(const float* D, const int* inv, int64_t T, int k, int H, float* out, hipStream_t stream);

// Optional start/stop events that the kernels of one FFN stage record themselves through their own
// dispatch (hipExtLaunchKernelGGL): the stage's first kernel records the start, every kernel the end
// (the last one's stands), so the pair times the stage's kernels without the launch gap before them.
// Both null: plain launches.
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
KernelEvents& kernel_events();   // this host thread's

template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream, Args... args) {
  KernelEvents& ev = kernel_events();
  if (ev.start || ev.stop) {
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, stream, ev.start, ev.stop, 0u, args...);
    ev.start = nullptr;
  } else {
    kernel<<<grid, block, lds, stream>>>(args...);
  }
}

}  // namespace moesq

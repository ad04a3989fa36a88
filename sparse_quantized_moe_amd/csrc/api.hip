// C ABI of the moesq library: argument checks, workspace layout and kernel launches.
#include <string>
#include <cstdio>

#include "moesq.h"
#include "moesq_internal.h"

namespace moesq {

namespace {
thread_local hipError_t g_pending_hip_error = hipSuccess;
}

void note_hip_error(hipError_t e) {
  if (g_pending_hip_error == hipSuccess) g_pending_hip_error = e;
}

hipError_t take_hip_error() {
  const hipError_t e = g_pending_hip_error;
  g_pending_hip_error = hipSuccess;
  return e;
}

}  // namespace moesq

namespace {

thread_local std::string g_last_error;

}  // namespace

moesq_status moesq::report(moesq_status s, const char* msg) {
  g_last_error = msg;
  return s;
}

namespace {

thread_local int64_t g_fused_spin_limit = -1;
thread_local hipEvent_t* g_stage_events = nullptr;
thread_local int g_stage_n = 0;

// With 13 stage events, events[5 + 2 i] and events[6 + 2 i] are recorded by stage i's own kernels
// (0 routing, 1 gate/up GEMM, 2 down GEMM, 3 combine), at the first one's start and the last one's end.
struct TimedKernel {
  explicit TimedKernel(int stage) {
    if (g_stage_events && g_stage_n >= 13)
      moesq::kernel_events() = {g_stage_events[5 + 2 * stage], g_stage_events[6 + 2 * stage]};
  }
  ~TimedKernel() { moesq::kernel_events() = {}; }
};

void stage_event(int i, hipStream_t stream) {
  if (g_stage_events) (void)hipEventRecord(g_stage_events[i], stream);
}

moesq_status fail(moesq_status s, const char* fmt, const char* what) {
  char buf[512];
  std::snprintf(buf, sizeof buf, fmt, what);
  g_last_error = buf;
  return s;
}
#define MOESQ_REQUIRE(cond, status, msg) \
  do { if (!(cond)) return fail(status, "%s", msg); } while (0)

moesq_status check_launch(hipStream_t stream, bool sync) {
  const hipError_t pending = moesq::take_hip_error();   // a launch skipped for a refused attribute
  hipError_t e = hipGetLastError();
  if (pending != hipSuccess) e = pending;
  if (e == hipSuccess && sync) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(MOESQ_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return MOESQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

moesq_status check_weights(const moesq_weights* w, const char* name) {
  if (!w) return fail(MOESQ_ERR_INVALID, "%s: null weights struct", name);
  if (w->layout != MOESQ_LAYOUT_PAIR_BITMASK && w->layout != MOESQ_LAYOUT_TILED)
    return fail(MOESQ_ERR_INVALID, "%s: unknown weight layout", name);
  const bool tiled = w->layout == MOESQ_LAYOUT_TILED;
  if (!w->packed || !w->global || (!tiled && (!w->mask || !w->scale)))
    return fail(MOESQ_ERR_INVALID, "%s: null weight pointer", name);
  if (w->E < 1 || w->N < 1 || w->K < 1) return fail(MOESQ_ERR_INVALID, "%s: E, N, K must be positive", name);
  if (w->G != 1 && w->G != 2) return fail(MOESQ_ERR_INVALID, "%s: G must be 1 or 2", name);
  if (w->K % 32) return fail(MOESQ_ERR_INVALID, "%s: K must be a multiple of 32", name);
  if (w->K % 256) return fail(MOESQ_ERR_UNSUPPORTED, "%s: the GEMM needs K % 256 == 0", name);
  if (w->N % 64) return fail(MOESQ_ERR_UNSUPPORTED, "%s: the GEMM needs N % 64 == 0", name);
  if (w->E > 1024) return fail(MOESQ_ERR_UNSUPPORTED, "%s: at most 1024 experts", name);
  if (!aligned16(w->packed) || (!tiled && (!aligned16(w->mask) || !aligned16(w->scale))))
    return fail(MOESQ_ERR_INVALID, "%s: weight tensors must be 16-byte aligned", name);
  return MOESQ_OK;
}

// Small batches (mean rows per expert <= 48) stream each expert's weights once per 32 rows with the
// activations of the whole K in LDS; large ones tile 128 rows and reuse each decoded weight fragment.
int ffn_tactic(int64_t rows, int32_t E, int32_t K1, int32_t K2) {
  const bool fits = moesq::gemm_lds_bytes(moesq::kTacticDecode, K1) <= moesq::kMaxLdsBytes &&
                    moesq::gemm_lds_bytes(moesq::kTacticDecode, K2) <= moesq::kMaxLdsBytes;
  return (rows <= (int64_t)48 * E && fits) ? moesq::kTacticDecode : moesq::kTacticPrefill;
}

// The one-launch decode path (ffn_fused.hip) for the decode tactic when the shapes and the device
// allow it and the caller asks for it.
bool ffn_fused(int64_t T, int32_t H, int32_t I, int32_t k, int32_t E, int tactic, uint32_t flags) {
  const bool want = (flags & MOESQ_FLAG_FUSED) && !(flags & MOESQ_FLAG_UNFUSED);
  return want && tactic == moesq::kTacticDecode && moesq::fused_applicable(T, H, I, k, E);
}

}  // namespace

extern "C" {

int moesq_abi_version(void) { return MOESQ_ABI_VERSION; }

const char* moesq_status_string(moesq_status s) {
  switch (s) {
    case MOESQ_OK: return "ok";
    case MOESQ_ERR_INVALID: return "invalid argument";
    case MOESQ_ERR_UNSUPPORTED: return "unsupported shape";
    case MOESQ_ERR_WORKSPACE: return "workspace too small";
    case MOESQ_ERR_HIP: return "HIP error";
    case MOESQ_ERR_DEVICE: return "device-side wait ran out";
  }
  return "unknown status";
}

const char* moesq_last_error(void) { return g_last_error.c_str(); }

moesq_status moesq_set_stage_events(hipEvent_t* events, int32_t n) {
  MOESQ_REQUIRE(!events || n >= 5, MOESQ_ERR_INVALID, "set_stage_events: need at least 5 events");
  g_stage_events = events;
  g_stage_n = events ? n : 0;
  return MOESQ_OK;
}

moesq_status moesq_set_fused_spin_limit(int64_t polls) {
  g_fused_spin_limit = polls < 0 ? -1 : (polls > 0xFFFFFFFFll ? 0xFFFFFFFFll : polls);
  return MOESQ_OK;
}

moesq_status moesq_route_topk(const void* logits, moesq_dtype dtype, int64_t T, int32_t E, int32_t k,
                              int32_t renormalize, int32_t* topk_ids, float* topk_weights, hipStream_t stream) {
  MOESQ_REQUIRE(T >= 0 && E >= 1 && E <= 1024 && k >= 1 && k <= E && k <= 64, MOESQ_ERR_INVALID,
                "route_topk: T >= 0, 1 <= E <= 1024, 1 <= k <= min(E, 64)");
  MOESQ_REQUIRE(dtype == MOESQ_BF16 || dtype == MOESQ_F32, MOESQ_ERR_INVALID, "route_topk: bad dtype");
  if (T == 0) return MOESQ_OK;
  MOESQ_REQUIRE(logits && topk_ids && topk_weights, MOESQ_ERR_INVALID, "route_topk: null pointer");
  moesq::launch_route_topk(logits, dtype == MOESQ_F32, T, E, k, renormalize != 0, topk_ids, topk_weights, stream);
  return check_launch(stream, false);
}

moesq_status moesq_probe_smfmac(int32_t blocks, int32_t iters, float* sink, int64_t* n_insts, hipStream_t stream) {
  MOESQ_REQUIRE(blocks >= 1 && iters >= 1 && sink && n_insts, MOESQ_ERR_INVALID,
                "probe_smfmac: blocks >= 1, iters >= 1, sink and n_insts required");
  *n_insts = moesq::launch_probe_smfmac(blocks, iters, sink, stream);
  return check_launch(stream, false);
}

moesq_status moesq_probe_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  MOESQ_REQUIRE(src && sink && bytes >= 16 && bytes % 16 == 0, MOESQ_ERR_INVALID,
                "probe_read: src and sink required, bytes a positive multiple of 16");
  MOESQ_REQUIRE((reinterpret_cast<uintptr_t>(src) & 15u) == 0, MOESQ_ERR_INVALID, "probe_read: src must be 16-byte aligned");
  moesq::launch_probe_read(src, bytes, sink, stream);
  return check_launch(stream, false);
}

moesq_status moesq_quantize_act(const void* x, moesq_dtype x_dtype, int64_t rows, int32_t K, int64_t x_row_stride,
                                const int32_t* src_row, const int32_t* expert_offsets, int32_t E, const float* global,
                                uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  MOESQ_REQUIRE(rows >= 0 && K > 0, MOESQ_ERR_INVALID, "quantize_act: rows >= 0 and K > 0 required");
  MOESQ_REQUIRE(K % 32 == 0, MOESQ_ERR_INVALID, "quantize_act: K must be a multiple of 32");
  MOESQ_REQUIRE(x_dtype == MOESQ_BF16 || x_dtype == MOESQ_F32, MOESQ_ERR_INVALID, "quantize_act: bad dtype");
  if (rows == 0) return MOESQ_OK;
  MOESQ_REQUIRE(x && global && codes && scales, MOESQ_ERR_INVALID, "quantize_act: null pointer");
  MOESQ_REQUIRE(x_row_stride >= K, MOESQ_ERR_INVALID, "quantize_act: x_row_stride < K");
  MOESQ_REQUIRE(aligned16(x) && aligned16(codes), MOESQ_ERR_INVALID, "quantize_act: x and codes must be 16-byte aligned");
  MOESQ_REQUIRE((x_row_stride * (x_dtype == MOESQ_F32 ? 4 : 2)) % 16 == 0, MOESQ_ERR_INVALID,
                "quantize_act: x row stride must be a multiple of 16 bytes");
  MOESQ_REQUIRE(!expert_offsets || E >= 1, MOESQ_ERR_INVALID, "quantize_act: E >= 1 with expert_offsets");
  moesq::launch_quantize(x, x_dtype == MOESQ_F32, rows, K, x_row_stride, src_row, expert_offsets, E, global, codes,
                         scales, stream);
  return check_launch(stream, false);
}

size_t moesq_permute_workspace_size(int64_t T, int32_t E) {
  if (T < 0 || E < 1) return 0;
  return moesq::route_scratch_bytes(T, E);
}

moesq_status moesq_permute(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t* counts, int32_t* offsets,
                           int32_t* sorted, int32_t* inv, int32_t* status, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  MOESQ_REQUIRE(T >= 0 && k >= 1 && k <= 32 && E >= 1, MOESQ_ERR_INVALID, "permute: T >= 0, 1 <= k <= 32, E >= 1");
  MOESQ_REQUIRE(E <= 1024, MOESQ_ERR_UNSUPPORTED, "permute: at most 1024 experts");
  MOESQ_REQUIRE(counts && offsets && status && (T == 0 || (topk_ids && sorted && inv)), MOESQ_ERR_INVALID,
                "permute: null pointer");
  MOESQ_REQUIRE(T * k < (int64_t)1 << 31, MOESQ_ERR_UNSUPPORTED, "permute: T*k must fit in int32");
  const size_t need = moesq::route_scratch_bytes(T, E);
  MOESQ_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), MOESQ_ERR_WORKSPACE, "permute: workspace too small");
  moesq::launch_route(topk_ids, T, k, E, counts, offsets, nullptr, 0, sorted, inv, status, workspace, nullptr, 0,
                      nullptr, nullptr, nullptr, stream);
  return check_launch(stream, false);
}

size_t moesq_grouped_gemm_workspace_size(int32_t E) { return align256((size_t)(E + 1 + moesq::kPrefillPools) * 4); }

moesq_status moesq_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
                                const int32_t* expert_offsets, int64_t rows, const moesq_weights* w, float* out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  moesq_status s = check_weights(w, "grouped_gemm");
  if (s != MOESQ_OK) return s;
  MOESQ_REQUIRE(rows >= 0, MOESQ_ERR_INVALID, "grouped_gemm: rows >= 0");
  if (rows == 0) return MOESQ_OK;
  MOESQ_REQUIRE(a_codes && a_scales && a_global && expert_offsets && out && workspace, MOESQ_ERR_INVALID,
                "grouped_gemm: null pointer");
  MOESQ_REQUIRE(workspace_bytes >= moesq_grouped_gemm_workspace_size(w->E), MOESQ_ERR_WORKSPACE,
                "grouped_gemm: workspace too small");
  MOESQ_REQUIRE(aligned16(out) && aligned16(a_codes) && ((uintptr_t)a_scales & 3) == 0, MOESQ_ERR_INVALID,
                "grouped_gemm: out and a_codes must be 16-byte aligned, a_scales 4-byte aligned");
  MOESQ_REQUIRE(rows * (w->K / 2) < ((int64_t)1 << 31), MOESQ_ERR_UNSUPPORTED,
                "grouped_gemm: activation codes must stay below 2 GiB (32-bit buffer offsets)");
  const int tactic = ffn_tactic(rows, w->E, w->K, w->K);
  int32_t* tile_offsets = static_cast<int32_t*>(workspace);
  moesq::launch_tile_offsets(expert_offsets, w->E, moesq::tactic_rows_per_mblock(tactic), tile_offsets, stream);
  moesq::GemmParams p{};
  p.a_codes = a_codes; p.a_scales = a_scales; p.a_global = a_global; p.offsets = expert_offsets;
  p.tile_offsets = tile_offsets; p.rows = rows;
  p.w_packed = w->packed; p.w_mask = w->mask; p.w_scale = w->scale; p.w_global = w->global;
  p.E = w->E; p.N = w->N; p.K = w->K; p.G = w->G; p.layout = w->layout; p.out = out;
  moesq::launch_grouped_gemm(p, moesq::kEpiStore, tactic, stream);
  return check_launch(stream, false);
}

moesq_status moesq_moe_ffn_layout(int64_t T, int32_t H, int32_t I, int32_t k, int32_t E, uint32_t flags,
                                  moesq_ffn_layout* L) {
  MOESQ_REQUIRE(L, MOESQ_ERR_INVALID, "moe_ffn_layout: null layout");
  MOESQ_REQUIRE(T >= 0 && H > 0 && I > 0 && k >= 1 && E >= 1, MOESQ_ERR_INVALID, "moe_ffn_layout: bad sizes");
  const size_t P = (size_t)T * k;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  L->counts = take((size_t)E * 4);
  L->offsets = take((size_t)(E + 1) * 4);
  L->tile_offsets = take((size_t)(E + 1 + moesq::kPrefillPools) * 4);
  L->status = take(4);
  L->sorted = take(P * 4);
  L->inv = take(P * 4);
  L->a13_codes = take(P * (size_t)(H / 2));
  L->a13_scales = take(P * (size_t)(H / 32));
  L->a2_codes = take(P * (size_t)(I / 2));
  L->a2_scales = take(P * (size_t)(I / 32));
  L->down_rows = take(P * (size_t)H * 4);
  L->route_scratch = take(moesq::route_scratch_bytes(T, E));
  L->sync = take(moesq::kFusedSyncBytes);
  L->total = off;
  const int tactic = ffn_tactic(T * k, E, H, I);
  L->rows_per_mblock = moesq::tactic_rows_per_mblock(tactic);
  L->fused = ffn_fused(T, H, I, k, E, tactic, flags) ? 1 : 0;
  return MOESQ_OK;
}

size_t moesq_moe_ffn_workspace_size(int64_t T, int32_t H, int32_t I, int32_t k, int32_t E, uint32_t flags) {
  moesq_ffn_layout L;
  if (moesq_moe_ffn_layout(T, H, I, k, E, flags, &L) != MOESQ_OK) return 0;
  return L.total;
}

}  // extern "C"

// The argument checks of moesq_moe_ffn that do not involve the workspace (shared with the
// allocation-free variant). MOESQ_OK with T == 0 means a no-op.
moesq_status moesq::validate_ffn_args(const void* x, int64_t T, int32_t H, const int32_t* topk_ids,
                                      const float* topk_weights, int32_t k, const moesq_weights* w13,
                                      const moesq_weights* w2, const float* a13_global, const float* a2_global,
                                      const float* out) {
  moesq_status s = check_weights(w13, "moe_ffn w13");
  if (s != MOESQ_OK) return s;
  s = check_weights(w2, "moe_ffn w2");
  if (s != MOESQ_OK) return s;
  MOESQ_REQUIRE(T >= 0 && k >= 1 && k <= 32, MOESQ_ERR_INVALID, "moe_ffn: T >= 0 and 1 <= k <= 32");
  const int32_t E = w13->E, I = w2->K;
  MOESQ_REQUIRE(w2->E == E, MOESQ_ERR_INVALID, "moe_ffn: w13 and w2 expert counts differ");
  MOESQ_REQUIRE(w13->G == 2 && w2->G == 1, MOESQ_ERR_INVALID, "moe_ffn: w13 needs G = 2 (gate|up), w2 G = 1");
  MOESQ_REQUIRE(w13->K == H && w2->N == H && w13->N == 2 * I, MOESQ_ERR_INVALID,
                "moe_ffn: shapes must be w13 [2I, H], w2 [H, I]");
  MOESQ_REQUIRE(I % 256 == 0 && H % 256 == 0, MOESQ_ERR_UNSUPPORTED, "moe_ffn: H and I must be multiples of 256");
  MOESQ_REQUIRE(T * k < ((int64_t)1 << 31), MOESQ_ERR_UNSUPPORTED, "moe_ffn: T*k must fit in int32");
  MOESQ_REQUIRE(T * k * ((H > I ? H : I) / 2) < ((int64_t)1 << 31), MOESQ_ERR_UNSUPPORTED,
                "moe_ffn: the gate/up and down input codes must stay below 2 GiB (32-bit buffer offsets)");
  if (T == 0) return MOESQ_OK;
  MOESQ_REQUIRE(x && topk_ids && topk_weights && a13_global && a2_global && out, MOESQ_ERR_INVALID,
                "moe_ffn: null pointer");
  MOESQ_REQUIRE(aligned16(x) && aligned16(out), MOESQ_ERR_INVALID, "moe_ffn: x and out must be 16-byte aligned");
  return MOESQ_OK;
}

extern "C" {

moesq_status moesq_moe_ffn(const void* x, int64_t T, int32_t H, const int32_t* topk_ids, const float* topk_weights,
                           int32_t k, const moesq_weights* w13, const moesq_weights* w2, const float* a13_global,
                           const float* a2_global, float* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                           hipStream_t stream) {
  moesq_status s = moesq::validate_ffn_args(x, T, H, topk_ids, topk_weights, k, w13, w2, a13_global, a2_global, out);
  if (s != MOESQ_OK || T == 0) return s;
  const int32_t E = w13->E, I = w2->K;
  MOESQ_REQUIRE(workspace, MOESQ_ERR_INVALID, "moe_ffn: null pointer");
  MOESQ_REQUIRE(aligned16(workspace), MOESQ_ERR_INVALID, "moe_ffn: x, out and workspace must be 16-byte aligned");
  moesq_ffn_layout L;
  moesq_moe_ffn_layout(T, H, I, k, E, flags, &L);
  MOESQ_REQUIRE(workspace_bytes >= L.total, MOESQ_ERR_WORKSPACE, "moe_ffn: workspace too small");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* tile_offsets = reinterpret_cast<int32_t*>(ws + L.tile_offsets);
  int32_t* status = reinterpret_cast<int32_t*>(ws + L.status);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);
  uint8_t* a13c = ws + L.a13_codes;
  uint8_t* a13s = ws + L.a13_scales;
  uint8_t* a2c = ws + L.a2_codes;
  uint8_t* a2s = ws + L.a2_scales;
  float* drows = reinterpret_cast<float*>(ws + L.down_rows);
  const int tactic = ffn_tactic(T * k, E, H, I);
  const int64_t P = T * k;

  if (L.fused && w13->layout == 1 && w2->layout == 1) {
    moesq::FusedLaunch f{};
    f.x = static_cast<const uint16_t*>(x); f.ids = topk_ids; f.topk_weights = topk_weights;
    f.a13_global = a13_global; f.a2_global = a2_global;
    f.w13 = w13->packed; f.w13_global = w13->global; f.w2 = w2->packed; f.w2_global = w2->global;
    f.T = T; f.H = H; f.I = I; f.k = k; f.E = E;
    f.counts = counts; f.offsets = offsets; f.sorted = sorted; f.inv = inv; f.status = status;
    f.a13c = a13c; f.a13s = a13s; f.a2c = a2c; f.a2s = a2s; f.D = drows; f.out = out; f.sync = ws + L.sync;
    f.spin_limit = g_fused_spin_limit;
    stage_event(0, stream);
    hipError_t err;
    unsigned ticket = 0;
    {
      const TimedKernel timed(0);
      err = moesq::launch_ffn_fused(f, stream, &ticket);
    }
    for (int i = 1; i <= 4; ++i) stage_event(i, stream);
    if (g_stage_events && g_stage_n >= 13)
      for (int i = 7; i <= 12; ++i) stage_event(i, stream);   // the other stages: empty, after the kernel
    if (err != hipSuccess) return fail(MOESQ_ERR_HIP, "moe_ffn: fused launch: %s", hipGetErrorString(err));
    const bool sync = (flags & MOESQ_FLAG_SYNC_CHECK) != 0;
    const moesq_status st = check_launch(stream, sync);
    if (st != MOESQ_OK || !sync) return st;
    // the kernel tags its error word with the launch's ticket when a barrier wait ran out
    unsigned word = 0;
    hipError_t e = hipMemcpyAsync(&word, ws + L.sync + moesq::kFusedErrOffset, sizeof word, hipMemcpyDeviceToHost,
                                  stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(MOESQ_ERR_HIP, "moe_ffn: reading the barrier error word: %s", hipGetErrorString(e));
    if (word == ticket)
      return fail(MOESQ_ERR_DEVICE, "%s", "moe_ffn: a barrier wait of the one-launch path ran out; outputs are not valid");
    return MOESQ_OK;
  }

  // routing: permutation + gate/up input quantization (pair order)
  stage_event(0, stream);
  {
    const TimedKernel timed(0);
    moesq::launch_route(topk_ids, T, k, E, counts, offsets, tile_offsets, L.rows_per_mblock, sorted, inv, status,
                        ws + L.route_scratch, static_cast<const uint16_t*>(x), H, a13_global, a13c, a13s, stream);
  }
  stage_event(1, stream);
  // gate/up GEMM, row r reading activation row sorted[r]; fused silu * up and down-input quantization
  moesq::GemmParams g{};
  g.a_codes = a13c; g.a_scales = a13s; g.a_global = a13_global; g.offsets = offsets; g.tile_offsets = tile_offsets;
  g.a_rows = sorted; g.rows = P; g.w_packed = w13->packed; g.w_mask = w13->mask; g.w_scale = w13->scale; g.w_global = w13->global;
  g.E = E; g.N = w13->N; g.K = H; g.G = 2; g.layout = w13->layout; g.h_codes = a2c; g.h_scales = a2s; g.h_global = a2_global;
  {
    const TimedKernel timed(1);
    moesq::launch_grouped_gemm(g, moesq::kEpiGateUp, tactic, stream);
  }
  stage_event(2, stream);
  moesq::GemmParams d{};
  d.a_codes = a2c; d.a_scales = a2s; d.a_global = a2_global; d.offsets = offsets; d.tile_offsets = tile_offsets;
  d.rows = P; d.w_packed = w2->packed; d.w_mask = w2->mask; d.w_scale = w2->scale; d.w_global = w2->global;
  d.E = E; d.N = H; d.K = I; d.G = 1; d.layout = w2->layout; d.out = drows; d.topk_weights = topk_weights; d.sorted = sorted;
  {
    const TimedKernel timed(2);
    moesq::launch_grouped_gemm(d, moesq::kEpiDown, tactic, stream);
  }
  stage_event(3, stream);
  {
    const TimedKernel timed(3);
    moesq::launch_combine(drows, inv, T, k, H, out, stream);
  }
  stage_event(4, stream);
  return check_launch(stream, (flags & MOESQ_FLAG_SYNC_CHECK) != 0);
}

moesq_status moesq_compress_weights(const float* w, int64_t N, int32_t K, uint8_t* packed, uint8_t* mask, uint8_t* scale,
                                    float* global, hipStream_t stream) {
  MOESQ_REQUIRE(N >= 1 && K >= 32 && K % 32 == 0, MOESQ_ERR_INVALID, "compress_weights: N >= 1, K % 32 == 0");
  MOESQ_REQUIRE(w && packed && mask && scale && global, MOESQ_ERR_INVALID, "compress_weights: null pointer");
  MOESQ_REQUIRE(aligned16(w) && ((uintptr_t)packed & 3) == 0 && ((uintptr_t)mask & 1) == 0 && ((uintptr_t)global & 3) == 0,
                MOESQ_ERR_INVALID, "compress_weights: w 16-byte, packed 4-byte, mask 2-byte aligned");
  moesq::launch_compress(w, N, K, packed, mask, scale, global, stream);
  return check_launch(stream, false);
}

size_t moesq_tiled_bytes(int32_t E, int32_t N, int32_t K) {
  if (E < 1 || N < 16 || K < 256 || N % 16 || K % 256) return 0;
  return moesq::tiled_bytes(E, N, K);
}

moesq_status moesq_prepare_weights(const moesq_weights* src, uint8_t* tiled, hipStream_t stream) {
  MOESQ_REQUIRE(src && tiled, MOESQ_ERR_INVALID, "prepare_weights: null pointer");
  MOESQ_REQUIRE(src->layout == MOESQ_LAYOUT_PAIR_BITMASK, MOESQ_ERR_INVALID, "prepare_weights: source must be pair-bitmask");
  MOESQ_REQUIRE(src->packed && src->mask && src->scale, MOESQ_ERR_INVALID, "prepare_weights: null weight pointer");
  MOESQ_REQUIRE(src->E >= 1 && src->N >= 16 && src->K >= 256, MOESQ_ERR_INVALID, "prepare_weights: bad sizes");
  MOESQ_REQUIRE(src->N % 16 == 0 && src->K % 256 == 0, MOESQ_ERR_UNSUPPORTED, "prepare_weights: needs N % 16 == 0, K % 256 == 0");
  MOESQ_REQUIRE(aligned16(src->packed) && ((uintptr_t)src->mask & 3) == 0 && ((uintptr_t)src->scale & 1) == 0 && aligned16(tiled),
                MOESQ_ERR_INVALID, "prepare_weights: alignment (packed, tiled 16 B; mask 4 B; scale 2 B)");
  moesq::launch_prepare(src->packed, src->mask, src->scale, src->E, src->N, src->K, tiled, stream);
  return check_launch(stream, false);
}

moesq_status moesq_unprepare_weights(const uint8_t* tiled, int32_t E, int32_t N, int32_t K, uint8_t* packed, uint8_t* mask,
                                     uint8_t* scale, hipStream_t stream) {
  MOESQ_REQUIRE(tiled && packed && mask && scale, MOESQ_ERR_INVALID, "unprepare_weights: null pointer");
  MOESQ_REQUIRE(E >= 1 && N >= 16 && K >= 256, MOESQ_ERR_INVALID, "unprepare_weights: bad sizes");
  MOESQ_REQUIRE(N % 16 == 0 && K % 256 == 0, MOESQ_ERR_UNSUPPORTED, "unprepare_weights: needs N % 16 == 0, K % 256 == 0");
  MOESQ_REQUIRE(aligned16(packed) && ((uintptr_t)mask & 3) == 0 && ((uintptr_t)scale & 1) == 0 && aligned16(tiled),
                MOESQ_ERR_INVALID, "unprepare_weights: alignment (packed, tiled 16 B; mask 4 B; scale 2 B)");
  moesq::launch_unprepare(tiled, E, N, K, packed, mask, scale, stream);
  return check_launch(stream, false);
}

moesq_status moesq_fold_gate_up_globals(uint8_t* scale, float* global, int32_t E, int32_t N, int32_t K,
                                        hipStream_t stream) {
  MOESQ_REQUIRE(E >= 0 && N >= 2 && N % 2 == 0 && K >= 32 && K % 32 == 0, MOESQ_ERR_INVALID,
                "fold_gate_up_globals: E >= 0, N even, K a positive multiple of 32");
  MOESQ_REQUIRE(E <= 65535, MOESQ_ERR_UNSUPPORTED, "fold_gate_up_globals: at most 65535 experts");
  if (E == 0) return MOESQ_OK;
  MOESQ_REQUIRE(scale && global, MOESQ_ERR_INVALID, "fold_gate_up_globals: null pointer");
  MOESQ_REQUIRE(((uintptr_t)global & 3) == 0, MOESQ_ERR_INVALID, "fold_gate_up_globals: global must be 4-byte aligned");
  moesq::launch_fold_gate_up(scale, global, E, N, K, stream);
  return check_launch(stream, false);
}

moesq_status moesq_validate_weights(const uint8_t* mask, int64_t rows, int32_t K, int32_t* bad, hipStream_t stream) {
  MOESQ_REQUIRE(rows >= 0 && K > 0 && K % 32 == 0, MOESQ_ERR_INVALID, "validate_weights: K % 32 == 0");
  MOESQ_REQUIRE(bad && (rows == 0 || mask), MOESQ_ERR_INVALID, "validate_weights: null pointer");
  moesq::launch_validate(mask, rows * (K / 16), bad, stream);
  return check_launch(stream, false);
}

moesq_status moesq_unpack_pair_bitmask(const uint8_t* packed, const uint8_t* mask, int64_t rows, int32_t K, uint8_t* dense,
                                       int32_t* bad, hipStream_t stream) {
  MOESQ_REQUIRE(rows >= 0 && K > 0 && K % 32 == 0, MOESQ_ERR_INVALID, "unpack: K % 32 == 0");
  MOESQ_REQUIRE(bad && (rows == 0 || (packed && mask && dense)), MOESQ_ERR_INVALID, "unpack: null pointer");
  MOESQ_REQUIRE(((uintptr_t)packed & 3) == 0 && ((uintptr_t)dense & 3) == 0, MOESQ_ERR_INVALID, "unpack: 4-byte alignment");
  moesq::launch_unpack(packed, mask, rows * (K / 16), dense, bad, stream);
  return check_launch(stream, false);
}

moesq_status moesq_pack_pair_bitmask(const uint8_t* dense, int64_t rows, int32_t K, uint8_t* packed, uint8_t* mask,
                                     int32_t* bad, hipStream_t stream) {
  MOESQ_REQUIRE(rows >= 0 && K > 0 && K % 32 == 0, MOESQ_ERR_INVALID, "pack: K % 32 == 0");
  MOESQ_REQUIRE(bad && (rows == 0 || (packed && mask && dense)), MOESQ_ERR_INVALID, "pack: null pointer");
  MOESQ_REQUIRE(((uintptr_t)packed & 3) == 0 && ((uintptr_t)dense & 3) == 0, MOESQ_ERR_INVALID, "pack: 4-byte alignment");
  moesq::launch_pack(dense, rows * (K / 16), packed, mask, bad, stream);
  return check_launch(stream, false);
}

}  // extern "C"

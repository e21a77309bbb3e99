// C ABI of the NVFP4 routed-expert library: argument validation, workspace
// layout and the launch sequence of each call (declared in include/nvfp4moe.h).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/nvfp4moe.h"
#include "kernels.h"

using namespace nvfp4;

namespace nvfp4 {
thread_local TimedLaunch g_timed_launch = {nullptr, nullptr};
}

namespace {

thread_local char g_last_error[512] = "";
thread_local hipEvent_t *g_stage_events = nullptr;
thread_local bool g_separate_h_quant = false;

// Records the profiling event of stage s (before: 2s, after: 2s+1), if set.
// Nothing is recorded while the stream is being captured into a graph.
void mark(int s, bool after, hipStream_t stream) {
  if (!g_stage_events) return;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
  (void)hipEventRecord(g_stage_events[2 * s + (after ? 1 : 0)], stream);
}

// For a stage that is exactly one kernel: its events ride on that kernel's
// dispatch (see launch_kernel), so the stage time is the kernel's own.
void mark_kernel(int s, hipStream_t stream) {
  if (!g_stage_events) return;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
  g_timed_launch = TimedLaunch{g_stage_events[2 * s], g_stage_events[2 * s + 1]};
}

nvfp4_status fail(nvfp4_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

nvfp4_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return NVFP4_OK;
  return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Sequential carving of a workspace into aligned regions.
struct Carver {
  char *base;
  size_t used = 0;
  explicit Carver(void *b) : base(static_cast<char *>(b)) {}
  template <typename T>
  T *take(size_t count) {
    T *p = base ? reinterpret_cast<T *>(base + used) : nullptr;
    used += round_up(count * sizeof(T));
    return p;
  }
};

#define CHECK_NULL(ptr)                                                         \
  do {                                                                          \
    if (!(ptr)) return fail(NVFP4_ERR_INVALID_ARGUMENT, "%s is NULL", #ptr);    \
  } while (0)
#define CHECK_ALIGN(ptr)                                                        \
  do {                                                                          \
    if (!aligned16(ptr))                                                        \
      return fail(NVFP4_ERR_MISALIGNED, "%s is not 16-byte aligned", #ptr);     \
  } while (0)

nvfp4_status check_k(int64_t k, const char *name) {
  if (k <= 0 || k % 32 != 0)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "%s = %lld must be a positive multiple of 32",
                name, (long long)k);
  if (k > (int64_t)1 << 30)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "%s = %lld is too large", name, (long long)k);
  return NVFP4_OK;
}

nvfp4_status check_workspace(void *ws, size_t have, size_t need) {
  if (have < need)
    return fail(NVFP4_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", have, need);
  if (need > 0) {
    CHECK_NULL(ws);
    CHECK_ALIGN(ws);
  }
  return NVFP4_OK;
}

#define TRY(expr)                          \
  do {                                     \
    const nvfp4_status st_ = (expr);       \
    if (st_ != NVFP4_OK) return st_;       \
  } while (0)
#define LAUNCH(expr, what) TRY(hip_status((expr), what))

// ---- workspace layouts ---------------------------------------------------------

struct QuantWs {
  float *partials;
};
QuantWs carve_quant(Carver &c) { return QuantWs{c.take<float>(kMaxPartials)}; }

struct LinearWs {
  _Float16 *x16;
  int32_t *shift;
  float *partials;
  float *g_x;
  float *split;   // partial sums of a K-split GEMM
};
// the dense row-streaming GEMV serves one or two rows (more would stream
// the weights once per row); larger M runs the tile GEMM
bool linear_rows(int64_t M, int64_t K, nvfp4_act_mode act) {
  return act == NVFP4_W4A16 && M <= 2 && row_gemv_supported((int)K);
}
// a few rows (up to 32) share one weight stream in the dense GEMV
bool linear_dense(int64_t M, int64_t K, nvfp4_act_mode act) {
  return !linear_rows(M, K, act) && dense_gemv_supported(M, K);
}
TilePlan linear_plan(int64_t M, int64_t N, int64_t K, nvfp4_act_mode act) {
  if (linear_dense(M, K, act)) return dense_gemv_plan(Epi::LINEAR, N, K, M);
  const int bm = gemm_block_rows(M);
  return tile_gemm_plan(Epi::LINEAR, N, K, (M + bm - 1) / bm, M);
}
LinearWs carve_linear(Carver &c, int64_t M, int64_t N, int64_t K, nvfp4_act_mode act) {
  LinearWs w;
  w.x16 = c.take<_Float16>((size_t)(M * K));
  w.shift = c.take<int32_t>((size_t)M);
  w.partials = c.take<float>(kMaxPartials);
  w.g_x = c.take<float>(4);
  w.split = c.take<float>(tile_gemm_supported((int)K) || linear_dense(M, K, act)
                              ? linear_plan(M, N, K, act).partial_floats
                              : 0);
  return w;
}

struct FfnWs {
  _Float16 *x16;
  int32_t *xshift;
  uint16_t *h;
  _Float16 *h16;
  int32_t *hshift;
  float *ypair;
  int4 *mblocks;
  int32_t *n_mblocks;
  int4 *mblocks_down;   // the down projection's blocks when their size differs
  int32_t *n_mblocks_down;
  uint32_t *slots;      // [0] running max |h| (float bits), [1] g_x, [2] g_h, [3] -
  float *partials;
  float *split;         // partial sums of a K-split GEMM
};
// Decode-sized batches: at most 256 (token, expert) pairs that average at
// most 16 per expert run as GEMVs over the pairs (a single expert, the dense
// MLP, only for one or two tokens, since the GEMVs stream an expert's rows
// once per pair).  Anything larger runs as a grouped GEMM over m-blocks of
// up to 128 rows, which streams every active expert's weights once per block
// however skewed the routing is (one expert holding almost every token of a
// prefill chunk costs a few blocks, not one weight stream per token).
bool ffn_small(int64_t T, int64_t E, int64_t k) {
  if (E == 1) return T * k <= 2;
  return T * k <= 256 && 2 * T * k <= 32 * E;
}
int ffn_bm(int64_t T, int64_t E, int64_t k) {
  if (ffn_small(T, E, k)) return 16;
  if (E == 1) return gemm_block_rows(T * k);
  // experts that average under 64 rows waste most of a 128-row block
  return T * k >= 64 * E ? 128 : 64;
}
// The down projection of light experts (64-row blocks above) runs faster on
// 32-row blocks: its K is the short intermediate size, so a block's weight
// stream is short and the smaller activation stage lets more workgroups share
// a CU.
int ffn_bm_down(int64_t T, int64_t E, int64_t k) {
  const int bm = ffn_bm(T, E, k);
  return E > 1 && bm == 64 ? 32 : bm;
}
// The fused decode path (W4A16 decode batch, H = 2048, I a multiple of 256)
// reads the routing in pair order when it is given no permutation.
bool ffn_pair_order_ok(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, nvfp4_act_mode act) {
  return act == NVFP4_W4A16 && ffn_small(T, E, k) && row_gemv_supported((int)H) &&
         row_gemv_supported((int)I) && row_ffn_supported((int)H, (int)I);
}
// A single expert (a dense MLP) with one row, W4A16: the gate/up rows and
// then the down rows dealt out evenly over the CUs (row_mlp_gate_up_kernel,
// row_mlp_down_kernel, which writes y itself)
bool ffn_row_mlp(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, nvfp4_act_mode act) {
  return act == NVFP4_W4A16 && E == 1 && T * k == 1 && row_mlp_supported((int)H, (int)I) &&
         row_mlp_down_supported((int)H, (int)I);
}
// A single expert (a dense MLP) with 3 to 32 rows: one weight stream shared
// by every row in the dense GEMV (K of both projections a multiple of 256).
bool ffn_dense(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  return E == 1 && !ffn_small(T, E, k) && dense_gemv_supported(T * k, H) &&
         dense_gemv_supported(T * k, I);
}
// m-blocks of up to bm rows over P pairs: each expert rounds up once (a
// single expert, the dense MLP, has exactly ceil(P / bm))
int64_t ffn_max_mblocks(int64_t P, int64_t E, int bm) {
  return (P + bm - 1) / bm + (E > 1 ? (E < P ? E : P) : 0);
}
struct FfnPlans {
  TilePlan gate_up, down;
};
FfnPlans ffn_plans(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  FfnPlans f;
  const int64_t P = T * k;
  const int64_t mb = ffn_max_mblocks(P, E, ffn_bm(T, E, k));
  const int64_t mb_down = ffn_max_mblocks(P, E, ffn_bm_down(T, E, k));
  if (ffn_dense(T, H, I, E, k)) {
    f.gate_up = dense_gemv_plan(Epi::SWIGLU, I, H, P);
    f.down = dense_gemv_plan(Epi::DOWN, H, I, P);
  } else if (!ffn_small(T, E, k)) {
    if (tile_gemm_supported((int)H)) f.gate_up = tile_gemm_plan(Epi::SWIGLU, I, H, mb, P);
    if (tile_gemm_supported((int)I)) f.down = tile_gemm_plan(Epi::DOWN, H, I, mb_down, P);
  }
  return f;
}
FfnWs carve_ffn(Carver &c, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  const int64_t P = T * k;
  FfnWs w;
  w.x16 = c.take<_Float16>((size_t)(T * H));
  w.xshift = c.take<int32_t>((size_t)T);
  w.h = c.take<uint16_t>((size_t)(P * I));
  w.h16 = c.take<_Float16>((size_t)(P * I));
  w.hshift = c.take<int32_t>((size_t)P);
  // (the fused decode FFN keeps a partial row per pair and 256-column slice of I)
  const int64_t ffn_parts = ffn_small(T, E, k) && row_ffn_supported((int)H, (int)I) ? I / 256 : 1;
  w.ypair = c.take<float>((size_t)(P * H * (ffn_parts > 1 ? ffn_parts : 1)));
  w.mblocks = c.take<int4>((size_t)ffn_max_mblocks(P, E, 16));
  w.n_mblocks = c.take<int32_t>(4);
  w.mblocks_down = c.take<int4>((size_t)ffn_max_mblocks(P, E, 16));
  w.n_mblocks_down = c.take<int32_t>(4);
  w.slots = c.take<uint32_t>(4);   // scratch words
  w.partials = c.take<float>(kMaxPartials);
  const FfnPlans pl = ffn_plans(T, H, I, E, k);
  w.split = c.take<float>(pl.gate_up.partial_floats > pl.down.partial_floats
                              ? pl.gate_up.partial_floats
                              : pl.down.partial_floats);
  return w;
}

struct SharedWs {
  Bf16Plan up_plan, down_plan;
  float *gu_part;
  uint16_t *h;
  float *y_part;
};
SharedWs carve_shared(Carver &c, int64_t T, int64_t H, int64_t I) {
  SharedWs w;
  w.up_plan = bf16_plan(T, H, 2 * I);
  w.down_plan = bf16_plan(T, I, H);
  w.gu_part = c.take<float>(w.up_plan.partial_floats);
  w.h = c.take<uint16_t>((size_t)(T * I));
  w.y_part = c.take<float>(w.down_plan.partial_floats);
  return w;
}

}  // namespace

extern "C" {

const char *nvfp4_status_string(nvfp4_status s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_INVALID_ARGUMENT: return "invalid argument";
    case NVFP4_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case NVFP4_ERR_MISALIGNED: return "misaligned pointer";
    case NVFP4_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case NVFP4_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *nvfp4_last_error(void) { return g_last_error; }

void nvfp4_set_ffn_stage_events(hipEvent_t *events) { g_stage_events = events; }

void nvfp4_set_ffn_separate_h_quant(int separate) { g_separate_h_quant = separate != 0; }

nvfp4_status nvfp4_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
  g_last_error[0] = 0;
  CHECK_NULL(buf);
  CHECK_NULL(sink);
  CHECK_ALIGN(buf);
  if (bytes == 0 || bytes % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "bytes = %zu must be a positive multiple of 16",
                bytes);
  LAUNCH(launch_read_probe(buf, (int64_t)bytes, sink, stream), "read probe");
  return NVFP4_OK;
}

// ---- nvfp4_quantize ----------------------------------------------------------------

size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols) {
  (void)rows;
  (void)cols;
  Carver c(nullptr);
  carve_quant(c);
  return c.used;
}

nvfp4_status nvfp4_quantize(const void *x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                            int64_t ld_x, uint8_t *codes, uint8_t *scales,
                            float *global_scale, nvfp4_global_mode mode, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  CHECK_NULL(x);
  CHECK_NULL(codes);
  CHECK_NULL(scales);
  CHECK_NULL(global_scale);
  if (x_dtype != NVFP4_DT_BF16 && x_dtype != NVFP4_DT_F32)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "x_dtype %d is not BF16 or F32", (int)x_dtype);
  if (mode != NVFP4_GLOBAL_COMPUTE && mode != NVFP4_GLOBAL_GIVEN)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "mode %d is not COMPUTE or GIVEN", (int)mode);
  if (rows < 1) return fail(NVFP4_ERR_INVALID_ARGUMENT, "rows = %lld < 1", (long long)rows);
  TRY(check_k(cols, "cols"));
  if (ld_x < cols || ld_x % 8 != 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "ld_x = %lld must be >= cols and a multiple of 8",
                (long long)ld_x);
  CHECK_ALIGN(x);
  CHECK_ALIGN(codes);
  CHECK_ALIGN(scales);
  if ((reinterpret_cast<uintptr_t>(global_scale) & 3u) != 0)
    return fail(NVFP4_ERR_MISALIGNED, "global_scale is not 4-byte aligned");
  TRY(check_workspace(workspace, workspace_bytes, nvfp4_quantize_workspace_size(rows, cols)));
  Carver c(workspace);
  const QuantWs w = carve_quant(c);
  const InType t = x_dtype == NVFP4_DT_BF16 ? InType::BF16 : InType::F32;
  if (mode == NVFP4_GLOBAL_COMPUTE) {
    const int n = amax_partials_grid(rows, cols);
    LAUNCH(launch_amax_partials(x, t, rows, cols, ld_x, w.partials, n, stream), "amax");
    LAUNCH(launch_quantize(x, t, rows, cols, ld_x, codes, scales, w.partials, n, nullptr,
                           global_scale, stream),
           "quantize");
  } else {
    LAUNCH(launch_quantize(x, t, rows, cols, ld_x, codes, scales, nullptr, 0, global_scale,
                           nullptr, stream),
           "quantize");
  }
  return NVFP4_OK;
}

// ---- nvfp4_dequantize --------------------------------------------------------------

static nvfp4_status check_matrix(const nvfp4_matrix *w) {
  CHECK_NULL(w);
  CHECK_NULL(w->codes);
  CHECK_NULL(w->scales);
  CHECK_NULL(w->global_scale);
  if (w->rows < 1) return fail(NVFP4_ERR_INVALID_ARGUMENT, "w->rows < 1");
  TRY(check_k(w->cols, "w->cols"));
  CHECK_ALIGN(w->codes);
  CHECK_ALIGN(w->scales);
  return NVFP4_OK;
}

nvfp4_status nvfp4_dequantize(const nvfp4_matrix *w, float *out, hipStream_t stream) {
  g_last_error[0] = 0;
  TRY(check_matrix(w));
  CHECK_NULL(out);
  CHECK_ALIGN(out);
  LAUNCH(launch_dequantize(w->codes, w->scales, w->global_scale, w->rows, w->cols, out, stream),
         "dequantize");
  return NVFP4_OK;
}

// ---- nvfp4_linear -------------------------------------------------------------------

size_t nvfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K, nvfp4_act_mode act) {
  if (M < 1 || K < 1 || N < 1) return 0;
  Carver c(nullptr);
  carve_linear(c, M, N, K, act);
  return c.used;
}

nvfp4_status nvfp4_linear(const void *x, int64_t M, const nvfp4_matrix *w,
                          nvfp4_act_mode act, nvfp4_global_mode act_global_mode,
                          float *act_global, void *y, nvfp4_dtype y_dtype, void *workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  if (M > 0) {   // (an empty batch may pass NULL for its empty arrays)
    CHECK_NULL(x);
    CHECK_NULL(y);
  }
  TRY(check_matrix(w));
  if (M < 0) return fail(NVFP4_ERR_INVALID_ARGUMENT, "M = %lld < 0", (long long)M);
  if (M > (1 << 30) || w->rows > (1 << 30))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "M or N exceeds 2^30");
  if (act != NVFP4_W4A16 && act != NVFP4_W4A4)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "act %d is not W4A16 or W4A4", (int)act);
  if (y_dtype != NVFP4_DT_BF16 && y_dtype != NVFP4_DT_F32)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "y_dtype %d is not BF16 or F32", (int)y_dtype);
  if (act == NVFP4_W4A4) {
    if (act_global_mode != NVFP4_GLOBAL_COMPUTE && act_global_mode != NVFP4_GLOBAL_GIVEN)
      return fail(NVFP4_ERR_INVALID_ARGUMENT, "act_global_mode %d invalid", (int)act_global_mode);
    if (act_global_mode == NVFP4_GLOBAL_GIVEN) CHECK_NULL(act_global);
  }
  CHECK_ALIGN(x);
  CHECK_ALIGN(y);
  const int64_t K = w->cols, N = w->rows;
  TRY(check_workspace(workspace, workspace_bytes, nvfp4_linear_workspace_size(M, N, K, act)));
  if (M == 0) return NVFP4_OK;   // nothing to compute (act_global is not written)
  Carver c(workspace);
  const LinearWs ws = carve_linear(c, M, N, K, act);
  const uint16_t *xb = static_cast<const uint16_t *>(x);
  // decode-sized W4A16: stream the weight rows against the bf16 rows as given
  if (linear_rows(M, K, act)) {
    GemmArgs a = {};
    a.A = static_cast<const _Float16 *>(x);
    a.lda = K;
    a.b_codes[0] = w->codes;
    a.b_scales[0] = w->scales;
    a.b_global[0] = w->global_scale;
    a.N = (int)N;
    a.K = (int)K;
    a.out = y;
    a.ldo = N;
    a.out_type = y_dtype == NVFP4_DT_F32 ? OutType::F32 : OutType::BF16;
    LAUNCH(launch_row_gemv(Epi::LINEAR, a, nullptr, nullptr, 1, (int)M, stream), "row gemv");
    return NVFP4_OK;
  }
  if (act == NVFP4_W4A16) {
    LAUNCH(launch_row_prep(xb, M, K, PrepMode::SHIFT, ws.x16, ws.shift, nullptr, 0, nullptr,
                           nullptr, nullptr, stream),
           "row_prep");
  } else if (act_global_mode == NVFP4_GLOBAL_GIVEN) {
    LAUNCH(launch_row_prep(xb, M, K, PrepMode::QUANT, ws.x16, nullptr, nullptr, 0, act_global,
                           ws.g_x, nullptr, stream),
           "row_prep");
  } else {
    const int n = amax_partials_grid(M, K);
    LAUNCH(launch_amax_partials(x, InType::BF16, M, K, K, ws.partials, n, stream), "amax");
    LAUNCH(launch_row_prep(xb, M, K, PrepMode::QUANT, ws.x16, nullptr, ws.partials, n, nullptr,
                           ws.g_x, act_global, stream),
           "row_prep");
  }
  GemmArgs a = {};
  a.A = ws.x16;
  a.lda = K;
  a.a_shift = act == NVFP4_W4A16 ? ws.shift : nullptr;
  a.b_codes[0] = w->codes;
  a.b_scales[0] = w->scales;
  a.b_global[0] = w->global_scale;
  a.N = (int)N;
  a.K = (int)K;
  const int bm = gemm_block_rows(M);
  a.mblocks = nullptr;
  a.dense_rows = M;
  a.n_mblocks = (int)((M + bm - 1) / bm);
  a.extra_scale = act == NVFP4_W4A4 ? ws.g_x : nullptr;
  a.out = y;
  a.ldo = N;
  a.out_type = y_dtype == NVFP4_DT_F32 ? OutType::F32 : OutType::BF16;
  if (linear_dense(M, K, act)) {
    const TilePlan plan = linear_plan(M, N, K, act);
    a.partial = ws.split;
    a.partial_rows = M;
    LAUNCH(launch_dense_gemv(Epi::LINEAR, a, (int)M, plan, nullptr, stream), "dense gemv");
  } else if (tile_gemm_supported((int)K)) {
    const TilePlan plan = linear_plan(M, N, K, act);
    a.partial = ws.split;
    a.partial_rows = M;
    LAUNCH(launch_tile_gemm(Epi::LINEAR, a, bm, plan, nullptr, (int)M, stream), "gemm");
  } else {
    LAUNCH(launch_gemm(Epi::LINEAR, a, bm, stream), "gemm");
  }
  return NVFP4_OK;
}

// ---- moe_route_topk -------------------------------------------------------------------

size_t moe_route_topk_workspace_size(int64_t T, int32_t E, int32_t k) {
  (void)T;
  (void)E;
  (void)k;
  return 256;   // word 0: the ticket counter of the one-launch decode routing
}

nvfp4_status moe_route_workspace_init(void *workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  g_last_error[0] = 0;
  CHECK_NULL(workspace);
  CHECK_ALIGN(workspace);
  if (workspace_bytes < sizeof(uint32_t))
    return fail(NVFP4_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs at least 4",
                workspace_bytes);
  LAUNCH(launch_ticket_reset(static_cast<uint32_t *>(workspace), stream), "workspace init");
  return NVFP4_OK;
}

nvfp4_status moe_route_topk(const float *logits, int64_t T, int32_t E, int32_t k,
                            int renormalize, int32_t *topk_ids, float *topk_weights,
                            int32_t *expert_offsets, int32_t *sorted_pairs, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  // both permutation outputs NULL: the top-k alone (moe_permute_pairs can
  // make the permutation later, e.g. on a second stream)
  const bool topk_only = !expert_offsets && !sorted_pairs;
  if (T > 0) {   // (an empty batch may pass NULL for its empty arrays)
    CHECK_NULL(logits);
    CHECK_NULL(topk_ids);
    CHECK_NULL(topk_weights);
    if (!topk_only) CHECK_NULL(sorted_pairs);
  }
  if (!topk_only) CHECK_NULL(expert_offsets);
  if (T < 0) return fail(NVFP4_ERR_INVALID_ARGUMENT, "T = %lld < 0", (long long)T);
  if (E < 1 || E > 1024)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "E = %d outside 1..1024", (int)E);
  if (k < 1 || k > E || k > 32)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "k = %d outside 1..min(E, 32)", (int)k);
  if (T * (int64_t)k > ((int64_t)1 << 24))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "T*k = %lld exceeds 2^24", (long long)(T * k));
  CHECK_ALIGN(logits);
  CHECK_ALIGN(topk_ids);
  CHECK_ALIGN(topk_weights);
  CHECK_ALIGN(expert_offsets);
  CHECK_ALIGN(sorted_pairs);
  if (topk_only) {   // (no ticket: the workspace is not used)
    if (T > 0)
      LAUNCH(launch_topk(LogitSrc{logits, 0, 1, nullptr, nullptr}, T, E, k, renormalize, topk_ids,
                         topk_weights, stream),
             "top-k");
    return NVFP4_OK;
  }
  TRY(check_workspace(workspace, workspace_bytes, moe_route_topk_workspace_size(T, E, k)));
  if (T == 0) {   // no pairs: every offset is 0
    LAUNCH(launch_permute(nullptr, 0, E, k, expert_offsets, nullptr, stream), "offsets");
    return NVFP4_OK;
  }
  LAUNCH(launch_route(LogitSrc{logits, 0, 1, nullptr, nullptr}, T, E, k, renormalize, topk_ids,
                      topk_weights, expert_offsets, sorted_pairs,
                      static_cast<uint32_t *>(workspace), stream),
         "route");
  return NVFP4_OK;
}

// ---- moe_router_topk ------------------------------------------------------------------

size_t moe_router_topk_workspace_size(int64_t T, int64_t H, int32_t E, int32_t k) {
  (void)k;
  if (T < 1 || H < 1 || E < 1) return 0;
  Carver c(nullptr);
  c.take<uint32_t>(64);   // word 0: the routing ticket
  c.take<float>(bf16_plan(T, H, E).partial_floats);
  return c.used;
}

nvfp4_status moe_router_topk(const void *x, int64_t T, int64_t H, const void *router_w,
                             const float *router_bias, int32_t E, int32_t k, int renormalize,
                             float *logits, int32_t *topk_ids, float *topk_weights,
                             int32_t *expert_offsets, int32_t *sorted_pairs, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  if (T > 0) {   // (an empty batch may pass NULL for its empty arrays)
    CHECK_NULL(x);
    CHECK_NULL(topk_ids);
    CHECK_NULL(topk_weights);
    CHECK_NULL(sorted_pairs);
  }
  CHECK_NULL(router_w);
  CHECK_NULL(expert_offsets);
  if (T < 0) return fail(NVFP4_ERR_INVALID_ARGUMENT, "T = %lld < 0", (long long)T);
  TRY(check_k(H, "H"));
  if (E < 1 || E > 1024)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "E = %d outside 1..1024", (int)E);
  if (k < 1 || k > E || k > 32)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "k = %d outside 1..min(E, 32)", (int)k);
  if (T * (int64_t)k > ((int64_t)1 << 24))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "T*k = %lld exceeds 2^24", (long long)(T * k));
  if (T * H > ((int64_t)1 << 40) || T * (int64_t)E > ((int64_t)1 << 31))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "T*H or T*E too large");
  CHECK_ALIGN(x);
  CHECK_ALIGN(router_w);
  if (router_bias) CHECK_ALIGN(router_bias);
  if (logits) CHECK_ALIGN(logits);
  CHECK_ALIGN(topk_ids);
  CHECK_ALIGN(topk_weights);
  CHECK_ALIGN(expert_offsets);
  CHECK_ALIGN(sorted_pairs);
  TRY(check_workspace(workspace, workspace_bytes, moe_router_topk_workspace_size(T, H, E, k)));
  if (T == 0) {   // no pairs: every offset is 0
    LAUNCH(launch_permute(nullptr, 0, E, k, expert_offsets, nullptr, stream), "offsets");
    return NVFP4_OK;
  }
  Carver c(workspace);
  uint32_t *ticket = c.take<uint32_t>(64);
  const Bf16Plan plan = bf16_plan(T, H, E);
  float *partial = c.take<float>(plan.partial_floats);
  LAUNCH(launch_bf16_partials(static_cast<const uint16_t *>(x),
                              static_cast<const uint16_t *>(router_w), nullptr, E, T, H, E, plan,
                              partial, stream),
         "router logits");
  LAUNCH(launch_route(LogitSrc{partial, T * (int64_t)E, plan.parts, router_bias, logits}, T, E,
                      k, renormalize, topk_ids, topk_weights, expert_offsets, sorted_pairs,
                      ticket, stream),
         "route");
  return NVFP4_OK;
}

// ---- expert paging ---------------------------------------------------------------------

nvfp4_status moe_expert_cache_init(int32_t *slot_of, int32_t E, int32_t *expert_of,
                                   uint32_t *last_use, int32_t *hand, int32_t S,
                                   hipStream_t stream) {
  g_last_error[0] = 0;
  CHECK_NULL(slot_of);
  CHECK_NULL(expert_of);
  CHECK_NULL(last_use);
  CHECK_NULL(hand);
  if (E < 1 || E > 1024 || S < 1 || S > 1024)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "E = %d, S = %d outside 1..1024", (int)E, (int)S);
  LAUNCH(launch_cache_init(slot_of, E, expert_of, last_use, hand, S, stream), "cache init");
  return NVFP4_OK;
}

nvfp4_status moe_expert_cache_plan(const int32_t *topk_ids, int64_t T, int32_t k, int32_t E,
                                   int32_t S, int32_t *slot_of, int32_t *expert_of,
                                   uint32_t *last_use, int32_t *hand, uint32_t step,
                                   uint32_t protect_from, int32_t max_fetch, int32_t *slot_ids,
                                   int32_t *fetch, int32_t *n_fetch, hipStream_t stream) {
  g_last_error[0] = 0;
  if (T > 0) {   // (an empty batch may pass NULL for its empty arrays)
    CHECK_NULL(topk_ids);
    CHECK_NULL(slot_ids);
  }
  CHECK_NULL(slot_of);
  CHECK_NULL(expert_of);
  CHECK_NULL(last_use);
  CHECK_NULL(hand);
  CHECK_NULL(fetch);
  CHECK_NULL(n_fetch);
  if (E < 1 || E > 1024 || S < 1 || S > 1024)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "E = %d, S = %d outside 1..1024", (int)E, (int)S);
  if (T < 0 || k < 1) return fail(NVFP4_ERR_INVALID_ARGUMENT, "need T >= 0 and k >= 1");
  if (step < 1 || protect_from > step)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "need 1 <= step and protect_from <= step");
  if (max_fetch < 0 || max_fetch > 1024)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "max_fetch = %d outside 0..1024", (int)max_fetch);
  const int64_t P = T * (int64_t)k;
  if (P > (int64_t)1 << 24) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "T*k too large");
  LAUNCH(launch_cache_plan(topk_ids, (int)P, E, S, slot_of, expert_of, last_use, hand, step,
                           protect_from, max_fetch, slot_ids, fetch, n_fetch, stream),
         "cache plan");
  return NVFP4_OK;
}

namespace {
nvfp4_status expert_ptrs(const nvfp4_expert_weights *w, ExpertPtrs &p, const char *what) {
  if (!w) return fail(NVFP4_ERR_INVALID_ARGUMENT, "%s is NULL", what);
  const void *q[9] = {w->gate_codes,  w->up_codes,  w->down_codes,  w->gate_scales, w->up_scales,
                      w->down_scales, w->gate_global, w->up_global, w->down_global};
  for (int j = 0; j < 9; ++j) {
    if (!q[j]) return fail(NVFP4_ERR_INVALID_ARGUMENT, "%s has a NULL array", what);
    if (j < 6 && !aligned16(q[j]))
      return fail(NVFP4_ERR_MISALIGNED, "%s: codes and scales must be 16-byte aligned", what);
    if (j >= 6 && (reinterpret_cast<uintptr_t>(q[j]) & 3u))
      return fail(NVFP4_ERR_MISALIGNED, "%s: globals must be 4-byte aligned", what);
    p.p[j] = static_cast<const uint8_t *>(q[j]);
  }
  return NVFP4_OK;
}
}  // namespace

nvfp4_status moe_expert_cache_fetch(const nvfp4_expert_weights *host_w,
                                    const nvfp4_expert_weights *pool, int64_t H, int64_t I,
                                    const int32_t *fetch, const int32_t *n_fetch,
                                    int32_t max_fetch, hipStream_t stream) {
  g_last_error[0] = 0;
  CHECK_NULL(fetch);
  CHECK_NULL(n_fetch);
  TRY(check_k(H, "H"));
  TRY(check_k(I, "I"));
  if (max_fetch < 0 || max_fetch > 1024)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "max_fetch = %d outside 0..1024", (int)max_fetch);
  ExpertPtrs hp, pp;
  TRY(expert_ptrs(host_w, hp, "host_w"));
  TRY(expert_ptrs(pool, pp, "pool"));
  // the kernel reads the host pages through their device mapping: each array
  // must be pinned host memory that the current device can address
  for (int j = 0; j < 9; ++j) {
    hipPointerAttribute_t at;
    const hipError_t e = hipPointerGetAttributes(&at, hp.p[j]);
    if (e != hipSuccess || at.type != hipMemoryTypeHost || !at.devicePointer) {
      (void)hipGetLastError();
      return fail(NVFP4_ERR_INVALID_ARGUMENT,
                  "host_w array %d is not pinned host memory mapped for the device", j);
    }
    hp.p[j] = static_cast<const uint8_t *>(at.devicePointer);
  }
  LAUNCH(launch_cache_fetch(hp, pp, H, I, fetch, n_fetch, max_fetch, stream), "cache fetch");
  return NVFP4_OK;
}

nvfp4_status moe_permute_pairs(const int32_t *topk_ids, int64_t T, int32_t E, int32_t k,
                               int32_t *expert_offsets, int32_t *sorted_pairs,
                               hipStream_t stream) {
  g_last_error[0] = 0;
  if (T > 0) {   // (an empty batch may pass NULL for its empty arrays)
    CHECK_NULL(topk_ids);
    CHECK_NULL(sorted_pairs);
  }
  CHECK_NULL(expert_offsets);
  if (T < 0) return fail(NVFP4_ERR_INVALID_ARGUMENT, "T = %lld < 0", (long long)T);
  if (E < 1 || E > 1024)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "E = %d outside 1..1024", (int)E);
  if (k < 1 || k > 32)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "k = %d outside 1..32", (int)k);
  if (T * (int64_t)k > ((int64_t)1 << 24))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "T*k = %lld exceeds 2^24", (long long)(T * k));
  CHECK_ALIGN(topk_ids);
  CHECK_ALIGN(expert_offsets);
  CHECK_ALIGN(sorted_pairs);
  LAUNCH(launch_permute(topk_ids, T, E, k, expert_offsets, sorted_pairs, stream), "permute");
  return NVFP4_OK;
}

// ---- moe_shared_expert_ffn -------------------------------------------------------------

size_t moe_shared_expert_ffn_workspace_size(int64_t T, int64_t H, int64_t I) {
  if (T < 1 || H < 1 || I < 1) return 0;
  Carver c(nullptr);
  carve_shared(c, T, H, I);
  return c.used;
}

nvfp4_status moe_shared_expert_ffn(const void *x, int64_t T, int64_t H, int64_t I,
                                   const void *w_gate, const void *w_up, const void *w_down,
                                   int accumulate, void *y, nvfp4_dtype y_dtype, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  if (T > 0) {   // (an empty batch may pass NULL for its empty arrays)
    CHECK_NULL(x);
    CHECK_NULL(y);
  }
  CHECK_NULL(w_gate);
  CHECK_NULL(w_up);
  CHECK_NULL(w_down);
  if (T < 0) return fail(NVFP4_ERR_INVALID_ARGUMENT, "T = %lld < 0", (long long)T);
  TRY(check_k(H, "H"));
  TRY(check_k(I, "I"));
  if (y_dtype != NVFP4_DT_BF16 && y_dtype != NVFP4_DT_F32)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "y_dtype must be bf16 or f32");
  if (T * H > ((int64_t)1 << 40) || T * 2 * I > ((int64_t)1 << 40) ||
      T > INT32_MAX / 2 || 2 * I > INT32_MAX / 2 || H > INT32_MAX / 2)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "shape too large");
  CHECK_ALIGN(x);
  CHECK_ALIGN(w_gate);
  CHECK_ALIGN(w_up);
  CHECK_ALIGN(w_down);
  CHECK_ALIGN(y);
  TRY(check_workspace(workspace, workspace_bytes, moe_shared_expert_ffn_workspace_size(T, H, I)));
  if (T == 0) return NVFP4_OK;   // nothing to compute
  Carver c(workspace);
  const SharedWs ws = carve_shared(c, T, H, I);
  const uint16_t *xb = static_cast<const uint16_t *>(x);
  LAUNCH(launch_bf16_partials(xb, static_cast<const uint16_t *>(w_gate),
                              static_cast<const uint16_t *>(w_up), I, T, H, 2 * I, ws.up_plan,
                              ws.gu_part, stream),
         "shared gate/up");
  LAUNCH(launch_shared_h(ws.gu_part, ws.up_plan.parts, T, I, ws.h, stream), "shared h");
  LAUNCH(launch_bf16_partials(ws.h, static_cast<const uint16_t *>(w_down), nullptr, H, T, I, H,
                              ws.down_plan, ws.y_part, stream),
         "shared down");
  LAUNCH(launch_shared_out(ws.y_part, ws.down_plan.parts, T, H, accumulate != 0, y,
                           y_dtype == NVFP4_DT_F32 ? OutType::F32 : OutType::BF16, stream),
         "shared out");
  return NVFP4_OK;
}

// ---- moe_grouped_nvfp4_ffn -----------------------------------------------------------

size_t moe_grouped_nvfp4_ffn_workspace_size(int64_t T, int64_t H, int64_t I, int32_t E,
                                            int32_t k, nvfp4_act_mode act) {
  (void)act;
  if (T < 1 || H < 1 || I < 1 || E < 1 || k < 1) return 0;
  Carver c(nullptr);
  carve_ffn(c, T, H, I, E, k);
  return c.used;
}

int moe_grouped_nvfp4_ffn_debug_h(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k,
                                  nvfp4_act_mode act, nvfp4_global_mode act_global_mode,
                                  size_t *h_offset, size_t *hq_offset) {
  if (h_offset) *h_offset = 0;
  if (hq_offset) *hq_offset = 0;
  if (T < 1 || H < 1 || I < 1 || E < 1 || k < 1 || k > E) return 0;
  // the offsets of carve_ffn's h and h16 regions
  Carver c(nullptr);
  c.take<_Float16>((size_t)(T * H));
  c.take<int32_t>((size_t)T);
  const size_t h_at = c.used;
  c.take<uint16_t>((size_t)(T * k * I));
  const size_t hq_at = c.used;
  if (h_offset) *h_offset = h_at;
  if (hq_offset) *hq_offset = hq_at;
  // which of them the call writes, by the dispatch of moe_grouped_nvfp4_ffn
  const bool small = ffn_small(T, E, k);
  if (act != NVFP4_W4A4) return small ? 0 : 1;   // (the row paths keep h elsewhere)
  const bool given = act_global_mode == NVFP4_GLOBAL_GIVEN;
  const FfnPlans plans = ffn_plans(T, H, I, E, k);
  const bool h_fused = given && !small && !ffn_dense(T, H, I, E, k) && !g_separate_h_quant &&
                       tile_gemm_supported((int)H) && plans.gate_up.ksplit == 1;
  return h_fused ? 2 : 3;
}

nvfp4_status moe_grouped_nvfp4_ffn(const void *x, int64_t T, int64_t H, int64_t I, int32_t E,
                                   int32_t k, const int32_t *topk_ids, const float *topk_weights,
                                   const int32_t *expert_offsets, const int32_t *sorted_pairs,
                                   const nvfp4_expert_weights *w, nvfp4_act_mode act,
                                   nvfp4_global_mode act_global_mode, float *act_globals,
                                   void *y, nvfp4_dtype y_dtype, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  // no permutation (both NULL): only on the fused decode path, which then
  // takes the pairs in pair order
  const bool pair_order = !expert_offsets && !sorted_pairs;
  if (T > 0) {   // (an empty batch may pass NULL for its empty arrays)
    CHECK_NULL(x);
    CHECK_NULL(topk_ids);
    CHECK_NULL(topk_weights);
    if (!pair_order) {
      CHECK_NULL(expert_offsets);
      CHECK_NULL(sorted_pairs);
    }
    CHECK_NULL(y);
  }
  CHECK_NULL(w);
  CHECK_NULL(w->gate_codes);
  CHECK_NULL(w->up_codes);
  CHECK_NULL(w->down_codes);
  CHECK_NULL(w->gate_scales);
  CHECK_NULL(w->up_scales);
  CHECK_NULL(w->down_scales);
  CHECK_NULL(w->gate_global);
  CHECK_NULL(w->up_global);
  CHECK_NULL(w->down_global);
  if (T < 0) return fail(NVFP4_ERR_INVALID_ARGUMENT, "T = %lld < 0", (long long)T);
  TRY(check_k(H, "H"));
  TRY(check_k(I, "I"));
  if (E < 1 || E > (1 << 20))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "E = %d outside 1..2^20", (int)E);
  if (k < 1 || k > E) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "k = %d outside 1..E", (int)k);
  if (T * (int64_t)k > ((int64_t)1 << 24))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "T*k exceeds 2^24");
  if (act != NVFP4_W4A16 && act != NVFP4_W4A4)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "act %d is not W4A16 or W4A4", (int)act);
  if (y_dtype != NVFP4_DT_BF16 && y_dtype != NVFP4_DT_F32)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "y_dtype %d is not BF16 or F32", (int)y_dtype);
  if (act == NVFP4_W4A4) {
    if (act_global_mode != NVFP4_GLOBAL_COMPUTE && act_global_mode != NVFP4_GLOBAL_GIVEN)
      return fail(NVFP4_ERR_INVALID_ARGUMENT, "act_global_mode %d invalid", (int)act_global_mode);
    if (act_global_mode == NVFP4_GLOBAL_GIVEN) CHECK_NULL(act_globals);
  }
  if (T > 0 && pair_order && !ffn_pair_order_ok(T, H, I, E, k, act))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "expert_offsets and sorted_pairs may be NULL only on the fused decode path "
                "(W4A16, H = 2048, I %% 256 == 0, T*k <= 256, 2*T*k <= 32*E)");
  CHECK_ALIGN(x);
  CHECK_ALIGN(y);
  CHECK_ALIGN(topk_ids);
  CHECK_ALIGN(topk_weights);
  CHECK_ALIGN(expert_offsets);
  CHECK_ALIGN(sorted_pairs);
  CHECK_ALIGN(w->gate_codes);
  CHECK_ALIGN(w->up_codes);
  CHECK_ALIGN(w->down_codes);
  CHECK_ALIGN(w->gate_scales);
  CHECK_ALIGN(w->up_scales);
  CHECK_ALIGN(w->down_scales);
  TRY(check_workspace(workspace, workspace_bytes,
                      moe_grouped_nvfp4_ffn_workspace_size(T, H, I, E, k, act)));
  if (T == 0) return NVFP4_OK;   // nothing to compute (act_globals is not written)
  Carver c(workspace);
  const FfnWs ws = carve_ffn(c, T, H, I, E, k);
  const int64_t P = T * k;
  const int bm = ffn_bm(T, E, k);
  const int bm_down = ffn_bm_down(T, E, k);
  const bool split_down = bm_down != bm;   // the down projection has blocks of its own
  const FfnPlans plans = ffn_plans(T, H, I, E, k);
  const bool a4 = act == NVFP4_W4A4;
  const bool given = a4 && act_global_mode == NVFP4_GLOBAL_GIVEN;
  float *slot_gx = reinterpret_cast<float *>(ws.slots + 1);
  float *slot_gh = reinterpret_cast<float *>(ws.slots + 2);

  const bool small = ffn_small(T, E, k);
  const OutType yt = y_dtype == NVFP4_DT_F32 ? OutType::F32 : OutType::BF16;
  const uint16_t *xb = static_cast<const uint16_t *>(x);

  // W4A16 decode: both projections stream whole weight rows against the bf16
  // activations as given (no fp16 operand passes)
  const bool rows = small && !a4 && row_gemv_supported((int)H) && row_gemv_supported((int)I);
  // ... and the down projection sums each token's slots itself (no combine)
  const bool fused_sum = rows && row_down_sum_supported((int)I, k);
  // A single expert (one slot per token) on the dense GEMV: bf16 x and h as
  // given (no fp16 operand passes), and the down projection's reduce writes y
  // itself (a combine of one slot is a copy), zeros for a dropped token.
  const bool dense = ffn_dense(T, H, I, E, k);
  const bool dense_direct = dense && !a4;
  const int64_t zero_words = 4;   // scratch words the plan zeroes

  // 1-2. plan (m-blocks per expert), zeroed scratch words and x -> fp16 rows
  if (rows) {   // no plan: the stream kernels read the routing directly
    mark(NVFP4_STAGE_PLAN, false, stream);
    mark(NVFP4_STAGE_PLAN, true, stream);
    mark(NVFP4_STAGE_X_PREP, false, stream);
    mark(NVFP4_STAGE_X_PREP, true, stream);
  } else if (dense_direct) {   // bf16 operands as given: no plan, no x pass
    mark(NVFP4_STAGE_PLAN, false, stream);
    mark(NVFP4_STAGE_PLAN, true, stream);
    mark(NVFP4_STAGE_X_PREP, false, stream);
    mark(NVFP4_STAGE_X_PREP, true, stream);
  } else if (!a4) {
    mark(NVFP4_STAGE_PLAN, false, stream);
    mark(NVFP4_STAGE_PLAN, true, stream);
    mark(NVFP4_STAGE_X_PREP, false, stream);
    LAUNCH(launch_moe_prep(xb, T, H, ws.x16, ws.xshift, expert_offsets, E, bm, ws.mblocks,
                           ws.n_mblocks, bm_down, split_down ? ws.mblocks_down : nullptr,
                           ws.n_mblocks_down, ws.slots, zero_words, stream),
           "plan + x prep");
    mark(NVFP4_STAGE_X_PREP, true, stream);
  } else {
    mark(NVFP4_STAGE_PLAN, false, stream);
    LAUNCH(launch_moe_plan(expert_offsets, E, bm, ws.mblocks, ws.n_mblocks, bm_down,
                           split_down ? ws.mblocks_down : nullptr, ws.n_mblocks_down, ws.slots,
                           (int)zero_words, stream),
           "plan");
    mark(NVFP4_STAGE_PLAN, true, stream);
    mark(NVFP4_STAGE_X_PREP, false, stream);
    if (given) {
      LAUNCH(launch_row_prep(xb, T, H, PrepMode::QUANT, ws.x16, nullptr, nullptr, 0, act_globals,
                             slot_gx, nullptr, stream),
             "x quant");
    } else {
      const int n = amax_partials_grid(T, H);
      LAUNCH(launch_amax_partials(x, InType::BF16, T, H, H, ws.partials, n, stream), "x amax");
      LAUNCH(launch_row_prep(xb, T, H, PrepMode::QUANT, ws.x16, nullptr, ws.partials, n, nullptr,
                             slot_gx, act_globals, stream),
             "x quant");
    }
    mark(NVFP4_STAGE_X_PREP, true, stream);
  }
  // 3. gate/up grouped GEMM with the SiLU * up epilogue -> h (bf16, expert-sorted rows)
  GemmArgs g = {};
  g.A = ws.x16;
  g.lda = H;
  g.a_rowmap = sorted_pairs;
  g.a_rowdiv = k;
  g.a_shift = a4 ? nullptr : ws.xshift;
  g.b_codes[0] = w->gate_codes;
  g.b_codes[1] = w->up_codes;
  g.b_scales[0] = w->gate_scales;
  g.b_scales[1] = w->up_scales;
  g.b_global[0] = w->gate_global;
  g.b_global[1] = w->up_global;
  g.b_codes_estride = I * (H / 2);
  g.b_scales_estride = I * (H / 16);
  g.N = (int)I;
  g.K = (int)H;
  g.mblocks = ws.mblocks;
  g.n_mblocks_dev = ws.n_mblocks;
  g.n_mblocks = (int)ffn_max_mblocks(P, E, bm);
  g.n_experts = E;
  g.extra_scale = a4 ? slot_gx : nullptr;
  g.out = ws.h;
  g.ldo = I;
  g.out_type = OutType::BF16;
  g.amax_slot = a4 ? ws.slots : nullptr;
  // W4A4 with a given h global on the tiled path: the gate/up epilogue
  // quantises h itself and writes the down GEMM's fp16 operand directly
  const bool h_fused = given && !small && !dense && !g_separate_h_quant &&
                       tile_gemm_supported((int)H) && plans.gate_up.ksplit == 1;
  if (h_fused) {
    g.h_quant_g = act_globals + 1;
    g.out = ws.h16;
    g.amax_slot = nullptr;
  }
  g.sorted_pairs = sorted_pairs;   // (split-K reduce: expert of each tile row)
  g.partial = ws.split;
  g.partial_rows = P;
  if (dense_direct) {
    g.A = reinterpret_cast<const _Float16 *>(x);   // bf16 rows, read as given
    g.a_shift = nullptr;
    g.a_bf16 = true;
  }
  if (rows) {
    g.A = reinterpret_cast<const _Float16 *>(x);   // bf16 rows, read as given
    g.a_shift = nullptr;
  }
  // W4A16 decode with H = 2048: both projections in one launch (one dense
  // row instead deals its gate/up rows out over every CU, below)
  if (rows && row_ffn_supported((int)H, (int)I) && !ffn_row_mlp(T, H, I, E, k, act)) {
    GemmArgs dd = {};
    dd.b_codes[0] = w->down_codes;
    dd.b_scales[0] = w->down_scales;
    dd.b_global[0] = w->down_global;
    dd.b_codes_estride = H * (I / 2);
    dd.b_scales_estride = H * (I / 16);
    dd.N = (int)H;
    dd.K = (int)I;
    dd.pair_weights = topk_weights;
    mark_kernel(NVFP4_STAGE_GATE_UP, stream);
    LAUNCH(launch_row_ffn(g, dd, sorted_pairs, topk_ids, k, (int)P, ws.ypair, stream),
           "gate/up + down");
    g_timed_launch = TimedLaunch{nullptr, nullptr};
    mark(NVFP4_STAGE_H_PREP, false, stream);
    mark(NVFP4_STAGE_H_PREP, true, stream);
    mark(NVFP4_STAGE_DOWN, false, stream);
    mark(NVFP4_STAGE_DOWN, true, stream);
    mark_kernel(NVFP4_STAGE_COMBINE, stream);
    LAUNCH(launch_ffn_combine(ws.ypair, (int)T, (int)H, (int)I, k, topk_ids, E, y, yt, stream),
           "combine");
    g_timed_launch = TimedLaunch{nullptr, nullptr};
    return NVFP4_OK;
  }
  mark_kernel(NVFP4_STAGE_GATE_UP, stream);
  if (rows && ffn_row_mlp(T, H, I, E, k, act))   // one dense row: rows dealt out evenly
    LAUNCH(launch_row_mlp_gate_up(g, topk_ids, stream), "gate/up");
  else if (rows)
    LAUNCH(launch_row_gemv(Epi::SWIGLU, g, sorted_pairs, topk_ids, k, (int)P, stream, fused_sum),
           "gate/up");
  else if (small)
    LAUNCH(launch_gemv(Epi::SWIGLU, g, false, stream), "gate/up");
  else if (dense)
    LAUNCH(launch_dense_gemv(Epi::SWIGLU, g, (int)P, plans.gate_up, nullptr, stream),
           "gate/up");
  else
    LAUNCH(tile_gemm_supported((int)H)
               ? launch_tile_gemm(Epi::SWIGLU, g, bm, plans.gate_up, topk_ids, (int)P, stream)
               : launch_gemm(Epi::SWIGLU, g, bm, stream),
           "gate/up");
  g_timed_launch = TimedLaunch{nullptr, nullptr};
  // 4. h rows -> fp16 operands (W4A16 small tiles convert inside the down kernel)
  mark(NVFP4_STAGE_H_PREP, false, stream);
  const bool h_inline = small && !a4;
  if (!a4) {
    if (!h_inline && !rows && !dense_direct)
      LAUNCH(launch_row_prep(ws.h, P, I, PrepMode::SHIFT, ws.h16, ws.hshift, nullptr, 0, nullptr,
                             nullptr, nullptr, stream),
             "h prep");
  } else if (h_fused) {
    // quantised in the gate/up epilogue (the down GEMM reads g_h from the caller)
  } else if (given) {
    LAUNCH(launch_row_prep(ws.h, P, I, PrepMode::QUANT, ws.h16, nullptr, nullptr, 0,
                           act_globals + 1, slot_gh, nullptr, stream),
           "h quant");
  } else {
    LAUNCH(launch_row_prep(ws.h, P, I, PrepMode::QUANT, ws.h16, nullptr,
                           reinterpret_cast<const float *>(ws.slots), 1, nullptr, slot_gh,
                           act_globals ? act_globals + 1 : nullptr, stream),
           "h quant");
  }
  mark(NVFP4_STAGE_H_PREP, true, stream);
  // 5. down grouped GEMM, weighted by the routing weight -> Y per pair (fp32)
  GemmArgs d = {};
  d.A = h_inline ? reinterpret_cast<const _Float16 *>(ws.h) : ws.h16;
  d.lda = I;
  d.a_shift = (a4 || h_inline) ? nullptr : ws.hshift;
  d.b_codes[0] = w->down_codes;
  d.b_scales[0] = w->down_scales;
  d.b_global[0] = w->down_global;
  d.b_codes_estride = H * (I / 2);
  d.b_scales_estride = H * (I / 16);
  d.N = (int)H;
  d.K = (int)I;
  d.mblocks = split_down ? ws.mblocks_down : ws.mblocks;
  d.n_mblocks_dev = split_down ? ws.n_mblocks_down : ws.n_mblocks;
  d.n_mblocks = (int)ffn_max_mblocks(P, E, bm_down);
  d.extra_scale = h_fused ? act_globals + 1 : a4 ? slot_gh : nullptr;
  d.out = ws.ypair;
  d.ldo = H;
  d.out_type = OutType::F32;
  d.pair_weights = topk_weights;
  d.sorted_pairs = sorted_pairs;
  d.n_experts = E;
  d.partial = ws.split;
  d.partial_rows = P;
  mark_kernel(NVFP4_STAGE_DOWN, stream);
  const bool mlp_row = rows && ffn_row_mlp(T, H, I, E, k, act);
  if (mlp_row) {
    d.A = reinterpret_cast<const _Float16 *>(ws.h);   // bf16 h, read as given
    d.a_shift = nullptr;
    LAUNCH(launch_row_mlp_down(d, topk_ids, y, yt, stream), "down");
  } else if (rows) {
    d.A = reinterpret_cast<const _Float16 *>(ws.h);   // bf16 h, read as given
    d.a_shift = nullptr;
    if (fused_sum) {
      d.out = y;
      d.ldo = H;
      d.out_type = yt;
      LAUNCH(launch_row_down_sum(d, topk_ids, k, (int)T, stream), "down + combine");
    } else {
      LAUNCH(launch_row_gemv(Epi::DOWN, d, sorted_pairs, topk_ids, k, (int)P, stream), "down");
    }
  } else if (small)
    LAUNCH(launch_gemv(Epi::DOWN, d, h_inline, stream), "down");
  else if (dense) {
    if (dense_direct) {   // bf16 h as given; the reduce writes y (pair t is token t)
      d.A = reinterpret_cast<const _Float16 *>(ws.h);
      d.a_shift = nullptr;
      d.a_bf16 = true;
      d.drop_ids = topk_ids;
      d.out = y;
      d.ldo = H;
      d.out_type = yt;
    }
    LAUNCH(launch_dense_gemv(Epi::DOWN, d, (int)P, plans.down, nullptr, stream), "down");
  }
  else
    LAUNCH(tile_gemm_supported((int)I)
               ? launch_tile_gemm(Epi::DOWN, d, bm_down, plans.down, topk_ids, (int)P, stream)
               : launch_gemm(Epi::DOWN, d, bm_down, stream),
           "down");
  g_timed_launch = TimedLaunch{nullptr, nullptr};
  // 6. combine the k pairs of every token in slot order
  if (fused_sum || dense_direct || mlp_row) {   // done by the down kernel: an empty stage
    mark(NVFP4_STAGE_COMBINE, false, stream);
    mark(NVFP4_STAGE_COMBINE, true, stream);
    return NVFP4_OK;
  }
  mark_kernel(NVFP4_STAGE_COMBINE, stream);
  LAUNCH(launch_combine(ws.ypair, T, H, k, topk_ids, E, y, yt, stream), "combine");
  g_timed_launch = TimedLaunch{nullptr, nullptr};
  return NVFP4_OK;
}

size_t moe_route_ffn_decode_workspace_size(int64_t T, int64_t H, int64_t I, int32_t E,
                                           int32_t k) {
  (void)E;
  if (T < 0 || H < 0 || I < 0 || k < 0) return 0;
  const int64_t parts = I / 256 > 0 ? I / 256 : 1;
  const size_t bytes = (size_t)(T * k * parts * H) * sizeof(float);
  return (bytes + 255) / 256 * 256 + 256;
}

nvfp4_status moe_route_ffn_decode(const float *logits, const void *x, int64_t T, int64_t H,
                                  int64_t I, int32_t E, int32_t k, int renormalize,
                                  int32_t *topk_ids, float *topk_weights,
                                  int32_t *expert_offsets, int32_t *sorted_pairs,
                                  const nvfp4_expert_weights *w, void *y, nvfp4_dtype y_dtype,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  if (T > 0) {   // (an empty batch may pass NULL for its empty arrays)
    CHECK_NULL(logits);
    CHECK_NULL(x);
    CHECK_NULL(topk_ids);
    CHECK_NULL(topk_weights);
    CHECK_NULL(sorted_pairs);
    CHECK_NULL(y);
  }
  CHECK_NULL(expert_offsets);
  CHECK_NULL(w);
  CHECK_NULL(w->gate_codes);
  CHECK_NULL(w->up_codes);
  CHECK_NULL(w->down_codes);
  CHECK_NULL(w->gate_scales);
  CHECK_NULL(w->up_scales);
  CHECK_NULL(w->down_scales);
  CHECK_NULL(w->gate_global);
  CHECK_NULL(w->up_global);
  CHECK_NULL(w->down_global);
  if (T < 0) return fail(NVFP4_ERR_INVALID_ARGUMENT, "T = %lld < 0", (long long)T);
  if (y_dtype != NVFP4_DT_BF16 && y_dtype != NVFP4_DT_F32)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "y_dtype %d is not BF16 or F32", (int)y_dtype);
  if (k < 1 || k > kMaxFfnRouteK || E < k || E > 512)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "k = %d, E = %d: needs 1 <= k <= 8, k <= E <= 512",
                (int)k, (int)E);
  if (!row_ffn_supported((int)H, (int)I) || !ffn_small(T, E, k))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE,
                "the fused decode path needs H = 2048, I %% 256 == 0 (I > 0), T*k <= 256 and "
                "2*T*k <= 32*E (H = %lld, I = %lld, T = %lld)",
                (long long)H, (long long)I, (long long)T);
  CHECK_ALIGN(logits);
  CHECK_ALIGN(x);
  CHECK_ALIGN(y);
  CHECK_ALIGN(topk_ids);
  CHECK_ALIGN(topk_weights);
  CHECK_ALIGN(expert_offsets);
  CHECK_ALIGN(sorted_pairs);
  CHECK_ALIGN(w->gate_codes);
  CHECK_ALIGN(w->up_codes);
  CHECK_ALIGN(w->down_codes);
  CHECK_ALIGN(w->gate_scales);
  CHECK_ALIGN(w->up_scales);
  CHECK_ALIGN(w->down_scales);
  TRY(check_workspace(workspace, workspace_bytes,
                      moe_route_ffn_decode_workspace_size(T, H, I, E, k)));
  if (T == 0) {   // no pairs: every offset is 0
    LAUNCH(launch_permute(nullptr, 0, E, k, expert_offsets, nullptr, stream), "offsets");
    return NVFP4_OK;
  }
  const int64_t P = T * k;
  float *ypart = static_cast<float *>(workspace);
  GemmArgs g = {};
  g.A = static_cast<const _Float16 *>(x);   // bf16 rows, read as given
  g.lda = H;
  g.b_codes[0] = w->gate_codes;
  g.b_codes[1] = w->up_codes;
  g.b_scales[0] = w->gate_scales;
  g.b_scales[1] = w->up_scales;
  g.b_global[0] = w->gate_global;
  g.b_global[1] = w->up_global;
  g.b_codes_estride = I * (H / 2);
  g.b_scales_estride = I * (H / 16);
  g.N = (int)I;
  g.K = (int)H;
  g.n_experts = E;
  GemmArgs dd = {};
  dd.b_codes[0] = w->down_codes;
  dd.b_scales[0] = w->down_scales;
  dd.b_global[0] = w->down_global;
  dd.b_codes_estride = H * (I / 2);
  dd.b_scales_estride = H * (I / 16);
  dd.N = (int)H;
  dd.K = (int)I;
  const FfnRoute fr{logits, (int)E, renormalize, topk_ids, topk_weights};
  // (the stage hook sees the same stages as moe_grouped_nvfp4_ffn; the plan,
  // preparation and separate down stages are empty here)
  mark(NVFP4_STAGE_PLAN, false, stream);
  mark(NVFP4_STAGE_PLAN, true, stream);
  mark(NVFP4_STAGE_X_PREP, false, stream);
  mark(NVFP4_STAGE_X_PREP, true, stream);
  mark_kernel(NVFP4_STAGE_GATE_UP, stream);
  LAUNCH(launch_row_ffn(g, dd, nullptr, topk_ids, k, (int)P, ypart, stream, &fr),
         "routing + gate/up + down");
  g_timed_launch = TimedLaunch{nullptr, nullptr};
  mark(NVFP4_STAGE_H_PREP, false, stream);
  mark(NVFP4_STAGE_H_PREP, true, stream);
  mark(NVFP4_STAGE_DOWN, false, stream);
  mark(NVFP4_STAGE_DOWN, true, stream);
  mark_kernel(NVFP4_STAGE_COMBINE, stream);
  LAUNCH(launch_ffn_combine(ypart, (int)T, (int)H, (int)I, k, topk_ids, E, y,
                            y_dtype == NVFP4_DT_F32 ? OutType::F32 : OutType::BF16, stream,
                            expert_offsets, sorted_pairs),
         "combine + permutation");
  g_timed_launch = TimedLaunch{nullptr, nullptr};
  return NVFP4_OK;
}

}  // extern "C"

// ---- moe_grouped_nvfp4_ffn_static: the FFN with the library's own scratch --------

namespace {
// Scratch of moe_grouped_nvfp4_ffn_static: a file-scope device array, one
// copy per device, held until the process ends.  Host code never uses the
// array's name as an address: the device address of each device's copy comes
// from hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxScratchDevices] = {};

nvfp4_status static_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "device %d outside 0..%d", dev,
                kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(NVFP4_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_OK;
}
}  // namespace

extern "C" {

size_t moe_grouped_nvfp4_ffn_static_max_bytes(void) { return kStaticScratchBytes; }

nvfp4_status moe_grouped_nvfp4_ffn_static(const void *x, int64_t T, int64_t H, int64_t I,
                                          int32_t E, int32_t k, const int32_t *topk_ids,
                                          const float *topk_weights,
                                          const int32_t *expert_offsets,
                                          const int32_t *sorted_pairs,
                                          const nvfp4_expert_weights *w, nvfp4_act_mode act,
                                          nvfp4_global_mode act_global_mode, float *act_globals,
                                          void *y, nvfp4_dtype y_dtype, hipStream_t stream) {
  g_last_error[0] = 0;
  // the scratch this call needs (a host computation: nothing is allocated)
  const size_t need = (T >= 1 && H >= 1 && I >= 1 && E >= 1 && k >= 1 && T <= ((int64_t)1 << 24) &&
                       H <= ((int64_t)1 << 30) && I <= ((int64_t)1 << 30))
                          ? moe_grouped_nvfp4_ffn_workspace_size(T, H, I, E, k, act)
                          : 0;
  if (need > kStaticScratchBytes)
    return fail(NVFP4_ERR_WORKSPACE_TOO_SMALL,
                "moe_grouped_nvfp4_ffn_static: this call needs %zu bytes of scratch, the "
                "library's static scratch holds %zu (use moe_grouped_nvfp4_ffn with a "
                "workspace)",
                need, kStaticScratchBytes);
  void *ws = nullptr;
  if (need > 0) TRY(static_scratch(&ws));
  return moe_grouped_nvfp4_ffn(x, T, H, I, E, k, topk_ids, topk_weights, expert_offsets,
                               sorted_pairs, w, act, act_global_mode, act_globals, y, y_dtype,
                               ws, need > 0 ? kStaticScratchBytes : 0, stream);
}

}  // extern "C"

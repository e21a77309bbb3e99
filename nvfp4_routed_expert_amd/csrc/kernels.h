// Host-side launchers of the NVFP4 kernels (internal to the library; the
// public C ABI is include/nvfp4moe.h).  Every launcher only enqueues work on
// `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace nvfp4 {

// Timing hook.  When a pair of events is attached, the next kernel launched
// through launch_kernel on this thread carries them in its own dispatch
// (start and end timestamps of that kernel), so their span is the kernel
// alone, without separate event packets around it.  The pair is used once.
struct TimedLaunch {
  hipEvent_t start, stop;
};
extern thread_local TimedLaunch g_timed_launch;

template <typename F, typename... Args>
void launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t shm, hipStream_t s, Args... args) {
  const TimedLaunch t = g_timed_launch;
  if (t.start) {
    g_timed_launch = TimedLaunch{nullptr, nullptr};
    hipExtLaunchKernelGGL(kernel, grid, block, shm, s, t.start, t.stop, 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shm, s, args...);
  }
}

enum class InType : int { BF16 = 0, F32 = 1 };
enum class OutType : int { BF16 = 0, F32 = 1 };

// ---- quantisation (quant.hip) ------------------------------------------------

// Partial maxima of |x| over a [rows, cols] matrix (row stride ld): one fp32
// per workgroup, `n_partials` workgroups.  Returns the launch status.
constexpr int kMaxPartials = 1024;
int amax_partials_grid(int64_t rows, int64_t cols);
hipError_t launch_amax_partials(const void *x, InType t, int64_t rows, int64_t cols,
                                int64_t ld, float *partials, int n_partials,
                                hipStream_t s);

// NVFP4 quantisation of x into codes/scales.  The decode scale g is either
// derived from `amax_src` (n_amax floats, maximum taken) or read from
// `g_given` when it is non-null.  g_out (if non-null) receives g.
hipError_t launch_quantize(const void *x, InType t, int64_t rows, int64_t cols,
                           int64_t ld, uint8_t *codes, uint8_t *scales,
                           const float *amax_src, int n_amax, const float *g_given,
                           float *g_out, hipStream_t s);

// Debug dequantisation to fp32.
hipError_t launch_dequantize(const uint8_t *codes, const uint8_t *scales,
                             const float *g, int64_t rows, int64_t cols,
                             float *out, hipStream_t s);

// Activation rows (bf16 [rows, cols], contiguous) -> fp16 MFMA operands.
//  SHIFT: per row r, s_r = floor(log2 amax_r) - 15, out = x * 2^-s_r, shift[r] = s_r.
//  QUANT: NVFP4-quantise with decode scale g (from amax_src/g_given as in
//         launch_quantize) and write e2m1 * e4m3 (without g) in fp16.
enum class PrepMode : int { SHIFT = 0, QUANT = 1 };
hipError_t launch_row_prep(const uint16_t *x, int64_t rows, int64_t cols,
                           PrepMode mode, _Float16 *out, int32_t *shift,
                           const float *amax_src, int n_amax, const float *g_given,
                           float *g_out, float *g_out2, hipStream_t s);

// ---- routing (route.hip, router.hip) ---------------------------------------------

// The fp32 logits [T, E] the top-k reads: logit (t, e) is the sum over parts
// s = 0 .. parts-1 (parts <= kMaxLogitParts), in that order, of
// part[s * part_stride + t * E + e], plus bias[e] when bias is set; out (when
// set) receives the logits.
constexpr int kMaxLogitParts = 4;
struct LogitSrc {
  const float *part;
  int64_t part_stride;
  int parts;
  const float *bias;
  float *out;
};

// Top-k ids/weights and the expert-sorted permutation (a top-k grid, then the
// permutation by one workgroup or by a grid split over experts).  ticket: a
// zero uint32 in the caller's workspace (left zero on return); with it,
// decode-sized batches (route_decode_supported) route in one launch.
bool route_decode_supported(int64_t T, int E, int k);
hipError_t launch_ticket_reset(uint32_t *ticket, hipStream_t s);
// The top-k alone (ids and weights, no permutation).
hipError_t launch_topk(const LogitSrc &logits, int64_t T, int E, int k, int renormalize,
                       int32_t *ids, float *weights, hipStream_t s);
hipError_t launch_route(const LogitSrc &logits, int64_t T, int E, int k, int renormalize,
                        int32_t *ids, float *weights, int32_t *offsets, int32_t *sorted_pairs,
                        uint32_t *ticket, hipStream_t s);

// x [T, H] bf16 . W^T as fp32 partial sums over `parts` K ranges of kpart
// columns: partial[s][t][n] (partial_floats floats), W [N, H] bf16 row-major,
// or (W1 set) rows n < N0 from W0 and rows n >= N0 from W1 (row n - N0).
// Tiles of 16 ms tokens x 16 nb rows of W per wavefront (ms = nb = 1 or 2).
// Needs H % 32 == 0.
struct Bf16Plan {
  int ms = 1, nb = 1;
  int kpart = 64;
  int parts = 1;
  size_t partial_floats = 0;
};
Bf16Plan bf16_plan(int64_t T, int64_t H, int64_t N);
hipError_t launch_bf16_partials(const uint16_t *x, const uint16_t *W0, const uint16_t *W1,
                                int64_t N0, int64_t T, int64_t H, int64_t N, const Bf16Plan &p,
                                float *partial, hipStream_t s);

// Shared expert (shared.hip).  h[t][i] = bf16(silu(G) * U) with G and U the
// part sums (in part order) of gp[s][t][i] and gp[s][t][I + i]; then
// y[t][n] = (accumulate ? y[t][n] : 0) + (part sums of yp[s][t][n]), rounded
// once to y's type.
hipError_t launch_shared_h(const float *gp, int parts, int64_t T, int64_t I, uint16_t *h,
                           hipStream_t s);
hipError_t launch_shared_out(const float *yp, int parts, int64_t T, int64_t H, bool accumulate,
                             void *y, OutType t, hipStream_t s);

// Permutation only (the second half of launch_route): expert offsets and the
// expert-sorted pairs of given ids.
hipError_t launch_permute(const int32_t *ids, int64_t T, int E, int k, int32_t *offsets,
                          int32_t *sorted_pairs, hipStream_t s);

// ---- expert paging (cache.hip) ----------------------------------------------------

// An expert set's nine arrays in nvfp4_expert_weights order: gate, up, down
// codes; gate, up, down scales; gate, up, down globals.
struct ExpertPtrs {
  const uint8_t *p[9];
};
hipError_t launch_cache_init(int32_t *slot_of, int E, int32_t *expert_of, uint32_t *last_use,
                             int32_t *hand, int S, hipStream_t s);
hipError_t launch_cache_plan(const int32_t *ids, int P, int E, int S, int32_t *slot_of,
                             int32_t *expert_of, uint32_t *last_use, int32_t *hand, uint32_t step,
                             uint32_t protect_from, int max_fetch, int32_t *slot_ids,
                             int32_t *fetch, int32_t *n_fetch, hipStream_t s);
hipError_t launch_cache_fetch(const ExpertPtrs &host, const ExpertPtrs &pool, int64_t H,
                              int64_t I, const int32_t *fetch, const int32_t *n_fetch,
                              int max_fetch, hipStream_t s);

// ---- grouped GEMM and FFN glue (gemm.hip) ---------------------------------------

enum class Epi : int { LINEAR = 0, SWIGLU = 1, DOWN = 2 };

struct GemmArgs {
  // A operand: fp16 rows.  Tile row `pos` reads A row
  //   a_rowmap ? a_rowmap[pos] / a_rowdiv : pos
  const _Float16 *A;
  int64_t lda;
  const int32_t *a_rowmap;
  int a_rowdiv;
  const int32_t *a_shift;   // per A row power-of-two exponent, or null
  // B operand(s): NVFP4 [E][N][K]; matrix 1 is `up` for SWIGLU
  const uint8_t *b_codes[2];
  const uint8_t *b_scales[2];
  const float *b_global[2];
  int64_t b_codes_estride, b_scales_estride;
  int N, K;
  // work list: int4 {expert, first tile row, rows, 0}; null = dense mode,
  // blocks of BM consecutive rows out of dense_rows, expert 0
  const int4 *mblocks;
  int64_t dense_rows;
  const int32_t *n_mblocks_dev;   // device count, or null to use n_mblocks
  int n_mblocks;                  // host count, or an upper bound when dev != null
  // epilogue
  const float *extra_scale;       // device scalar multiplier (W4A4 act scale) or null
  void *out;
  int64_t ldo;
  OutType out_type;
  uint32_t *amax_slot;            // SWIGLU: running max of |h| (float bits) or null
  // SWIGLU, tile GEMM without a K split: when set, h is quantised to NVFP4
  // with this (given) global in the epilogue and out receives the exact fp16
  // products e2m1 * e4m3 (what the down GEMM consumes) instead of bf16 h
  const float *h_quant_g;
  const float *pair_weights;      // DOWN: routing weight of pair p
  const int32_t *sorted_pairs;    // DOWN: pair of each tile row
  int n_experts;                  // E: ids outside 0..E-1 mark dropped pairs
  // split K (tile GEMM): raw fp32 sums of part kz at partial[kz][pos][col]
  // (SWIGLU: gate columns 0..N-1, up columns N..2N-1); partial_rows = rows
  // per part
  int ksplit;
  float *partial;
  int64_t partial_rows;
  // dense GEMV (SWIGLU / DOWN): A holds bf16 rows as given (no shift), the
  // weights are dequantised to bf16 and multiplied by bf16 MFMA
  bool a_bf16;
  // dense GEMV, DOWN: rows t of out whose id drop_ids[t] lies outside
  // 0..n_experts-1 (tokens of one slot each) are written as zeros
  const int32_t *drop_ids;
};

hipError_t launch_gemm(Epi epi, const GemmArgs &a, int bm, hipStream_t s);

// Grouped GEMM with both operands staged through an LDS ring (tile_gemm.hip):
// m-blocks of bm (16, 32, 64 or 128) rows, 256 (or 64) weight rows per
// workgroup.  Needs K % 64 == 0 (tile_gemm_supported); other K use
// launch_gemm.  tile_gemm_plan picks the workgroup width and the K split for
// a problem (n_mblocks_bound: the m-block count or a bound on it; rows: tile
// rows, the partial buffer's rows); a split needs partial_floats floats of
// workspace in GemmArgs::partial (partial_rows >= rows).  ids (grouped mode,
// with a K split): expert of tile row pos is ids[sorted_pairs[pos]].
struct TilePlan {
  int waves = 4;
  int ksplit = 1;
  size_t partial_floats = 0;
};
bool tile_gemm_supported(int K);
TilePlan tile_gemm_plan(Epi epi, int64_t N, int64_t K, int64_t n_mblocks_bound, int64_t rows);
hipError_t launch_tile_gemm(Epi epi, const GemmArgs &a, int bm, const TilePlan &plan,
                            const int32_t *ids, int rows, hipStream_t s);
// The split-K reduce alone: adds the a.ksplit parts of a.partial in part
// order for `rows` tile rows and applies the epilogue.
hipError_t launch_split_reduce(Epi epi, const GemmArgs &a, int rows, const int32_t *ids,
                               hipStream_t s);

// Dense GEMV for M <= 32 rows (densegemv.hip): one weight stream shared by
// all rows (dense mode: A rows pos = 0..M-1 through a_rowmap / a_shift as in
// the tile GEMM, expert 0), weights in 128-byte row lines through an LDS
// ring, MFMA 16x16x32 f16 (or bf16 with a_bf16).  Needs K % 256 == 0.  dense_gemv_plan picks the
// K split (partial_floats floats of workspace in GemmArgs::partial).
bool dense_gemv_supported(int64_t M, int64_t K);
TilePlan dense_gemv_plan(Epi epi, int64_t N, int64_t K, int64_t M);
hipError_t launch_dense_gemv(Epi epi, const GemmArgs &a, int M, const TilePlan &plan,
                             const int32_t *ids, hipStream_t s);

// Small-M grouped GEMV (tiles of 16 rows): waves of a workgroup split K and
// keep several 128-wide chunks of weight loads in flight.  a_bf16: A rows are
// bf16 and each workgroup derives their power-of-two shift from the row
// maximum itself.  Output tiles are gemv_tile_cols(epi, N, K) columns wide.
hipError_t launch_gemv(Epi epi, const GemmArgs &a, bool a_bf16, hipStream_t s);
int gemv_tile_cols(Epi epi, int N, int K);

// Row-streaming GEMV for W4A16 decode: A rows are bf16 (used as given).
// Work items are (tile row, block of output rows); tile row pos is the pair
// sorted_pairs[pos] of expert ids[pair] and token pair / k (sorted_pairs ==
// null: a dense matrix, pair = token = pos, expert 0).  SWIGLU reads A row
// token and writes row pos; DOWN reads A row pos and writes row pair; LINEAR
// reads and writes row pos.  n_pos tile rows.  Supported K: 256, 512, 1024
// and 2048..32768 (multiples of 32).
bool row_gemv_supported(int K);
hipError_t launch_row_gemv(Epi epi, const GemmArgs &a, const int32_t *sorted_pairs,
                           const int32_t *ids, int k, int n_pos, hipStream_t s,
                           bool h_by_pair = false);

// Fused decode FFN (W4A16, H = 2048, I a multiple of 256): gate/up and down
// (sorted_pairs null: pairs in pair order, ids outside 0..g.n_experts-1 skipped)
// in one launch (a workgroup per tile row and 256-column slice of I, h kept
// in LDS), partial rows in ypart [P][I / 256][H] (fp32), then a combine
// that adds each token's slots and slices in order into y.  g: the gate/up
// arguments (A = bf16 x rows), d: the down arguments (pair weights set).
// With a route (logits set, sorted_pairs null, E <= 512, k <= 8), each
// workgroup takes the top-k of its own token from the fp32 logits [T, E]
// (what the routing kernels compute, bit for bit) and the workgroup of slot
// 0, slice 0 writes the token's ids_out / weights_out; ids and the pair
// weights of g / d are then unused.  The combine given offsets (and
// sorted_pairs) adds one workgroup that makes the permutation of the ids
// (T k <= 256, E <= 512) beside the sums.
struct FfnRoute {
  const float *logits;
  int E;
  int renormalize;
  int32_t *ids_out;
  float *weights_out;
};
constexpr int kMaxFfnRouteK = 8;
bool row_ffn_supported(int H, int I);
hipError_t launch_row_ffn(const GemmArgs &g, const GemmArgs &d, const int32_t *sorted_pairs,
                          const int32_t *ids, int k, int P, float *ypart, hipStream_t s,
                          const FfnRoute *route = nullptr);
hipError_t launch_ffn_combine(const float *ypart, int T, int H, int I, int k, const int32_t *ids,
                              int E, void *y, OutType yt, hipStream_t s,
                              int32_t *offsets = nullptr, int32_t *sorted_pairs = nullptr);

// Gate/up projection of a dense MLP's one row (W4A16, one expert, one
// token; H a multiple of 1024 up to 5120, I a multiple of 16 up to 32768):
// h = bf16(silu(g_gate x Wg^T) * g_up x Wu^T) into g.out [I] (bf16), the
// rows dealt out as whole 16-column blocks of I over at most 256
// workgroups.  Writes nothing when ids[0] lies outside 0..g.n_experts-1.
// g: A = the bf16 x row, b_* the gate (0) and up (1) matrices of expert 0.
bool row_mlp_supported(int H, int I);
hipError_t launch_row_mlp_gate_up(const GemmArgs &g, const int32_t *ids, hipStream_t s);

// Down projection of the same row: y [H] = g_down w (h . Wd^T) in y's type
// (zeros when ids[0] lies outside 0..d.n_experts-1), the output rows dealt
// out evenly over at most 256 workgroups; d: A = h [I] (bf16), the down
// matrix of expert 0, pair_weights[0] = w.  I a multiple of 32 up to 31744,
// H up to 8192.
bool row_mlp_down_supported(int H, int I);
hipError_t launch_row_mlp_down(const GemmArgs &d, const int32_t *ids, void *y, OutType yt,
                               hipStream_t s);

// Token-major down projection for decode with the combine folded in: y[t] =
// sum over slots j (in order) of w[t k + j] * g * (h[t k + j] . W_down[e]);
// A = h rows in pair order (bf16), out = y.  Supported for K (= I) in
// {256, 512, 1024, 2048} and k <= 32.
bool row_down_sum_supported(int K, int k);
hipError_t launch_row_down_sum(const GemmArgs &a, const int32_t *ids, int k, int T,
                               hipStream_t s);

// FFN prep for W4A16: x rows -> fp16 + shift (SHIFT), plus (one extra
// workgroup) the m-block plan and zeroing of `zero_words` words at `zero`.
// (mblocks2 set: also a list of bm2-row blocks, for the down projection)
hipError_t launch_moe_prep(const uint16_t *x, int64_t T, int64_t H, _Float16 *x16,
                           int32_t *xshift, const int32_t *offsets, int E, int bm,
                           int4 *mblocks, int32_t *n_mblocks, int bm2, int4 *mblocks2,
                           int32_t *n_mblocks2, uint32_t *zero, int64_t zero_words,
                           hipStream_t s);
int gemm_block_rows(int64_t rows_hint);   // M-tile (multiple of 16) for a workload

// FFN plan: m-blocks from expert offsets; zeroes `zero_words` words at `zero`.
hipError_t launch_moe_plan(const int32_t *offsets, int E, int bm, int4 *mblocks,
                           int32_t *n_mblocks, int bm2, int4 *mblocks2, int32_t *n_mblocks2,
                           uint32_t *zero, int zero_words, hipStream_t s);

// y[t] = sum_j Y[t*k + j] over the kept slots (ids[t*k + j] in 0..E-1),
// j ascending, fp32 -> out type.
hipError_t launch_combine(const float *ypair, int64_t T, int64_t H, int k, const int32_t *ids,
                          int E, void *y, OutType t, hipStream_t s);

// ---- measurement aid (probe.hip) ---------------------------------------------------

// Streaming read of `bytes` (a multiple of 16) at buf; sink: >= 1024 words.
hipError_t launch_read_probe(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t s);

}  // namespace nvfp4

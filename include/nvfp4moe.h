/*
 * nvfp4moe.h - C ABI of the NVFP4 routed-expert FFN library for MI355X (gfx950).
 *
 * The library implements the quantised routed-expert (mixture-of-experts)
 * feed-forward path over NVFP4 weights: 4-bit E2M1 elements, one FP8 E4M3
 * scale per 16 consecutive elements along K and one fp32 scale per tensor.
 * The routed experts of the Flash-Next NVFP4 checkpoint are NVFP4 "W4A4"
 * (Qwen3.8-Flash-Next-NVFP4-SSD-Stream model card, "What this model is");
 * other NVFP4 parts are quantised weight-only, "W4A16"
 * (Qwen3.8-27B-nvfp4full-dflash2-NInfer model card, "Limits").  Decode runs
 * it as a memory-bound grouped GEMV and prefill as an expert-grouped GEMM
 * over chunks of up to 512 tokens that reuse the routed expert weights
 * (Eider page, "Performance").
 *
 * Encodings (the pages name NVFP4 but do not define its bits; these are the
 * OCP Microscaling Formats v1.0 element types):
 *   E2M1 code c (4 bits): sign bit 3, exponent bits 2..1 (bias 1), mantissa
 *     bit 0; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *   E4M3 byte: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0,
 *     subnormals, largest finite 448 (0x7E).  Block scales are >= 0.
 *   An NVFP4 matrix W[N, K] is
 *     codes  uint8 [N, K/2]  row-major; element 2i of a row in the low nibble
 *                            of byte i, element 2i+1 in the high nibble
 *                            (each byte holds two NVFP4 values: same model
 *                            card, "Why Hugging Face shows 68B parameters");
 *     scales uint8 [N, K/16] row-major, one E4M3 per 16 elements, no swizzle;
 *     global float           the decode multiplier g;
 *   and W[n][k] = e2m1(code) * e4m3(scale[n][k/16]) * g.
 *
 * Conventions shared by every call:
 *   - Every data pointer is a DEVICE pointer, 16-byte aligned, and owned by
 *     the caller.  Struct arguments (nvfp4_matrix, nvfp4_expert_weights) are
 *     host structs holding device pointers; they are read during the call
 *     only.  The library allocates nothing, frees nothing and keeps no
 *     pointer after returning; scratch memory comes from `workspace`, at
 *     least the size the matching *_workspace_size query returns.
 *   - All work is enqueued on `stream` (0 = the null stream).  No call
 *     synchronises or copies between host and device, so buffers must stay
 *     valid until the stream's work completes.
 *   - Arguments are validated on the host before anything is enqueued.  On
 *     failure the call returns the status, records a message for
 *     nvfp4_last_error() and writes nothing.  A failed kernel launch returns
 *     NVFP4_ERR_HIP.  Faults inside kernels surface at the caller's next
 *     synchronisation, as usual in HIP.
 *   - Calls are deterministic: the same inputs give bit-identical outputs
 *     (no floating-point atomics; maxima use order-independent integer
 *     atomics).  The library's state is per thread (the last-error message
 *     and the two switches below), except for moe_grouped_nvfp4_ffn_static's
 *     scratch array, one per device (see there).
 *   - K (the contraction length: cols, H or I) must be a positive multiple
 *     of 32, otherwise NVFP4_ERR_UNSUPPORTED_SHAPE.
 *   - Inputs must be finite; NaN or infinite activations, logits or weights
 *     are not checked and give unspecified results.
 *   - An empty batch (T = 0 tokens, or M = 0 rows for nvfp4_linear) is
 *     valid: the other arguments are checked as usual, the batch's empty
 *     arrays may be NULL, and nothing is computed.  The routing calls
 *     (moe_route_topk, moe_router_topk, moe_permute_pairs) then set the
 *     E + 1 expert offsets to 0 and moe_expert_cache_plan sets *n_fetch to
 *     0; every other output is left untouched (act_globals included).
 *     Negative sizes are NVFP4_ERR_INVALID_ARGUMENT.
 *   - The library ships a thread-local execution switch and a timing hook
 *     (nvfp4_set_ffn_separate_h_quant, nvfp4_set_ffn_stage_events); they
 *     change no result.
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad enum */
  NVFP4_ERR_UNSUPPORTED_SHAPE = 2,  /* K % 32 != 0, k > E, limits exceeded   */
  NVFP4_ERR_MISALIGNED = 3,         /* a pointer is not 16-byte aligned       */
  NVFP4_ERR_WORKSPACE_TOO_SMALL = 4,
  NVFP4_ERR_HIP = 5                 /* a HIP launch failed                    */
} nvfp4_status;

typedef enum { NVFP4_DT_BF16 = 0, NVFP4_DT_F32 = 1 } nvfp4_dtype;

/* Where the fp32 tensor scale of a quantised activation comes from. */
typedef enum {
  NVFP4_GLOBAL_COMPUTE = 0,  /* g = amax / 2688 over the tensor; written out */
  NVFP4_GLOBAL_GIVEN = 1     /* g is read from the caller's pointer          */
} nvfp4_global_mode;

typedef enum {
  NVFP4_W4A16 = 0,  /* weights NVFP4, activations bf16                      */
  NVFP4_W4A4 = 1    /* activations also quantised to NVFP4 before each GEMM */
} nvfp4_act_mode;

/* One NVFP4 matrix [rows, cols] (layout in the header comment). */
typedef struct {
  const uint8_t *codes;        /* [rows, cols/2]                        */
  const uint8_t *scales;       /* [rows, cols/16] E4M3                  */
  const float *global_scale;   /* device pointer to the decode scale g  */
  int64_t rows, cols;
} nvfp4_matrix;

/* E experts' gated-FFN weights, stacked along a leading expert axis. */
typedef struct {
  const uint8_t *gate_codes, *up_codes, *down_codes;    /* [E,I,H/2] [E,I,H/2] [E,H,I/2]    */
  const uint8_t *gate_scales, *up_scales, *down_scales; /* [E,I,H/16] [E,I,H/16] [E,H,I/16] */
  const float *gate_global, *up_global, *down_global;   /* [E] each                         */
} nvfp4_expert_weights;

/*
 * nvfp4_quantize: quantise x [rows, cols] (row stride ld_x elements, bf16 or
 * f32) to NVFP4.  codes [rows, cols/2], scales [rows, cols/16] are written,
 * two 4-bit values per code byte (Qwen3.8-Flash-Next-NVFP4-SSD-Stream model
 * card, "Why Hugging Face shows 68B parameters and 8-bit precision": each
 * packed byte holds two NVFP4 values); the same encoder serves the offline
 * weights and the online W4A4 activations (same card, "What this model is").
 * mode COMPUTE: g = amax(|x|) / 2688 (1.0 for an all-zero x), written to
 * *global_scale.  mode GIVEN: g is read from *global_scale.
 * Per 16-block: s = E4M3_rne_saturate(amax_b / (6 g)); per element:
 * code = E2M1_rne_saturate(x * (1 / (e4m3(s) g))), sign kept, 0 codes when
 * e4m3(s) g == 0; every step is an fp32 operation rounded to nearest-even.
 * Requires cols % 32 == 0, ld_x >= cols, ld_x % 8 == 0.
 */
nvfp4_status nvfp4_quantize(const void *x, nvfp4_dtype x_dtype, int64_t rows,
                            int64_t cols, int64_t ld_x, uint8_t *codes,
                            uint8_t *scales, float *global_scale,
                            nvfp4_global_mode mode, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);
size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols);

/*
 * nvfp4_dequantize: out [rows, cols] f32 = e2m1 * e4m3 * g, each element the
 * correctly rounded fp32 product (a debug and test aid; not on the hot path).
 * The value of a packed NVFP4 element (Qwen3.8-Flash-Next-NVFP4-SSD-Stream
 * model card, "Why Hugging Face shows 68B parameters and 8-bit precision").
 * Errors: NULL or misaligned pointers, cols % 32 != 0.  out is caller-owned.
 */
nvfp4_status nvfp4_dequantize(const nvfp4_matrix *w, float *out,
                              hipStream_t stream);

/*
 * nvfp4_linear: y [M, N] = x [M, K] . W^T for an NVFP4 W [N, K], fp32
 * accumulation, y in bf16 (round-to-nearest-even) or f32.  The dense NVFP4
 * linear of the MLP weights (Eider page, "Qwen3.8 27B": NVFP4 for most MLP
 * weights); W4A16 is the weight-only form (Qwen3.8-27B-nvfp4full-dflash2-
 * NInfer model card, "Limits": NVFP4 parents quantised weight-only), W4A4
 * the activation-quantised one (Qwen3.8-Flash-Next-NVFP4-SSD-Stream model
 * card, "What this model is").  x is bf16,
 * row-major, contiguous.  act W4A4: x is first quantised to NVFP4 with one
 * tensor scale over all of x (mode COMPUTE writes it to *act_global, GIVEN
 * reads it), and the product uses the dequantised x.  act_global may be
 * NULL for W4A16.
 */
nvfp4_status nvfp4_linear(const void *x, int64_t M, const nvfp4_matrix *w,
                          nvfp4_act_mode act, nvfp4_global_mode act_global_mode,
                          float *act_global, void *y, nvfp4_dtype y_dtype,
                          void *workspace, size_t workspace_bytes,
                          hipStream_t stream);
size_t nvfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K,
                                   nvfp4_act_mode act);

/*
 * moe_route_topk: the routing step in front of the routed experts (Eider
 * page, "Qwen3.8 Flash Next": all 512 MoE experts of the model are served).
 * Per token t of logits [T, E] (f32), the k experts with the
 * largest logits in descending order, equal logits going to the lower expert
 * index -> topk_ids [T, k] int32.  topk_weights [T, k] f32: with renormalize,
 * exp(l_j - l_max) / sum over the k chosen (top-k of softmax, renormalised);
 * without, softmax over all E.  The pairs p = t*k + j are then sorted by
 * expert, ties by token: expert_offsets [E+1] int32 (rows of expert e are
 * offsets[e] .. offsets[e+1]-1), sorted_pairs [T*k] int32.
 * The ids, offsets and permutation are exact integers; the weights are fp32.
 * Requires 1 <= k <= E <= 1024, k <= 32, 1 <= T <= 2^24 / k.
 * workspace (moe_route_topk_workspace_size bytes, device, 16-byte aligned):
 * its first 32-bit word must be zero when the call runs, and every call
 * leaves it zero, so a workspace zeroed once serves successive calls on one
 * stream; calls that may run at the same time need separate workspaces.
 * (Decode-sized batches route in one launch whose last finishing wavefront
 * builds the permutation; the word counts finished wavefronts.)
 * Top-k only: with expert_offsets and sorted_pairs both NULL the call writes
 * the ids and weights and nothing else; workspace may then be NULL (it is
 * not touched).  The permutation can follow later from moe_permute_pairs on
 * the ids, e.g. on another stream beside the fused decode FFN, which takes
 * the pairs in pair order (moe_grouped_nvfp4_ffn).  Exactly one of the two
 * NULL is NVFP4_ERR_INVALID_ARGUMENT.
 */
nvfp4_status moe_route_topk(const float *logits, int64_t T, int32_t E,
                            int32_t k, int renormalize, int32_t *topk_ids,
                            float *topk_weights, int32_t *expert_offsets,
                            int32_t *sorted_pairs, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);
size_t moe_route_topk_workspace_size(int64_t T, int32_t E, int32_t k);

/*
 * moe_route_workspace_init: makes a workspace ready for moe_route_topk and
 * moe_router_topk by zeroing its first 32-bit word on `stream` (a one-
 * wavefront kernel, no memset, so it may be captured into a graph).  Call it
 * once after allocating a workspace, or whenever its contents are unknown
 * (reused from another call, or a routing launch that did not finish);
 * successive routing calls on one stream then keep it ready.  A workspace
 * whose first word is not zero makes the one-launch decode routing skip its
 * permutation (sorted_pairs and expert_offsets are left as they were).
 * Errors: NULL or misaligned workspace, workspace_bytes < 4.
 */
nvfp4_status moe_route_workspace_init(void *workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * moe_router_topk: the router in front of moe_route_topk.  Logits
 *   l[t][e] = sum_h x[t][h] * R[e][h]  (+ router_bias[e])
 * with x [T, H] bf16 and the router matrix R [E, H] bf16 (one row per
 * expert, row-major).  The router stays BF16 next to the NVFP4 routed
 * experts (Qwen3.8-Flash-Next-NVFP4-SSD-Stream model card, "What this model
 * is") and is replicated on every device that holds experts (DwarfStar
 * page, GPU pairs).  Every product is exact in fp32 and the sums are fp32,
 * in an order fixed by the shapes (deterministic run to run, not bitwise
 * equal to a sequential sum).  router_bias: f32 [E] or NULL.  On those fp32
 * logits the call then computes exactly what moe_route_topk computes
 * (top-k ids / weights, expert_offsets, sorted_pairs).  logits: f32 [T, E]
 * receives the logits when non-NULL (NULL skips the write).
 * Requires H % 32 == 0 and moe_route_topk's limits on T, E and k.
 * workspace (moe_router_topk_workspace_size bytes, device, 16-byte aligned):
 * holds the K-split partial sums; its first 32-bit word must be zero when
 * the call runs and is left zero, as for moe_route_topk.
 */
nvfp4_status moe_router_topk(const void *x, int64_t T, int64_t H, const void *router_w,
                             const float *router_bias, int32_t E, int32_t k,
                             int renormalize, float *logits, int32_t *topk_ids,
                             float *topk_weights, int32_t *expert_offsets,
                             int32_t *sorted_pairs, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);
size_t moe_router_topk_workspace_size(int64_t T, int64_t H, int32_t E, int32_t k);

/*
 * Expert paging.  The pages keep selected experts resident and page the
 * others in from slower memory when the GPU cannot hold them all (Eider page,
 * "Why Eider exists": bounded page pools, selected experts resident, the rest
 * paged from disk; Qwen3.8-Flash-Next-NVFP4-SSD-Stream model card, 24-32 GB
 * GPUs: expert blocks prefetched while the GPU computes).  Here every
 * expert's NVFP4 weights live in host memory allocated pinned
 * (hipHostMalloc), laid out as nvfp4_expert_weights with E experts, and a
 * device pool of S slots (the same layout with S experts) holds the resident
 * ones.  Per step:
 *   moe_expert_cache_plan   ids of the step -> slot ids, and the experts to
 *                           fetch with their slots (on the device, no host
 *                           round trip);
 *   moe_expert_cache_fetch  copies those experts from host memory into their
 *                           slots (a kernel reading the pinned pages);
 *   moe_permute_pairs       the expert-sorted pair order of the slot ids;
 *   moe_grouped_nvfp4_ffn   on the pool (E = S) with the slot ids.
 * The FFN's result is bit-identical to the one over all E experts in device
 * memory.  State (caller-owned device arrays, set by moe_expert_cache_init):
 * slot_of [E] int32 (slot of each expert, -1 = not resident), expert_of [S]
 * int32 (-1 = empty), last_use [S] uint32 (step stamp), hand [1] int32.
 */
nvfp4_status moe_expert_cache_init(int32_t *slot_of, int32_t E, int32_t *expert_of,
                                   uint32_t *last_use, int32_t *hand, int32_t S,
                                   hipStream_t stream);

/*
 * moe_expert_cache_plan: for topk_ids [T, k] (experts of the step),
 * step = the step's stamp (>= 1, increasing): every needed resident expert is
 * kept and stamped; every needed missing expert gets a slot that holds no
 * expert needed now and whose stamp is below protect_from (a step whose FFN
 * may still be running keeps its experts: pass its stamp; else pass step),
 * taken in slot order from the clock hand on (empty slots count as free).
 * Writes slot_ids [T, k] (slot of each pair's expert), fetch [2 S] int32
 * (pairs {expert, slot} of the experts to copy), in ascending expert order, and
 * *n_fetch (device int32) = their number.  max_fetch is the most experts the
 * following moe_expert_cache_fetch will copy (pass the same value to both).
 * S must exceed the distinct experts of a step (twice over while a previous
 * step's FFN may still run).  A plan that does not fit (fewer free slots
 * than missing experts, or more missing experts than max_fetch) moves
 * nothing: *n_fetch = -1 (the device-side status of the step), the resident
 * experts keep their slots and stamps, and the missing experts' pairs (like
 * ids outside 0..E-1) get slot id -1.  Every later call drops such pairs
 * (moe_permute_pairs leaves them out, moe_grouped_nvfp4_ffn gives them no
 * contribution), so the step's output is the FFN over its placed pairs
 * only, with no read outside the pool.  Requires 1 <= E, S <= 1024, T >= 0,
 * k >= 1, 1 <= step, protect_from <= step, 0 <= max_fetch <= 1024.  One
 * workgroup; integer-exact.  step and protect_from are host values: a HIP
 * graph that captures this call replays it with the stamps of the capture,
 * so slots stamped by one replay are never free in the next (with
 * protect_from = step); call it outside the graph, or capture one graph per
 * step.
 */
nvfp4_status moe_expert_cache_plan(const int32_t *topk_ids, int64_t T, int32_t k,
                                   int32_t E, int32_t S, int32_t *slot_of,
                                   int32_t *expert_of, uint32_t *last_use,
                                   int32_t *hand, uint32_t step, uint32_t protect_from,
                                   int32_t max_fetch, int32_t *slot_ids, int32_t *fetch,
                                   int32_t *n_fetch, hipStream_t stream);

/*
 * moe_expert_cache_fetch: copies the first *n_fetch experts of fetch (from
 * moe_expert_cache_plan with the same max_fetch; nothing when *n_fetch is -1)
 * from host_w (E experts, pinned
 * host memory) into their slots of pool (S experts, device memory, written
 * by this call): codes, scales and globals of gate, up and down.  H, I as
 * in moe_grouped_nvfp4_ffn.  Every host_w array must be pinned host memory
 * mapped for the current device (hipHostMalloc); any other pointer is
 * rejected with NVFP4_ERR_INVALID_ARGUMENT before a launch.  The copy runs
 * on stream like a kernel (no host synchronisation); host_w must not change
 * until it has run.
 */
nvfp4_status moe_expert_cache_fetch(const nvfp4_expert_weights *host_w,
                                    const nvfp4_expert_weights *pool, int64_t H,
                                    int64_t I, const int32_t *fetch,
                                    const int32_t *n_fetch, int32_t max_fetch,
                                    hipStream_t stream);

/*
 * moe_permute_pairs: moe_route_topk's expert offsets [E+1] and sorted pairs
 * [T*k] for given ids [T, k] (stable: pairs of one expert in ascending
 * order), the pair order of a step on the expert pool (Eider page, "Why
 * Eider exists": selected experts resident in bounded page pools).  Same
 * limits as moe_route_topk.  The kept ids of one token must be distinct (as
 * the ids of moe_route_topk and the slot ids of moe_expert_cache_plan are);
 * this is not checked, and repeated ids leave the pair order undefined.  An id
 * outside 0..E-1 drops its pair: it takes
 * no position, offsets[E] counts the kept pairs only, and the positions
 * offsets[E] .. T*k-1 of sorted_pairs are set to -1.
 */
nvfp4_status moe_permute_pairs(const int32_t *topk_ids, int64_t T, int32_t E, int32_t k,
                               int32_t *expert_offsets, int32_t *sorted_pairs,
                               hipStream_t stream);

/*
 * moe_shared_expert_ffn: the shared expert that runs beside the routed ones
 * on every token; it stays BF16 (Qwen3.8-Flash-Next-NVFP4-SSD-Stream model
 * card, "What this model is") and is replicated on every device (DwarfStar
 * page, GPU pairs).  For x [T, H] bf16 and bf16 weights w_gate, w_up
 * [I, H] and w_down [H, I] (row-major):
 *   h_t = bf16_rne( silu(x_t Wg^T) * (x_t Wu^T) )
 *   y_t = h_t Wd^T                       (accumulate = 0)
 *   y_t = y_t + h_t Wd^T                 (accumulate != 0: y is read first,
 *                                         e.g. the routed output)
 * Products are exact in fp32 and the sums fp32; the result is rounded once
 * to y's type (bf16 round-to-nearest-even or f32).
 * Requires H % 32 == 0, I % 32 == 0, T >= 0.  workspace:
 * moe_shared_expert_ffn_workspace_size bytes (device, 16-byte aligned).
 */
nvfp4_status moe_shared_expert_ffn(const void *x, int64_t T, int64_t H, int64_t I,
                                   const void *w_gate, const void *w_up,
                                   const void *w_down, int accumulate, void *y,
                                   nvfp4_dtype y_dtype, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);
size_t moe_shared_expert_ffn_workspace_size(int64_t T, int64_t H, int64_t I);

/*
 * moe_grouped_nvfp4_ffn: routed-expert gated FFN, a grouped GEMV in decode
 * and an expert-grouped GEMM over prefill chunks (Eider page, "Performance":
 * prefill takes up to 512 prompt tokens per iteration so that the routed
 * expert weights are reused; the routed experts are NVFP4 W4A4 in the
 * Flash-Next checkpoint: Qwen3.8-Flash-Next-NVFP4-SSD-Stream model card,
 * "What this model is").  For each pair p = t*k + j
 * routed to expert e = topk_ids[p] (moe_route_topk's ids / weights / offsets /
 * sorted_pairs, which must be consistent with each other):
 *   h_p = bf16_rne( silu(g_gate[e] x_t D_gate[e]^T) * (g_up[e] x_t D_up[e]^T) )
 *   y_t = sum_j topk_weights[p] * g_down[e] h_p D_down[e]^T   (j ascending)
 * with D the e2m1*e4m3 part of each NVFP4 matrix and fp32 accumulation.
 * x [T, H] bf16; y [T, H] bf16 or f32.  act W4A4 quantises x (one scale over
 * all T rows) and h (one scale over all T*k pairs) to NVFP4 before the gate/up
 * and down products; act_globals[0..1] = {g_x, g_h} are written (COMPUTE) or
 * read (GIVEN).  act_globals may be NULL for W4A16.
 * Requires H % 32 == 0, I % 32 == 0, 1 <= k <= E, T >= 0.
 * Dropped pairs: a pair whose id lies outside 0..E-1 (a slot id of -1 from a
 * failed moe_expert_cache_plan, or a pair that another device's experts
 * serve) contributes nothing: y_t sums only the token's kept pairs (0 when
 * it has none), and in W4A4 g_h is taken over the kept pairs only.  The
 * offsets and sorted pairs must then come from moe_permute_pairs on the
 * same ids (it leaves dropped pairs out).
 * Pair order: expert_offsets and sorted_pairs may both be NULL where the
 * decode batch runs on the fused per-row kernels (W4A16, H = 2048,
 * I % 256 == 0, T*k <= 256, 2*T*k <= 32*E); each pair p then takes its expert
 * from topk_ids[p] directly, dropped ids included, and y is bit-identical to
 * the call with the permutation (the combine sums a token's pairs in j order
 * either way).  Elsewhere, or with one of the two NULL,
 * NVFP4_ERR_INVALID_ARGUMENT.
 * workspace: moe_grouped_nvfp4_ffn_workspace_size bytes (device, 16-byte
 * aligned), scratch only; its contents after the call are unspecified
 * except as moe_grouped_nvfp4_ffn_debug_h describes.
 */
nvfp4_status moe_grouped_nvfp4_ffn(const void *x, int64_t T, int64_t H,
                                   int64_t I, int32_t E, int32_t k,
                                   const int32_t *topk_ids,
                                   const float *topk_weights,
                                   const int32_t *expert_offsets,
                                   const int32_t *sorted_pairs,
                                   const nvfp4_expert_weights *w,
                                   nvfp4_act_mode act,
                                   nvfp4_global_mode act_global_mode,
                                   float *act_globals, void *y,
                                   nvfp4_dtype y_dtype, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);
size_t moe_grouped_nvfp4_ffn_workspace_size(int64_t T, int64_t H, int64_t I,
                                            int32_t E, int32_t k,
                                            nvfp4_act_mode act);

/*
 * moe_route_ffn_decode: the routing and the routed-expert FFN of a decode
 * batch in two launches instead of three.  Decode streams the routed
 * experts' weights once per step, so the step's time is that stream plus
 * whatever runs before it (Eider page, "Performance"; "Qwen3.8 Flash Next":
 * the 512 experts).  Computes exactly what moe_route_topk(logits, T, E, k,
 * renormalize) followed by moe_grouped_nvfp4_ffn(act W4A16) computes on the
 * same inputs: topk_ids, topk_weights, expert_offsets, sorted_pairs and y
 * are bit-identical to theirs.  Each workgroup of the fused FFN kernel takes
 * the top-k of its own token (the same merge network) before it streams
 * that pair's expert, so the stream does not wait for a routing launch; the
 * permutation is made by one more workgroup of the combine launch.
 * logits f32 [T, E]; x bf16 [T, H]; y [T, H] bf16 or f32; the other
 * outputs as moe_route_topk's.
 * Requires the fused decode shapes: H = 2048, I % 256 == 0, 1 <= k <= 8,
 * k <= E <= 512, T*k <= 256, 2*T*k <= 32*E (NVFP4_ERR_UNSUPPORTED_SHAPE
 * otherwise; use the two calls there).  T = 0 writes E + 1 zero offsets.
 * workspace: moe_route_ffn_decode_workspace_size bytes (device, 16-byte
 * aligned), scratch only (no state between calls).
 */
nvfp4_status moe_route_ffn_decode(const float *logits, const void *x, int64_t T, int64_t H,
                                  int64_t I, int32_t E, int32_t k, int renormalize,
                                  int32_t *topk_ids, float *topk_weights,
                                  int32_t *expert_offsets, int32_t *sorted_pairs,
                                  const nvfp4_expert_weights *w, void *y, nvfp4_dtype y_dtype,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);
size_t moe_route_ffn_decode_workspace_size(int64_t T, int64_t H, int64_t I, int32_t E,
                                           int32_t k);

/*
 * moe_grouped_nvfp4_ffn_static: moe_grouped_nvfp4_ffn without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops and harnesses that forbid hipMalloc.
 * Its scratch is a file-scope device array inside the library, one copy per
 * device (each device holds it, moe_grouped_nvfp4_ffn_static_max_bytes()
 * = 64 MiB, from the library's load until the process ends); the device
 * address of the current device's copy is looked up once per device on the
 * first call there.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine) and computes exactly what
 * moe_grouped_nvfp4_ffn computes with a workspace (bit-identical outputs).
 * Shapes whose moe_grouped_nvfp4_ffn_workspace_size exceeds the maximum
 * return NVFP4_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (the
 * routed decode and 512-token prefill shapes fit; a 2048-token W4A4 batch
 * with H = 4096 does not).  Every call on a device shares that device's
 * array and leaves its contents behind; the call clears what it needs
 * cleared itself.  Calls that may overlap on one device (several streams
 * or host threads) race on the array: serialise them.
 */
nvfp4_status moe_grouped_nvfp4_ffn_static(const void *x, int64_t T, int64_t H, int64_t I,
                                          int32_t E, int32_t k, const int32_t *topk_ids,
                                          const float *topk_weights,
                                          const int32_t *expert_offsets,
                                          const int32_t *sorted_pairs,
                                          const nvfp4_expert_weights *w, nvfp4_act_mode act,
                                          nvfp4_global_mode act_global_mode, float *act_globals,
                                          void *y, nvfp4_dtype y_dtype, hipStream_t stream);
size_t moe_grouped_nvfp4_ffn_static_max_bytes(void);

/*
 * moe_grouped_nvfp4_ffn_debug_h: a test aid (not part of the computation)
 * for checking h element by element where it decides an integer: its bf16
 * rounding and, in W4A4, its NVFP4 codes (Qwen3.8-Flash-Next-NVFP4-SSD-
 * Stream model card, "What this model is": W4A4 routed experts).  For a
 * moe_grouped_nvfp4_ffn call with these arguments, made on the calling
 * thread, *h_offset receives the byte offset in its workspace of h in bf16
 * and *hq_offset that of h's W4A4 operand (fp16 values e2m1 * e4m3 of the
 * quantised h, without g_h); both are [T*k, I] row-major with row pos
 * holding pair sorted_pairs[pos] (rows past the kept pairs are
 * unspecified).  Returns a bit mask of what the call leaves there: 1 = the
 * bf16 h, 2 = the W4A4 operand; 0 when the call keeps h elsewhere (the
 * decode row kernels).  Either pointer may be NULL.
 */
int moe_grouped_nvfp4_ffn_debug_h(int64_t T, int64_t H, int64_t I, int32_t E, int32_t k,
                                  nvfp4_act_mode act, nvfp4_global_mode act_global_mode,
                                  size_t *h_offset, size_t *hq_offset);

/*
 * Profiling aid (not part of the computation).  While a non-NULL array is
 * set, every moe_grouped_nvfp4_ffn call made on the calling thread records
 * events[2*s] on its stream just before stage s and events[2*s+1] just after
 * it, for the NVFP4_FFN_STAGES stages below; the caller creates the events
 * (hipEventCreate) and reads them with hipEventElapsedTime.  NULL disables
 * recording.  Nothing is recorded while the stream is being captured into a
 * graph.  The setting is per thread and holds no other state.
 */
enum {
  NVFP4_STAGE_PLAN = 0,     /* m-block list from the expert offsets              */
  NVFP4_STAGE_X_PREP = 1,   /* x -> fp16 operands (W4A4: amax + quantisation)    */
  NVFP4_STAGE_GATE_UP = 2,  /* grouped gate/up GEMM with the SiLU * up epilogue  */
  NVFP4_STAGE_H_PREP = 3,   /* h -> fp16 operands (W4A4: quantisation)           */
  NVFP4_STAGE_DOWN = 4,     /* grouped down GEMM times the routing weight        */
  NVFP4_STAGE_COMBINE = 5,  /* sum of each token's k pairs                       */
  NVFP4_FFN_STAGES = 6
};
void nvfp4_set_ffn_stage_events(hipEvent_t *events);

/*
 * Execution choice (not part of the computation).  With act W4A4 and GIVEN
 * globals, moe_grouped_nvfp4_ffn quantises h inside the gate/up GEMM's
 * epilogue wherever the tiled kernel computes a whole h row block without a
 * K split: the 16-element block maxima are reduced across lanes and h never
 * goes to memory in bf16.  nvfp4_set_ffn_separate_h_quant(1) makes later
 * calls on the calling thread write bf16 h and quantise it in a pass of its
 * own instead (0 restores the default).  Both orders compute the same h and
 * the same codes with the same fp32 operations, so their outputs are
 * bit-identical; the choice only changes the kernels that run.
 */
void nvfp4_set_ffn_separate_h_quant(int separate);

/*
 * Measurement aid (not part of the computation): a plain streaming read of
 * `bytes` (a positive multiple of 16) of device memory at buf, 16-byte
 * non-temporal loads, four in flight per thread, up to 8192 workgroups.
 * Its rate is the practical HBM read ceiling the decode kernels are
 * compared with, beside the 8 TB/s peak.  sink: >= 1024 device words,
 * written only in the (data-dependent, practically never met) case that
 * keeps the loads from being optimised away.
 */
nvfp4_status nvfp4_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Text of a status code; never NULL. */
const char *nvfp4_status_string(nvfp4_status s);
/* Detail of the last failure on the calling thread ("" if none). */
const char *nvfp4_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4MOE_H */

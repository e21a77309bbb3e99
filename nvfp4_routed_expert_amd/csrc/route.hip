// Top-k routing and the expert-sorted pair permutation.
//
// The Flash-Next model routes every token to a few of its 512 MoE experts
// (Eider page, "Qwen3.8 Flash Next"); the grouped expert kernels need the
// (token, slot) pairs grouped by expert.  Both steps are integer-exact:
// selection compares the fp32 logits (ties to the lower expert index) and
// the permutation is a stable counting sort whose ranks come from per-expert
// token bitmaps and population counts, so no atomic ordering can leak into
// the result.
#include "common.h"
#include "kernels.h"

namespace nvfp4 {
namespace {

constexpr int kMaxExperts = 1024;
constexpr int kMaxPerLane = kMaxExperts / kWave;  // 16 logits per lane
constexpr int kTopkThreads = 256;

// a beats b: larger logit, or equal logit and lower index (branch-free)
__device__ __forceinline__ bool beats(float av, int ai, float bv, int bi) {
  return (av > bv) | ((av == bv) & (ai < bi));
}

// Takes the partner lane's (value, index) when it beats this lane's.  Lanes
// of rows outside ROW_MASK keep theirs.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_best(float &v, int &i) {
  const float ov = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      __builtin_bit_cast(int, v), __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROW_MASK, 0xF, false);
  const bool t = beats(ov, oi, v, i);
  v = t ? ov : v;
  i = t ? oi : i;
}

// Wave-wide best (value, index) with DPP: within rows of 16 lanes, then
// row_bcast15 / row_bcast31 carry the row winners up to lane 63, whose result
// is broadcast.  Every lane gets the result.
__device__ __forceinline__ void wave_best(float &v, int &i) {
  dpp_best<0xB1, 0xF>(v, i);    // lane ^ 1
  dpp_best<0x4E, 0xF>(v, i);    // lane ^ 2
  dpp_best<0x141, 0xF>(v, i);   // the other quad of 8
  dpp_best<0x140, 0xF>(v, i);   // the other 8 of 16
  dpp_best<0x142, 0xA>(v, i);   // rows 1, 3 take lane 15 of the row below
  dpp_best<0x143, 0xC>(v, i);   // rows 2, 3 take lane 31
  v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

// Top-k of one token's logits by one wavefront.  Lane l holds logits
// l, l+64, ...; k rounds of a wave-wide argmax pick the experts in
// descending order.  Lane j < k writes the j-th id and weight.
__device__ void wave_topk(const float *row, int E, int k, int renormalize, int32_t *ids,
                          float *weights, int32_t *ids_copy) {
  const int lane = threadIdx.x & 63;
  float v[kMaxPerLane];
  const int per_lane = (E + 63) / 64;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = (i < per_lane && e < E) ? row[e] : 0.0f;
  }
  uint32_t taken = 0;
  float my_val = 0.0f;   // lane j < k keeps the j-th selected logit
  int my_idx = 0;
  for (int r = 0; r < k; ++r) {
    // this lane's best untaken candidate; indices rise with i, so a strict
    // comparison keeps the lower index on ties (branch-free selects)
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      const bool ok = (i < per_lane) & (e < E) & !((taken >> i) & 1u) & (v[i] > bv);
      bv = ok ? v[i] : bv;
      bi = ok ? e : bi;
    }
    wave_best(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == r) { my_val = bv; my_idx = bi; }
  }
  const float lmax = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_val), 0));
  const float ex = lane < k ? expf(my_val - lmax) : 0.0f;
  float denom;
  if (renormalize) {
    denom = wave_sum(ex);
  } else {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (i < per_lane && e < E) s += expf(v[i] - lmax);
    }
    denom = wave_sum(s);
  }
  if (lane < k) {
    ids[lane] = my_idx;
    weights[lane] = ex / denom;
    if (ids_copy) ids_copy[lane] = my_idx;
  }
}

// One wavefront per token.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float *logits, int64_t T, int E, int k, int renormalize, int32_t *ids,
    float *weights) {
  const int64_t t = (int64_t)blockIdx.x * (kTopkThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  wave_topk(logits + t * E, E, k, renormalize, ids + t * k, weights + t * k, nullptr);
}

// Single workgroup.  Pass 1 counts pairs per expert and writes the offsets.
// Pass 2 walks tokens in chunks: a bitmap per expert marks the chunk's tokens
// routed to it; the rank of pair (t, j) inside its expert is the number of
// earlier tokens of that expert = tokens in earlier chunks + set bits before t.
constexpr int kPermThreads = 1024;
constexpr int kBitmapWords = 16384;   // experts * words-per-expert per chunk

struct PermuteLds {
  uint32_t bitmap[kBitmapWords];
  uint16_t prefix[kBitmapWords];
  int32_t cnt[kMaxExperts];
  int32_t off[kMaxExperts];
  int32_t base[kMaxExperts];
  int32_t chunk_cnt[kMaxExperts];
  int32_t wave_tot[kPermThreads / 64];
};

// ids: the [T, k] expert ids (global or LDS).  One workgroup of any
// multiple of 64 threads up to kPermThreads.
__device__ void permute_block(const int32_t *ids, int64_t T, int E, int k, int W,
                              int32_t *offsets, int32_t *sorted_pairs, PermuteLds &L) {
  uint32_t *bitmap = L.bitmap;
  uint16_t *prefix = L.prefix;
  int32_t *cnt = L.cnt, *off = L.off, *base = L.base, *chunk_cnt = L.chunk_cnt;
  int32_t *wave_tot = L.wave_tot;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int64_t P = T * k;

  for (int e = tid; e < E; e += nthr) { cnt[e] = 0; base[e] = 0; }
  __syncthreads();
  for (int64_t p = tid; p < P; p += nthr) atomicAdd(&cnt[ids[p]], 1);
  __syncthreads();

  // exclusive scan of cnt over E <= 1024 experts: thread tid owns the ept
  // consecutive experts tid * ept ..
  {
    const int ept = (E + nthr - 1) / nthr;
    const int e0 = tid * ept;
    int c = 0;
    for (int i = 0; i < ept; ++i)
      if (e0 + i < E) c += cnt[e0 + i];
    int incl = c;
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int run = incl - c;
    for (int w = 0; w < wave; ++w) run += wave_tot[w];
    for (int i = 0; i < ept; ++i) {
      const int e = e0 + i;
      if (e < E) {
        off[e] = run;
        offsets[e] = run;
        run += cnt[e];
      }
    }
    if (tid == 0) offsets[E] = (int32_t)P;
  }
  __syncthreads();

  const int64_t chunk_tokens = (int64_t)W * 32;
  for (int64_t t0 = 0; t0 < T; t0 += chunk_tokens) {
    const int64_t t1 = t0 + chunk_tokens < T ? t0 + chunk_tokens : T;
    for (int i = tid; i < E * W; i += nthr) bitmap[i] = 0u;
    __syncthreads();
    for (int64_t p = t0 * k + tid; p < t1 * k; p += nthr) {
      const int64_t tl = p / k - t0;
      atomicOr(&bitmap[ids[p] * W + (int)(tl >> 5)], 1u << (tl & 31));
    }
    __syncthreads();
    for (int e = tid; e < E; e += nthr) {
      int run = 0;
      for (int w = 0; w < W; ++w) {
        prefix[e * W + w] = (uint16_t)run;
        run += __popc(bitmap[e * W + w]);
      }
      chunk_cnt[e] = run;
    }
    __syncthreads();
    for (int64_t p = t0 * k + tid; p < t1 * k; p += nthr) {
      const int e = ids[p];
      const int64_t tl = p / k - t0;
      const int w = (int)(tl >> 5);
      const uint32_t below = bitmap[e * W + w] & ((1u << (tl & 31)) - 1u);
      const int rank = base[e] + prefix[e * W + w] + __popc(below);
      sorted_pairs[off[e] + rank] = (int32_t)p;
    }
    __syncthreads();
    for (int e = tid; e < E; e += nthr) base[e] += chunk_cnt[e];
    __syncthreads();
  }
}


__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t *ids, int64_t T, int E, int k, int W, int32_t *offsets,
    int32_t *sorted_pairs) {
  __shared__ PermuteLds L;
  permute_block(ids, T, E, k, W, offsets, sorted_pairs, L);
}

int permute_words(int64_t T, int E) {
  // words per expert per chunk: E * W <= kBitmapWords, and W * 32 tokens
  // per chunk keep every per-word prefix below 2^16
  int W = kBitmapWords / E;
  if (W > 2048) W = 2048;
  const int64_t need = (T + 31) / 32;
  if (W > need) W = (int)need;
  if (W < 1) W = 1;
  return W;
}

}  // namespace

hipError_t launch_route(const float *logits, int64_t T, int E, int k, int renormalize,
                        int32_t *ids, float *weights, int32_t *offsets, int32_t *sorted_pairs,
                        hipStream_t s) {
  // top-k: one wavefront per token, four per workgroup, so a decode batch
  // spreads over several CUs (one wave per SIMD) instead of sharing one
  const int W = permute_words(T, E);
  const int64_t blocks = (T + 3) / 4;
  launch_kernel(topk_kernel, dim3((unsigned)blocks), dim3(kTopkThreads), 0, s, logits, T, E, k,
                renormalize, ids, weights);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // permutation: one workgroup, small for decode-sized batches (fewer
  // waves make its barriers cheaper)
  const int threads = T * k <= 1024 ? 256 : kPermThreads;
  launch_kernel(permute_kernel, dim3(1), dim3(threads), 0, s, ids, T, E, k, W, offsets,
                sorted_pairs);
  return hipGetLastError();
}

}  // namespace nvfp4

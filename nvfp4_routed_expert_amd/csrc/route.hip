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

// a beats b: larger logit, or equal logit and lower index
__device__ __forceinline__ bool beats(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// One wavefront per token.  Lane l holds logits l, l+64, ...; k rounds of a
// wave-wide argmax pick the experts in descending order.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float *logits, int64_t T, int E, int k, int renormalize, int32_t *ids,
    float *weights) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (kTopkThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *row = logits + t * E;
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
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (i < per_lane && e < E && !((taken >> i) & 1u) && beats(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (beats(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == r) { my_val = bv; my_idx = bi; }
  }
  const float lmax = __shfl(my_val, 0, kWave);
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
    ids[t * k + lane] = my_idx;
    weights[t * k + lane] = ex / denom;
  }
}

// Single workgroup.  Pass 1 counts pairs per expert and writes the offsets.
// Pass 2 walks tokens in chunks: a bitmap per expert marks the chunk's tokens
// routed to it; the rank of pair (t, j) inside its expert is the number of
// earlier tokens of that expert = tokens in earlier chunks + set bits before t.
constexpr int kPermThreads = 1024;
constexpr int kBitmapWords = 16384;   // experts * words-per-expert per chunk

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t *ids, int64_t T, int E, int k, int W, int32_t *offsets,
    int32_t *sorted_pairs) {
  __shared__ uint32_t bitmap[kBitmapWords];
  __shared__ uint16_t prefix[kBitmapWords];
  __shared__ int32_t cnt[kMaxExperts];
  __shared__ int32_t off[kMaxExperts];
  __shared__ int32_t base[kMaxExperts];
  __shared__ int32_t chunk_cnt[kMaxExperts];
  __shared__ int32_t wave_tot[kPermThreads / 64];
  const int tid = threadIdx.x;
  const int64_t P = T * k;

  for (int e = tid; e < E; e += kPermThreads) { cnt[e] = 0; base[e] = 0; }
  __syncthreads();
  for (int64_t p = tid; p < P; p += kPermThreads) atomicAdd(&cnt[ids[p]], 1);
  __syncthreads();

  // exclusive scan of cnt over E <= 1024 experts (one per thread)
  {
    const int c = tid < E ? cnt[tid] : 0;
    int incl = c;
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wave_tot[w];
    if (tid < E) {
      off[tid] = wbase + incl - c;
      offsets[tid] = wbase + incl - c;
    }
    if (tid == 0) offsets[E] = (int32_t)P;
  }
  __syncthreads();

  const int64_t chunk_tokens = (int64_t)W * 32;
  for (int64_t t0 = 0; t0 < T; t0 += chunk_tokens) {
    const int64_t t1 = t0 + chunk_tokens < T ? t0 + chunk_tokens : T;
    for (int i = tid; i < E * W; i += kPermThreads) bitmap[i] = 0u;
    __syncthreads();
    for (int64_t p = t0 * k + tid; p < t1 * k; p += kPermThreads) {
      const int64_t tl = p / k - t0;
      atomicOr(&bitmap[ids[p] * W + (int)(tl >> 5)], 1u << (tl & 31));
    }
    __syncthreads();
    for (int e = tid; e < E; e += kPermThreads) {
      int run = 0;
      for (int w = 0; w < W; ++w) {
        prefix[e * W + w] = (uint16_t)run;
        run += __popc(bitmap[e * W + w]);
      }
      chunk_cnt[e] = run;
    }
    __syncthreads();
    for (int64_t p = t0 * k + tid; p < t1 * k; p += kPermThreads) {
      const int e = ids[p];
      const int64_t tl = p / k - t0;
      const int w = (int)(tl >> 5);
      const uint32_t below = bitmap[e * W + w] & ((1u << (tl & 31)) - 1u);
      const int rank = base[e] + prefix[e * W + w] + __popc(below);
      sorted_pairs[off[e] + rank] = (int32_t)p;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kPermThreads) base[e] += chunk_cnt[e];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_route_topk(const float *logits, int64_t T, int E, int k,
                             int renormalize, int32_t *ids, float *weights,
                             hipStream_t s) {
  const int64_t blocks = (T + 3) / 4;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)blocks), dim3(kTopkThreads), 0, s,
                     logits, T, E, k, renormalize, ids, weights);
  return hipGetLastError();
}

hipError_t launch_route_permute(const int32_t *ids, int64_t T, int E, int k,
                                int32_t *offsets, int32_t *sorted_pairs,
                                hipStream_t s) {
  // words per expert per chunk: E * W <= kBitmapWords, and W * 32 tokens
  // per chunk keep every per-word prefix below 2^16
  int W = kBitmapWords / E;
  if (W > 2048) W = 2048;
  const int64_t need = (T + 31) / 32;
  if (W > need) W = (int)need;
  if (W < 1) W = 1;
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, s, ids, T, E, k, W,
                     offsets, sorted_pairs);
  return hipGetLastError();
}

}  // namespace nvfp4
